"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module only makes bytes; it holds none of the permutation's arithmetic.

Byte stream: the little-endian concatenation of the 64-bit words
``splitmix64(seed ^ (j * 0x9E3779B97F4A7C15))`` for j = 0, 1, 2, ...,
truncated to the requested length.  splitmix64 is Vigna's published mixer
(add the golden-ratio increment, then two xor-shift-multiply rounds and a
final xor-shift).  The stream does not depend on the element width, the
chunking or the thread count.
"""

from __future__ import annotations

import numpy as np

GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)

# fp32 encodings forced into the scale-factor workload: +-Inf, quiet NaNs
# (one with a payload), signalling NaNs, denormals, -0 and +0.
F32_SPECIALS = np.array(
    [0x7F800000, 0xFF800000, 0x7FC00000, 0xFFC00000, 0x7FC00001, 0x7F800001,
     0x7FBFFFFF, 0x00000001, 0x007FFFFF, 0x80000001, 0x80000000, 0x00000000],
    dtype=np.uint32,
)


def splitmix64(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = x + GOLDEN
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def random_bytes(seed: int, nbytes: int, chunk_words: int = 1 << 22) -> np.ndarray:
    """``nbytes`` bytes of the seeded stream, as a uint8 array."""
    nwords = (nbytes + 7) // 8
    out = np.empty(nwords, dtype=np.uint64)
    s = np.uint64(seed & 0xFFFFFFFFFFFFFFFF)
    for j0 in range(0, nwords, chunk_words):
        j = np.arange(j0, min(nwords, j0 + chunk_words), dtype=np.uint64)
        with np.errstate(over="ignore"):
            out[j0:j0 + len(j)] = splitmix64(s ^ (j * GOLDEN))
    return out.view(np.uint8)[:nbytes]


def inject_f32_specials(words: np.ndarray, seed: int, rate_log2: int = 6,
                        chunk: int = 1 << 22) -> np.ndarray:
    """Overwrite element i of a uint32 array when splitmix64(seed ^ i) % 2**rate_log2 == 0.

    The replacement is ``F32_SPECIALS[i % 12]``.  Works in place; returns ``words``.
    """
    assert words.dtype == np.uint32
    s = np.uint64(seed & 0xFFFFFFFFFFFFFFFF)
    m = np.uint64((1 << rate_log2) - 1)
    for i0 in range(0, words.size, chunk):
        i = np.arange(i0, min(words.size, i0 + chunk), dtype=np.uint64)
        hit = (splitmix64(s ^ i) & m) == 0
        idx = i[hit]
        words[idx.astype(np.int64)] = F32_SPECIALS[(idx % np.uint64(len(F32_SPECIALS))).astype(np.int64)]
    return words
