/*
 * oracle_permute.c -- the plain, slow CPU oracle for permute_layout.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or
 * load this file or the library built from it; only the tests, the smoke
 * check and the benchmark's CPU-baseline leg do.  It shares no code, header,
 * table or helper with the HIP library: it is a second, independent statement
 * of what the operation computes.
 *
 * What it computes (the definition, written out):
 *
 *   Buffers and memory page, "Declaring buffers": a buffer is a pointer plus a
 *   layout, and an element's address is the data pointer plus the element
 *   offset plus the layout's offset of the coordinate; a shape:stride layout
 *   maps coordinate c to sum_i c_i * stride_i, in elements.
 *
 *   permute_layout page, intro and "Algorithm" step 3: every element of the
 *   region is read through the source layout and written back through the
 *   destination layout.  The XOR swizzle of step 2 only reorders the accesses
 *   (each register is written and read back at the same iteration), so the
 *   value that lands at every destination address is the value read from the
 *   source address of the same logical coordinate.  The warp-sync between the
 *   two phases makes the result that of reading everything before writing
 *   anything, also when source and destination alias.
 *
 * So, for every batch index b and every coordinate c (row-major odometer):
 *
 *   so = off_src + b * span_src + sum_i c_i * src_stride_i
 *   do = off_dst + b * span_dst + sum_i c_i * dst_stride_i
 *   dst bytes [do*w, do*w + w)  :=  src bytes [so*w, so*w + w)
 *
 * where span_x = 1 + sum_i (extent_i - 1) * stride_x_i is the side's cosize
 * (a "contiguous batch": batch item b starts right after item b-1 ends).
 * Bytes are copied verbatim; nothing is interpreted as a number, so NaN
 * payloads, signed zeros and denormals pass through unchanged.
 *
 * The source is snapshotted first when its byte range overlaps the
 * destination's, which gives the read-all-then-write-all result.
 *
 * Swizzled operands (oracle_permute_swizzled).  The pages allocate
 * MMA-compatible tiles whose layout is a plain layout composed with an XOR
 * swizzle (buffers page, "Pool sugar", alloc_mma) and exclude such operands
 * from permute_layout ("What it accepts": no swizzle wrapper); they do not
 * spell the function out.  Here a swizzle is the usual XOR function of the
 * layout offset, given by three numbers (bits, base, shift):
 *
 *   swz(m) = m XOR (((m >> (base + shift)) mod 2^bits) << base)
 *
 * i.e. the `bits`-bit field of m starting at bit base + shift is XORed into
 * the field starting at bit base; with shift >= bits the two fields are
 * disjoint, so swz is its own inverse.  bits = 0 is the plain layout.  It
 * acts on the side's layout offset with the batch as an outermost mode,
 * before the element offset is added:
 *
 *   so = off_src + swz_src(b * span_src + sum_i c_i * src_stride_i)
 *
 * (when span is a multiple of 2^(base + shift + bits), this equals
 * swizzling each batch item's offsets on their own).
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum {
    ORACLE_OK = 0,
    ORACLE_E_ARG = 1,      /* null pointer, bad rank, bad width, negative extent/batch */
    ORACLE_E_RANGE = 2,    /* some access falls outside the given buffer length */
    ORACLE_E_NOMEM = 3
};

/* permute_layout page, "What it accepts": widths 1, 2, 4, 8 and 16 bytes. */
static int width_ok(int w)
{
    return w == 1 || w == 2 || w == 4 || w == 8 || w == 16;
}

/* Cosize of one side: 1 + sum (e_i - 1) * s_i  (0 when any extent is 0). */
static int64_t cosize(int rank, const int64_t *ext, const int64_t *str)
{
    int64_t span = 1;
    for (int i = 0; i < rank; ++i) {
        if (ext[i] == 0)
            return 0;
        span += (ext[i] - 1) * str[i];
    }
    return span;
}

/* Buffers and memory page, "Declaring buffers": offset of a coordinate. */
static int64_t layout_apply(int rank, const int64_t *coord, const int64_t *str)
{
    int64_t m = 0;
    for (int i = 0; i < rank; ++i)
        m += coord[i] * str[i];
    return m;
}

/* A swizzle descriptor {bits, base, shift}; NULL or bits == 0 is none. */
static int swizzle_ok(const int32_t *z)
{
    if (!z || z[0] == 0)
        return 1;
    return z[0] > 0 && z[0] <= 16 && z[1] >= 0 && z[2] >= z[0] && z[1] + z[2] + z[0] <= 48;
}

static int64_t swizzle(const int32_t *z, int64_t m)
{
    if (!z || z[0] == 0)
        return m;
    const int64_t field = (m >> (z[1] + z[2])) & (((int64_t)1 << z[0]) - 1);
    return m ^ (field << z[1]);
}

/*
 * src_len / dst_len are the buffer lengths in bytes; every access is checked
 * against them before anything is written.  Returns ORACLE_OK or an error.
 */
int oracle_permute_swizzled(const void *src, int64_t src_len, void *dst, int64_t dst_len,
                            int w, int rank, const int64_t *extents,
                            const int64_t *src_strides, const int64_t *dst_strides,
                            const int64_t *elem_offsets, int64_t batch,
                            const int32_t *src_swz, const int32_t *dst_swz)
{
    if (!src || !dst || !extents || !src_strides || !dst_strides || !elem_offsets)
        return ORACLE_E_ARG;
    if (!width_ok(w) || rank < 1 || rank > 16 || batch < 0)
        return ORACLE_E_ARG;
    if (!swizzle_ok(src_swz) || !swizzle_ok(dst_swz))
        return ORACLE_E_ARG;
    int64_t n = batch;
    for (int i = 0; i < rank; ++i) {
        if (extents[i] < 0)
            return ORACLE_E_ARG;
        n *= extents[i];
    }
    if (n == 0)
        return ORACLE_OK;

    const int64_t span_s = cosize(rank, extents, src_strides);
    const int64_t span_d = cosize(rank, extents, dst_strides);
    int64_t coord[16];

    /* Pass 1: check every source and destination access is in range. */
    for (int64_t b = 0; b < batch; ++b) {
        memset(coord, 0, sizeof coord);
        for (;;) {
            int64_t so = elem_offsets[0] + swizzle(src_swz, b * span_s + layout_apply(rank, coord, src_strides));
            int64_t d_o = elem_offsets[1] + swizzle(dst_swz, b * span_d + layout_apply(rank, coord, dst_strides));
            if (so < 0 || (so + 1) * w > src_len || d_o < 0 || (d_o + 1) * w > dst_len)
                return ORACLE_E_RANGE;
            int i = rank - 1;
            while (i >= 0 && ++coord[i] == extents[i]) {
                coord[i] = 0;
                --i;
            }
            if (i < 0)
                break;
        }
    }

    /* Snapshot the source when the two byte ranges overlap. */
    const uint8_t *s = (const uint8_t *)src;
    uint8_t *copy = NULL;
    uintptr_t s0 = (uintptr_t)src, s1 = s0 + (uintptr_t)src_len;
    uintptr_t d0 = (uintptr_t)dst, d1 = d0 + (uintptr_t)dst_len;
    if (s0 < d1 && d0 < s1) {
        copy = (uint8_t *)malloc((size_t)src_len);
        if (!copy)
            return ORACLE_E_NOMEM;
        memcpy(copy, src, (size_t)src_len);
        s = copy;
    }

    /* Pass 2: the copy itself, one element at a time. */
    uint8_t *d = (uint8_t *)dst;
    for (int64_t b = 0; b < batch; ++b) {
        memset(coord, 0, sizeof coord);
        for (;;) {
            int64_t so = elem_offsets[0] + swizzle(src_swz, b * span_s + layout_apply(rank, coord, src_strides));
            int64_t d_o = elem_offsets[1] + swizzle(dst_swz, b * span_d + layout_apply(rank, coord, dst_strides));
            memcpy(d + d_o * w, s + so * w, (size_t)w);
            int i = rank - 1;
            while (i >= 0 && ++coord[i] == extents[i]) {
                coord[i] = 0;
                --i;
            }
            if (i < 0)
                break;
        }
    }
    free(copy);
    return ORACLE_OK;
}

int oracle_permute(const void *src, int64_t src_len, void *dst, int64_t dst_len,
                   int w, int rank, const int64_t *extents,
                   const int64_t *src_strides, const int64_t *dst_strides,
                   const int64_t *elem_offsets, int64_t batch)
{
    return oracle_permute_swizzled(src, src_len, dst, dst_len, w, rank, extents, src_strides,
                                   dst_strides, elem_offsets, batch, NULL, NULL);
}

/* The swizzle of one layout offset, exported so tests can pin it. */
int64_t oracle_swizzle(int32_t bits, int32_t base, int32_t shift, int64_t m)
{
    const int32_t z[3] = {bits, base, shift};
    return swizzle(z, m);
}

/* Element offset of one coordinate, exported so tests can pin the address
 * rule against the worked address examples of the buffers page. */
int64_t oracle_address(int rank, const int64_t *coord, const int64_t *strides,
                       int64_t elem_offset)
{
    return elem_offset + layout_apply(rank, coord, strides);
}
