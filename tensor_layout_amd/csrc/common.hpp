// common.hpp -- types shared by the host planner and the gfx950 kernels.
//
// Everything here is plain data plus small __host__ __device__ index helpers.
// The lane -> LDS address maps of the tiled kernel live here so that the
// planner's bank simulation runs exactly the addresses the kernel issues.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#include <hip/hip_runtime.h>
#define TPL_HD __host__ __device__ __forceinline__
#else
#define TPL_HD inline
#endif

namespace tpl {

constexpr int kMaxShard = 10;   // shard modes (8 user modes + batch + slack)
constexpr int kMaxBatch = 10;   // modes a kernel decomposes (at most the whole shard)
constexpr int kWave = 64;       // gfx950 wavefront

// Division by an invariant 31-bit integer with a multiply and a shift
// (Granlund & Montgomery, "Division by invariant integers using
// multiplication", 1994, round-up variant): for 0 <= n < 2^31 and
// 1 <= d < 2^31, n / d = (umulhi(n, m) + n) >> s with s = ceil(log2 d) and
// m = floor(2^32 * (2^s - d) / d) + 1.
struct FastDiv {
    uint32_t d, m, s;
};

inline FastDiv make_fastdiv(uint32_t d) {
    FastDiv f;
    f.d = d;
    uint32_t s = 0;
    while ((1ull << s) < d) ++s;
    f.s = s;
    f.m = (uint32_t)((((1ull << s) - d) << 32) / d + 1);
    return f;
}

TPL_HD uint32_t fdiv(uint32_t n, const FastDiv& f) {
#if defined(__HIP_DEVICE_COMPILE__)
    uint32_t hi = __umulhi(n, f.m);
#else
    uint32_t hi = (uint32_t)(((uint64_t)n * f.m) >> 32);
#endif
    return (hi + n) >> f.s;
}

// Row-major decomposition of a linear index over up to kMaxBatch modes,
// returning the source and destination element offsets of that index.
struct Modes {
    int n;
    FastDiv div[kMaxBatch];   // extents, innermost last
    int64_t ext[kMaxBatch];
    int64_t ss[kMaxBatch];    // source strides (elements)
    int64_t ds[kMaxBatch];    // destination strides (elements)
};

template <bool BIG>
TPL_HD void modes_step(const Modes& m, int i, int64_t& idx, int64_t& so, int64_t& d_o) {
    int64_t q, r;
    if (BIG) {
        q = idx / m.ext[i];
        r = idx - q * m.ext[i];
    } else {
        uint32_t qq = fdiv((uint32_t)idx, m.div[i]);
        r = (int64_t)((uint32_t)idx - qq * m.div[i].d);
        q = qq;
    }
    so += r * m.ss[i];
    d_o += r * m.ds[i];
    idx = q;
}

// NB >= 0: the kernel was built for exactly NB modes, so the loop unrolls and
// the mode table is read once; NB < 0: m.n modes, decided at run time.
template <int NB, bool BIG>
TPL_HD void modes_offsets(const Modes& m, int64_t idx, int64_t& so, int64_t& d_o) {
    so = 0;
    d_o = 0;
    if constexpr (NB >= 0) {
#pragma unroll
        for (int i = NB - 1; i >= 0; --i) modes_step<BIG>(m, i, idx, so, d_o);
    } else {
        for (int i = m.n - 1; i >= 0; --i) modes_step<BIG>(m, i, idx, so, d_o);
    }
}

// Kernels are built for 0, 1 and 2 batch modes and for any count.
inline int nb_class(int n) { return n <= 2 ? n : -1; }

// ---------------------------------------------------------------------------
// XOR swizzle of an operand, on byte offsets from the operand's base (the
// element swizzle (bits, base, shift) of width-w elements is the byte swizzle
// (bits, base + log2 w, shift)): P -> P ^ ((P >> shift) & ymask), with ymask
// = (2^bits - 1) << (base + log2 w).  ymask == 0: plain layout.  Offsets
// below 2^(base + log2 w) apart inside one aligned granule stay adjacent.
struct Swz {
    int64_t ymask;
    int32_t shift;
    int32_t pad;
};

TPL_HD int64_t swz_apply(const Swz& z, int64_t p) { return p ^ ((p >> z.shift) & z.ymask); }

// ---------------------------------------------------------------------------
// Kernel argument blocks (passed by value).

struct GatherArgs {
    const uint8_t* src;
    uint8_t* dst;
    int64_t total;   // elements
    Modes modes;     // the whole shard
    int unit;        // bytes moved per access (divides the element width)
    int w;
    Swz zs, zd;          // operand swizzles (byte form)
};

struct CopyArgs {
    const uint8_t* src;
    uint8_t* dst;
    int64_t nchunks;     // vectors overall
    FastDiv div_cpr;     // vectors per run
    int64_t cpr;
    Modes rows;          // the modes outside the contiguous run
    int w;
    int vec;             // vector bytes: 16, 8 or 4
    Swz zs, zd;          // operand swizzles (byte form)
};

struct QuadArgs {
    const uint8_t* src;
    uint8_t* dst;
    int64_t nunits;      // work units overall (4x32 blocks when wide, else 4x4 blocks)
    FastDiv div_upr;     // units per batch item
    int64_t upr;
    int64_t s_b;         // source stride of the 4-row mode (elements)
    int64_t d_a;         // destination stride of the contiguous-source mode (elements)
    int32_t wide;        // 1: 4 rows x 8 chunks per half-wave, lane-ordered 128-byte row loads
    int32_t split;       // 1: sub-dword columns stored one by one (not adjacent in the destination)
    Modes batch;
    Swz zs, zd;          // operand swizzles (byte form)
};

// Element tiles (TB x TA elements of w bytes), in two forms.
//
// Element form (swizzled operands): one element per access; the LDS row
// pitch is the row plus one element of at least 4 bytes, an odd number of
// such units, so that the lanes of a column read (neighbouring rows) hit
// distinct banks.
//
// Vector form (plain operands, w <= 4): each source row piece is read as the
// 16-byte aligned chunks that cover it, at most TA w / 16 + 1, and kept in
// LDS as read: row bb starts at vrow(bb) = bb rp + sk (bb >> le), and its
// element aa sits lead(bb) + aa w bytes further, lead(bb) being the row
// piece's address mod 16.  Destination row pieces are written as aligned
// 16-byte chunks, element by element only in a chunk the piece covers in
// part.  rp, sk and le are chosen on the measured gfx950 bank geometry so
// that neither the chunk writes (pieces of g bytes: b128, b64 pairs or b32)
// nor the element reads of a destination chunk (16 / w rows of one column
// per lane) meet a bank conflict.
struct EtileShape {
    int w, tb, ta;
    int rp, sk, le, g;   // vector form: LDS row pitch, skew bytes per 2^le rows, write piece
    constexpr TPL_HD int unit() const { return w < 4 ? 4 : w; }
    constexpr TPL_HD int pitch() const { return ta * w + unit(); }
    constexpr TPL_HD int vrow(int bb) const { return bb * rp + sk * (bb >> le); }
    // rows: TB and up to 16 / w - 1 more (destination rows not on 16 bytes)
    constexpr TPL_HD int vbytes() const { return vrow(tb + 16 / w - 1); }
};

// One shape per width: TA elements of a source row make 128 or 256 bytes, TB
// of a destination row 128 to 1024; 16 KiB per tile; TA and TB divide the
// 256 threads of a workgroup.  8- and 16-byte elements take the element
// form only (an 8-byte element per lane measured as fast as or faster than
// 16-byte chunks with their realignment).
constexpr EtileShape kEtileShapes[5] = {
    {1, 128, 128, 144, 16, 4, 16},
    {2, 128, 64, 152, 8, 3, 8},
    {4, 128, 32, 148, 4, 2, 4},
    {8, 64, 32, 0, 0, 0, 0},
    {16, 64, 16, 0, 0, 0, 0},
};
constexpr TPL_HD int etile_index(int w) { return w == 1 ? 0 : w == 2 ? 1 : w == 4 ? 2 : w == 8 ? 3 : 4; }

// Tall vector-form tiles: twice the rows, so destination row pieces of 256
// bytes (u8) and 512 bytes (bf16), and half the extra rows per tile that
// unaligned destination rows need.  The placement constants were searched
// on the same CPU model of the gfx950 passes.  bf16 writes LDS in 4-byte
// pieces: with 8- or 16-byte pieces the row pitch and skew are multiples of
// 8 bytes, and the 32 rows one column's half-wave reads then fall on 16
// banks.  The search found no conflict-free tall placement for 4-byte
// elements (256 x 32).
constexpr EtileShape kEtileTall[2] = {
    {1, 256, 128, 152, 8, 4, 8},
    {2, 256, 64, 148, 4, 3, 4},
};
constexpr TPL_HD EtileShape etile_vshape(int w, bool tall) {
    return tall && w <= 2 ? kEtileTall[w - 1] : kEtileShapes[etile_index(w)];
}

// In-place pair swaps walk tile pairs in blocks of kSwapG x kSwapG tiles.
constexpr int kSwapLogG = 3;
constexpr int kSwapG = 1 << kSwapLogG;

struct LdsArgs {
    const uint8_t* src;
    uint8_t* dst;
    int64_t e_b, e_a;    // b: destination-contiguous mode, a: source-contiguous mode
    int64_t s_b, d_a;    // the two non-unit strides (elements)
    int64_t ntiles;
    int64_t ntb, nta;
    FastDiv div_nta, div_ntb;
    Modes batch;
    int32_t pitch;       // LDS row pitch, bytes
    int32_t shift_r, mask_r, shift_w, mask_w;
    // In-place pair swaps only: work units per batch item, blocks of
    // kSwapG x kSwapG tiles per side, and whether every tile goes element by
    // element (bases or pitches not 16-byte aligned).
    int64_t npair;
    FastDiv div_npair;
    int64_t nbl;
    FastDiv div_nbl;
    int32_t scalar;
    // Element tiles only: 0 for the element form; the vector form (16-byte
    // chunks kept in LDS as read) 1 with every destination row on 16 bytes,
    // 2 with destination rows whose tile ranges shift to 16-byte boundaries.
    int32_t vform;
    Swz zs, zd;          // operand swizzles (byte form)
};

// Records kernel: a tile of TR consecutive records of F fields each, the
// dense side (whole records one after the other) moved as one contiguous
// block, the other side one row per field.
struct RecArgs {
    const uint8_t* src;
    uint8_t* dst;
    int64_t nrec;        // records per batch item
    int64_t ntr;         // tiles per batch item
    FastDiv div_ntr;
    int64_t ntiles;      // tiles overall
    int64_t fstride;     // field stride on the sparse side (elements)
    int32_t F;           // fields per record
    int32_t TR;          // records per full tile (a multiple of 16 / w)
    Modes batch;
};

struct Reg16Args {
    const uint8_t* src;
    uint8_t* dst;
    int64_t e_b, e_a, s_b, d_a;
    int64_t nblocks;     // 8x8 element blocks overall
    int64_t nbb, nba;
    FastDiv div_nba, div_nbb;
    Modes batch;
};

// ---------------------------------------------------------------------------
// Tiled LDS kernel geometry: one workgroup moves one TB x TA tile
// (TB along the destination-contiguous mode b, TA along the
// source-contiguous mode a).  NT = tile_bytes / (16 * cpt) threads, each
// thread loading cpt 16-byte chunks.  The read phase gathers, per lane, one
// 16-byte destination chunk: 4*g dwords (w <= 4, g elements per dword),
// two 8-byte elements (w = 8) or one 16-byte element (w = 16).

struct LdsShape {
    int w, tb, ta, cpt;
    constexpr TPL_HD int row_bytes() const { return ta * w; }            // one source row in the tile
    constexpr TPL_HD int chunks_per_row() const { return ta * w / 16; }
    constexpr TPL_HD int tile_bytes() const { return tb * ta * w; }
    constexpr TPL_HD int threads() const { return tile_bytes() / (16 * cpt); }
    constexpr TPL_HD int g() const { return w >= 4 ? 1 : 4 / w; }         // elements per dword
    constexpr TPL_HD int read_bytes() const { return w >= 8 ? w : 4; }    // LDS read width
    constexpr TPL_HD int reads_per_group() const { return w >= 8 ? 16 / w : 4 * g(); }  // P of the read phase
    constexpr TPL_HD int nq() const { return tb * w / 16; }              // 16-byte chunks per destination row
    // chunks along b in neighbouring lanes: a wave's store covers 256-byte
    // runs of destination rows (measured against 128- and 512-byte runs)
    constexpr TPL_HD int ql() const { return nq() < 16 ? nq() : 16; }
    constexpr TPL_HD int cols() const { return w >= 8 ? ta : ta * w / 4; } // read columns (dwords, or 8-byte elements)
    constexpr TPL_HD int groups() const { return cols() * nq(); }
    constexpr TPL_HD int groups_per_thread() const { return (groups() + threads() - 1) / threads(); }
};

// Write phase: thread t, chunk slot k (0..3), piece step r of the chunk.
// Returns the LDS byte address; `piece` receives the piece index written.
TPL_HD int lds_write_addr(const LdsShape& sh, int pitch, int ww, int t, int k, int r,
                          int shift_w, int mask_w, int* piece) {
    int cid = t + k * sh.threads();
    int row = cid / sh.chunks_per_row();
    int c = cid % sh.chunks_per_row();
    int lane = t & (kWave - 1);
    int h = r ^ ((lane >> shift_w) & mask_w);
    if (piece) *piece = h;
    return row * pitch + c * 16 + h * ww;
}

// Read phase: thread t, group slot k2, unrolled read step r.
// Group gid -> (column col, chunk q): lanes run along q first (ql() of them),
// then along col, then over the rest of q.
TPL_HD void lds_group(const LdsShape& sh, int t, int k2, int* col, int* q) {
    int gid = t + k2 * sh.threads();
    int ql = sh.ql();
    int seg = gid % ql;
    int rest = gid / ql;
    *col = rest % sh.cols();
    *q = (rest / sh.cols()) * ql + seg;
}

// Returns -1 when slot k2 of thread t holds no group (the last slot may be partial).
TPL_HD int lds_read_addr(const LdsShape& sh, int pitch, int t, int k2, int r,
                         int shift_r, int mask_r, int* row_step) {
    if (t + k2 * sh.threads() >= sh.groups()) return -1;
    int col, q;
    lds_group(sh, t, k2, &col, &q);
    int lane = t & (kWave - 1);
    int j = r ^ ((lane >> shift_r) & mask_r);
    if (row_step) *row_step = j;
    int b0 = q * sh.reads_per_group();
    return (b0 + j) * pitch + col * sh.read_bytes();
}

}  // namespace tpl
