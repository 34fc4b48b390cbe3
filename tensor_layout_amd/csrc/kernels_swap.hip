// kernels_swap.hip -- in-place square transposes by mirrored tile-pair
// swaps through LDS.
#include "device.hpp"
#include "tile.hpp"

namespace tpl {

// ---------------------------------------------------------------------------
// In-place square transpose across tiles: tile (b-tile c, a-tile r) and its
// mirror (b-tile r, a-tile c) occupy each other's destination, so one
// workgroup reads both into LDS before it writes either.  Work units are the
// pairs c <= r of every batch item (diagonal tiles pair with themselves);
// distinct units touch disjoint memory.
//
// Unit order: the m x m tiles form M x M blocks of G x G tiles (G = kSwapG,
// M = ceil(m / G)).  Block pairs (C, R = C + D) walk the block diagonals:
// unit row kb of M holds block diagonal kb (M - kb blocks) followed by block
// diagonal M - kb (kb blocks); rows kb = 0 .. M/2 cover every block
// diagonal once, except that for even M the second half of row M/2 repeats
// block diagonal M/2 and does nothing.  Each block pair is G x G units, tile
// pair (C G + u, R G + v); on the block diagonal D = 0 only u <= v, and
// tiles past the edge, do anything.  Neighbouring blocks thus read
// different row and column bands (a column band shared by many concurrent
// workgroups piles their reads onto the same HBM channels when the row
// pitch is a power of two), while the G x G pairs of one block share their
// DRAM rows.  On the 16384^2 bf16 transpose: G = 8 +3% against walking
// single tiles diagonally (G = 1); G = 16 -5%, G = 32 -16%.
template <int W, int T, int CPT, int WW, int NB, bool BIG>
__global__ void __launch_bounds__(T * T * W / (16 * CPT)) k_swap(LdsArgs a) {
    constexpr LdsShape SH{W, T, T, CPT};
    constexpr int NT = SH.threads();
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

    const int t = threadIdx.x;
    const int lane = t & (kWave - 1);
    const int key_w = (lane >> a.shift_w) & a.mask_w;
    const int key_r = (lane >> a.shift_r) & a.mask_r;
    const int pitch = a.pitch;
    uint8_t* l0 = lds;
    uint8_t* l1 = lds + T * pitch;

    for (int64_t unit = blockIdx.x; unit < a.ntiles; unit += gridDim.x) {
        int64_t item, pr, kb, jb;
        split<BIG>(unit, a.npair, a.div_npair, item, pr);
        split<BIG>(pr >> (2 * kSwapLogG), a.nbl, a.div_nbl, kb, jb);
        const int u = (int)(pr >> kSwapLogG) & (kSwapG - 1), v = (int)pr & (kSwapG - 1);
        const int64_t M = a.nbl;
        int64_t cb, db;   // block pair (cb, cb + db)
        if (jb < M - kb) {
            db = kb;
            cb = jb;
        } else {
            db = M - kb;
            cb = jb - (M - kb);
            if (db == kb) continue;   // even M, row M/2: block diagonal M/2 again (uniform)
        }
        if (db == 0 && u > v) continue;   // block diagonal: each pair once
        const int64_t c = cb * kSwapG + u, r = (cb + db) * kSwapG + v;
        if (r >= a.ntb) continue;   // past the edge (c <= r)
        int64_t so, d_o;
        modes_offsets<NB, BIG>(a.batch, item, so, d_o);
        const bool two = c != r;
        // Tile X: b-tile c, a-tile r.  Tile Y: b-tile r, a-tile c.
        const int64_t lo = c * T, hi = r * T;
        const int64_t px = (so + lo * a.s_b + hi) * W, py = (so + hi * a.s_b + lo) * W;
        const int64_t qx = (d_o + hi * a.d_a + lo) * W, qy = (d_o + lo * a.d_a + hi) * W;
        const uint8_t* sx = a.src + px;
        const uint8_t* sy = a.src + py;
        uint8_t* dx = a.dst + qx;
        uint8_t* dy = a.dst + qy;
        if (!a.scalar && hi + T <= a.e_a) {
            // Both tiles' loads are issued before either is written to LDS.
            u32x4 vx[CPT], vy[CPT];
            tile_load<W, T, T, CPT>(vx, a.src, px, a.s_b * W, t);
            if (two) tile_load<W, T, T, CPT>(vy, a.src, py, a.s_b * W, t);
            tile_put<W, T, T, CPT, WW>(l0, vx, pitch, t, key_w);
            if (two) tile_put<W, T, T, CPT, WW>(l1, vy, pitch, t, key_w);
            __syncthreads();
            tile_from_lds<W, T, T, CPT>(l0, a.dst, qx, a.d_a, pitch, t, key_r);
            if (two) tile_from_lds<W, T, T, CPT>(l1, a.dst, qy, a.d_a, pitch, t, key_r);
        } else {
            // Ragged (the last tile row and column) or unaligned: element by
            // element through LDS.  nlo / nhi: valid extents along the modes
            // whose tile index is c / r.
            const int nlo = (int)(a.e_a - lo < T ? a.e_a - lo : T), nhi = (int)(a.e_a - hi < T ? a.e_a - hi : T);
            for (int idx = t; idx < T * T; idx += NT) {
                const int bb = idx / T, aa = idx % T;
                if (bb < nlo && aa < nhi) copy_elem<W>(l0 + bb * pitch + aa * W, sx + (bb * a.s_b + aa) * W);
                if (two && bb < nhi && aa < nlo) copy_elem<W>(l1 + bb * pitch + aa * W, sy + (bb * a.s_b + aa) * W);
            }
            __syncthreads();
            for (int idx = t; idx < T * T; idx += NT) {
                const int bb = idx % T, aa = idx / T;
                if (bb < nlo && aa < nhi) copy_elem<W>(dx + (aa * a.d_a + bb) * W, l0 + bb * pitch + aa * W);
                if (two && bb < nhi && aa < nlo) copy_elem<W>(dy + (aa * a.d_a + bb) * W, l1 + bb * pitch + aa * W);
            }
        }
        __syncthreads();   // LDS is reused by the next pair of this workgroup
    }
}

// ---------------------------------------------------------------------------
// Launcher.

template <int NB, bool BIG>
static hipError_t launch_swap_shape(const Plan& p, const LdsArgs& a, hipStream_t st) {
    dim3 grid((unsigned)cap_grid(p.grid, p.block)), block((unsigned)p.block);
    const int w = p.w, tb = p.tile_b, ww = p.ww;
#define TPL_SWAP_CASE(W_, T_, WW_)                                                                     \
    if (w == W_ && tb == T_ && ww == WW_) {                                                           \
        hipLaunchKernelGGL((k_swap<W_, T_, 2, WW_, NB, BIG>), grid, block, p.lds_bytes, st, a);       \
        return hipGetLastError();                                                                     \
    }
#define TPL_SWAP_SHAPE(W_, T_) TPL_SWAP_CASE(W_, T_, 16) TPL_SWAP_CASE(W_, T_, 8) TPL_SWAP_CASE(W_, T_, 4)
    TPL_SWAP_SHAPE(1, 128)
    TPL_SWAP_SHAPE(2, 64)
    TPL_SWAP_SHAPE(4, 64)
    TPL_SWAP_SHAPE(8, 32)
    TPL_SWAP_SHAPE(16, 16)
#undef TPL_SWAP_SHAPE
#undef TPL_SWAP_CASE
    return hipErrorInvalidConfiguration;
}

template <int NB, bool BIG>
hipError_t launch_swap(const Plan& p, const uint8_t* src, uint8_t* dst, hipStream_t st) {
    LdsArgs a = p.lds;
    a.src = src;
    a.dst = dst;
    return launch_swap_shape<NB, BIG>(p, a, st);
}

TPL_LAUNCHER_INSTANCES(launch_swap)

}  // namespace tpl
