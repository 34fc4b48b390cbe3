// kernels_lds_impl.hpp -- the tiled transpose through LDS: the kernel and
// its launcher for one element width, included by the translation units
// that instantiate it (kernels_lds_w*.hip, a few widths each).
#pragma once

#include "lds.hpp"
#include "tile.hpp"

namespace tpl {

// ---------------------------------------------------------------------------
// LDS kernel: one workgroup moves a TB x TA tile (TB along the destination-
// contiguous mode b, TA along the source-contiguous mode a).
//
// Phase 1: every thread loads CPT (two) 16-byte chunks of source rows and writes
// them to LDS (row pitch chosen by the planner) in 16/WW pieces, the piece
// order XOR-rotated per lane: piece = r ^ ((lane >> shift_w) & mask_w).
// Barrier.  Phase 2: every thread gathers, for one column of the tile and
// one 16-byte destination chunk, the rows b0 .. b0+P-1 of that column, in the
// order j = r ^ ((lane >> shift_r) & mask_r), restores row order in
// registers, packs sub-dword elements into destination-order dwords and
// stores 16 bytes.  Both XORs are the planner's smallest conflict-free k for
// the measured gfx950 LDS banks.  Tiles of 4- to 16-byte elements store with
// device scope (st16_dev): 4096^2 x 16 B 90.3 -> 88.0 us, the 32 MiB and
// 64 MiB 4-D permutes (4- and 8-byte elements) 1.2 % faster; 1- and 2-byte
// tiles measured the same or up to 2 % slower that way and keep st16.

template <int W, int TB, int TA, int CPT, int WW, int NB, bool BIG, bool SWZ>
__device__ __forceinline__ void lds_loop(const LdsArgs& a, uint8_t* lds) {
    constexpr LdsShape SH{W, TB, TA, CPT};
    constexpr int NT = SH.threads();

    const int t = threadIdx.x;
    const int lane = t & (kWave - 1);
    const int key_w = (lane >> a.shift_w) & a.mask_w;
    const int key_r = (lane >> a.shift_r) & a.mask_r;
    const int pitch = a.pitch;

    for (int64_t tile = blockIdx.x; tile < a.ntiles; tile += gridDim.x) {
        // Tile order: b fastest, so that neighbouring workgroups write
        // neighbouring pieces of the same destination rows; and diagonal in
        // a (the a-tile index is shifted by the b-tile index), so that
        // neighbouring workgroups read source rows at different column
        // offsets.  With power-of-two row pitches the plain order sends every
        // concurrent read of a column band to the same HBM channels.
        int64_t rest, tq, item, tbi, tai, wrap;
        split<BIG>(tile, a.ntb, a.div_ntb, rest, tbi);
        split<BIG>(rest, a.nta, a.div_nta, item, tq);
        split<BIG>(tq + tbi, a.nta, a.div_nta, wrap, tai);
        int64_t so, d_o;
        modes_offsets<NB, BIG>(a.batch, item, so, d_o);
        const int64_t b0 = tbi * TB, a0 = tai * TA;

        if (b0 + TB > a.e_b || a0 + TA > a.e_a) {
            // Ragged edge tile: element by element (never used in place).
            const int nb = (int)(a.e_b - b0 < TB ? a.e_b - b0 : TB), na = (int)(a.e_a - a0 < TA ? a.e_a - a0 : TA);
            for (int idx = t; idx < TB * TA; idx += NT) {
                const int bb = idx / TA, aa = idx % TA;
                if (bb >= nb || aa >= na) continue;
                const uint8_t* s = at<SWZ>(a.src, (so + (b0 + bb) * a.s_b + a0 + aa) * W, a.zs);
                uint8_t* d = at<SWZ>(a.dst, (d_o + (a0 + aa) * a.d_a + b0 + bb) * W, a.zd);
                if constexpr (W == 16) *reinterpret_cast<u32x4*>(d) = *reinterpret_cast<const u32x4*>(s);
                else copy_elem<W>(d, s);
            }
            continue;   // uniform across the workgroup
        }

        tile_to_lds<W, TB, TA, CPT, WW, SWZ>(lds, a.src, (so + b0 * a.s_b + a0) * W, a.s_b * W, pitch, t, key_w,
                                             a.zs);
        __syncthreads();
        tile_from_lds<W, TB, TA, CPT, SWZ, (W >= 4)>(lds, a.dst, (d_o + a0 * a.d_a + b0) * W, a.d_a, pitch, t, key_r,
                                                    a.zd);
        __syncthreads();   // LDS is reused by the next tile of this workgroup
    }
}

// Plain and swizzled operands are separate kernels: with both loops in one
// kernel behind a uniform branch, the plain fp16 tile workload (65536 tiles
// of 128 x 64) ran 342.3 us against 337.7 for the plain loop alone.
template <int W, int TB, int TA, int CPT, int WW, int NB, bool BIG, bool SWZ>
__global__ void __launch_bounds__(TB * TA * W / (16 * CPT)) k_lds(LdsArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    lds_loop<W, TB, TA, CPT, WW, NB, BIG, SWZ>(a, lds);
}

// ---------------------------------------------------------------------------
// Launcher for the tile shapes of width W.

template <int W, int NB, bool BIG>
hipError_t launch_lds_width(const Plan& p, const LdsArgs& a, hipStream_t st) {
    dim3 grid((unsigned)cap_grid(p.grid, p.block)), block((unsigned)p.block);
    const int tb = p.tile_b, ta = p.tile_a, cpt = p.cpt, ww = p.ww;
    const bool swz = (a.zs.ymask | a.zd.ymask) != 0;
#define TPL_LDS_CASE(W_, TB_, TA_, CPT_, WW_)                                                                \
    if (tb == TB_ && ta == TA_ && cpt == CPT_ && ww == WW_) {                                                \
        if (swz) hipLaunchKernelGGL((k_lds<W_, TB_, TA_, CPT_, WW_, NB, BIG, true>), grid, block, p.lds_bytes, st, a); \
        else hipLaunchKernelGGL((k_lds<W_, TB_, TA_, CPT_, WW_, NB, BIG, false>), grid, block, p.lds_bytes, st, a);   \
        return hipGetLastError();                                                                              \
    }
#define TPL_LDS_SHAPE(W_, TB_, TA_, CPT_) \
    TPL_LDS_CASE(W_, TB_, TA_, CPT_, 16) TPL_LDS_CASE(W_, TB_, TA_, CPT_, 8) TPL_LDS_CASE(W_, TB_, TA_, CPT_, 4)
    if constexpr (W == 1) {
        TPL_LDS_SHAPE(1, 128, 128, 4)
        TPL_LDS_SHAPE(1, 128, 128, 2)
        TPL_LDS_SHAPE(1, 64, 128, 2)
    }
    if constexpr (W == 2) {
        TPL_LDS_SHAPE(2, 256, 64, 4)
        TPL_LDS_SHAPE(2, 256, 64, 2)
        TPL_LDS_SHAPE(2, 128, 128, 4)
        TPL_LDS_SHAPE(2, 128, 64, 2)
        TPL_LDS_SHAPE(2, 32, 64, 2)
    }
    if constexpr (W == 4) {
        TPL_LDS_SHAPE(4, 128, 64, 4)
        TPL_LDS_SHAPE(4, 64, 64, 2)
        TPL_LDS_SHAPE(4, 32, 256, 2)
        TPL_LDS_SHAPE(4, 32, 32, 2)
    }
    if constexpr (W == 8) {
        TPL_LDS_SHAPE(8, 64, 64, 4)
        TPL_LDS_SHAPE(8, 32, 64, 2)
        TPL_LDS_SHAPE(8, 16, 32, 2)
    }
    if constexpr (W == 16) {
        TPL_LDS_SHAPE(16, 64, 16, 2)
        TPL_LDS_SHAPE(16, 16, 64, 2)
        TPL_LDS_SHAPE(16, 16, 16, 2)
    }
#undef TPL_LDS_SHAPE
#undef TPL_LDS_CASE
    return hipErrorInvalidConfiguration;
}

}  // namespace tpl

#define TPL_LDS_WIDTH_INSTANCES(W)                                                                  \
    template hipError_t tpl::launch_lds_width<W, 0, false>(const tpl::Plan&, const tpl::LdsArgs&, hipStream_t); \
    template hipError_t tpl::launch_lds_width<W, 1, false>(const tpl::Plan&, const tpl::LdsArgs&, hipStream_t); \
    template hipError_t tpl::launch_lds_width<W, 2, false>(const tpl::Plan&, const tpl::LdsArgs&, hipStream_t); \
    template hipError_t tpl::launch_lds_width<W, -1, false>(const tpl::Plan&, const tpl::LdsArgs&, hipStream_t); \
    template hipError_t tpl::launch_lds_width<W, 0, true>(const tpl::Plan&, const tpl::LdsArgs&, hipStream_t); \
    template hipError_t tpl::launch_lds_width<W, 1, true>(const tpl::Plan&, const tpl::LdsArgs&, hipStream_t); \
    template hipError_t tpl::launch_lds_width<W, 2, true>(const tpl::Plan&, const tpl::LdsArgs&, hipStream_t); \
    template hipError_t tpl::launch_lds_width<W, -1, true>(const tpl::Plan&, const tpl::LdsArgs&, hipStream_t);
