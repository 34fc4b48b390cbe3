// kernels_etile.hip -- 2-D transposes through LDS one element per access.
#include "device.hpp"

namespace tpl {

// ---------------------------------------------------------------------------
// Element tiles: a TB x TA tile (TB along the destination-contiguous mode b,
// TA along the source-contiguous mode a) staged through LDS one element per
// access, for 2-D transposes whose row pitches, bases or swizzle granules
// rule out the 16-byte vectors of k_lds.  Loading, neighbouring lanes walk
// a source row (TA elements: 128 or 256 bytes); storing, they walk a
// destination row.  TA and TB divide the 256 threads, so each thread keeps
// one column on each side and steps by whole rows: its addresses advance by
// a constant.  The LDS pitch is the row plus one unit of max(w, 4) bytes, an
// odd number of units, so the column read of phase 2 (lanes on neighbouring
// rows) meets no bank conflict; the row write of phase 1 is contiguous.
// Tiles follow the k_lds order.

template <int W> struct Elem;
template <> struct Elem<1> { typedef uint8_t type; };
template <> struct Elem<2> { typedef uint16_t type; };
template <> struct Elem<4> { typedef uint32_t type; };
template <> struct Elem<8> { typedef u32x2 type; };
template <> struct Elem<16> { typedef u32x4 type; };

template <int W, int NB, bool BIG, bool SWZ>
__device__ __forceinline__ void etile_loop(const LdsArgs& a, uint8_t* lds) {
    typedef typename Elem<W>::type T;
    constexpr EtileShape ES = kEtileShapes[etile_index(W)];
    constexpr int TB = ES.tb, TA = ES.ta, P = ES.pitch(), NT = 256;
    constexpr int RA = NT / TA, RB = NT / TB;   // rows per step, phase 1 and 2
    static_assert(NT % TA == 0 && NT % TB == 0 && TB % RA == 0 && TA % RB == 0, "tile must tile the threads");
    const int t = threadIdx.x;
    const int aa1 = t % TA, bb1 = t / TA;   // phase 1: column aa1, rows bb1 + i RA
    const int bb2 = t % TB, aa2 = t / TB;   // phase 2: column bb2, rows aa2 + i RB
    for (int64_t tile = blockIdx.x; tile < a.ntiles; tile += gridDim.x) {
        int64_t rest, tq, item, tbi, tai, wrap;
        split<BIG>(tile, a.ntb, a.div_ntb, rest, tbi);
        split<BIG>(rest, a.nta, a.div_nta, item, tq);
        split<BIG>(tq + tbi, a.nta, a.div_nta, wrap, tai);
        int64_t so, d_o;
        modes_offsets<NB, BIG>(a.batch, item, so, d_o);
        const int64_t b0 = tbi * TB, a0 = tai * TA;
        const int nb = (int)(a.e_b - b0 < TB ? a.e_b - b0 : TB), na = (int)(a.e_a - a0 < TA ? a.e_a - a0 : TA);
        {
            int64_t off = (so + (b0 + bb1) * a.s_b + a0 + aa1) * W;
            const int64_t step = (int64_t)RA * a.s_b * W;
#pragma unroll 16
            for (int i = 0; i < TB / RA; ++i, off += step) {
                const int bb = bb1 + i * RA;
                if (aa1 < na && bb < nb)
                    *reinterpret_cast<T*>(lds + bb * P + aa1 * W) =
                        __builtin_nontemporal_load(reinterpret_cast<const T*>(at<SWZ>(a.src, off, a.zs)));
            }
        }
        __syncthreads();
        {
            int64_t off = (d_o + (a0 + aa2) * a.d_a + b0 + bb2) * W;
            const int64_t step = (int64_t)RB * a.d_a * W;
#pragma unroll 16
            for (int i = 0; i < TA / RB; ++i, off += step) {
                const int aa = aa2 + i * RB;
                if (bb2 < nb && aa < na)
                    __builtin_nontemporal_store(*reinterpret_cast<const T*>(lds + bb2 * P + aa * W),
                                                reinterpret_cast<T*>(at<SWZ>(a.dst, off, a.zd)));
            }
        }
        __syncthreads();   // LDS is reused by the next tile of this workgroup
    }
}

template <int W, int NB, bool BIG>
__global__ void __launch_bounds__(256) k_etile(LdsArgs a) {
    constexpr EtileShape ES = kEtileShapes[etile_index(W)];
    __shared__ __attribute__((aligned(16))) uint8_t lds[ES.tb * ES.pitch()];
    // Plain operands take the code without swizzle arithmetic (a uniform branch).
    if ((a.zs.ymask | a.zd.ymask) == 0) etile_loop<W, NB, BIG, false>(a, lds);
    else etile_loop<W, NB, BIG, true>(a, lds);
}

// ---------------------------------------------------------------------------
// Launcher.

template <int NB, bool BIG>
hipError_t launch_etile(const Plan& p, const uint8_t* src, uint8_t* dst, hipStream_t st) {
    LdsArgs a = p.lds;
    a.src = src;
    a.dst = dst;
    dim3 grid((unsigned)cap_grid(p.grid, 256)), block(256);
    switch (p.w) {
    case 1: hipLaunchKernelGGL((k_etile<1, NB, BIG>), grid, block, 0, st, a); break;
    case 2: hipLaunchKernelGGL((k_etile<2, NB, BIG>), grid, block, 0, st, a); break;
    case 4: hipLaunchKernelGGL((k_etile<4, NB, BIG>), grid, block, 0, st, a); break;
    case 8: hipLaunchKernelGGL((k_etile<8, NB, BIG>), grid, block, 0, st, a); break;
    default: hipLaunchKernelGGL((k_etile<16, NB, BIG>), grid, block, 0, st, a); break;
    }
    return hipGetLastError();
}

TPL_LAUNCHER_INSTANCES(launch_etile)

}  // namespace tpl
