// kernels_stream.hip -- the kernels without an exchange: element gather,
// run copy and the 16-byte lane remap.
#include "device.hpp"

namespace tpl {

// ---------------------------------------------------------------------------
// Gather/scatter: one element per thread per iteration, any layout.

template <typename T>
struct Unit;
template <> struct Unit<uint8_t> { static constexpr int bytes = 1; };
template <> struct Unit<uint16_t> { static constexpr int bytes = 2; };
template <> struct Unit<uint32_t> { static constexpr int bytes = 4; };
template <> struct Unit<uint64_t> { static constexpr int bytes = 8; };
template <> struct Unit<u32x4> { static constexpr int bytes = 16; };

template <typename T, bool BIG>
__global__ void __launch_bounds__(256) k_gather(GatherArgs a) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int nu = a.w / Unit<T>::bytes;
    for (int64_t n = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; n < a.total; n += stride) {
        int64_t so, d_o;
        modes_offsets<-1, BIG>(a.modes, n, so, d_o);
        const T* s = reinterpret_cast<const T*>(at<true>(a.src, so * a.w, a.zs));
        T* d = reinterpret_cast<T*>(at<true>(a.dst, d_o * a.w, a.zd));
        for (int u = 0; u < nu; ++u) d[u] = s[u];
    }
}

// ---------------------------------------------------------------------------
// Copy: both sides contiguous along one mode (the contiguous-chunk case of
// the dsmem page, "Algorithm" step 1): every run is moved in V-byte vectors,
// one per lane, one wave per workgroup.

template <int V> struct Vec;
template <> struct Vec<4> { typedef uint32_t type; };
template <> struct Vec<8> { typedef u32x2 type; };
template <> struct Vec<16> { typedef u32x4 type; };

template <int V, int NB, bool BIG, bool SWZ>
__global__ void __launch_bounds__(64) k_copy(CopyArgs a) {
    typedef typename Vec<V>::type T;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; id < a.nchunks; id += stride) {
        int64_t row, c;
        split<BIG>(id, a.cpr, a.div_cpr, row, c);
        int64_t so, d_o;
        modes_offsets<NB, BIG>(a.rows, row, so, d_o);
        const T v = __builtin_nontemporal_load(reinterpret_cast<const T*>(at<SWZ>(a.src, so * a.w + c * V, a.zs)));
        if constexpr (V == 16) st16_dev(at<SWZ>(a.dst, d_o * a.w + c * V, a.zd), v);   // device-scope store
        else __builtin_nontemporal_store(v, reinterpret_cast<T*>(at<SWZ>(a.dst, d_o * a.w + c * V, a.zd)));
    }
}

// ---------------------------------------------------------------------------
// 16-byte elements: a wave takes an 8x8 element block; lane (i, j) loads
// source row b0+i, element a0+j (eight lanes per 128-byte source line) and
// stores it at destination row a0+j, element b0+i (eight lanes per 128-byte
// destination line).  An element is one dwordx4, so no exchange is needed.

template <int NB, bool BIG>
__global__ void __launch_bounds__(256) k_reg16(Reg16Args a) {
    const int lane = threadIdx.x & 63;
    const int i = lane >> 3, j = lane & 7;
    for (int64_t blk = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); blk < a.nblocks;
         blk += (int64_t)gridDim.x * 4) {
        int64_t rest, tai, item, tbi;
        split<BIG>(blk, a.nba, a.div_nba, rest, tai);
        split<BIG>(rest, a.nbb, a.div_nbb, item, tbi);
        int64_t so, d_o;
        modes_offsets<NB, BIG>(a.batch, item, so, d_o);
        const int64_t bb = tbi * 8 + i, aa = tai * 8 + j;
        if (bb < a.e_b && aa < a.e_a)
            st16(a.dst + (d_o + aa * a.d_a + bb) * 16, ld16(a.src + (so + bb * a.s_b + aa) * 16));
    }
}

// ---------------------------------------------------------------------------
// Launchers.

template <bool BIG>
hipError_t launch_gather(const Plan& p, const uint8_t* src, uint8_t* dst, hipStream_t st) {
    GatherArgs a = p.gather;
    a.src = src;
    a.dst = dst;
    dim3 grid((unsigned)cap_grid(p.grid, 256)), block(256);
    switch (a.unit) {
    case 1: hipLaunchKernelGGL((k_gather<uint8_t, BIG>), grid, block, 0, st, a); break;
    case 2: hipLaunchKernelGGL((k_gather<uint16_t, BIG>), grid, block, 0, st, a); break;
    case 4: hipLaunchKernelGGL((k_gather<uint32_t, BIG>), grid, block, 0, st, a); break;
    case 8: hipLaunchKernelGGL((k_gather<uint64_t, BIG>), grid, block, 0, st, a); break;
    default: hipLaunchKernelGGL((k_gather<u32x4, BIG>), grid, block, 0, st, a); break;
    }
    return hipGetLastError();
}

template <int NB, bool BIG>
hipError_t launch_copy(const Plan& p, const uint8_t* src, uint8_t* dst, hipStream_t st) {
    CopyArgs a = p.copy;
    a.src = src;
    a.dst = dst;
    dim3 grid((unsigned)cap_grid(p.grid, 64)), block(64);
    if ((a.zs.ymask | a.zd.ymask) == 0) {
        if (a.vec == 16) hipLaunchKernelGGL((k_copy<16, NB, BIG, false>), grid, block, 0, st, a);
        else if (a.vec == 8) hipLaunchKernelGGL((k_copy<8, NB, BIG, false>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((k_copy<4, NB, BIG, false>), grid, block, 0, st, a);
    } else {
        if (a.vec == 16) hipLaunchKernelGGL((k_copy<16, NB, BIG, true>), grid, block, 0, st, a);
        else if (a.vec == 8) hipLaunchKernelGGL((k_copy<8, NB, BIG, true>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((k_copy<4, NB, BIG, true>), grid, block, 0, st, a);
    }
    return hipGetLastError();
}

template <int NB, bool BIG>
hipError_t launch_reg16(const Plan& p, const uint8_t* src, uint8_t* dst, hipStream_t st) {
    Reg16Args a = p.reg16;
    a.src = src;
    a.dst = dst;
    hipLaunchKernelGGL((k_reg16<NB, BIG>), dim3((unsigned)cap_grid(p.grid, 256)), dim3(256), 0, st, a);
    return hipGetLastError();
}

template hipError_t launch_gather<false>(const Plan&, const uint8_t*, uint8_t*, hipStream_t);
template hipError_t launch_gather<true>(const Plan&, const uint8_t*, uint8_t*, hipStream_t);
TPL_LAUNCHER_INSTANCES(launch_copy)
TPL_LAUNCHER_INSTANCES(launch_reg16)

}  // namespace tpl
