// staged.hip -- tpl_permute_staged: the pages' warp primitive, one batch item
// per 32-lane half-wave, staged through LDS (permute_layout page,
// "Algorithm"; the device program is tpl_wave::group_permute in tpl_wave.h).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <string>

#include "../../include/tpl_wave.h"
#include "common.hpp"
#include "planner.hpp"

namespace tpl {

int fail_status(int status, const std::string& why);   // kernels.hip

typedef uint32_t sx4 __attribute__((ext_vector_type(4)));

// Workgroups (two half-waves each) of the staged kernel; each loops over
// its share of the items.  On the 2^20-tile SF workload, with the pipelined
// loop: 3072 (12 per CU) 180.3 us; 2304 193.4, 2560 187.5, 2816 183.2,
// 3328 179.8, 3584 180.9, 4096 185.1, 8192 211, 16384 229.  The items in
// flight span a few MiB of each buffer, so the rate also depends on where
// the buffers lie: with source and destination allocated in another order
// 3072 took 186.5 us, 3328 184.1, 4096 186.3.  (Before the loop was
// pipelined 4096 was best, 5.58 TB/s.)
constexpr int64_t kStagedGrid = 3072;

struct StagedArgs {
    const uint8_t* src;
    uint8_t* dst;
    int64_t batch;
    int64_t span_s, span_d;     // item spacing on each side, bytes
    int32_t src_bytes;          // source footprint copied into LDS (multiple of vec)
    int32_t dst_bytes;          // destination footprint copied back (multiple of vec)
    int32_t src_region;         // LDS bytes reserved for the source footprint (16-aligned)
    int32_t group_bytes;        // LDS bytes per half-wave
    int32_t vec;                // copy vector: 16, 4 or 1 bytes
    int32_t shift, mask;
    tpl_wave::Shard sh;
    tpl_wave::Swizzle zs, zd;
};

template <int V> struct CopyT;
template <> struct CopyT<1> { typedef uint8_t type; };
template <> struct CopyT<4> { typedef uint32_t type; };
template <> struct CopyT<16> { typedef sx4 type; };

template <int V>
__device__ __forceinline__ void group_copy(uint8_t* d, const uint8_t* s, int bytes, int lane) {
    typedef typename CopyT<V>::type T;
    for (int off = lane * V; off < bytes; off += 32 * V)
        *reinterpret_cast<T*>(d + off) = *reinterpret_cast<const T*>(s + off);
}

__device__ __forceinline__ void group_copy_v(uint8_t* d, const uint8_t* s, int bytes, int lane, int vec) {
    if (vec == 16) group_copy<16>(d, s, bytes, lane);
    else if (vec == 4) group_copy<4>(d, s, bytes, lane);
    else group_copy<1>(d, s, bytes, lane);
}

// Each half-wave moves items grp, grp + 2 gridDim.x, ... in turn.  The
// program's offsets depend only on the shard, the lane and the XOR, so they
// are computed once, before the first item.  Item order in LDS: the copy-in
// of the next item writes the source region, which this item's permute read
// before the second barrier; its permute writes the destination region after
// the next first barrier, by which time this item's copy-out has read it.
template <typename T, int P>
__global__ void __launch_bounds__(64) k_staged(StagedArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int lane = threadIdx.x & 31, grp = threadIdx.x >> 5;
    uint8_t* ls = lds + grp * a.group_bytes;
    uint8_t* ld = ls + a.src_region;
    const tpl_wave::Offsets<P> o = tpl_wave::group_offsets<P>(a.sh, lane, a.shift, a.mask, a.zs, a.zd);
    const int64_t step = (int64_t)gridDim.x * 2;
    int64_t first = (int64_t)blockIdx.x * 2;
    if (a.vec == 16 && a.src_bytes == 32 * 16 && a.dst_bytes == 32 * 16 && first + 1 < a.batch) {
        // Items of one 16-byte chunk per lane each way, software pipelined
        // over the iterations in which both half-waves have an item: the
        // next item's chunk is loaded while this one is permuted and stored.
        // Every load and store of the loop is unconditional (a load past
        // the last item reads the last item again), so the wait for the
        // next chunk before it enters LDS does not also wait for the store
        // issued after that load.
        const uint8_t* sp = a.src + lane * 16;
        const int64_t last = a.batch - 1;
        *reinterpret_cast<sx4*>(ls + lane * 16) =
            *reinterpret_cast<const sx4*>(sp + (first + grp) * a.span_s);
        sx4 v = *reinterpret_cast<const sx4*>(sp + min(first + step + grp, last) * a.span_s);
        auto iteration = [&]() {
            __syncthreads();
            tpl_wave::group_permute<T, P>(reinterpret_cast<T*>(ld), reinterpret_cast<const T*>(ls), o);
            __syncthreads();
            const sx4 r = *reinterpret_cast<const sx4*>(ld + lane * 16);
            const bool more = first + step + 1 < a.batch;   // the next iteration is full too
            if (more) {
                *reinterpret_cast<sx4*>(ls + lane * 16) = v;
                v = *reinterpret_cast<const sx4*>(sp + min(first + 2 * step + grp, last) * a.span_s);
            }
            *reinterpret_cast<sx4*>(a.dst + (first + grp) * a.span_d + lane * 16) = r;
            first += step;
            return more;
        };
        // The first iteration runs on its own, so that the loop is entered,
        // as it is re-entered, with a load and then a store outstanding.
        if (iteration())
            while (iteration()) {
            }
    }
    for (; first < a.batch; first += step) {
        const int64_t item = first + grp;
        const bool act = item < a.batch;   // uniform across the half-wave
        if (act) group_copy_v(ls, a.src + item * a.span_s, a.src_bytes, lane, a.vec);
        __syncthreads();
        if (act) tpl_wave::group_permute<T, P>(reinterpret_cast<T*>(ld), reinterpret_cast<const T*>(ls), o);
        __syncthreads();
        if (act) group_copy_v(a.dst + item * a.span_d, ld, a.dst_bytes, lane, a.vec);
    }
}

template <typename T>
static hipError_t launch_staged_t(const StagedArgs& a, int P, dim3 grid, int lds, hipStream_t st) {
    switch (P) {
    case 1: hipLaunchKernelGGL((k_staged<T, 1>), grid, dim3(64), lds, st, a); break;
    case 2: hipLaunchKernelGGL((k_staged<T, 2>), grid, dim3(64), lds, st, a); break;
    case 4: hipLaunchKernelGGL((k_staged<T, 4>), grid, dim3(64), lds, st, a); break;
    case 8: hipLaunchKernelGGL((k_staged<T, 8>), grid, dim3(64), lds, st, a); break;
    case 16: hipLaunchKernelGGL((k_staged<T, 16>), grid, dim3(64), lds, st, a); break;
    default: hipLaunchKernelGGL((k_staged<T, 32>), grid, dim3(64), lds, st, a); break;
    }
    return hipGetLastError();
}

static int align_of(uintptr_t x) {
    int a = 1;
    while (a < 16 && (x % (2 * a)) == 0) a *= 2;
    return a;
}

static SwzSpec staged_spec(const tpl_swizzle* z) {
    SwzSpec s;
    if (z) {
        s.bits = z->bits;
        s.base = z->base;
        s.shift = z->shift;
    }
    return s;
}

static int64_t swz_of(const SwzSpec& z, int64_t m) {
    if (z.bits == 0) return m;
    return m ^ (((m >> (z.base + z.shift)) & (((int64_t)1 << z.bits) - 1)) << z.base);
}

static int staged_impl(const void* src, void* dst, int w, int rank, const int64_t* ext, const int64_t* ss,
                       const int64_t* ds, const int64_t* offs_in, int64_t batch, const tpl_swizzle* zs_in,
                       const tpl_swizzle* zd_in, int xor_k, hipStream_t stream) {
    const SwzSpec zs = staged_spec(zs_in), zd = staged_spec(zd_in);
    if (!swz_valid(zs) || !swz_valid(zd))
        return fail_status(TPL_E_ARG,
                           "a swizzle needs 0 <= bits <= 16, base >= 0, shift >= bits, base + shift + bits <= 48");
    if (rank < 1 || rank > TPL_MAX_RANK || !ext || !ss || !ds) return fail_status(TPL_E_ARG, "rank must be in 1..8");
    if (w != 1 && w != 2 && w != 4 && w != 8 && w != 16)
        return fail_status(TPL_E_DTYPE_WIDTH, "unsupported dtype byte width (must be 1, 2, 4, 8 or 16)");
    if (batch < 0) return fail_status(TPL_E_ARG, "batch must be >= 0");
    static const int64_t zero[2] = {0, 0};
    const int64_t* offs = offs_in ? offs_in : zero;
    int64_t n = 0;
    for (int i = 0; i < rank; ++i)
        if (ext[i] < 0) return fail_status(TPL_E_ARG, "extents must be >= 0");
    if (!count_elements(rank, ext, batch, &n))
        return fail_status(TPL_E_LAYOUT, "layouts must slice/canonicalize: element count overflows");
    if (n == 0) return TPL_OK;
    if (!src || !dst) return fail_status(TPL_E_ARG, "src and dst must not be NULL");
    if (offs[0] < 0 || offs[1] < 0) return fail_status(TPL_E_LAYOUT, "layouts must slice/canonicalize: negative offsets");

    // The item size rule first (the warp plan's search simulates every step).
    int64_t item_n = 1;
    for (int i = 0; i < rank; ++i) item_n = ext[i] > 1024 ? 1025 : std::min<int64_t>(item_n * ext[i], 1025);
    if (item_n % 32 != 0 || item_n > 1024)
        return fail_status(TPL_E_LAYOUT, "staged permute needs prod(extents) = 32 * P with P a power of two <= 32");
    // The per-item program: the pages' warp plan on the half-wave bank model.
    Plan p = plan_halfwave(w, rank, ext, ss, ds, 1, zs, zd);
    if (p.status != TPL_OK && p.status != TPL_E_NO_K) return fail_status(p.status, p.reason);
    const int64_t P = p.P;
    if (P < 1 || P > 32 || (P & (P - 1)))
        return fail_status(TPL_E_LAYOUT, "staged permute needs prod(extents) = 32 * P with P a power of two <= 32");
    int64_t cos_s = 1, cos_d = 1, prod = 1;
    for (int i = 0; i < rank; ++i) {
        cos_s += (ext[i] - 1) * ss[i];
        cos_d += (ext[i] - 1) * ds[i];
        prod *= ext[i];
    }
    if (cos_d != prod) return fail_status(TPL_E_LAYOUT, "staged permute needs a dense destination footprint");
    if (cos_s * w > 8192 || cos_d * w > 8192)
        return fail_status(TPL_E_LAYOUT, "staged permute footprints must fit 8 KiB");
    // Swizzled sides: every swizzled offset of an item stays inside the item's
    // footprint [0, span) (a bijection of it, so the destination stays
    // dense), and with several items the span is a multiple of the swizzle
    // period, so that item b's offsets are b * span plus those of item 0.
    for (int side = 0; side < 2; ++side) {
        const SwzSpec& z = side ? zd : zs;
        if (z.bits == 0) continue;
        const int64_t span = side ? cos_d : cos_s;
        const int64_t period = (int64_t)1 << (z.base + z.shift + z.bits);
        if (batch > 1 && span % period != 0)
            return fail_status(TPL_E_LAYOUT, "staged permute: with batch > 1 a swizzled side's item span must be "
                                             "a multiple of the swizzle period");
        for (int64_t m = 0; m < span; ++m)
            if (swz_of(z, m) >= span)
                return fail_status(TPL_E_LAYOUT, "staged permute: the swizzle leaves the item footprint");
    }
    const tpl_wave::Swizzle wzs{zs.bits ? (int)((((int64_t)1 << zs.bits) - 1) << zs.base) : 0, zs.shift};
    const tpl_wave::Swizzle wzd{zd.bits ? (int)((((int64_t)1 << zd.bits) - 1) << zd.base) : 0, zd.shift};
    int shift = p.shift, mask = p.mask;
    if (xor_k >= 0) {
        if ((1ll << xor_k) > P || xor_k > 5) return fail_status(TPL_E_ARG, "forced k exceeds log2(P)");
        mask = (1 << xor_k) - 1;
        shift = 5 - xor_k;
    } else if (p.status == TPL_E_NO_K) {
        return fail_status(TPL_E_NO_K, p.reason);
    }

    StagedArgs a{};
    a.src = static_cast<const uint8_t*>(src) + offs[0] * w;
    a.dst = static_cast<uint8_t*>(dst) + offs[1] * w;
    a.batch = batch;
    a.span_s = cos_s * w;
    a.span_d = cos_d * w;
    // Overlap of the two byte ranges is refused (the staged path is out of place).
    const uint8_t* s_hi = a.src + batch * a.span_s;
    const uint8_t* d_hi = a.dst + batch * a.span_d;
    if (a.src < d_hi && a.dst < s_hi) return fail_status(TPL_E_ALIAS, "staged permute is out of place only");
    // Copy vector: the widest of 16, 4 and 1 bytes that divides every item's
    // base address and both footprint lengths.
    int vec = 16;
    for (uintptr_t x : {(uintptr_t)a.src, (uintptr_t)a.dst, (uintptr_t)a.span_s, (uintptr_t)a.span_d}) {
        const int al = align_of(x);
        if (al < vec) vec = al;
    }
    vec = vec >= 16 ? 16 : vec >= 4 ? 4 : 1;
    a.src_bytes = (int32_t)a.span_s;
    a.dst_bytes = (int32_t)a.span_d;
    a.src_region = (int32_t)((a.span_s + 15) / 16 * 16);
    a.group_bytes = a.src_region + (int32_t)((a.span_d + 15) / 16 * 16);
    a.vec = vec;
    a.shift = shift;
    a.mask = mask;
    a.zs = wzs;
    a.zd = wzd;
    a.sh.rank = p.shard.rank;
    for (int i = 0; i < p.shard.rank; ++i) {
        a.sh.extent[i] = (int)p.shard.m[i].e;
        a.sh.src_str[i] = (int)p.shard.m[i].s;
        a.sh.dst_str[i] = (int)p.shard.m[i].d;
    }
    const int64_t groups = (batch + 1) / 2;
    dim3 grid((unsigned)std::min<int64_t>(groups, kStagedGrid));
    const int lds = 2 * a.group_bytes;
    hipError_t e;
    switch (w) {
    case 1: e = launch_staged_t<uint8_t>(a, (int)P, grid, lds, stream); break;
    case 2: e = launch_staged_t<uint16_t>(a, (int)P, grid, lds, stream); break;
    case 4: e = launch_staged_t<uint32_t>(a, (int)P, grid, lds, stream); break;
    case 8: e = launch_staged_t<uint64_t>(a, (int)P, grid, lds, stream); break;
    default: e = launch_staged_t<sx4>(a, (int)P, grid, lds, stream); break;
    }
    if (e != hipSuccess) return fail_status(TPL_E_HIP, std::string("HIP launch failed: ") + hipGetErrorString(e));
    return TPL_OK;
}

}  // namespace tpl

extern "C" int tpl_permute_staged(const void* src, void* dst, int dtype_bytes, int rank, const int64_t* extents,
                                  const int64_t* src_strides, const int64_t* dst_strides,
                                  const int64_t* elem_offsets, int64_t batch, const tpl_swizzle* src_swizzle,
                                  const tpl_swizzle* dst_swizzle, int xor_k, hipStream_t stream) {
    try {
        return tpl::staged_impl(src, dst, dtype_bytes, rank, extents, src_strides, dst_strides, elem_offsets, batch,
                                src_swizzle, dst_swizzle, xor_k, stream);
    } catch (...) {
        return tpl::fail_status(TPL_E_ARG, "internal error");
    }
}
