// device.hpp -- what the kernel families share: vector types, 16-byte
// non-temporal accesses, swizzled addressing, index splits, element copies,
// the launch-grid cap, and the launchers each family's translation unit
// defines (explicitly instantiated there for every batch-mode class and
// index width).
#pragma once

#include <hip/hip_runtime.h>

#include "common.hpp"
#include "planner.hpp"

namespace tpl {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int64_t kMaxThreads = (int64_t)1 << 31;   // grid * block kept below 2^32

__device__ __forceinline__ u32x4 ld16(const uint8_t* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void st16(uint8_t* p, u32x4 v) {
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}

// A 16-byte store with device scope (sc1) besides the non-temporal hint.  A
// plain 512 MiB copy measured 6.77 TB/s that way against 6.66 with the hint
// alone (MI355X); across the kernels it helps the quad kernel (+1-2 % on the
// scale-factor and record tiles) and costs the LDS-tile and record kernels
// up to 4 % on some layouts, so only the quad kernel and the 16-byte run
// copy (the plain copy the others are measured against) use it.  No builtin
// sets sc1 on a global store, hence the asm.  A store of more than 8 bytes
// reads its data registers after issue, and the compiler cannot see into the
// asm to keep a following VALU write to them 2 wait states away, so the asm
// ends with that wait itself (s_nop 1, what the compiler emits after its own
// 16-byte stores).  The memory clobber keeps the store in program order with
// every other memory access.
__device__ __forceinline__ void st16_dev(uint8_t* p, u32x4 v) {
    asm volatile("global_store_dwordx4 %0, %1, off sc1 nt\n\ts_nop 1" ::"v"(p), "v"(v) : "memory");
}

// base + P, or base + swz(P) for a swizzled operand.
template <bool SWZ>
__device__ __forceinline__ uint8_t* at(const uint8_t* base, int64_t p, const Swz& z) {
    return const_cast<uint8_t*>(base) + (SWZ ? swz_apply(z, p) : p);
}

template <bool BIG>
__device__ __forceinline__ void split(int64_t idx, int64_t n, const FastDiv& f, int64_t& q, int64_t& r) {
    if (BIG) {
        q = idx / n;
        r = idx - q * n;
    } else {
        uint32_t qq = fdiv((uint32_t)idx, f);
        q = qq;
        r = (int64_t)((uint32_t)idx - qq * f.d);
    }
}

template <int W>
__device__ __forceinline__ void copy_elem(uint8_t* d, const uint8_t* s) {
    if constexpr (W == 1) {
        *d = *s;
    } else if constexpr (W == 2) {
        *reinterpret_cast<uint16_t*>(d) = *reinterpret_cast<const uint16_t*>(s);
    } else {
#pragma unroll
        for (int i = 0; i < W / 4; ++i)
            reinterpret_cast<uint32_t*>(d)[i] = reinterpret_cast<const uint32_t*>(s)[i];
    }
}

inline int64_t cap_grid(int64_t grid, int64_t block) {
    int64_t lim = kMaxThreads / block;
    return grid < lim ? (grid < 1 ? 1 : grid) : lim;
}

// Launchers: enqueue the plan's kernel on st with the operands' bases.
template <bool BIG>
hipError_t launch_gather(const Plan& p, const uint8_t* src, uint8_t* dst, hipStream_t st);
template <int NB, bool BIG>
hipError_t launch_copy(const Plan& p, const uint8_t* src, uint8_t* dst, hipStream_t st);
template <int NB, bool BIG>
hipError_t launch_reg16(const Plan& p, const uint8_t* src, uint8_t* dst, hipStream_t st);
template <int NB, bool BIG>
hipError_t launch_quad(const Plan& p, const uint8_t* src, uint8_t* dst, hipStream_t st);
template <int NB, bool BIG>
hipError_t launch_lds(const Plan& p, const uint8_t* src, uint8_t* dst, hipStream_t st);
template <int NB, bool BIG>
hipError_t launch_swap(const Plan& p, const uint8_t* src, uint8_t* dst, hipStream_t st);
template <int NB, bool BIG>
hipError_t launch_rec(const Plan& p, const uint8_t* src, uint8_t* dst, hipStream_t st);
template <int NB, bool BIG>
hipError_t launch_etile(const Plan& p, const uint8_t* src, uint8_t* dst, hipStream_t st);

}  // namespace tpl

// Instances for 0, 1, 2 and any number of batch modes, 32- and 64-bit indices.
#define TPL_LAUNCHER_INSTANCES(fn)                                                        \
    template hipError_t fn<0, false>(const Plan&, const uint8_t*, uint8_t*, hipStream_t);  \
    template hipError_t fn<1, false>(const Plan&, const uint8_t*, uint8_t*, hipStream_t);  \
    template hipError_t fn<2, false>(const Plan&, const uint8_t*, uint8_t*, hipStream_t);  \
    template hipError_t fn<-1, false>(const Plan&, const uint8_t*, uint8_t*, hipStream_t); \
    template hipError_t fn<0, true>(const Plan&, const uint8_t*, uint8_t*, hipStream_t);   \
    template hipError_t fn<1, true>(const Plan&, const uint8_t*, uint8_t*, hipStream_t);   \
    template hipError_t fn<2, true>(const Plan&, const uint8_t*, uint8_t*, hipStream_t);   \
    template hipError_t fn<-1, true>(const Plan&, const uint8_t*, uint8_t*, hipStream_t);
