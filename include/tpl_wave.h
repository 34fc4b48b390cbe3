/*
 * tpl_wave.h -- the register-staged, XOR-swizzled permute of one lane group,
 * as a device function for HIP kernels on gfx950 (header only).
 *
 * The per-lane program of the permute_layout page, "Algorithm" step 3.  At
 * unrolled step r (0 <= r < P) a lane of a 32-lane group takes iteration
 * j = r ^ ((lane >> shift) & mask); the linear index lane + 32 * j, split
 * row-major over the shard extent and dotted with the source strides, gives
 * the element it loads into register r.  Once every lane holds its P
 * registers (a wave barrier), the same indices dotted with the destination
 * strides give where each register is stored.  Both
 * operands normally live in LDS; src and dst may be the same buffer.  Either
 * side may be XOR-swizzled (an MMA-style LDS tile): its offsets then go
 * through swz(m) = m ^ ((m >> shift) & ymask) before the access.
 *
 * On a 64-lane gfx950 wave the two half-waves run two independent groups.
 * For every LDS access width the hardware serves each half-wave in passes of
 * its own (b32: 32 lanes, b64 reads: 32 lanes, b64 writes: 16 lanes, b128
 * reads: 16 lanes of one half, b128 writes: 8 lanes), so the bank pattern of
 * one group is that of the pages' 32-lane warp, and the (shift, mask) that
 * tpl_plan(..., TPL_GEOM_GFX950_HALFWAVE, ...) returns keeps it free of bank
 * conflicts.
 */
#ifndef TPL_WAVE_H
#define TPL_WAVE_H

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tpl_wave {

/* The shard of one region: row-major iteration extent (last mode fastest)
 * and per-side strides, in elements; rank <= 8, prod(extent) == 32 * P. */
struct Shard {
    int rank;
    int extent[8];
    int src_str[8];
    int dst_str[8];
};

/* A side's swizzle on element offsets: ymask = (2^bits - 1) << base and
 * shift is the distance of the XORed field; ymask = 0 is a plain side. */
struct Swizzle {
    int ymask;
    int shift;
};

__device__ __forceinline__ int swizzle(const Swizzle& z, int m) { return m ^ ((m >> z.shift) & z.ymask); }

/* Element offsets of iteration n on both sides. */
__device__ __forceinline__ void project(const Shard& sh, int n, int* so, int* d_o) {
    int s = 0, d = 0;
#pragma unroll
    for (int i = 7; i >= 0; --i) {
        if (i >= sh.rank) continue;
        const int e = sh.extent[i];
        const int digit = n % e;
        n /= e;
        s += digit * sh.src_str[i];
        d += digit * sh.dst_str[i];
    }
    *so = s;
    *d_o = d;
}

/* A lane's element offsets for its P iterations on both sides, in the order
 * the program visits them (step r: iteration lane + 32 * (r ^ key)), with
 * the sides' swizzles applied.  They depend only on the shard, the lane and
 * the XOR, so a kernel that moves many regions with one layout computes them
 * once and reuses them for every region. */
template <int P>
struct Offsets {
    int src[P];
    int dst[P];
};

template <int P>
__device__ __forceinline__ Offsets<P> group_offsets(const Shard& sh, int lane, int shift, int mask,
                                                    Swizzle zs = Swizzle{0, 0}, Swizzle zd = Swizzle{0, 0}) {
    Offsets<P> o;
    const int key = (lane >> shift) & mask;
#pragma unroll
    for (int r = 0; r < P; ++r) {
        int so, d_o;
        project(sh, lane + (r ^ key) * 32, &so, &d_o);
        o.src[r] = swizzle(zs, so);
        o.dst[r] = swizzle(zd, d_o);
    }
    return o;
}

/* One 32-lane group permutes src into dst (element type T, P elements per
 * lane) with offsets from group_offsets. */
template <typename T, int P>
__device__ __forceinline__ void group_permute(T* dst, const T* src, const Offsets<P>& o) {
    T regs[P];
#pragma unroll
    for (int r = 0; r < P; ++r) regs[r] = src[o.src[r]];
    // Every lane's reads are issued, and their data consumed below, before any
    // write of this wave reaches LDS: in-place operands are safe.
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int r = 0; r < P; ++r) dst[o.dst[r]] = regs[r];
    __builtin_amdgcn_wave_barrier();
}

/* The same for a single region: offsets computed on the spot.  lane is the
 * lane index inside the group (0..31). */
template <typename T, int P>
__device__ __forceinline__ void group_permute(T* dst, const T* src, const Shard& sh, int lane, int shift,
                                              int mask, Swizzle zs = Swizzle{0, 0}, Swizzle zd = Swizzle{0, 0}) {
    group_permute<T, P>(dst, src, group_offsets<P>(sh, lane, shift, mask, zs, zd));
}

}  // namespace tpl_wave

#endif /* TPL_WAVE_H */
