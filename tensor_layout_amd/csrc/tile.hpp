// tile.hpp -- the two phases of an LDS tile (global rows into LDS with
// XOR-ordered pieces; LDS columns out to global rows with XOR-ordered rows),
// shared by the tiled transpose and the in-place pair swap.
#pragma once

#include "device.hpp"

namespace tpl {

template <int N>
__device__ __forceinline__ void unrotate(uint32_t (&d)[N], int key) {
    // d[r] holds row r ^ key; afterwards d[m] holds row m.
#pragma unroll
    for (int bi = 0; (1 << bi) < N; ++bi) {
        const bool sw = (key >> bi) & 1;
#pragma unroll
        for (int x = 0; x < N; ++x) {
            if (x & (1 << bi)) continue;
            uint32_t p0 = d[x], p1 = d[x | (1 << bi)];
            d[x] = sw ? p1 : p0;
            d[x | (1 << bi)] = sw ? p0 : p1;
        }
    }
}

// Phase 1 of an LDS tile: the TB x TA source tile at pt (rows srow bytes
// apart) through registers into LDS, element (b, a) at b * pitch + a * W.
// Each thread loads CPT 16-byte chunks (tile_load), then writes them in
// 16 / WW pieces whose order is rotated by key_w (tile_put).
template <int W, int TB, int TA, int CPT, bool SWZ = false>
__device__ __forceinline__ void tile_load(u32x4 (&v)[CPT], const uint8_t* gsrc, int64_t pt, int64_t srow, int t,
                                          const Swz& z = Swz{}) {
    constexpr LdsShape SH{W, TB, TA, CPT};
    constexpr int NT = SH.threads();
    constexpr int CPR = TA * W / 16;
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
        const int cid = t + k * NT;
        v[k] = ld16(at<SWZ>(gsrc, pt + (cid / CPR) * srow + (cid % CPR) * 16, z));
    }
}

template <int W, int TB, int TA, int CPT, int WW>
__device__ __forceinline__ void tile_put(uint8_t* lds, const u32x4 (&v)[CPT], int pitch, int t, int key_w) {
    constexpr LdsShape SH{W, TB, TA, CPT};
    constexpr int NT = SH.threads();
    constexpr int CPR = TA * W / 16;
    constexpr int NP = 16 / WW;   // pieces per chunk
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
        const int cid = t + k * NT;
        uint8_t* row = lds + (cid / CPR) * pitch + (cid % CPR) * 16;
        if constexpr (NP == 1) {
            *reinterpret_cast<u32x4*>(row) = v[k];
        } else if constexpr (NP == 2) {
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                const int h = r ^ key_w;
                u32x2 p = h ? u32x2{v[k].z, v[k].w} : u32x2{v[k].x, v[k].y};
                *reinterpret_cast<u32x2*>(row + h * 8) = p;
            }
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int h = r ^ key_w;
                uint32_t p = h == 0 ? v[k].x : h == 1 ? v[k].y : h == 2 ? v[k].z : v[k].w;
                *reinterpret_cast<uint32_t*>(row + h * 4) = p;
            }
        }
    }
}

template <int W, int TB, int TA, int CPT, int WW, bool SWZ = false>
__device__ __forceinline__ void tile_to_lds(uint8_t* lds, const uint8_t* gsrc, int64_t pt, int64_t srow, int pitch,
                                            int t, int key_w, const Swz& z = Swz{}) {
    u32x4 v[CPT];
    tile_load<W, TB, TA, CPT, SWZ>(v, gsrc, pt, srow, t, z);
    tile_put<W, TB, TA, CPT, WW>(lds, v, pitch, t, key_w);
}

// Phase 2 of an LDS tile: LDS through registers to the destination tile at
// dt (destination rows d_a elements apart).  A thread reads R words of one
// LDS column per group, rows in the order r ^ key_r, restores their order,
// packs them into 16-byte destination chunks and stores them.  Every LDS
// and global address is computed first; then all of a thread's LDS reads
// issue back to back, then the packing, then all of its stores back to back
// (scheduling barriers keep the three apart).  With two or more groups per
// thread the compiler otherwise interleaves the groups' reads, address
// arithmetic and stores, which measured 2-4 % slower on the 16384^2 bf16
// transpose at two workgroups per CU (183.6 us interleaved group by group,
// 181.2 us with address arithmetic between the stores, 176.7 us unbroken).
// DEV selects the device-scope non-temporal store (st16_dev) over st16.
template <int W, int TB, int TA, int CPT, bool SWZ = false, bool DEV = false>
__device__ __forceinline__ void tile_from_lds(const uint8_t* lds, uint8_t* gdst, int64_t pt, int64_t d_a, int pitch,
                                              int t, int key_r, const Swz& z = Swz{}) {
    constexpr LdsShape SH{W, TB, TA, CPT};
    constexpr int NT = SH.threads();
    constexpr int R = SH.reads_per_group();       // LDS reads per group: 4 dwords per element byte, two
                                                  // 8-byte elements, or one 16-byte element
    constexpr int GPT = SH.groups_per_thread();   // groups per thread
    constexpr bool PARTIAL = SH.groups() % NT != 0;   // the last slot is empty for some threads
    constexpr int NS = W == 1 ? 4 : W == 2 ? 2 : 1;   // 16-byte stores per group
    bool live[GPT];
    const uint8_t* src[GPT][R];
    uint8_t* dst[GPT][NS];
#pragma unroll
    for (int k2 = 0; k2 < GPT; ++k2) {
        live[k2] = !PARTIAL || t + k2 * NT < SH.groups();
        int col, q;
        lds_group(SH, t, k2, &col, &q);
        const uint8_t* base = lds + (q * R) * pitch + col * SH.read_bytes();
#pragma unroll
        for (int r = 0; r < R; ++r) src[k2][r] = base + (R == 1 ? 0 : (r ^ key_r) * pitch);
        // destination chunk of store s of group k2: row NS * col + s, chunk q
        const int64_t out = pt + (int64_t)(NS * col) * d_a * W + q * 16;
#pragma unroll
        for (int s2 = 0; s2 < NS; ++s2) dst[k2][s2] = at<SWZ>(gdst, out + s2 * d_a * W, z);
    }
    __builtin_amdgcn_sched_barrier(0);
    u32x4 o[GPT][NS];
    if constexpr (W == 16) {
#pragma unroll
        for (int k2 = 0; k2 < GPT; ++k2)
            if (live[k2]) o[k2][0] = *reinterpret_cast<const u32x4*>(src[k2][0]);
        __builtin_amdgcn_sched_barrier(0);
    } else if constexpr (W == 8) {
        u32x2 x[GPT][2];
#pragma unroll
        for (int k2 = 0; k2 < GPT; ++k2)
            if (live[k2])
#pragma unroll
                for (int r = 0; r < 2; ++r) x[k2][r] = *reinterpret_cast<const u32x2*>(src[k2][r]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int k2 = 0; k2 < GPT; ++k2) {
            if (!live[k2]) continue;
            uint32_t lo[2] = {x[k2][0].x, x[k2][1].x}, hi[2] = {x[k2][0].y, x[k2][1].y};
            unrotate<2>(lo, key_r);
            unrotate<2>(hi, key_r);
            o[k2][0] = u32x4{lo[0], hi[0], lo[1], hi[1]};
        }
    } else {
        uint32_t d[GPT][R];
#pragma unroll
        for (int k2 = 0; k2 < GPT; ++k2)
            if (live[k2])
#pragma unroll
                for (int r = 0; r < R; ++r) d[k2][r] = *reinterpret_cast<const uint32_t*>(src[k2][r]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int k2 = 0; k2 < GPT; ++k2) {
            if (!live[k2]) continue;
            unrotate<R>(d[k2], key_r);
            if constexpr (W == 4) {
                o[k2][0] = u32x4{d[k2][0], d[k2][1], d[k2][2], d[k2][3]};
            } else if constexpr (W == 2) {
                // d[m] = (b0+m, a=2col) | (b0+m, a=2col+1) << 16
                uint32_t* p0 = reinterpret_cast<uint32_t*>(&o[k2][0]);
                uint32_t* p1 = reinterpret_cast<uint32_t*>(&o[k2][1]);
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    const uint32_t x = d[k2][2 * kk], y = d[k2][2 * kk + 1];
                    p0[kk] = (x & 0xffffu) | (y << 16);
                    p1[kk] = (x >> 16) | (y & 0xffff0000u);
                }
            } else {
                // W == 1: d[m] holds bytes (b0+m, a=4col+t), t = 0..3.
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) {
                    uint32_t* p = reinterpret_cast<uint32_t*>(&o[k2][tt]);
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk) {
                        const int sh = 8 * tt;
                        p[kk] = ((d[k2][4 * kk] >> sh) & 0xffu) | (((d[k2][4 * kk + 1] >> sh) & 0xffu) << 8) |
                                (((d[k2][4 * kk + 2] >> sh) & 0xffu) << 16) | (((d[k2][4 * kk + 3] >> sh) & 0xffu) << 24);
                    }
                }
            }
        }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k2 = 0; k2 < GPT; ++k2)
        if (live[k2])
#pragma unroll
            for (int s2 = 0; s2 < NS; ++s2) {
                if constexpr (DEV) st16_dev(dst[k2][s2], o[k2][s2]);
                else st16(dst[k2][s2], o[k2][s2]);
            }
}

// One element of W bytes, moved in pieces of min(W, 4) bytes (the LDS pitch
// and the element bases are multiples of that).
}  // namespace tpl
