// kernels_quad.hip -- the quad kernel: 4x4 dword blocks transposed in
// registers across lanes.
#include "device.hpp"

namespace tpl {

// ---------------------------------------------------------------------------
// Quad kernel: fp32 tiles whose destination-contiguous mode b has extent 4.
// Each 4x4 block (4 rows of b, 4 consecutive columns of a) sits in four lanes
// that each hold one row (16 bytes); two exchange stages transpose it so that
// each lane holds one column, i.e. 16 contiguous destination bytes.  One wave
// per workgroup, one 16-byte load and store per lane.
//
// Wide units (a-extent a multiple of 32): a half-wave takes a 4x32 block,
// lane l = 8r + q loading row r, columns 4q..4q+3, so each row's 128 bytes
// are read by eight neighbouring lanes.  The rows of a 4x4 block are then 8
// and 16 lanes apart: the first stage uses a DPP row rotation by 8 (lanes
// l^8 inside a 16-lane row), the second v_permlane16_swap (lanes l^16);
// both are VALU operations, so the kernel issues no LDS instruction at all.
// Narrow units: a lane quad takes one 4x4 block (lane i = row i) and both
// stages are DPP quad permutations.  A stage swaps, between the two lanes,
// the entries whose column bit differs from the lane's row bit.

__device__ __forceinline__ uint32_t xchg_q1(uint32_t x) {   // quad_perm [1,0,3,2]: lane i^1
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0xB1, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t xchg_q2(uint32_t x) {   // quad_perm [2,3,0,1]: lane i^2
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x4E, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t xchg_l8(uint32_t x) {   // row_ror:8: lane l^8 in its 16-lane row
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x128, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t xchg_l16(uint32_t x, int lane) {  // lane l^16
    // v_permlane16_swap(x, x) swaps the odd 16-lane rows of its first operand
    // with the even rows of its second: the second result holds x[l+16] in
    // even rows, the first holds x[l-16] in odd rows.
    auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    return (lane & 16) ? r[0] : r[1];
}

template <bool WIDE>
__device__ __forceinline__ u32x4 transpose4(u32x4 v, int row, int lane) {
    const bool b0 = row & 1, b1 = row & 2;
    uint32_t x0 = v.x, x1 = v.y, x2 = v.z, x3 = v.w;
    uint32_t s0 = b0 ? x0 : x1, s1 = b0 ? x2 : x3;
    uint32_t u0 = WIDE ? xchg_l8(s0) : xchg_q1(s0);
    uint32_t u1 = WIDE ? xchg_l8(s1) : xchg_q1(s1);
    uint32_t a0 = b0 ? u0 : x0, a1 = b0 ? x1 : u0;
    uint32_t a2 = b0 ? u1 : x2, a3 = b0 ? x3 : u1;
    uint32_t s2 = b1 ? a0 : a2, s3 = b1 ? a1 : a3;
    uint32_t u2 = WIDE ? xchg_l16(s2, lane) : xchg_q2(s2);
    uint32_t u3 = WIDE ? xchg_l16(s3, lane) : xchg_q2(s3);
    u32x4 y;
    y.x = b1 ? u2 : a0;
    y.y = b1 ? u3 : a1;
    y.z = b1 ? a2 : u2;
    y.w = b1 ? a3 : u3;
    return y;
}

// After transpose4 a lane holds, for rows 0..3, dword j of each row's chunk
// (d[r] = row r, the 4 / W elements of columns c .. c + 4/W - 1).  Sub-dword
// elements are then regrouped so that the lane holds those columns one after
// the other, each as its 4 rows: the 16 destination bytes of 4 / W adjacent
// columns.
template <int W>
__device__ __forceinline__ u32x4 columns_from_rows(u32x4 d) {
    if constexpr (W == 4) {
        return d;
    } else if constexpr (W == 2) {
        return u32x4{(d.x & 0xffffu) | (d.y << 16), (d.z & 0xffffu) | (d.w << 16),
                     (d.x >> 16) | (d.y & 0xffff0000u), (d.z >> 16) | (d.w & 0xffff0000u)};
    } else {
        u32x4 o;
        uint32_t* op = reinterpret_cast<uint32_t*>(&o);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int s = 8 * k;
            op[k] = ((d.x >> s) & 0xffu) | (((d.y >> s) & 0xffu) << 8) | (((d.z >> s) & 0xffu) << 16) |
                    (((d.w >> s) & 0xffu) << 24);
        }
        return o;
    }
}

// SPLIT (W < 4 only): the lane's 4/W columns are not adjacent in the
// destination; each column's 4 rows (4 W bytes) are stored on their own.
template <int W, bool WIDE, int NB, bool BIG, bool SWZ, bool SPLIT>
__global__ void __launch_bounds__(64) k_quad(QuadArgs a) {
    static_assert(!SPLIT || W < 4, "split stores are for sub-dword elements");
    constexpr int CE = 16 / W;   // elements per 16-byte row chunk
    const int lane = threadIdx.x & 63;
    // WIDE: half-wave h takes unit 2g+h; row r = (lane>>3)&3, column group q = lane&7.
    // narrow: quad qi takes unit 16g+qi; row r = lane&3.
    const int r = WIDE ? (lane >> 3) & 3 : lane & 3;
    const int cq = WIDE ? lane & 7 : 0;
    const int slot = WIDE ? lane >> 5 : lane >> 2;
    constexpr int per_wave = WIDE ? 2 : 16;
    for (int64_t g = blockIdx.x; g * per_wave < a.nunits; g += gridDim.x) {
        const int64_t U = g * per_wave + slot;
        const bool act = U < a.nunits;
        u32x4 v = u32x4{0, 0, 0, 0};
        int64_t dofs = 0;
        if (act) {
            int64_t item, ua;
            split<BIG>(U, a.upr, a.div_upr, item, ua);
            int64_t so, d_o;
            modes_offsets<NB, BIG>(a.batch, item, so, d_o);
            const int64_t a0 = WIDE ? (8 * ua + cq) * CE : ua * CE;   // first column this lane loads
            v = ld16(at<SWZ>(a.src, (so + r * a.s_b + a0) * W, a.zs));
            // after the exchange: columns a0 + r * 4/W onwards (adjacent unless SPLIT)
            dofs = (d_o + (a0 + r * (4 / W)) * a.d_a) * W;
        }
        const u32x4 y = columns_from_rows<W>(transpose4<WIDE>(v, r, lane));
        if (act) {
            if constexpr (!SPLIT) {
                st16_dev(at<SWZ>(a.dst, dofs, a.zd), y);
            } else if constexpr (W == 2) {
                __builtin_nontemporal_store(u32x2{y.x, y.y}, reinterpret_cast<u32x2*>(at<SWZ>(a.dst, dofs, a.zd)));
                __builtin_nontemporal_store(u32x2{y.z, y.w},
                                            reinterpret_cast<u32x2*>(at<SWZ>(a.dst, dofs + a.d_a * 2, a.zd)));
            } else {
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    __builtin_nontemporal_store(y[k], reinterpret_cast<uint32_t*>(at<SWZ>(a.dst, dofs + k * a.d_a, a.zd)));
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Launcher.

template <int NB, bool BIG>
hipError_t launch_quad(const Plan& p, const uint8_t* src, uint8_t* dst, hipStream_t st) {
    QuadArgs a = p.quad;
    a.src = src;
    a.dst = dst;
    dim3 grid((unsigned)cap_grid(p.grid, 64)), block(64);
    const bool swz = (a.zs.ymask | a.zd.ymask) != 0;
#define TPL_QUAD_W(W_, SP_)                                                                                   \
    if (p.w == W_ && a.split == (SP_ ? 1 : 0)) {                                                             \
        if (!swz) {                                                                                          \
            if (a.wide) hipLaunchKernelGGL((k_quad<W_, true, NB, BIG, false, SP_>), grid, block, 0, st, a);   \
            else hipLaunchKernelGGL((k_quad<W_, false, NB, BIG, false, SP_>), grid, block, 0, st, a);         \
        } else {                                                                                             \
            if (a.wide) hipLaunchKernelGGL((k_quad<W_, true, NB, BIG, true, SP_>), grid, block, 0, st, a);    \
            else hipLaunchKernelGGL((k_quad<W_, false, NB, BIG, true, SP_>), grid, block, 0, st, a);          \
        }                                                                                                    \
    }
    TPL_QUAD_W(4, false)
    TPL_QUAD_W(2, false)
    TPL_QUAD_W(1, false)
    TPL_QUAD_W(2, true)
    TPL_QUAD_W(1, true)
#undef TPL_QUAD_W
    return hipGetLastError();
}

TPL_LAUNCHER_INSTANCES(launch_quad)

}  // namespace tpl
