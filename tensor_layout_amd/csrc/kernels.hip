// kernels.hip -- gfx950 kernels of permute_layout and the C entry points.
//
// permute_layout page, "Algorithm" step 3: each lane reads its elements
// through the source layout into registers, the lanes synchronise, and the
// registers are written back through the destination layout.  On gfx950 the
// reads and writes go to HBM, so both sides are 16-byte vector accesses that
// cover whole 128-byte lines, and the element exchange between them happens
// in registers (lane quads, DPP) or through LDS with XOR-ordered phases.
// Data moves as integers only; no floating-point instruction touches it.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <unordered_map>

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
        __builtin_nontemporal_store(v, reinterpret_cast<T*>(at<SWZ>(a.dst, d_o * a.w + c * V, a.zd)));
    }
}

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
                st16(at<SWZ>(a.dst, dofs, a.zd), y);
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
// the measured gfx950 LDS banks.

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

// Phase 1 of an LDS tile: the TB x TA source tile at st (rows srow bytes
// apart) through registers into LDS, element (b, a) at b * pitch + a * W.
// Each thread loads CPT 16-byte chunks, then writes them in 16 / WW pieces
// whose order is rotated by key_w.
template <int W, int TB, int TA, int CPT, int WW, bool SWZ = false>
__device__ __forceinline__ void tile_to_lds(uint8_t* lds, const uint8_t* gsrc, int64_t pt, int64_t srow, int pitch,
                                            int t, int key_w, const Swz& z = Swz{}) {
    constexpr LdsShape SH{W, TB, TA, CPT};
    constexpr int NT = SH.threads();
    constexpr int CPR = TA * W / 16;
    constexpr int NP = 16 / WW;   // pieces per chunk
    u32x4 v[CPT];
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
        const int cid = t + k * NT;
        v[k] = ld16(at<SWZ>(gsrc, pt + (cid / CPR) * srow + (cid % CPR) * 16, z));
    }
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

// Phase 2 of an LDS tile: LDS through registers to the destination tile at
// dt (destination rows d_a elements apart).  A thread reads R words of one
// LDS column, rows in the order r ^ key_r, restores their order, packs them
// and stores 16-byte destination chunks.
template <int W, int TB, int TA, int CPT, bool SWZ = false>
__device__ __forceinline__ void tile_from_lds(const uint8_t* lds, uint8_t* gdst, int64_t pt, int64_t d_a, int pitch,
                                              int t, int key_r, const Swz& z = Swz{}) {
    constexpr LdsShape SH{W, TB, TA, CPT};
    constexpr int NT = SH.threads();
    constexpr int R = SH.reads_per_group();       // reads per group
    constexpr int GPT = SH.groups_per_thread();   // groups per thread
#pragma unroll
    for (int k2 = 0; k2 < GPT; ++k2) {
        if (SH.groups() % NT != 0 && t + k2 * NT >= SH.groups()) break;
        int col, q;
        lds_group(SH, t, k2, &col, &q);
        const uint8_t* base = lds + (q * R) * pitch + col * SH.read_bytes();
        if constexpr (W == 16) {
            const u32x4 x = *reinterpret_cast<const u32x4*>(base);
            st16(at<SWZ>(gdst, pt + (int64_t)col * d_a * 16 + q * 16, z), x);
        } else if constexpr (W == 8) {
            uint32_t lo[2], hi[2];
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                const int j = r ^ key_r;
                u32x2 x = *reinterpret_cast<const u32x2*>(base + j * pitch);
                lo[r] = x.x;
                hi[r] = x.y;
            }
            unrotate<2>(lo, key_r);
            unrotate<2>(hi, key_r);
            st16(at<SWZ>(gdst, pt + (int64_t)col * d_a * W + q * 16, z), u32x4{lo[0], hi[0], lo[1], hi[1]});
        } else {
            uint32_t d[R];
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int j = r ^ key_r;
                d[r] = *reinterpret_cast<const uint32_t*>(base + j * pitch);
            }
            unrotate<R>(d, key_r);
            if constexpr (W == 4) {
                st16(at<SWZ>(gdst, pt + (int64_t)col * d_a * 4 + q * 16, z), u32x4{d[0], d[1], d[2], d[3]});
            } else if constexpr (W == 2) {
                // d[m] = (b0+m, a=2col) | (b0+m, a=2col+1) << 16
                u32x4 o0, o1;
                uint32_t* p0 = reinterpret_cast<uint32_t*>(&o0);
                uint32_t* p1 = reinterpret_cast<uint32_t*>(&o1);
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    const uint32_t x = d[2 * kk], y = d[2 * kk + 1];
                    p0[kk] = (x & 0xffffu) | (y << 16);
                    p1[kk] = (x >> 16) | (y & 0xffff0000u);
                }
                const int64_t out = pt + (int64_t)(2 * col) * d_a * 2 + q * 16;
                st16(at<SWZ>(gdst, out, z), o0);
                st16(at<SWZ>(gdst, out + d_a * 2, z), o1);
            } else {
                // W == 1: d[m] holds bytes (b0+m, a=4col+t), t = 0..3.
                u32x4 o[4];
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) {
                    uint32_t* p = reinterpret_cast<uint32_t*>(&o[tt]);
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk) {
                        const int sh = 8 * tt;
                        p[kk] = ((d[4 * kk] >> sh) & 0xffu) | (((d[4 * kk + 1] >> sh) & 0xffu) << 8) |
                                (((d[4 * kk + 2] >> sh) & 0xffu) << 16) | (((d[4 * kk + 3] >> sh) & 0xffu) << 24);
                    }
                }
                const int64_t out = pt + (int64_t)(4 * col) * d_a + q * 16;
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) st16(at<SWZ>(gdst, out + tt * d_a, z), o[tt]);
            }
        }
    }
}

// One element of W bytes, moved in pieces of min(W, 4) bytes (the LDS pitch
// and the element bases are multiples of that).
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
        tile_from_lds<W, TB, TA, CPT, SWZ>(lds, a.dst, (d_o + a0 * a.d_a + b0) * W, a.d_a, pitch, t, key_r, a.zd);
        __syncthreads();   // LDS is reused by the next tile of this workgroup
    }
}

template <int W, int TB, int TA, int CPT, int WW, int NB, bool BIG>
__global__ void __launch_bounds__(TB * TA * W / (16 * CPT)) k_lds(LdsArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    // Plain operands take the code without swizzle arithmetic (a uniform branch).
    if ((a.zs.ymask | a.zd.ymask) == 0) lds_loop<W, TB, TA, CPT, WW, NB, BIG, false>(a, lds);
    else lds_loop<W, TB, TA, CPT, WW, NB, BIG, true>(a, lds);
}

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
            tile_to_lds<W, T, T, CPT, WW>(l0, a.src, px, a.s_b * W, pitch, t, key_w);
            if (two) tile_to_lds<W, T, T, CPT, WW>(l1, a.src, py, a.s_b * W, pitch, t, key_w);
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
// Records kernel (layouts whose short side is a whole record of F fields,
// any F: float3 or RGB records to field arrays and back).  The tile holds
// TR consecutive records in LDS in record order, byte b = (r F + f) W of
// the tile's dense block in 16-byte chunk b / 16.  DENSE_SRC: the source
// tile is one contiguous block (records one after the other), loaded as
// 16-byte chunks; every field's TR elements then leave as 16-byte pieces of
// that field's destination row.  Otherwise the mirror: 16-byte pieces of
// each field's source row in, the contiguous destination block out.  A
// tile with fewer than TR records goes element by element (plain record
// order in both phases).
//
// Lane q of the piece phase touches record q CE + k, so neighbouring lanes
// are 16 F bytes apart, a whole number of chunks: in plain record order
// they share at most 8 of the 32 banks (4-way conflicts).  TURN places
// chunk c turned by dwords (c / 8) mod 4 (elements of at most 4 bytes) or
// by halves (c / 16) mod 2 (8-byte elements), which spreads lanes with
// equal c mod 8 (resp. 16) over the other positions: no conflicts for odd
// F, half of them for even F, and the chunk phase still moves whole
// aligned chunks.  It pays only where the piece phase writes LDS with
// elements of 4 bytes or more (fields to records: +5% for fp32); where the
// piece phase reads, or elements are narrower, the slot arithmetic per
// element costs more than the conflicts (up to -16% for bytes), so the
// other instances keep plain record order.

template <int W>
__device__ __forceinline__ int rec_turn(int c) {   // bytes
    constexpr int TM = W <= 4 ? 12 : W == 8 ? 8 : 0;
    return (c >> 1) & TM;
}

template <int W, bool TURN>
__device__ __forceinline__ int rec_slot(int b) {
    if constexpr (!TURN) return b;
    else return (b & ~15) | ((b + rec_turn<W>(b >> 4)) & 15);
}

// The contents of chunk c read back out of its (turned) slot.
template <int W, bool TURN>
__device__ __forceinline__ u32x4 rec_unturn(u32x4 v, int c) {
    if constexpr (TURN) {
        const int r = rec_turn<W>(c) >> 2;   // dwords
        if (r & 1) v = v.yzwx;
        if (r & 2) v = v.zwxy;
    }
    return v;
}

template <int W, bool DENSE_SRC, int NB, bool BIG>
__global__ void __launch_bounds__(256) k_rec(RecArgs a) {
    constexpr int NT = 256;
    constexpr int CE = 16 / W;   // elements per 16-byte piece
    constexpr bool TURN = !DENSE_SRC && W >= 4;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int t = threadIdx.x;
    const int F = a.F;
    for (int64_t tile = blockIdx.x; tile < a.ntiles; tile += gridDim.x) {
        int64_t item, ti;
        split<BIG>(tile, a.ntr, a.div_ntr, item, ti);
        int64_t so, d_o;
        modes_offsets<NB, BIG>(a.batch, item, so, d_o);
        const int64_t r0 = ti * a.TR;
        const int nr = (int)(a.nrec - r0 < a.TR ? a.nrec - r0 : a.TR);
        const int nel = nr * F;
        // element (r, f) of this tile: dense side at block + r F + f, sparse
        // side at row f: f * fstride + r0 + r
        const int64_t block = DENSE_SRC ? so + r0 * F : d_o + r0 * F;
        const int64_t rows = DENSE_SRC ? d_o + r0 : so + r0;
        if (nr == a.TR) {
            const int nchunks = nel * W / 16;    // == F * TR / CE
            const int nq = a.TR / CE;            // pieces per field row
            if constexpr (DENSE_SRC) {
                // Four chunk loads in flight per lane before their LDS writes
                // (a plain loop waits on each load): +10% on float3 records,
                // neutral for bytes.  The mirror direction measured faster
                // with one piece at a time.
                constexpr int U = 4;
                for (int c0 = 0; c0 < nchunks; c0 += U * NT) {
                    u32x4 v[U];
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        const int c = c0 + u * NT + t;
                        if (c < nchunks) v[u] = ld16(a.src + block * W + (int64_t)c * 16);
                    }
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        const int c = c0 + u * NT + t;
                        if (c < nchunks) *reinterpret_cast<u32x4*>(lds + c * 16) = v[u];
                    }
                }
            } else {
                for (int g = t; g < nchunks; g += NT) {
                    const int q = g % nq, f = g / nq;
                    const u32x4 v = ld16(a.src + (rows + f * a.fstride + (int64_t)q * CE) * W);
                    const uint8_t* vb = reinterpret_cast<const uint8_t*>(&v);
#pragma unroll
                    for (int k = 0; k < CE; ++k)
                        copy_elem<W>(lds + rec_slot<W, TURN>(((q * CE + k) * F + f) * W), vb + k * W);
                }
            }
            __syncthreads();
            if constexpr (DENSE_SRC) {
                for (int g = t; g < nchunks; g += NT) {
                    const int q = g % nq, f = g / nq;
                    u32x4 v;
                    uint8_t* vb = reinterpret_cast<uint8_t*>(&v);
#pragma unroll
                    for (int k = 0; k < CE; ++k)
                        copy_elem<W>(vb + k * W, lds + rec_slot<W, TURN>(((q * CE + k) * F + f) * W));
                    st16(a.dst + (rows + f * a.fstride + (int64_t)q * CE) * W, v);
                }
            } else {
                for (int c = t; c < nchunks; c += NT)
                    st16(a.dst + block * W + (int64_t)c * 16,
                         rec_unturn<W, TURN>(*reinterpret_cast<const u32x4*>(lds + c * 16), c));
            }
        } else {
            for (int i = t; i < nel; i += NT) {
                const int f = i / nr, r = i % nr;
                const uint8_t* sp = DENSE_SRC ? a.src + (block + r * F + f) * W : a.src + (rows + f * a.fstride + r) * W;
                copy_elem<W>(lds + (r * F + f) * W, sp);
            }
            __syncthreads();
            for (int i = t; i < nel; i += NT) {
                const int f = i / nr, r = i % nr;
                uint8_t* dp = DENSE_SRC ? a.dst + (rows + f * a.fstride + r) * W : a.dst + (block + r * F + f) * W;
                copy_elem<W>(dp, lds + (r * F + f) * W);
            }
        }
        __syncthreads();   // LDS is reused by the next tile of this workgroup
    }
}

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
// Launch.

static int64_t cap_grid(int64_t grid, int64_t block) {
    int64_t lim = kMaxThreads / block;
    return grid < lim ? (grid < 1 ? 1 : grid) : lim;
}

template <int NB, bool BIG>
static hipError_t launch_lds(const Plan& p, const LdsArgs& a, hipStream_t st) {
    dim3 grid((unsigned)cap_grid(p.grid, p.block)), block((unsigned)p.block);
    const int w = p.w, tb = p.tile_b, ta = p.tile_a, cpt = p.cpt, ww = p.ww;
#define TPL_LDS_CASE(W_, TB_, TA_, CPT_, WW_)                                                          \
    if (w == W_ && tb == TB_ && ta == TA_ && cpt == CPT_ && ww == WW_) {                                 \
        hipLaunchKernelGGL((k_lds<W_, TB_, TA_, CPT_, WW_, NB, BIG>), grid, block, p.lds_bytes, st, a); \
        return hipGetLastError();                                                                        \
    }
#define TPL_LDS_SHAPE(W_, TB_, TA_, CPT_) \
    TPL_LDS_CASE(W_, TB_, TA_, CPT_, 16) TPL_LDS_CASE(W_, TB_, TA_, CPT_, 8) TPL_LDS_CASE(W_, TB_, TA_, CPT_, 4)
    TPL_LDS_SHAPE(1, 128, 128, 2)
    TPL_LDS_SHAPE(1, 64, 128, 2)
    TPL_LDS_SHAPE(2, 256, 64, 2)
    TPL_LDS_SHAPE(2, 128, 64, 2)
    TPL_LDS_SHAPE(2, 32, 64, 2)
    TPL_LDS_SHAPE(4, 64, 64, 2)
    TPL_LDS_SHAPE(4, 32, 32, 2)
    TPL_LDS_SHAPE(8, 32, 64, 2)
    TPL_LDS_SHAPE(8, 16, 32, 2)
    TPL_LDS_SHAPE(16, 64, 16, 2)
    TPL_LDS_SHAPE(16, 16, 64, 2)
    TPL_LDS_SHAPE(16, 16, 16, 2)
#undef TPL_LDS_SHAPE
#undef TPL_LDS_CASE
    return hipErrorInvalidConfiguration;
}

template <int NB, bool BIG>
static hipError_t launch_swap(const Plan& p, const LdsArgs& a, hipStream_t st) {
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
static hipError_t launch_nb(const Plan& p, const uint8_t* src, uint8_t* dst, hipStream_t st) {
    switch (p.kernel) {
    case TPL_KERNEL_COPY: {
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
    case TPL_KERNEL_QUAD: {
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
    case TPL_KERNEL_LDS: {
        LdsArgs a = p.lds;
        a.src = src;
        a.dst = dst;
        return launch_lds<NB, BIG>(p, a, st);
    }
    case TPL_KERNEL_SWAP: {
        LdsArgs a = p.lds;
        a.src = src;
        a.dst = dst;
        return launch_swap<NB, BIG>(p, a, st);
    }
    case TPL_KERNEL_REC: {
        RecArgs a = p.rec;
        a.src = src;
        a.dst = dst;
        dim3 grid((unsigned)cap_grid(p.grid, 256)), block(256);
#define TPL_REC_W(W_)                                                                                   \
    if (p.w == W_) {                                                                                    \
        if (p.rec_dense_src) hipLaunchKernelGGL((k_rec<W_, true, NB, BIG>), grid, block, p.lds_bytes, st, a); \
        else hipLaunchKernelGGL((k_rec<W_, false, NB, BIG>), grid, block, p.lds_bytes, st, a);         \
    }
        TPL_REC_W(1)
        TPL_REC_W(2)
        TPL_REC_W(4)
        TPL_REC_W(8)
        TPL_REC_W(16)
#undef TPL_REC_W
        return hipGetLastError();
    }
    case TPL_KERNEL_ETILE: {
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
    case TPL_KERNEL_REG16: {
        Reg16Args a = p.reg16;
        a.src = src;
        a.dst = dst;
        hipLaunchKernelGGL((k_reg16<NB, BIG>), dim3((unsigned)cap_grid(p.grid, 256)), dim3(256), 0, st, a);
        return hipGetLastError();
    }
    default:
        return hipSuccess;
    }
}

template <bool BIG>
static hipError_t launch_big(const Plan& p, const uint8_t* src, uint8_t* dst, hipStream_t st) {
    if (p.kernel == TPL_KERNEL_GATHER) {
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
    switch (nb_class(p.batch_modes)) {
    case 0: return launch_nb<0, BIG>(p, src, dst, st);
    case 1: return launch_nb<1, BIG>(p, src, dst, st);
    case 2: return launch_nb<2, BIG>(p, src, dst, st);
    default: return launch_nb<-1, BIG>(p, src, dst, st);
    }
}

// ---------------------------------------------------------------------------
// Plan cache and error text.

static thread_local std::string g_last_error;

// Records the reason text of a non-OK return for tpl_last_error().
int fail_status(int status, const std::string& why) {
    g_last_error = why;
    return status;
}

static int fail(int status, const std::string& why) { return fail_status(status, why); }

struct PlanCache {
    std::mutex mu;
    std::unordered_map<std::string, Plan> map;
};

static PlanCache& cache() {
    static PlanCache c;
    return c;
}

static bool log_enabled() {
    static int on = -1;
    if (on < 0) {
        const char* e = getenv("TPL_LOG");
        on = (e && *e && *e != '0') ? 1 : 0;
    }
    return on == 1;
}

static const char* kernel_name(int k) {
    switch (k) {
    case TPL_KERNEL_GATHER: return "gather";
    case TPL_KERNEL_QUAD: return "quad";
    case TPL_KERNEL_LDS: return "lds";
    case TPL_KERNEL_REG16: return "reg16";
    case TPL_KERNEL_COPY: return "copy";
    case TPL_KERNEL_SWAP: return "swap";
    case TPL_KERNEL_REC: return "rec";
    case TPL_KERNEL_ETILE: return "etile";
    default: return "none";
    }
}

// The planning inputs of one call, zero-padded to a fixed size so that two
// calls compare with memcmp.
struct PlanKey {
    int32_t w, rank, sa, da, inplace, pad;
    int32_t zs[3], zd[3];
    int64_t ext[TPL_MAX_RANK], ss[TPL_MAX_RANK], ds[TPL_MAX_RANK], offs[2], batch;
};

static Plan get_plan_shared(int w, int rank, const int64_t* ext, const int64_t* ss, const int64_t* ds,
                            const int64_t* offs, int64_t batch, int sa, int da, bool inplace, const SwzSpec& zs,
                            const SwzSpec& zd);

// Repeated calls with one layout (the usual case in a loop) skip the shared
// cache: each thread remembers its last plan of each kind (src != dst, and
// src == dst).
static const Plan& get_plan(int w, int rank, const int64_t* ext, const int64_t* ss, const int64_t* ds,
                            const int64_t* offs, int64_t batch, int sa, int da, bool inplace, const SwzSpec& zs,
                            const SwzSpec& zd) {
    thread_local PlanKey last_key[2];
    thread_local Plan last_plan[2];
    thread_local bool have[2] = {false, false};
    const int slot = inplace ? 1 : 0;
    PlanKey k;
    std::memset(&k, 0, sizeof k);
    k.w = w;
    k.rank = rank;
    k.sa = sa;
    k.da = da;
    k.inplace = inplace;
    k.zs[0] = zs.bits;
    k.zs[1] = zs.base;
    k.zs[2] = zs.shift;
    k.zd[0] = zd.bits;
    k.zd[1] = zd.base;
    k.zd[2] = zd.shift;
    for (int i = 0; i < rank; ++i) {
        k.ext[i] = ext[i];
        k.ss[i] = ss[i];
        k.ds[i] = ds[i];
    }
    k.offs[0] = offs[0];
    k.offs[1] = offs[1];
    k.batch = batch;
    if (have[slot] && std::memcmp(&k, &last_key[slot], sizeof k) == 0) return last_plan[slot];
    last_plan[slot] = get_plan_shared(w, rank, ext, ss, ds, offs, batch, sa, da, inplace, zs, zd);
    last_key[slot] = k;
    have[slot] = true;
    return last_plan[slot];
}

static Plan get_plan_shared(int w, int rank, const int64_t* ext, const int64_t* ss, const int64_t* ds,
                            const int64_t* offs, int64_t batch, int sa, int da, bool inplace, const SwzSpec& zs,
                            const SwzSpec& zd) {
    std::string key;
    key.reserve(64 + rank * 24);
    auto put = [&](int64_t x) { key.append(reinterpret_cast<const char*>(&x), sizeof x); };
    put(w);
    put(rank);
    for (int i = 0; i < rank; ++i) {
        put(ext[i]);
        put(ss[i]);
        put(ds[i]);
    }
    put(offs[0]);
    put(offs[1]);
    put(batch);
    put(sa);
    put(da);
    put(inplace ? 1 : 0);
    put(zs.bits);
    put(zs.base);
    put(zs.shift);
    put(zd.bits);
    put(zd.base);
    put(zd.shift);
    PlanCache& c = cache();
    {
        std::lock_guard<std::mutex> lk(c.mu);
        auto it = c.map.find(key);
        if (it != c.map.end()) return it->second;
    }
    Plan p = inplace ? plan_inplace(w, rank, ext, ss, ds, offs, batch, sa, da, zs, zd)
                     : plan_gfx950(w, rank, ext, ss, ds, offs, batch, sa, da, zs, zd);
    if (log_enabled()) {
        std::fprintf(stderr, "[tpl] plan w=%d kernel=%s status=%d shard=", w, kernel_name(p.kernel), p.status);
        for (int i = 0; i < p.shard.rank; ++i)
            std::fprintf(stderr, "(%lld:%lld,%lld)", (long long)p.shard.m[i].e, (long long)p.shard.m[i].s,
                         (long long)p.shard.m[i].d);
        std::fprintf(stderr, " P=%lld k=%d shift=%d mask=%d k_w=%d shift_w=%d tile=%dx%d pitch=%d grid=%lld block=%lld\n",
                     (long long)p.P, p.k, p.shift, p.mask, p.k_w, p.shift_w, p.tile_b, p.tile_a, p.pitch,
                     (long long)p.grid, (long long)p.block);
    }
    std::lock_guard<std::mutex> lk(c.mu);
    if (c.map.size() > 4096) c.map.clear();
    c.map.emplace(key, p);
    return p;
}

static int ptr_align(const void* p) {
    uintptr_t x = (uintptr_t)p;
    int a = 1;
    while (a < 256 && (x % (2 * a)) == 0) a *= 2;
    return a;
}

static int64_t cosize_side(const Shard& sh, bool src) {
    int64_t c = 1;
    for (int i = 0; i < sh.rank; ++i) c += (sh.m[i].e - 1) * (src ? sh.m[i].s : sh.m[i].d);
    return c;
}

// Bytes from a side's base to one past its last byte.  A swizzle only
// rewrites the bits below the top of its target field, so no swizzled offset
// of an offset <= last exceeds last with all those bits set.
static int64_t reach_bytes(const Plan& p, bool src) {
    const int64_t last = (cosize_side(p.shard, src) - 1) * p.w + (p.w - 1);
    const int64_t y = swz_bytes(src ? p.zs : p.zd, p.w).ymask;
    return (y ? (last | y | (y - 1)) : last) + 1;
}

static SwzSpec spec_of(const tpl_swizzle* z) {
    SwzSpec s;
    if (z) {
        s.bits = z->bits;
        s.base = z->base;
        s.shift = z->shift;
    }
    return s;
}

static int permute_impl(const void* src, void* dst, int w, int rank, const int64_t* ext,
                        const int64_t* ss, const int64_t* ds, const int64_t* offs_in, int64_t batch,
                        const tpl_swizzle* zs_in, const tpl_swizzle* zd_in, hipStream_t stream) {
    const SwzSpec zs = spec_of(zs_in), zd = spec_of(zd_in);
    if (rank < 1 || rank > TPL_MAX_RANK) return fail(TPL_E_ARG, "rank must be in 1..8");
    if (!ext || !ss || !ds) return fail(TPL_E_ARG, "extents/strides arrays must not be NULL");
    if (w != 1 && w != 2 && w != 4 && w != 8 && w != 16)
        return fail(TPL_E_DTYPE_WIDTH, "unsupported dtype byte width (must be 1, 2, 4, 8 or 16)");
    if (batch < 0) return fail(TPL_E_ARG, "batch must be >= 0");
    for (int i = 0; i < rank; ++i)
        if (ext[i] < 0) return fail(TPL_E_ARG, "extents must be >= 0");
    int64_t n = 0;
    if (!count_elements(rank, ext, batch, &n))
        return fail(TPL_E_LAYOUT, "layouts must slice/canonicalize: element count overflows 64-bit addressing");
    static const int64_t zero[2] = {0, 0};
    const int64_t* offs = offs_in ? offs_in : zero;
    if (n == 0) return TPL_OK;
    if (!src || !dst) return fail(TPL_E_ARG, "src and dst must not be NULL");

    const uint8_t* s = reinterpret_cast<const uint8_t*>(src);
    uint8_t* d = reinterpret_cast<uint8_t*>(dst);
    const Plan& p = get_plan(w, rank, ext, ss, ds, offs, batch, ptr_align(src), ptr_align(dst), false, zs, zd);
    if (p.status != TPL_OK) return fail(p.status, p.reason);
    if (p.kernel == TPL_KERNEL_NONE) return TPL_OK;

    const uint8_t* sb = s + p.src_off_bytes;
    uint8_t* db = d + p.dst_off_bytes;
    const uint8_t* s_hi = sb + reach_bytes(p, true);
    const uint8_t* d_hi = db + reach_bytes(p, false);
    const Plan* run = &p;
    if (sb < d_hi && db < s_hi) {
        if (sb != db) return fail(TPL_E_ALIAS, "source and destination overlap but do not start at one address");
        if (!inplace_by_unit(p)) {
            // Same memory on both sides: the in-place plan of the layouts,
            // planned from the common base (offsets already applied).
            static const int64_t none[2] = {0, 0};
            const int al = ptr_align(sb);
            const Plan& q = get_plan(w, rank, ext, ss, ds, none, batch, al, al, true, zs, zd);
            if (q.status != TPL_OK) return fail(q.status, q.reason);
            run = &q;
        }
    }

    hipError_t e = run->big ? launch_big<true>(*run, sb, db, stream) : launch_big<false>(*run, sb, db, stream);
    if (e != hipSuccess) return fail(TPL_E_HIP, std::string("HIP launch failed: ") + hipGetErrorString(e));
    return TPL_OK;
}

}  // namespace tpl

// ---------------------------------------------------------------------------
// C ABI.

extern "C" {

int tpl_permute(const void* src, void* dst, int dtype_bytes, int rank, const int64_t* extents,
                const int64_t* src_strides, const int64_t* dst_strides, const int64_t* elem_offsets,
                int64_t batch, hipStream_t stream) {
    try {
        return tpl::permute_impl(src, dst, dtype_bytes, rank, extents, src_strides, dst_strides,
                                 elem_offsets, batch, nullptr, nullptr, stream);
    } catch (...) {
        return tpl::fail(TPL_E_ARG, "internal error");
    }
}

int tpl_permute_swizzled(const void* src, void* dst, int dtype_bytes, int rank, const int64_t* extents,
                         const int64_t* src_strides, const int64_t* dst_strides, const int64_t* elem_offsets,
                         int64_t batch, const tpl_swizzle* src_swizzle, const tpl_swizzle* dst_swizzle,
                         hipStream_t stream) {
    try {
        return tpl::permute_impl(src, dst, dtype_bytes, rank, extents, src_strides, dst_strides,
                                 elem_offsets, batch, src_swizzle, dst_swizzle, stream);
    } catch (...) {
        return tpl::fail(TPL_E_ARG, "internal error");
    }
}

int tpl_plan_swizzled(int dtype_bytes, int rank, const int64_t* extents, const int64_t* src_strides,
                      const int64_t* dst_strides, const int64_t* elem_offsets, int64_t batch,
                      const tpl_swizzle* src_swizzle, const tpl_swizzle* dst_swizzle, int geometry,
                      tpl_plan_info* out) {
    try {
        tpl::Plan p;
        static const int64_t zero[2] = {0, 0};
        const int64_t* offs = elem_offsets ? elem_offsets : zero;
        const tpl::SwzSpec zs = tpl::spec_of(src_swizzle), zd = tpl::spec_of(dst_swizzle);
        if (rank < 1 || rank > TPL_MAX_RANK || !extents || !src_strides || !dst_strides || batch < 0) {
            p.status = TPL_E_ARG;
            p.reason = "rank must be in 1..8, arrays non-NULL, batch >= 0";
        } else if (geometry == TPL_GEOM_PAGES32) {
            p = tpl::plan_pages32(dtype_bytes, rank, extents, src_strides, dst_strides, batch, zs, zd);
        } else if (geometry == TPL_GEOM_GFX950_HALFWAVE) {
            p = tpl::plan_halfwave(dtype_bytes, rank, extents, src_strides, dst_strides, batch, zs, zd);
        } else if (geometry == TPL_GEOM_GFX950_INPLACE) {
            p = tpl::plan_inplace(dtype_bytes, rank, extents, src_strides, dst_strides, offs, batch, 256, 256, zs,
                                  zd);
        } else if (geometry == TPL_GEOM_GFX950) {
            p = tpl::plan_gfx950(dtype_bytes, rank, extents, src_strides, dst_strides, offs, batch, 256, 256, zs,
                                 zd);
        } else {
            p.status = TPL_E_ARG;
            p.reason = "unknown geometry";
        }
        if (out) tpl::fill_info(p, out);
        if (p.status != TPL_OK) return tpl::fail(p.status, p.reason);
        return TPL_OK;
    } catch (...) {
        return tpl::fail(TPL_E_ARG, "internal error");
    }
}

int tpl_plan(int dtype_bytes, int rank, const int64_t* extents, const int64_t* src_strides,
             const int64_t* dst_strides, const int64_t* elem_offsets, int64_t batch, int geometry,
             tpl_plan_info* out) {
    return tpl_plan_swizzled(dtype_bytes, rank, extents, src_strides, dst_strides, elem_offsets, batch, nullptr,
                             nullptr, geometry, out);
}

const char* tpl_status_string(int status) {
    switch (status) {
    case TPL_OK: return "ok";
    case TPL_E_ARG: return "invalid argument";
    case TPL_E_DTYPE_WIDTH: return "unsupported dtype byte width";
    case TPL_E_DTYPE: return "dtype mismatch";
    case TPL_E_EXTENT: return "extent mismatch";
    case TPL_E_LAYOUT: return "layouts must slice/canonicalize";
    case TPL_E_NO_K: return "no conflict-free XOR swizzle";
    case TPL_E_ALIAS: return "source and destination overlap";
    case TPL_E_HIP: return "HIP error";
    default: return "unknown status";
    }
}

const char* tpl_last_error(void) { return tpl::g_last_error.c_str(); }

}  // extern "C"
