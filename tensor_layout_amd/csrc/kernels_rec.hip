// kernels_rec.hip -- records of any field count to field rows and back.
#include "device.hpp"
#include "tile.hpp"

namespace tpl {

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
// other instances keep plain record order.  Where the piece phase reads
// 4-byte fields (records to fields) and F is odd, lanes instead read their
// four records in a per-lane order (below), which spreads them over all
// banks at the cost of a register reorder: no conflicts on float3 records
// (0.6 conflict cycles per LDS-active cycle before), at the same speed
// within 1 %.

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
                // 4-byte fields, F odd: lane groups of 8 take their piece's
                // four records in the order k ^ x (x = the group within 32
                // lanes), which puts the four lanes 8 apart, whose record
                // rows would share banks, on dwords F (k ^ x) apart: distinct
                // banks.  The registers are put back in record order after.
                const int x = (W == 4 && (F & 1)) ? (t >> 3) & 3 : 0;
                for (int g = t; g < nchunks; g += NT) {
                    const int q = g % nq, f = g / nq;
                    u32x4 v;
                    if constexpr (W == 4) {
                        uint32_t e[4];
#pragma unroll
                        for (int k = 0; k < 4; ++k)
                            e[k] = *reinterpret_cast<const uint32_t*>(lds + ((q * 4 + (k ^ x)) * F + f) * 4);
                        unrotate<4>(e, x);
                        v = u32x4{e[0], e[1], e[2], e[3]};
                    } else {
                        uint8_t* vb = reinterpret_cast<uint8_t*>(&v);
#pragma unroll
                        for (int k = 0; k < CE; ++k)
                            copy_elem<W>(vb + k * W, lds + rec_slot<W, TURN>(((q * CE + k) * F + f) * W));
                    }
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
// Launcher.

template <int NB, bool BIG>
hipError_t launch_rec(const Plan& p, const uint8_t* src, uint8_t* dst, hipStream_t st) {
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

TPL_LAUNCHER_INSTANCES(launch_rec)

}  // namespace tpl
