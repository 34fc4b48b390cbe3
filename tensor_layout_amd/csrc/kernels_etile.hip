// kernels_etile.hip -- 2-D transposes through LDS whose rows are not aligned
// to 16 bytes (or whose swizzle granules are shorter than 16 bytes).
#include "device.hpp"

namespace tpl {

// ---------------------------------------------------------------------------
// Element tiles: a TB x TA tile (TB along the destination-contiguous mode b,
// TA along the source-contiguous mode a) staged through LDS, for 2-D
// transposes whose row pitches, bases or swizzle granules rule out the
// 16-byte vectors of k_lds.  Plain operands take the vector form
// (etile_vec_loop): 16-byte aligned chunks in and out, the rows' offsets
// from 16 bytes absorbed in the LDS addresses.  Swizzled operands take the
// element form (etile_loop): one element per access; loading, neighbouring
// lanes walk a source row (TA elements: 128 or 256 bytes); storing, they
// walk a destination row.  TA and TB divide the 256 threads, so each thread
// keeps one column on each side and steps by whole rows: its addresses
// advance by a constant.  The LDS pitch is the row plus one unit of
// max(w, 4) bytes, an odd number of units, so the column read of phase 2
// (lanes on neighbouring rows) meets no bank conflict; the row write of
// phase 1 is contiguous.  Tiles follow the k_lds order in both forms.

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
    constexpr int U1 = TB / RA < 16 ? TB / RA : 16, U2 = TA / RB < 16 ? TA / RB : 16;   // steps per batch
    static_assert(NT % TA == 0 && NT % TB == 0 && TB % RA == 0 && TA % RB == 0 && (TB / RA) % U1 == 0 &&
                      (TA / RB) % U2 == 0,
                  "tile must tile the threads");
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
            // U steps at a time: U loads back to back, then their LDS writes.
            // A lane outside the item loads the tile's first element and
            // writes it to its own slot, which phase 2 never reads: with
            // unconditional writes no load stays outstanding on any path, so
            // the loads need not wait for one another.
            const int64_t first = (so + b0 * a.s_b + a0) * W;
            int64_t off = (so + (b0 + bb1) * a.s_b + a0 + aa1) * W;
            const int64_t step = (int64_t)RA * a.s_b * W;
#pragma unroll
            for (int i0 = 0; i0 < TB / RA; i0 += U1) {
                T v[U1];
#pragma unroll
                for (int u = 0; u < U1; ++u) {
                    const int bb = bb1 + (i0 + u) * RA;
                    const bool on = aa1 < na && bb < nb;
                    v[u] = __builtin_nontemporal_load(
                        reinterpret_cast<const T*>(at<SWZ>(a.src, on ? off + u * step : first, a.zs)));
                }
#pragma unroll
                for (int u = 0; u < U1; ++u)
                    *reinterpret_cast<T*>(lds + (bb1 + (i0 + u) * RA) * P + aa1 * W) = v[u];
                off += U1 * step;
            }
        }
        __syncthreads();
        {
            // U steps at a time: the LDS reads (in bounds for every lane), then
            // the stores of the elements inside the item.
            int64_t off = (d_o + (a0 + aa2) * a.d_a + b0 + bb2) * W;
            const int64_t step = (int64_t)RB * a.d_a * W;
#pragma unroll
            for (int i0 = 0; i0 < TA / RB; i0 += U2) {
                T v[U2];
#pragma unroll
                for (int u = 0; u < U2; ++u)
                    v[u] = *reinterpret_cast<const T*>(lds + bb2 * P + (aa2 + (i0 + u) * RB) * W);
#pragma unroll
                for (int u = 0; u < U2; ++u) {
                    if (bb2 < nb && aa2 + (i0 + u) * RB < na)
                        __builtin_nontemporal_store(v[u], reinterpret_cast<T*>(at<SWZ>(a.dst, off + u * step, a.zd)));
                }
                off += U2 * step;
            }
        }
        __syncthreads();   // LDS is reused by the next tile of this workgroup
    }
}

// Vector form (plain operands, W <= 4).  Loading, thread t takes chunk
// t % QS of rows t / QS + i RS, then thread t < TB the one extra chunk that
// a row piece not starting on 16 bytes reaches into, of row t / L + (TB / L)
// (t % L): the L lanes of one LDS write pass (128 / g) take rows TB / L
// apart, whose extra chunks fall in distinct banks.  A chunk may hold
// bytes outside the layout; they share its aligned 16 bytes, hence its page,
// with bytes of the layout, and are never stored.  Storing, thread t takes
// chunk t % QD of the destination rows (tile columns) t / QD + i CS; 16
// neighbouring lanes (8 for bytes, 32 for 4-byte elements) cover a column's
// row piece.  A column owns the rows [delta, delta + TB) from b0, delta being
// the elements from its destination row's address at b0 to the next 16-byte
// boundary, so that its chunks are whole; the item's first tile also owns
// rows [0, delta), stored by thread t < TA for column t.  When a column has
// delta > 0 the tile loads TB + 16 / W - 1 rows, the last ones in one more
// step.  Partial chunks, stored element by element, are left only at an
// item's first and last rows.  SHIFT = false compiles the case where every
// destination row is on 16 bytes (delta = 0, TB rows) without the shift
// arithmetic.  TALL takes the tall tile of the width (kEtileTall).
template <int W, int NB, bool BIG, bool SHIFT, bool TALL, int G>
__device__ __forceinline__ void etile_vec_loop(const LdsArgs& a, uint8_t* lds) {
    typedef typename Elem<W>::type T;
    static_assert(!TALL || W <= 2, "tall tiles exist for 1- and 2-byte elements");
    constexpr EtileShape ES = etile_vshape(W, TALL);
    constexpr int TB = ES.tb, TA = ES.ta, NT = 256, E = 16 / W;
    constexpr int QS = TA * W / 16, QD = TB * W / 16;   // chunks of a whole source / destination row piece
    constexpr int RS = NT / QS, CS = NT / QD;           // rows / columns per step
    constexpr int NS = TB / RS, ND = TA / CS;           // steps
    constexpr int L = 128 / ES.g;                       // lanes per LDS write pass
    constexpr int XR = E - 1;                           // rows loaded past TB for shifted columns
    static_assert(NT % QS == 0 && NT % QD == 0 && TB % RS == 0 && TA % CS == 0 && TB <= NT && TA <= NT &&
                      TB % L == 0 && XR * (QS + 1) <= NT && ND % G == 0,
                  "tile must tile the threads");
    static_assert(ES.rp >= (QS + 1) * 16 && ES.vrow(1) % ES.g == 0 && ES.rp % ES.g == 0 && ES.sk % ES.g == 0,
                  "LDS rows must hold every chunk at the write piece's alignment");
    const int t = threadIdx.x;
    const int q1 = t % QS, r1 = t / QS;
    const int q2 = t % QD, c2 = t / QD;
    const uint32_t pm = (uint32_t)(a.s_b * W) & 15;   // lead change per source row
    for (int64_t tile = blockIdx.x; tile < a.ntiles; tile += gridDim.x) {
        int64_t rest, tq, item, tbi, tai, wrap;
        split<BIG>(tile, a.ntb, a.div_ntb, rest, tbi);
        split<BIG>(rest, a.nta, a.div_nta, item, tq);
        split<BIG>(tq + tbi, a.nta, a.div_nta, wrap, tai);
        int64_t so, d_o;
        modes_offsets<NB, BIG>(a.batch, item, so, d_o);
        const int64_t b0 = tbi * TB, a0 = tai * TA;
        const int nb = (int)(a.e_b - b0 < TB ? a.e_b - b0 : TB), na = (int)(a.e_a - a0 < TA ? a.e_a - a0 : TA);
        const uint8_t* s0 = a.src + (so + b0 * a.s_b + a0) * W;   // row 0 of the tile's source piece
        const uint32_t L0 = (uint32_t)(uintptr_t)s0 & 15;
        const int64_t srow = a.s_b * W;
        // rows to load: XR more when some column's destination row is not on 16 bytes
        const bool shifted =
            SHIFT && (((uint32_t)(uintptr_t)(a.dst + (d_o + a0 * a.d_a + b0) * W) | (uint32_t)(a.d_a * W)) & 15) != 0;
        const int nl = shifted ? (int)(a.e_b - b0 < TB + XR ? a.e_b - b0 : TB + XR) : nb;
        // One 16-byte chunk into LDS at byte offset `at`, chunk slot q of its row,
        // written in pieces of g bytes.
        auto put = [&](int at, int q, const u32x4& v) {
            uint8_t* l = lds + at;
            if constexpr (ES.g == 16) {
                *reinterpret_cast<u32x4*>(l) = v;
            } else if constexpr (ES.g == 8) {
                // Lanes 8 chunks apart write their halves in opposite order.
                const u32x2 lo = {v.x, v.y}, hi = {v.z, v.w};
                const bool h = (q >> 3) & 1;
                *reinterpret_cast<u32x2*>(l + (h ? 8 : 0)) = h ? hi : lo;
                *reinterpret_cast<u32x2*>(l + (h ? 0 : 8)) = h ? lo : hi;
            } else {
                uint32_t* d = reinterpret_cast<uint32_t*>(l);
                d[0] = v.x;
                d[1] = v.y;
                d[2] = v.z;
                d[3] = v.w;
            }
        };
        {
            // Every lane loads and writes to LDS in each of the NS steps: a lane
            // whose chunk lies past its row piece or whose row lies past the
            // item loads the tile's first chunk instead and writes it to its
            // own slot, bytes that phase 2 never reads.  With the writes
            // unconditional no load is left outstanding on any path through
            // the loop, and the compiler issues the NS loads back to back;
            // conditional writes made it wait for each load before issuing
            // the next (16384^2 bf16, source pitch 16385: 212 -> 206 us).
            u32x4 v[NS];
            int at_lds[NS];
            const uint8_t* first = s0 - L0;
#pragma unroll
            for (int i = 0; i < NS; ++i) {
                const int bb = r1 + i * RS;
                const int lead = (int)((L0 + (uint32_t)bb * pm) & 15);
                const bool on = bb < nl && q1 * 16 < lead + na * W;
                at_lds[i] = ES.vrow(bb) + q1 * 16;
                const uint8_t* g = on ? s0 + bb * srow - lead + q1 * 16 : first;
                // The first and last chunk of a row piece may hold bytes of
                // the neighbouring tiles' pieces: ordinary loads keep them in
                // L2 for those tiles (non-temporal ones let the 16384^2 bf16
                // transpose with pitch 16385 fetch 1.8x).
                if (q1 == 0 || q1 * 16 + 16 > lead + na * W) v[i] = *reinterpret_cast<const u32x4*>(g);
                else v[i] = ld16(g);
            }
            if (t < TB) {
                // the extra chunk of a row piece not starting on 16 bytes
                const int bb = t / L + (TB / L) * (t % L);
                const int lead = (int)((L0 + (uint32_t)bb * pm) & 15);
                if (bb < nl && QS * 16 < lead + na * W)
                    put(ES.vrow(bb) + QS * 16, QS, *reinterpret_cast<const u32x4*>(s0 + bb * srow - lead + QS * 16));
            }
            if (shifted && t < XR * (QS + 1)) {
                // rows TB.. of shifted columns: thread t takes chunk t % (QS + 1) of
                // row TB + t / (QS + 1); the next tile reads them too (ordinary loads)
                const int bb = TB + t / (QS + 1), q = t % (QS + 1);
                const int lead = (int)((L0 + (uint32_t)bb * pm) & 15);
                if (bb < nl && q * 16 < lead + na * W)
                    put(ES.vrow(bb) + q * 16, q, *reinterpret_cast<const u32x4*>(s0 + bb * srow - lead + q * 16));
            }
#pragma unroll
            for (int i = 0; i < NS; ++i) put(at_lds[i], q1, v[i]);
        }
        __syncthreads();
        {
            uint8_t* d0 = a.dst + (d_o + a0 * a.d_a + b0) * W;   // the tile's destination row 0
            const int64_t drow = a.d_a * W;
            const int rows = (int)(a.e_b - b0 < TB + XR ? a.e_b - b0 : TB + XR);   // of the item, from b0
            union Chunk {
                u32x4 v;
                T e[E];
            };
            // The rows [lo, hi) a column stores and its chunk's start (bytes from
            // its destination row at b0).
            auto span = [&](int aa, int& rel, int& lo, int& hi) {
                if constexpr (SHIFT) {
                    const int lead = (int)((uint32_t)(uintptr_t)(d0 + aa * drow) & 15);
                    const int dw = (16 - lead) & 15;   // bytes to the next 16-byte boundary: delta W
                    rel = dw + q2 * 16;
                    lo = dw / W;
                    hi = lo + TB < rows ? lo + TB : rows;
                } else {
                    rel = q2 * 16;
                    lo = 0;
                    hi = nb;
                }
            };
            // Element (bb, aa) sits at its row's lead; rows outside [lo, hi)
            // read row lo (a partial chunk stores no such element).
            auto gather = [&](int aa, int rel, int lo, int hi, Chunk& u) {
                const int bbf = rel / W;   // exact: lead is a multiple of W
#pragma unroll
                for (int j = 0; j < E; ++j) {
                    const int bb = (unsigned)(bbf + j - lo) < (unsigned)(hi - lo) ? bbf + j : lo;
                    const int ls = (int)((L0 + (uint32_t)bb * pm) & 15);
                    u.e[j] = *reinterpret_cast<const T*>(lds + ES.vrow(bb) + ls + aa * W);
                }
            };
            auto emit = [&](uint8_t* D, int rel, int lo, int hi, const Chunk& u) {
                if (rel >= lo * W && rel + 16 <= hi * W) {
                    st16(D + rel, u.v);
                } else {
                    // A chunk the row piece covers in part: its elements one by one.
                    const int bbf = rel / W;
#pragma unroll
                    for (int j = 0; j < E; ++j) {
                        // Ordinary stores: the chunk's other bytes may come
                        // from another workgroup (a neighbouring item), and L2
                        // can merge the two before writing the line.
                        if ((unsigned)(bbf + j - lo) < (unsigned)(hi - lo))
                            *reinterpret_cast<T*>(D + rel + j * W) = u.e[j];
                    }
                }
            };
            // The LDS reads of G steps first, then their stores: columns past
            // the item read in-bounds LDS bytes and store nothing.
#pragma unroll
            for (int i0 = 0; i0 < ND; i0 += G) {
                Chunk u[G];
#pragma unroll
                for (int i = 0; i < G; ++i) {
                    int rel, lo, hi;
                    span(c2 + (i0 + i) * CS, rel, lo, hi);
                    gather(c2 + (i0 + i) * CS, rel, lo, hi, u[i]);
                }
#pragma unroll
                for (int i = 0; i < G; ++i) {
                    const int aa = c2 + (i0 + i) * CS;
                    int rel, lo, hi;
                    span(aa, rel, lo, hi);
                    if (aa < na && rel < hi * W) emit(d0 + aa * drow, rel, lo, hi, u[i]);
                }
            }
            if constexpr (SHIFT) {
                // The item's first tile also stores rows [0, delta) of each
                // column whose destination row is not on 16 bytes (thread t:
                // column t).
                if (t < TA && t < na && tbi == 0) {
                    uint8_t* D = d0 + t * drow;
                    const int lead = (int)((uint32_t)(uintptr_t)D & 15);
                    const int dw = (16 - lead) & 15;
                    const int hi = dw / W < rows ? dw / W : rows;
                    if (lead != 0 && -lead < hi * W) {
                        Chunk c;
                        gather(t, -lead, 0, hi, c);
                        emit(D, -lead, 0, hi, c);
                    }
                }
            }
        }
        __syncthreads();   // LDS is reused by the next tile of this workgroup
    }
}

// Destination steps of the vector form whose LDS reads are issued together,
// before their stores: all of them, but one at a time for 1-byte elements in
// the shifted form, where each element holds a register until packed (all
// four steps took 178 VGPRs and ran 6 % slower than the one-step form on
// u8 16384^2 with destination pitch 16387; two steps 1 % slower).
template <int W, bool SHIFT, bool TALL>
constexpr int etile_read_group() {
    constexpr EtileShape ES = etile_vshape(W, TALL);
    constexpr int ND = ES.ta / (256 / (ES.tb * W / 16));
    return W == 1 && SHIFT ? 1 : ND;
}

// The two forms are separate kernels: the element form's swizzle branch
// would otherwise set the vector form's register count.
template <int W, int NB, bool BIG, bool SHIFT, bool TALL, int G_ = etile_read_group<W, SHIFT, TALL>()>
__global__ void __launch_bounds__(256) k_etile_vec(LdsArgs a) {
    // the plan's LDS bytes: vrow(TB) (vrow(TB + 16 / W - 1) shifted) or more
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    etile_vec_loop<W, NB, BIG, SHIFT, TALL, G_>(a, lds);
}

template <int W, int NB, bool BIG>
__global__ void __launch_bounds__(256) k_etile(LdsArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];   // TB x pitch bytes
    // Plain operands take the code without swizzle arithmetic (a uniform branch).
    if ((a.zs.ymask | a.zd.ymask) == 0) etile_loop<W, NB, BIG, false>(a, lds);
    else etile_loop<W, NB, BIG, true>(a, lds);
}

// ---------------------------------------------------------------------------
// Launcher: the plan picks the form (plain operands of up to 4 bytes take
// the vector form).

// The vector form of width W: aligned (vform 1) or shifted (2) destination
// rows, the width's tile or its tall tile (the plan's TB says which).
template <int W, int NB, bool BIG>
static void launch_etile_vec(const Plan& p, const LdsArgs& a, dim3 grid, dim3 block, hipStream_t st) {
    constexpr bool CT = W <= 2;   // a tall tile exists
    const bool tall = CT && p.tile_b == etile_vshape(W, true).tb;
    if (a.vform == 1) {
        if (tall) hipLaunchKernelGGL((k_etile_vec<W, NB, BIG, false, CT>), grid, block, p.lds_bytes, st, a);
        else hipLaunchKernelGGL((k_etile_vec<W, NB, BIG, false, false>), grid, block, p.lds_bytes, st, a);
    } else {
        if (tall) hipLaunchKernelGGL((k_etile_vec<W, NB, BIG, true, CT>), grid, block, p.lds_bytes, st, a);
        else hipLaunchKernelGGL((k_etile_vec<W, NB, BIG, true, false>), grid, block, p.lds_bytes, st, a);
    }
}

template <int NB, bool BIG>
hipError_t launch_etile(const Plan& p, const uint8_t* src, uint8_t* dst, hipStream_t st) {
    LdsArgs a = p.lds;
    a.src = src;
    a.dst = dst;
    dim3 grid((unsigned)cap_grid(p.grid, 256)), block(256);
#define TPL_ETILE_CASE(W_)                                                                   \
    case W_:                                                                                 \
        if (a.vform != 0) launch_etile_vec<W_, NB, BIG>(p, a, grid, block, st);             \
        else hipLaunchKernelGGL((k_etile<W_, NB, BIG>), grid, block, p.lds_bytes, st, a);   \
        break;
    switch (p.w) {
        TPL_ETILE_CASE(1)
        TPL_ETILE_CASE(2)
        TPL_ETILE_CASE(4)
    case 8: hipLaunchKernelGGL((k_etile<8, NB, BIG>), grid, block, p.lds_bytes, st, a); break;
    default: hipLaunchKernelGGL((k_etile<16, NB, BIG>), grid, block, p.lds_bytes, st, a); break;
    }
#undef TPL_ETILE_CASE
    return hipGetLastError();
}

TPL_LAUNCHER_INSTANCES(launch_etile)

}  // namespace tpl
