// planner.cpp -- host-side steps of permute_layout.
//
// permute_layout page, "Algorithm": (1) slice and canonicalise both layouts
// and regroup them onto one shard, P = elements per lane; (2) choose the XOR
// swizzle by simulating the banks of both staged phases and taking the
// smallest k that is conflict-free, else decline; (3) the two register-staged
// phases themselves, which here are the gfx950 kernels.  The operand rules
// are those of the page's "What it accepts" section.
#include "planner.hpp"

#include <algorithm>
#include <cstring>
#include <mutex>
#include <sstream>
#include <unordered_map>

namespace tpl {

// ---------------------------------------------------------------------------
// Bank geometries.

static int log2_bytes(int bytes) {
    int l = 0;
    while ((1 << l) < bytes) ++l;
    return l;
}

const Geometry& geometry_pages32() {
    // The pages' warp: 32 lanes, 32 banks of 4 bytes, element-granular (two
    // lanes in one bank conflict even inside one word).  An access of
    // w > 4 bytes spans w/4 banks and the warp is served 128/w lanes at a time.
    static const Geometry g = {
        32, 4, false,
        {32, 32, 32, 32, 32}, {32, 32, 32, 16, 8},
        {32, 32, 32, 32, 32}, {32, 32, 32, 16, 8},
        {0, 0, 0, 0, 0}, {0, 0, 0, 0, 0},
    };
    return g;
}

const Geometry& geometry_gfx950() {
    // Measured on MI355X with the LDS bank-conflict counter, two lanes at a
    // time (which lanes share a pass, which addresses share a bank) and whole
    // waves (strides, lane groups, tile maps): b32 accesses see 32 banks of
    // 4 bytes in two passes of 32 consecutive lanes; ds_read_b64 sees 64
    // banks in passes of 32 lanes; ds_read_b128 sees 64 banks in four passes
    // of 16 lanes, a pass being the lanes with equal lane bit 5 and equal
    // parity of lane bits 2, 3 and 4; writes see 32 banks with passes of 32,
    // 16 and 8 consecutive lanes for b32, b64 and b128.  Lanes reading the
    // same dword are served together.  Sub-dword accesses are modelled as b32.
    static const Geometry g = {
        64, 4, true,
        {32, 32, 32, 64, 64}, {32, 32, 32, 32, 16},
        {32, 32, 32, 32, 32}, {32, 32, 32, 16, 8},
        {0, 0, 0, 0, 1}, {0, 0, 0, 0, 0},
    };
    return g;
}

static int pass_of(const Geometry& g, bool is_write, int li, int lane) {
    const int grouping = is_write ? g.group_write[li] : g.group_read[li];
    if (grouping == 1) return ((lane >> 5) & 1) * 2 + (((lane >> 2) ^ (lane >> 3) ^ (lane >> 4)) & 1);
    return lane / (is_write ? g.pass_write[li] : g.pass_read[li]);
}

bool step_conflict_free(const Geometry& g, bool is_write, int bytes, const int64_t* addr,
                        const bool* active, int lanes) {
    const int li = log2_bytes(bytes);
    const int banks = is_write ? g.banks_write[li] : g.banks_read[li];
    const int words = bytes > g.bank_bytes ? bytes / g.bank_bytes : 1;
    // owner[pass][bank] = word using the bank in that pass, or -1; a pass
    // index is below the lane count (at most 64)
    static thread_local int64_t owner[64][64];
    for (int p = 0; p < 64; ++p)
        for (int b = 0; b < banks; ++b) owner[p][b] = -1;
    for (int l = 0; l < lanes; ++l) {
        if (active && !active[l]) continue;
        const int p = pass_of(g, is_write, li, l);
        const int64_t w0 = addr[l] / g.bank_bytes;
        for (int k = 0; k < words; ++k) {
            const int64_t word = w0 + k;
            const int bank = (int)(word % banks);
            if (owner[p][bank] >= 0 && !(g.same_word_ok && owner[p][bank] == word)) return false;
            owner[p][bank] = word;
        }
    }
    return true;
}

// ---------------------------------------------------------------------------
// Canonical shard.

Shard make_shard(int rank, const int64_t* ext, const int64_t* ss, const int64_t* ds,
                 int64_t batch) {
    Mode tmp[kMaxShard];
    int n = 0;
    if (batch > 1) {
        int64_t span_s = 1, span_d = 1;
        for (int i = 0; i < rank; ++i) {
            span_s += (ext[i] - 1) * ss[i];
            span_d += (ext[i] - 1) * ds[i];
        }
        tmp[n++] = {batch, span_s, span_d};
    }
    for (int i = 0; i < rank; ++i)
        if (ext[i] != 1) tmp[n++] = {ext[i], ss[i], ds[i]};
    Shard sh;
    if (n == 0) {
        sh.rank = 1;
        sh.m[0] = {1, 1, 1};
        return sh;
    }
    // Neighbours i, i+1 merge when both sides see one longer run.
    sh.m[0] = tmp[0];
    sh.rank = 1;
    for (int i = 1; i < n; ++i) {
        Mode& last = sh.m[sh.rank - 1];
        if (last.s == tmp[i].e * tmp[i].s && last.d == tmp[i].e * tmp[i].d) {
            last.e *= tmp[i].e;
            last.s = tmp[i].s;
            last.d = tmp[i].d;
        } else {
            sh.m[sh.rank++] = tmp[i];
        }
    }
    return sh;
}

bool dst_injective(const Shard& sh) {
    // Sufficient test: sorted by destination stride, every stride exceeds the
    // largest offset reachable with the smaller modes.
    Mode m[kMaxShard];
    int n = 0;
    for (int i = 0; i < sh.rank; ++i)
        if (sh.m[i].e > 1) m[n++] = sh.m[i];
    std::sort(m, m + n, [](const Mode& a, const Mode& b) { return a.d < b.d; });
    int64_t span = 0;
    for (int i = 0; i < n; ++i) {
        if (m[i].d <= span) return false;
        span += (m[i].e - 1) * m[i].d;
    }
    return true;
}

static int64_t shard_elements(const Shard& sh) {
    int64_t n = 1;
    for (int i = 0; i < sh.rank; ++i) n *= sh.m[i].e;
    return n;
}

static bool set_modes(Modes& out, const Shard& sh, const int* idx, int n) {
    // n never exceeds the shard rank, which make_shard keeps <= kMaxShard.
    static_assert(kMaxBatch >= kMaxShard, "mode table must hold a whole shard");
    if (n > kMaxBatch) return false;
    out.n = n;
    for (int i = 0; i < n; ++i) {
        const Mode& m = sh.m[idx[i]];
        out.ext[i] = m.e;
        out.ss[i] = m.s;
        out.ds[i] = m.d;
        out.div[i] = make_fastdiv((uint32_t)std::min<int64_t>(m.e, 0x7fffffff));
    }
    return true;
}

// ---------------------------------------------------------------------------
// The pages' plan (32-lane warp program).

static void decompose(int64_t n, const Shard& sh, int64_t* digits) {
    for (int i = sh.rank - 1; i >= 0; --i) {
        digits[i] = n % sh.m[i].e;
        n /= sh.m[i].e;
    }
}

Plan plan_pages32(int w, int rank, const int64_t* ext, const int64_t* ss, const int64_t* ds,
                  int64_t batch, const SwzSpec& zs, const SwzSpec& zd) {
    return plan_warp32(geometry_pages32(), w, rank, ext, ss, ds, batch, zs, zd);
}

Plan plan_halfwave(int w, int rank, const int64_t* ext, const int64_t* ss, const int64_t* ds,
                   int64_t batch, const SwzSpec& zs, const SwzSpec& zd) {
    return plan_warp32(geometry_gfx950(), w, rank, ext, ss, ds, batch, zs, zd);
}

static bool offsets_fit(int w, int rank, const int64_t* ext, const int64_t* ss, const int64_t* ds,
                        const int64_t* offs, int64_t batch);

// Largest P (elements per lane) the warp plan accepts.
static constexpr int64_t kWarpPlanMaxP = 4096;

// A swizzle applied to an element offset.
static int64_t swz_elem(const SwzSpec& z, int64_t m) {
    if (z.bits == 0) return m;
    return m ^ (((m >> (z.base + z.shift)) & (((int64_t)1 << z.bits) - 1)) << z.base);
}

// The pages' warp program for one region: 32 lanes, n = lane + 32 j, with
// the bank model of the given hardware (its first 32 lanes).  Swizzled
// operands: each side's offsets go through its swizzle before the bank model
// sees them.
Plan plan_warp32(const Geometry& g, int w, int rank, const int64_t* ext, const int64_t* ss,
                 const int64_t* ds, int64_t batch, const SwzSpec& zs, const SwzSpec& zd) {
    Plan p;
    p.w = w;
    p.zs = zs;
    p.zd = zd;
    if (w != 1 && w != 2 && w != 4 && w != 8 && w != 16) {
        p.status = TPL_E_DTYPE_WIDTH;
        p.reason = "unsupported dtype byte width";
        return p;
    }
    if (!swz_valid(zs) || !swz_valid(zd)) {
        p.status = TPL_E_ARG;
        p.reason = "a swizzle needs 0 <= bits <= 16, base >= 0, shift >= bits and base + shift + bits <= 48";
        return p;
    }
    for (int i = 0; i < rank; ++i) {
        if (ext[i] < 1 || ss[i] < 0 || ds[i] < 0) {
            p.status = TPL_E_LAYOUT;
            p.reason = "layouts must slice/canonicalize: extents must be >= 1 and strides >= 0";
            return p;
        }
    }
    if (batch < 1) {
        p.status = TPL_E_LAYOUT;
        p.reason = "layouts must slice/canonicalize: batch must be >= 1";
        return p;
    }
    static const int64_t no_offsets[2] = {0, 0};
    int64_t n = 0;
    if (!count_elements(rank, ext, batch, &n) || !offsets_fit(w, rank, ext, ss, ds, no_offsets, batch)) {
        p.status = TPL_E_LAYOUT;
        p.reason = "layouts must slice/canonicalize: offsets overflow 64-bit addressing";
        return p;
    }
    p.shard = make_shard(rank, ext, ss, ds, batch);
    if (!dst_injective(p.shard)) {
        p.status = TPL_E_LAYOUT;
        p.reason = "layouts must slice/canonicalize: destination is not one-to-one";
        return p;
    }
    const int lanes = 32;
    int64_t total = shard_elements(p.shard);
    if (total % lanes) {
        p.status = TPL_E_LAYOUT;
        p.reason = "layouts must slice/canonicalize: elements are not a multiple of 32 lanes";
        return p;
    }
    int64_t P = total / lanes;
    p.P = P;
    // The search simulates all P steps of the warp for every candidate k, so
    // its cost grows with the region; a register-staged program holds far
    // fewer elements per lane than this bound.
    if (P > kWarpPlanMaxP) {
        p.status = TPL_E_LAYOUT;
        p.reason = "the warp program stages at most 4096 elements per lane (P = elements / 32)";
        return p;
    }
    int kmax = 0;
    while ((2ll << kmax) <= P && kmax < 5) ++kmax;
    int64_t digits[kMaxShard];
    int64_t addr[64];
    for (int k = 0; k <= kmax; ++k) {
        if (P % (1ll << k)) continue;
        int mask = (1 << k) - 1, shift = 5 - k;
        bool ok = true;
        for (int phase = 0; phase < 2 && ok; ++phase) {
            for (int64_t r = 0; r < P && ok; ++r) {
                for (int lane = 0; lane < lanes; ++lane) {
                    int64_t j = r ^ ((lane >> shift) & mask);
                    decompose(lane + j * lanes, p.shard, digits);
                    int64_t off = 0;
                    for (int i = 0; i < p.shard.rank; ++i)
                        off += digits[i] * (phase == 0 ? p.shard.m[i].s : p.shard.m[i].d);
                    addr[lane] = swz_elem(phase == 0 ? zs : zd, off) * w;
                }
                ok = step_conflict_free(g, phase == 1, w, addr, nullptr, lanes);
            }
        }
        if (ok) {
            p.k = k;
            p.mask = mask;
            p.shift = shift;
            p.status = TPL_OK;
            return p;
        }
    }
    p.status = TPL_E_NO_K;
    p.reason = "no XOR k makes both phases bank-conflict-free";
    return p;
}

// ---------------------------------------------------------------------------
// gfx950 LDS kernel: choose the pitch and the XOR of both LDS phases.

struct LdsChoice {
    bool ok = false;
    int pitch = 0, ww = 0;
    int k_w = 0, shift_w = 0, k_r = 0, shift_r = 0;
};

// Smallest k (then largest shift) whose XOR makes every step of a phase
// conflict-free over every wave of the workgroup.
template <typename AddrFn>
static bool choose_phase(const Geometry& g, bool is_write, int bytes, int steps, int slots,
                         int threads, AddrFn addr_of, int* k_out, int* shift_out) {
    int kmax = 0;
    while ((2 << kmax) <= steps) ++kmax;
    int64_t addr[64];
    bool active[64];
    for (int k = 0; k <= kmax; ++k) {
        if (steps % (1 << k)) continue;
        int mask = (1 << k) - 1;
        for (int shift = 6 - k; shift >= 0; --shift) {
            bool ok = true;
            for (int wv = 0; wv < threads / kWave && ok; ++wv)
                for (int slot = 0; slot < slots && ok; ++slot)
                    for (int r = 0; r < steps && ok; ++r) {
                        for (int l = 0; l < kWave; ++l) {
                            addr[l] = addr_of(wv * kWave + l, slot, r, shift, mask);
                            active[l] = addr[l] >= 0;
                        }
                        ok = step_conflict_free(g, is_write, bytes, addr, active, kWave);
                    }
            if (ok) {
                *k_out = k;
                *shift_out = shift;
                return true;
            }
            if (k == 0) break;   // with mask 0 the shift does not matter
        }
    }
    return false;
}

static LdsChoice choose_lds(const LdsShape& sh) {
    const Geometry& g = geometry_gfx950();
    const int row = sh.row_bytes();
    const int pads[] = {16, 8, 4, 0, 32, 48, 64};
    for (int pad : pads) {
        int pitch = row + pad;
        int ww = (pitch % 16 == 0) ? 16 : (pitch % 8 == 0) ? 8 : 4;
        if (sh.tb * pitch > 64 * 1024) continue;
        LdsChoice c;
        c.pitch = pitch;
        c.ww = ww;
        bool okw = choose_phase(
            g, true, ww, 16 / ww, sh.cpt, sh.threads(),
            [&](int t, int slot, int r, int shift, int mask) {
                return (int64_t)lds_write_addr(sh, pitch, ww, t, slot, r, shift, mask, nullptr);
            },
            &c.k_w, &c.shift_w);
        if (!okw) continue;
        bool okr = choose_phase(
            g, false, sh.read_bytes(), sh.reads_per_group(), sh.groups_per_thread(), sh.threads(),
            [&](int t, int slot, int r, int shift, int mask) {
                return (int64_t)lds_read_addr(sh, pitch, t, slot, r, shift, mask, nullptr);
            },
            &c.k_r, &c.shift_r);
        if (!okr) continue;
        c.ok = true;
        return c;
    }
    return LdsChoice{};
}

const EtileShape* etile_shape(int w) {
    for (const EtileShape& e : kEtileShapes)
        if (e.w == w) return &e;
    return nullptr;
}

const EtileShape* etile_tall_shape(int w) {
    for (const EtileShape& e : kEtileTall)
        if (e.w == w) return &e;
    return nullptr;
}

// Tile shapes the library instantiates: (w, TB, TA, CPT), largest first.
// Two 16-byte chunks per thread: measured a little faster than four on the
// large transposes (more waves, each with less data in flight).
static const LdsShape kLdsShapes[] = {
    {1, 128, 128, 2}, {1, 64, 128, 2},
    {2, 256, 64, 2}, {2, 128, 64, 2}, {2, 32, 64, 2},
    {4, 64, 64, 2}, {4, 32, 32, 2},
    {8, 32, 64, 2}, {8, 16, 32, 2},
    {16, 64, 16, 2}, {16, 16, 64, 2}, {16, 16, 16, 2},
};

// Shapes tried first when destination rows are short next to source rows
// (the source-contiguous extent at least four times the destination-
// contiguous one): longer source pieces then pay more than longer
// destination pieces.  On MI355X, on 64 transposes of 128 x 1024, the
// fp16 tile 128 x 128 (256-byte source pieces, whole 256-byte destination
// rows, four chunks per thread) moved the 16 MiB in 7.0 us against 8.2 us
// for 128 x 64, and the fp32 tile 32 x 256 (1 KiB source pieces) in
// 13.0 us against 13.7 us for 64 x 64.
static const LdsShape kLdsShortDst[] = {
    {2, 128, 128, 4},
    {4, 32, 256, 2},
};

// Shapes for transposes whose tiles are strided on both sides (each tile
// reads and writes row pieces of a larger matrix), one per width: 32 KiB
// tiles of 512 threads (16 KiB for 16-byte elements), with dynamic LDS
// reserved so that at most two workgroups share a CU (kTwoPerCuLds: more
// than a third, at most half of the 160 KiB).  Fewer tiles in flight per CU
// relieve the L2 crossbar and the DRAM credit stalls that bound these
// layouts.  Measured on MI355X against the same transposes with the shapes
// below and up to four workgroups per CU: bf16 16384^2 176 us (was 185),
// fp32 8192^2 89.5 us (95.0), u64 4096^2 43.9 us (48.4), u8 16384^2
// 96.0 us (98.3), 16-byte 4096^2 90.5 us (92.2); never slower down to
// 32 MiB each way.  Tiles whose footprint is one contiguous block on a side
// (whole rows of adjacent destination rows) measured slower with the cap,
// and keep the shapes below.
static const LdsShape kLdsStrided[] = {
    {1, 128, 128, 4}, {2, 256, 64, 4}, {4, 128, 64, 4}, {8, 64, 64, 4}, {16, 64, 16, 2},
};
static constexpr int kTwoPerCuLds = 55 * 1024;
static constexpr int kThreePerCuLds = 41 * 1024;

static std::mutex g_choice_mu;

static LdsChoice cached_choice(const LdsShape& sh) {
    static std::unordered_map<int, LdsChoice> cache;
    int key = ((sh.w * 1024 + sh.tb) * 1024 + sh.ta) * 8 + sh.cpt;
    std::lock_guard<std::mutex> lk(g_choice_mu);
    auto it = cache.find(key);
    if (it != cache.end()) return it->second;
    LdsChoice c = choose_lds(sh);
    cache[key] = c;
    return c;
}

// ---------------------------------------------------------------------------
// Device plan.

// The records kernel decomposes the batch modes only (at most the shard).
static bool rank_ok_for_rec(const Shard& sh) { return sh.rank <= kMaxBatch + 2; }

static int pow2_align(int64_t x) {
    // largest power of two (<= 256) dividing x (x == 0 counts as 256)
    int a = 1;
    while (a < 256 && (x % (2 * a)) == 0) a *= 2;
    return a;
}

static bool all_aligned(const Shard& sh, int skip_a, int skip_b, int w, bool src_side, int align) {
    for (int i = 0; i < sh.rank; ++i) {
        int64_t st = src_side ? sh.m[i].s : sh.m[i].d;
        if (i == skip_a || i == skip_b) continue;
        if ((st * w) % align) return false;
    }
    return true;
}

// Overflow: the largest byte offset on each side (non-negative strides,
// extents >= 1) must stay below 2^58, so that every sum of terms fits.
static bool offsets_fit(int w, int rank, const int64_t* ext, const int64_t* ss, const int64_t* ds,
                        const int64_t* offs, int64_t batch) {
    const int64_t lim = (int64_t)1 << 58;
    for (int side = 0; side < 2; ++side) {
        long double span = 1;
        for (int i = 0; i < rank; ++i) span += (long double)(ext[i] - 1) * (side ? ds[i] : ss[i]);
        const long double hi = ((long double)offs[side] + (long double)batch * span) * w;
        if (hi > (long double)lim) return false;
    }
    return true;
}

bool count_elements(int rank, const int64_t* ext, int64_t batch, int64_t* out) {
    // Product of the extents and the batch; false when it exceeds 2^62
    // (a zero extent anywhere makes the product 0 and is never an overflow),
    // or when an extent or the batch is negative.
    if (batch < 0) return false;
    for (int i = 0; i < rank; ++i)
        if (ext[i] < 0) return false;
    bool zero = batch == 0;
    for (int i = 0; i < rank; ++i) zero = zero || ext[i] == 0;
    if (zero) {
        *out = 0;
        return true;
    }
    __int128 n = batch;
    for (int i = 0; i < rank; ++i) {
        n *= ext[i];
        if (n > ((__int128)1 << 62)) return false;
    }
    *out = (int64_t)n;
    return true;
}

static constexpr int kSwzGranuleLog2Cap = 30;
static constexpr int64_t kPlainGranule = (int64_t)1 << 40;

// granule_s / granule_d: bytes that stay adjacent under each side's swizzle
// (a vector access must not straddle one), at most 2^kSwzGranuleLog2Cap for a
// swizzled side; kPlainGranule for a plain side.
static Plan plan_core(int w, int rank, const int64_t* ext, const int64_t* ss, const int64_t* ds,
                      const int64_t* offs, int64_t batch, int src_align, int dst_align, int64_t granule_s,
                      int64_t granule_d) {
    Plan p;
    p.w = w;
    const bool plain = granule_s == kPlainGranule && granule_d == kPlainGranule;
    const bool vec16 = granule_s >= 16 && granule_d >= 16;
    if (w != 1 && w != 2 && w != 4 && w != 8 && w != 16) {
        p.status = TPL_E_DTYPE_WIDTH;
        p.reason = "unsupported dtype byte width (must be 1, 2, 4, 8 or 16)";
        return p;
    }
    bool neg = batch < 0;
    for (int i = 0; i < rank; ++i) neg = neg || ext[i] < 0;
    if (neg) {
        p.status = TPL_E_ARG;
        p.reason = "extents and batch must be >= 0";
        return p;
    }
    int64_t n = 0;
    if (!count_elements(rank, ext, batch, &n)) {
        p.status = TPL_E_LAYOUT;
        p.reason = "layouts must slice/canonicalize: element count overflows 64-bit addressing";
        return p;
    }
    if (n == 0) {
        p.kernel = TPL_KERNEL_NONE;
        p.shard.rank = 0;
        return p;
    }
    for (int i = 0; i < rank; ++i) {
        if (ss[i] < 0 || ds[i] < 0) {
            p.status = TPL_E_LAYOUT;
            p.reason = "layouts must slice/canonicalize: negative strides are not supported";
            return p;
        }
    }
    if (offs[0] < 0 || offs[1] < 0) {
        p.status = TPL_E_LAYOUT;
        p.reason = "layouts must slice/canonicalize: negative element offsets";
        return p;
    }
    if (!offsets_fit(w, rank, ext, ss, ds, offs, batch)) {
        p.status = TPL_E_LAYOUT;
        p.reason = "layouts must slice/canonicalize: offsets overflow 64-bit addressing";
        return p;
    }
    p.shard = make_shard(rank, ext, ss, ds, batch);
    const Shard& sh = p.shard;
    if (!dst_injective(sh)) {
        p.status = TPL_E_LAYOUT;
        p.reason = "layouts must slice/canonicalize: destination layout is not one-to-one";
        return p;
    }
    p.src_off_bytes = offs[0] * w;
    p.dst_off_bytes = offs[1] * w;
    int sa = std::min(src_align, pow2_align(p.src_off_bytes));
    int da = std::min(dst_align, pow2_align(p.dst_off_bytes));
    p.big = n >= ((int64_t)1 << 31);
    int64_t max_off = 0;
    for (int i = 0; i < sh.rank; ++i)
        max_off = std::max(max_off, (sh.m[i].e - 1) * std::max(sh.m[i].s, sh.m[i].d));
    if (max_off >= ((int64_t)1 << 31)) p.big = true;

    // The two contiguous modes.
    int a = -1, b = -1;
    for (int i = 0; i < sh.rank; ++i) {
        if (sh.m[i].e > 1 && sh.m[i].s == 1) a = i;
        if (sh.m[i].e > 1 && sh.m[i].d == 1) b = i;
    }
    p.mode_a = a;
    p.mode_b = b;
    int others[kMaxShard];
    int no = 0;
    for (int i = 0; i < sh.rank; ++i)
        if (i != a && i != b) others[no++] = i;
    p.batch_modes = no;

    auto choose_gather = [&]() {
        p.kernel = TPL_KERNEL_GATHER;
        int unit = w;
        while (unit > 1 && ((sa % unit) || (da % unit))) unit /= 2;
        int idx[kMaxShard];
        for (int i = 0; i < sh.rank; ++i) idx[i] = i;
        GatherArgs& ga = p.gather;
        set_modes(ga.modes, sh, idx, sh.rank);
        ga.total = n;
        ga.unit = unit;
        ga.w = w;
        p.P = 1;
        p.block = 256;
        p.grid = std::min<int64_t>((n + 255) / 256, 1 << 16);
        if (p.big) p.grid = std::min<int64_t>(p.grid, 1 << 15);
    };

    // 16-byte elements too small for an LDS tile: one element is one dwordx4;
    // lanes form 8x8 blocks.
    if (plain && w == 16 && a >= 0 && b >= 0 && a != b && sa % 16 == 0 && da % 16 == 0 &&
        (sh.m[b].e < 16 || sh.m[a].e < 16)) {
        p.kernel = TPL_KERNEL_REG16;
        Reg16Args& r = p.reg16;
        r.e_b = sh.m[b].e;
        r.e_a = sh.m[a].e;
        r.s_b = sh.m[b].s;
        r.d_a = sh.m[a].d;
        r.nbb = (r.e_b + 7) / 8;
        r.nba = (r.e_a + 7) / 8;
        int64_t items = 1;
        for (int i = 0; i < no; ++i) items *= sh.m[others[i]].e;
        r.nblocks = items * r.nbb * r.nba;
        if (r.nblocks >= ((int64_t)1 << 31)) p.big = true;
        r.div_nba = make_fastdiv((uint32_t)std::min<int64_t>(r.nba, 0x7fffffff));
        r.div_nbb = make_fastdiv((uint32_t)std::min<int64_t>(r.nbb, 0x7fffffff));
        set_modes(r.batch, sh, others, no);
        p.P = 1;
        p.tile_b = 8;
        p.tile_a = 8;
        p.block = 256;
        p.grid = (r.nblocks + 3) / 4;
        p.unit_is_item = (r.nbb == 1 && r.nba == 1);
        return p;
    }

    // Both sides contiguous along the same mode: copy runs in the widest
    // vector (16, 8 or 4 bytes) that divides the run and every run start.
    if (a >= 0 && a == b) {
        const int64_t run = sh.m[a].e * w;
        int vec = 0;
        for (int v : {16, 8, 4}) {
            if (v <= granule_s && v <= granule_d && run % v == 0 && sa % v == 0 && da % v == 0 && all_aligned(sh, a, -1, w, true, v) &&
                all_aligned(sh, a, -1, w, false, v)) {
                vec = v;
                break;
            }
        }
        if (vec) {
            p.kernel = TPL_KERNEL_COPY;
            CopyArgs& c = p.copy;
            c.cpr = run / vec;
            c.div_cpr = make_fastdiv((uint32_t)std::min<int64_t>(c.cpr, 0x7fffffff));
            c.nchunks = n * w / vec;
            c.w = w;
            c.vec = vec;
            if (c.nchunks >= ((int64_t)1 << 31)) p.big = true;
            // Rows in destination order (the row mode with the smallest
            // destination stride fastest): neighbouring lanes and workgroups
            // then write one sequential stream, and the reads jump instead.
            // Measured on the (1,0,2,3) axis swap of 64x128x32x32 fp32 (4 KiB
            // runs): 4.84 TB/s against 4.17 with the reads sequential.
            std::sort(others, others + no, [&](int x, int y) { return sh.m[x].d > sh.m[y].d; });
            set_modes(c.rows, sh, others, no);
            p.P = vec / w > 0 ? vec / w : 1;
            p.block = 64;
            p.grid = (c.nchunks + 63) / 64;
            return p;
        }
        choose_gather();
        return p;
    }

    if (a >= 0 && b >= 0) {
        const Mode& ma = sh.m[a];
        const Mode& mb = sh.m[b];
        bool src_ok = sa % 16 == 0 && all_aligned(sh, a, -1, w, true, 16);
        bool dst_ok = da % 16 == 0 && all_aligned(sh, b, -1, w, false, 16);
        // Blocks of 4 rows x one 16-byte chunk transposed inside lane quads.
        // A lane ends up with 16 destination bytes: one column of 4-byte
        // elements, or 4/w columns of 1- or 2-byte elements, stored as one
        // piece when adjacent in the destination (column stride 4) and one
        // column at a time otherwise.
        const int ce = 16 / w;   // elements per 16-byte chunk
        // Sub-dword columns that are not adjacent in the destination are
        // stored one by one, 4 w bytes each (every destination offset a
        // multiple of 4 elements), but only where neighbouring lanes' pieces
        // fill whole lines: along a destination-contiguous mode longer than
        // the 4-row block.  Isolated pieces (a tile of 4 rows with gaps
        // between its columns) measured slower than the element-wise kernel.
        const bool split = w < 4 && ma.d != 4;
        const bool quad_w = w == 4 || (w < 4 && (!split || mb.e > 4));
        const bool dst_ok_q = split ? (da % (4 * w) == 0 && all_aligned(sh, b, -1, w, false, 4 * w))
                                    : (da % 16 == 0 && all_aligned(sh, b, w < 4 ? a : -1, w, false, 16));
        // A longer destination-contiguous mode (records of 16-48 bytes to
        // field arrays, or back) when the LDS tile does not apply: blocks of
        // 4 rows along it become one more batch mode.
        const bool lds_fits = ma.e * w >= 64 && mb.e * w >= 64;
        const bool quad_rows = mb.e == 4 || (mb.e % 4 == 0 && !lds_fits && sh.rank + 2 <= kMaxShard);
        if (vec16 && quad_w && quad_rows && ma.e % ce == 0 && src_ok && dst_ok_q) {
            p.kernel = TPL_KERNEL_QUAD;
            QuadArgs& q = p.quad;
            q.split = split ? 1 : 0;
            // Wide units (4 rows x 8 chunks, one per 32-lane half-wave) when the
            // rows allow it: each row's 128 bytes are then one lane-ordered load.
            q.wide = (ma.e * w % 128 == 0) ? 1 : 0;
            q.upr = q.wide ? ma.e * w / 128 : ma.e / ce;
            q.div_upr = make_fastdiv((uint32_t)std::min<int64_t>(q.upr, 0x7fffffff));
            q.s_b = mb.s;
            q.d_a = ma.d;
            Shard qs = sh;
            int qidx[kMaxShard + 2];
            int nq = 0;
            for (int i = 0; i < no; ++i) qidx[nq++] = others[i];
            if (mb.e > 4 && mb.e / 4 < ma.e / ce) {
                // Few row blocks, many chunks (a field array to records of 8
                // or 12 floats): chunks and then row blocks, fastest, as batch
                // modes of narrow units, so a wave writes whole records.
                q.wide = 0;
                q.upr = 1;
                q.div_upr = make_fastdiv(1);
                qs.m[qs.rank] = Mode{ma.e / ce, ce * ma.s, ce * ma.d};
                qidx[nq++] = qs.rank++;
                qs.m[qs.rank] = Mode{mb.e / 4, 4 * mb.s, 4 * mb.d};
                qidx[nq++] = qs.rank++;
            } else if (mb.e > 4) {
                // Many row blocks (records to field arrays): the blocks as the
                // fastest batch mode, the few chunks of a record inside a unit.
                qs.m[qs.rank] = Mode{mb.e / 4, 4 * mb.s, 4 * mb.d};
                qidx[nq++] = qs.rank++;
            }
            int64_t items = 1;
            for (int i = 0; i < nq; ++i) items *= qs.m[qidx[i]].e;
            q.nunits = items * q.upr;
            if (q.nunits >= ((int64_t)1 << 31)) p.big = true;
            set_modes(q.batch, qs, qidx, nq);
            p.batch_modes = nq;
            p.P = 4;
            p.tile_b = 4;
            p.tile_a = q.wide ? 128 / w : ce;
            p.block = 64;   // one wave per workgroup
            const int64_t per_wave = q.wide ? 2 : 16;
            p.grid = (q.nunits + per_wave - 1) / per_wave;
            // One wave-instruction moves each batch item (all its loads complete
            // before its stores) when the item's units tile the wave evenly.
            p.unit_is_item = mb.e == 4 && (q.wide ? (q.upr <= 2) : (q.upr <= 16 && 16 % q.upr == 0));
            return p;
        }
        // Tiled LDS transpose.
        if (vec16 && ma.e * w >= 64 && mb.e * w >= 64 && src_ok && dst_ok) {
            const LdsShape* pick = nullptr;
            bool two_per_cu = false;
            if (ma.e >= 4 * mb.e) {
                for (const LdsShape& s : kLdsShortDst)
                    if (s.w == w && s.tb <= mb.e && s.ta <= ma.e) {
                        pick = &s;
                        break;
                    }
            } else {
                for (const LdsShape& s : kLdsStrided) {
                    if (s.w != w || s.tb > mb.e || s.ta > ma.e) continue;
                    // a tile's destination (source) footprint is one block when
                    // it spans whole destination (source) rows that are adjacent
                    const bool dst_block = s.tb == mb.e && ma.d == mb.e;
                    const bool src_block = s.ta == ma.e && mb.s == ma.e;
                    if (!dst_block && !src_block) {
                        pick = &s;
                        two_per_cu = true;
                    }
                    break;
                }
            }
            for (const LdsShape& s : kLdsShapes) {
                if (pick) break;
                if (s.w != w) continue;
                if (s.tb <= mb.e && s.ta <= ma.e) {
                    pick = &s;
                    break;
                }
            }
            if (!pick) {
                for (const LdsShape& s : kLdsShapes)
                    if (s.w == w) pick = &s;   // smallest of this width; partial tiles
            }
            LdsChoice c = cached_choice(*pick);
            if (!c.ok) {
                p.status = TPL_E_NO_K;
                p.reason = "no XOR k makes both LDS phases bank-conflict-free for this tile";
                return p;
            }
            p.kernel = TPL_KERNEL_LDS;
            LdsArgs& l = p.lds;
            l.e_b = mb.e;
            l.e_a = ma.e;
            l.s_b = mb.s;
            l.d_a = ma.d;
            l.ntb = (mb.e + pick->tb - 1) / pick->tb;
            l.nta = (ma.e + pick->ta - 1) / pick->ta;
            int64_t items = 1;
            for (int i = 0; i < no; ++i) items *= sh.m[others[i]].e;
            l.ntiles = items * l.ntb * l.nta;
            if (l.ntiles >= ((int64_t)1 << 31)) p.big = true;
            l.div_nta = make_fastdiv((uint32_t)std::min<int64_t>(l.nta, 0x7fffffff));
            l.div_ntb = make_fastdiv((uint32_t)std::min<int64_t>(l.ntb, 0x7fffffff));
            set_modes(l.batch, sh, others, no);
            l.pitch = c.pitch;
            l.shift_r = c.shift_r;
            l.mask_r = (1 << c.k_r) - 1;
            l.shift_w = c.shift_w;
            l.mask_w = (1 << c.k_w) - 1;
            p.tile_b = pick->tb;
            p.tile_a = pick->ta;
            p.cpt = pick->cpt;
            p.pitch = c.pitch;
            p.ww = c.ww;
            p.k = c.k_r;
            p.shift = c.shift_r;
            p.mask = l.mask_r;
            p.k_w = c.k_w;
            p.shift_w = c.shift_w;
            p.mask_w = l.mask_w;
            p.P = pick->reads_per_group();
            p.block = pick->threads();
            p.grid = l.ntiles;
            p.lds_bytes = pick->tb * c.pitch;
            if (two_per_cu && p.lds_bytes < kTwoPerCuLds) p.lds_bytes = kTwoPerCuLds;
            p.unit_is_item = (l.ntb == 1 && l.nta == 1 && mb.e == pick->tb && ma.e == pick->ta);
            return p;
        }
        // Records: the shorter of the two contiguous modes is a record of F
        // fields that is dense on its side (records one after the other),
        // the longer one counts records.  The dense side moves as one block.
        if (plain && rank_ok_for_rec(sh)) {
            const bool src_records = ma.e <= mb.e;   // records dense in the source
            const Mode& mf = src_records ? ma : mb;    // field mode
            const Mode& mr = src_records ? mb : ma;    // record mode
            const int64_t F = mf.e;
            const bool dense = src_records ? (mr.s == F) : (mr.d == F);
            const int64_t fstride = src_records ? mf.d : mf.s;   // field rows on the sparse side
            // 16-byte pieces on both sides of a full tile: base, batch strides
            // and field rows aligned; the block start moves by TR F w bytes.
            const bool aligned = sa % 16 == 0 && da % 16 == 0 && (fstride * w) % 16 == 0 &&
                                 all_aligned(sh, a, b, w, true, 16) && all_aligned(sh, a, b, w, false, 16);
            if (dense && F * w <= 1024 && aligned && mr.e >= ce) {
                int64_t tr = 1;
                while (tr * 2 * F * w <= 16384) tr *= 2;
                tr = std::max<int64_t>(tr, ce);
                tr = std::min<int64_t>(tr, mr.e / ce * ce);
                p.kernel = TPL_KERNEL_REC;
                p.rec_dense_src = src_records;
                RecArgs& r = p.rec;
                r.F = (int32_t)F;
                r.TR = (int32_t)tr;
                r.nrec = mr.e;
                r.ntr = (mr.e + tr - 1) / tr;
                r.div_ntr = make_fastdiv((uint32_t)std::min<int64_t>(r.ntr, 0x7fffffff));
                r.fstride = fstride;
                int64_t items = 1;
                for (int i = 0; i < no; ++i) items *= sh.m[others[i]].e;
                r.ntiles = items * r.ntr;
                if (r.ntiles >= ((int64_t)1 << 31)) p.big = true;
                set_modes(r.batch, sh, others, no);
                p.P = ce;
                p.tile_b = src_records ? (int)tr : (int)F;
                p.tile_a = src_records ? (int)F : (int)tr;
                p.block = 256;
                p.grid = r.ntiles;
                p.lds_bytes = (int)(tr * F * w);
                return p;
            }
        }
        // Element tiles: a 2-D transpose whose row pitches, bases or swizzle
        // granules rule out the 16-byte vectors of the tile kernel still moves
        // through an LDS tile: the aligned 16-byte chunks covering each row
        // piece for plain operands, one element per access otherwise;
        // neighbouring lanes along source rows on the way in and along
        // destination rows on the way out.
        const EtileShape* es = etile_shape(w);
        if (es && sa % w == 0 && da % w == 0 && ma.e >= 8 && mb.e >= 8) {
            p.kernel = TPL_KERNEL_ETILE;
            // Plain operands take the kernel's vector form (16-byte chunks
            // kept in LDS as read), swizzled ones its element form.
            const bool vform = plain && w <= 4;
            int64_t items = 1;
            for (int i = 0; i < no; ++i) items *= sh.m[others[i]].e;
            // Tall tiles (twice the rows) where they measured faster: the
            // shifted form at 2048 tall tiles or more (u8 8192^2 with
            // destination pitch 8195 75 -> 53 us, bf16 8192^2 with pitch 8193
            // 84 -> 71, u8 and bf16 16384^2 with pitches 16387 and 16385 258 ->
            // 183 and 352 -> 251; bf16 4096^2 with pitch 4097, 1024 tall
            // tiles, 21.3 -> 22.0), and bf16 with aligned destination rows at
            // 16384 or more (16384^2 with source pitch 16385 198.8 -> 195.0;
            // 8192^2 with pitch 8196, 4096 tall tiles, 51.3 -> 56.1; u8
            // 16384^2 with pitch 16387 113 -> 116).
            if (vform && w <= 2) {
                const EtileShape* tall = etile_tall_shape(w);
                const int64_t nt = items * ((mb.e + tall->tb - 1) / tall->tb) * ((ma.e + tall->ta - 1) / tall->ta);
                if ((!dst_ok && nt >= 2048) || (dst_ok && w == 2 && nt >= 16384)) es = tall;
            }
            LdsArgs& l = p.lds;
            l = LdsArgs{};
            l.e_b = mb.e;
            l.e_a = ma.e;
            l.s_b = mb.s;
            l.d_a = ma.d;
            l.ntb = (mb.e + es->tb - 1) / es->tb;
            l.nta = (ma.e + es->ta - 1) / es->ta;
            l.ntiles = items * l.ntb * l.nta;
            if (l.ntiles >= ((int64_t)1 << 31)) p.big = true;
            l.div_nta = make_fastdiv((uint32_t)std::min<int64_t>(l.nta, 0x7fffffff));
            l.div_ntb = make_fastdiv((uint32_t)std::min<int64_t>(l.ntb, 0x7fffffff));
            set_modes(l.batch, sh, others, no);
            l.pitch = vform ? es->rp : es->pitch();
            l.vform = !vform ? 0 : dst_ok ? 1 : 2;
            p.tile_b = es->tb;
            p.tile_a = es->ta;
            p.pitch = l.pitch;
            p.P = vform ? 16 / w : 1;
            p.block = 256;
            p.grid = l.ntiles;
            p.lds_bytes = !vform ? es->tb * es->pitch() : dst_ok ? es->vrow(es->tb) : es->vbytes();
            // Launches of 8192 tiles or more in the vector form with aligned
            // destination rows run at most three workgroups per CU (reserved
            // LDS): 16384^2 bf16 with source pitch 16385 (32768 tiles) 206 ->
            // 198 us, u8 16384^2 with pitch 16387 116 -> 114, fp32 8192^2
            // with pitch 8193 99.4 -> 96.3, bf16 8192^2 with pitch 8196
            // 52.9 -> 51.6.  At 2048-4096 tiles it cost up to 27 %; the
            // shifted form gained nothing at three (bf16 16384^2 with
            // destination pitch 16385) and u8 lost 4 %.
            if (dst_ok && vform && p.grid >= 8192 && p.lds_bytes < kThreePerCuLds)
                p.lds_bytes = kThreePerCuLds;
            // a whole item in one tile is read into LDS before any of it is written
            p.unit_is_item = l.ntb == 1 && l.nta == 1;
            return p;
        }
    }
    choose_gather();
    return p;
}

static int log2_width(int w) {
    int l = 0;
    while ((1 << l) < w) ++l;
    return l;
}

Swz swz_bytes(const SwzSpec& z, int w) {
    Swz b{};
    if (z.bits > 0) {
        b.ymask = (((int64_t)1 << z.bits) - 1) << (z.base + log2_width(w));
        b.shift = z.shift;
    }
    return b;
}

bool swz_valid(const SwzSpec& z) {
    if (z.bits == 0) return true;
    return z.bits > 0 && z.bits <= 16 && z.base >= 0 && z.shift >= z.bits && z.base + z.shift + z.bits <= 48;
}

Plan plan_gfx950(int w, int rank, const int64_t* ext, const int64_t* ss, const int64_t* ds,
                 const int64_t* offs, int64_t batch, int src_align, int dst_align, const SwzSpec& zs,
                 const SwzSpec& zd) {
    if (!swz_valid(zs) || !swz_valid(zd)) {
        Plan p;
        p.w = w;
        p.status = TPL_E_ARG;
        p.reason = "a swizzle needs 0 <= bits <= 16, base >= 0, shift >= bits and base + shift + bits <= 48";
        return p;
    }
    const int lw = (w == 1 || w == 2 || w == 4 || w == 8 || w == 16) ? log2_width(w) : 0;
    // A swizzle whose field starts at byte bit 30 or above still makes its
    // side swizzled: the kernels without swizzle arithmetic must not take it.
    const int64_t gs = zs.bits ? ((int64_t)1 << std::min(kSwzGranuleLog2Cap, zs.base + lw)) : kPlainGranule;
    const int64_t gd = zd.bits ? ((int64_t)1 << std::min(kSwzGranuleLog2Cap, zd.base + lw)) : kPlainGranule;
    Plan p = plan_core(w, rank, ext, ss, ds, offs, batch, src_align, dst_align, gs, gd);
    p.zs = zs;
    p.zd = zd;
    if (p.status != TPL_OK) return p;
    const Swz bs = swz_bytes(zs, w), bd = swz_bytes(zd, w);
    p.gather.zs = p.copy.zs = p.quad.zs = p.lds.zs = bs;
    p.gather.zd = p.copy.zd = p.quad.zd = p.lds.zd = bd;
    // A swizzle rewrites only bits below the top of its target field, so a
    // swizzled offset of an offset <= mx is at most mx with all those bits
    // set: 64-bit index math when that passes 2^31 elements.
    if (zs.bits || zd.bits) {
        int64_t mx = 0;
        for (int i = 0; i < p.shard.rank; ++i) {
            mx += (p.shard.m[i].e - 1) * std::max(p.shard.m[i].s, p.shard.m[i].d);
        }
        const int top = std::max(zs.bits ? zs.base + zs.bits : 0, zd.bits ? zd.base + zd.bits : 0);
        if ((mx | (((int64_t)1 << top) - 1)) >= ((int64_t)1 << 31)) p.big = true;
    }
    return p;
}

// Overlap is allowed unit-for-unit: every batch item is moved by one work
// unit that reads all before writing (the planner's unit_is_item), items sit
// at the same offsets on both sides and do not overlap each other, and an
// item covers the same span on both sides.
bool inplace_by_unit(const Plan& p) {
    if (!p.unit_is_item || p.src_off_bytes != p.dst_off_bytes) return false;
    const Shard& sh = p.shard;
    int64_t in_s = 1, in_d = 1;
    int others = 0;
    int64_t ostride = 0;
    for (int i = 0; i < sh.rank; ++i) {
        if (i == p.mode_a || i == p.mode_b) {
            in_s += (sh.m[i].e - 1) * sh.m[i].s;
            in_d += (sh.m[i].e - 1) * sh.m[i].d;
        } else {
            if (sh.m[i].s != sh.m[i].d) return false;
            ++others;
            ostride = sh.m[i].s;
        }
    }
    if (others > 1) return false;
    if (in_s != in_d) return false;
    if (others == 1 && ostride < in_s) return false;
    return true;
}

// Square tiles for in-place pair swaps, one per element width: 128-byte
// (w <= 2) or 256-byte (w >= 4) rows.
static const LdsShape kSwapShapes[] = {
    {1, 128, 128, 2}, {2, 64, 64, 2}, {4, 64, 64, 2}, {8, 32, 32, 2}, {16, 16, 16, 2},
};

const LdsShape* swap_shapes(int* n) {
    *n = (int)(sizeof(kSwapShapes) / sizeof(kSwapShapes[0]));
    return kSwapShapes;
}

Plan plan_inplace(int w, int rank, const int64_t* ext, const int64_t* ss, const int64_t* ds,
                  const int64_t* offs, int64_t batch, int src_align, int dst_align, const SwzSpec& zs,
                  const SwzSpec& zd) {
    Plan p = plan_gfx950(w, rank, ext, ss, ds, offs, batch, src_align, dst_align, zs, zd);
    auto decline = [&](const char* why) {
        p.status = TPL_E_ALIAS;
        p.reason = std::string("source and destination are the same memory: ") + why;
        p.kernel = TPL_KERNEL_NONE;
        return p;
    };
    if (p.status != TPL_OK || p.kernel == TPL_KERNEL_NONE) return p;
    if (zs.bits || zd.bits) {
        const bool same = zs.bits == zd.bits && (zs.bits == 0 || (zs.base == zd.base && zs.shift == zd.shift));
        bool identity = same;
        for (int i = 0; i < p.shard.rank; ++i) identity = identity && p.shard.m[i].s == p.shard.m[i].d;
        if (identity && p.src_off_bytes == p.dst_off_bytes) {
            p.kernel = TPL_KERNEL_NONE;
            p.grid = p.block = 0;
            return p;
        }
        return decline("swizzled operands are not permuted in place");
    }
    if (inplace_by_unit(p)) return p;
    if (p.src_off_bytes != p.dst_off_bytes) return decline("offsets differ");
    const Shard& sh = p.shard;
    bool identity = true;
    for (int i = 0; i < sh.rank; ++i) identity = identity && sh.m[i].s == sh.m[i].d;
    if (identity) {
        // Every element already sits where the destination layout puts it.
        p.kernel = TPL_KERNEL_NONE;
        p.grid = p.block = 0;
        return p;
    }
    const int a = p.mode_a, b = p.mode_b;
    if (a < 0 || b < 0 || a == b)
        return decline("only a square transpose of two modes runs in place across tiles");
    const Mode ma = sh.m[a], mb = sh.m[b];
    if (ma.e != mb.e || mb.s != ma.d)
        return decline("the transpose must be square, with one row pitch on both sides");
    // Every other mode maps each item onto itself, and items are disjoint:
    // sorted by stride, each mode's stride covers everything inside it.
    int others[kMaxShard];
    int no = 0;
    for (int i = 0; i < sh.rank; ++i) {
        if (i == a || i == b) continue;
        if (sh.m[i].s != sh.m[i].d) return decline("batch modes must have equal strides on both sides");
        others[no++] = i;
    }
    std::sort(others, others + no, [&](int x, int y) { return sh.m[x].s < sh.m[y].s; });
    int64_t span = 1 + (ma.e - 1) * (mb.s + 1);
    for (int i = 0; i < no; ++i) {
        const Mode& m = sh.m[others[i]];
        if (m.s < span) return decline("batch items overlap");
        span += (m.e - 1) * m.s;
    }
    const int sa = std::min(src_align, pow2_align(p.src_off_bytes));
    if (sa % std::min(w, 4)) return decline("the base is not aligned to the element (or 4 bytes)");
    const bool vec = sa % 16 == 0 && all_aligned(sh, a, -1, w, true, 16);
    const LdsShape* pick = nullptr;
    for (const LdsShape& x : kSwapShapes)
        if (x.w == w) pick = &x;
    LdsChoice c = cached_choice(*pick);
    if (!c.ok) return decline("no bank-conflict-free LDS plan for the square tile");

    const int T = pick->tb;
    p.kernel = TPL_KERNEL_SWAP;
    LdsArgs& l = p.lds;
    l = LdsArgs{};
    l.e_b = mb.e;
    l.e_a = ma.e;
    l.s_b = mb.s;
    l.d_a = ma.d;
    l.ntb = l.nta = (ma.e + T - 1) / T;
    // units per item: (M/2 + 1) M block units of G x G pairs (block order, see k_swap)
    l.nbl = (l.ntb + kSwapG - 1) / kSwapG;
    l.npair = (l.nbl / 2 + 1) * l.nbl * kSwapG * kSwapG;
    l.div_nbl = make_fastdiv((uint32_t)std::min<int64_t>(l.nbl, 0x7fffffff));
    int64_t items = 1;
    for (int i = 0; i < no; ++i) items *= sh.m[others[i]].e;
    l.ntiles = items * l.npair;
    if (l.ntiles >= ((int64_t)1 << 31)) p.big = true;
    l.div_npair = make_fastdiv((uint32_t)std::min<int64_t>(l.npair, 0x7fffffff));
    set_modes(l.batch, sh, others, no);
    l.pitch = c.pitch;
    l.shift_r = c.shift_r;
    l.mask_r = (1 << c.k_r) - 1;
    l.shift_w = c.shift_w;
    l.mask_w = (1 << c.k_w) - 1;
    l.scalar = vec ? 0 : 1;
    p.batch_modes = no;
    p.tile_b = p.tile_a = T;
    p.cpt = pick->cpt;
    p.pitch = c.pitch;
    p.ww = c.ww;
    p.k = c.k_r;
    p.shift = c.shift_r;
    p.mask = l.mask_r;
    p.k_w = c.k_w;
    p.shift_w = c.shift_w;
    p.mask_w = l.mask_w;
    p.P = pick->reads_per_group();
    p.block = pick->threads();
    p.grid = l.ntiles;
    p.lds_bytes = 2 * T * c.pitch;
    // Long launches run at most three pair-swap workgroups per CU (reserved
    // LDS: more than a quarter, at most a third of the 160 KiB): on the
    // 16384^2 bf16 transpose in place (34816 workgroups of 256 lanes) 191 us
    // against 200.6 us with up to eight per CU; four per CU measured 191.7,
    // five 199.3.  Below 8 rounds of three per CU on 256 CUs the cap would
    // only lengthen the launch's tail, so it applies from 6144 workgroups.
    if (p.grid >= 6144 && p.lds_bytes < kThreePerCuLds) p.lds_bytes = kThreePerCuLds;
    p.unit_is_item = false;
    return p;
}

void fill_info(const Plan& p, tpl_plan_info* out) {
    std::memset(out, 0, sizeof(*out));
    out->status = p.status;
    out->rank = p.shard.rank;
    for (int i = 0; i < p.shard.rank && i < TPL_MAX_SHARD; ++i) {
        out->extent[i] = p.shard.m[i].e;
        out->src_str[i] = p.shard.m[i].s;
        out->dst_str[i] = p.shard.m[i].d;
    }
    out->P = p.P;
    out->k = p.k;
    out->shift = p.shift;
    out->mask = p.mask;
    out->k_w = p.k_w;
    out->shift_w = p.shift_w;
    out->mask_w = p.mask_w;
    out->kernel = p.kernel;
    out->tile[0] = p.tile_b;
    out->tile[1] = p.tile_a;
    out->chunks_per_thread = p.cpt;
    out->lds_pitch = p.pitch;
    out->grid = p.grid;
    out->block = p.block;
}

}  // namespace tpl
