// kernels.hip -- permute_layout on gfx950: dispatch to the kernel families
// (kernels_*.hip, one translation unit each), the plan cache and the C entry
// points.
//
// The method is the register-staged exchange of the permute_layout page,
// "Algorithm" step 3.  Here both ends are HBM: every kernel loads whole
// 16-byte vectors along the source-contiguous mode, regroups elements across
// lanes (DPP and permlane within lane quads, or an LDS tile whose two phases
// use the XOR-ordered visiting order), and stores whole 16-byte vectors along
// the destination-contiguous mode, so each side moves full 128-byte lines.
// Data moves as integers only; no floating-point instruction touches it.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <unordered_map>

#include "device.hpp"

namespace tpl {


// ---------------------------------------------------------------------------
// Dispatch: the plan's kernel family, compiled for its number of batch modes.

template <int NB, bool BIG>
static hipError_t launch_nb(const Plan& p, const uint8_t* src, uint8_t* dst, hipStream_t st) {
    switch (p.kernel) {
    case TPL_KERNEL_COPY: return launch_copy<NB, BIG>(p, src, dst, st);
    case TPL_KERNEL_QUAD: return launch_quad<NB, BIG>(p, src, dst, st);
    case TPL_KERNEL_LDS: return launch_lds<NB, BIG>(p, src, dst, st);
    case TPL_KERNEL_SWAP: return launch_swap<NB, BIG>(p, src, dst, st);
    case TPL_KERNEL_REC: return launch_rec<NB, BIG>(p, src, dst, st);
    case TPL_KERNEL_ETILE: return launch_etile<NB, BIG>(p, src, dst, st);
    case TPL_KERNEL_REG16: return launch_reg16<NB, BIG>(p, src, dst, st);
    default: return hipSuccess;
    }
}

template <bool BIG>
static hipError_t launch_big(const Plan& p, const uint8_t* src, uint8_t* dst, hipStream_t st) {
    if (p.kernel == TPL_KERNEL_GATHER) return launch_gather<BIG>(p, src, dst, st);
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
        bool neg = false;
        if (rank >= 1 && rank <= TPL_MAX_RANK && extents)
            for (int i = 0; i < rank; ++i) neg = neg || extents[i] < 0;
        if (rank < 1 || rank > TPL_MAX_RANK || !extents || !src_strides || !dst_strides || batch < 0) {
            p.status = TPL_E_ARG;
            p.reason = "rank must be in 1..8, arrays non-NULL, batch >= 0";
        } else if (neg) {
            p.status = TPL_E_ARG;
            p.reason = "extents must be >= 0";
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
