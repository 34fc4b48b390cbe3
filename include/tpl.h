/*
 * tpl.h -- C ABI of the permute_layout library for MI355X (gfx950).
 *
 * The operation (permute_layout page, intro and "Algorithm"; address rule from
 * the "Buffers and memory" page, "Declaring buffers"): every element of a
 * tensor held under a source shape:stride layout is copied, bit for bit, to
 * the place the destination layout gives the same logical coordinate.
 *
 * For every batch index b < batch and every coordinate c of `extents`:
 *
 *   dst[off_d + b*span_d + sum_i c_i*dst_strides[i]] :=
 *       src[off_s + b*span_s + sum_i c_i*src_strides[i]]
 *
 * with strides and offsets counted in elements of `dtype_bytes` bytes, and
 * span_x = 1 + sum_i (extents[i]-1)*x_strides[i] (the side's cosize: batch
 * items follow each other with no gap).  A batch with another spacing is one
 * more leading mode with batch = 1.  The bytes move verbatim; nothing is
 * interpreted as a number.
 *
 * Operand rules (permute_layout page, "What it accepts"): one element width
 * for both sides, equal extents (a single `extents` array here), width in
 * {1, 2, 4, 8, 16}, plain shape:stride layouts, and a conflict-free XOR
 * swizzle must exist for the staged exchange, else the call declines.
 */
#ifndef TPL_H
#define TPL_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes.  Every check runs before anything is enqueued: on a non-OK
 * return nothing was launched and dst is untouched. */
typedef enum {
    TPL_OK = 0,
    TPL_E_ARG = 1,          /* null pointer, rank outside 1..8, negative extent or batch */
    TPL_E_DTYPE_WIDTH = 2,  /* dtype_bytes not in {1, 2, 4, 8, 16} */
    TPL_E_DTYPE = 3,        /* element types differ (raised by the Python binding) */
    TPL_E_EXTENT = 4,       /* extents differ (raised by the Python binding) */
    TPL_E_LAYOUT = 5,       /* layout cannot be canonicalised: negative stride or offset,
                               destination not provably one-to-one, offsets overflow */
    TPL_E_NO_K = 6,         /* no XOR swizzle makes both staged phases conflict-free */
    TPL_E_ALIAS = 7,        /* src and dst overlap other than unit-for-unit in place */
    TPL_E_HIP = 8           /* the HIP runtime refused the launch; see tpl_last_error() */
} tpl_status;

/* Bank geometry for tpl_plan. */
enum {
    TPL_GEOM_GFX950 = 0,   /* the kernels this library launches on gfx950 (64-lane waves,
                              LDS banks as measured on MI355X) */
    TPL_GEOM_PAGES32 = 1,  /* the pages' warp program: 32 lanes, 32 banks of 4 bytes */
    TPL_GEOM_GFX950_HALFWAVE = 2, /* the pages' warp program run by one 32-lane half of a
                                     gfx950 wave on LDS (tpl_permute_staged, tpl_wave.h) */
    TPL_GEOM_GFX950_INPLACE = 3   /* the plan tpl_permute launches when src == dst: a kernel
                                     whose work units each read before they write, or the
                                     pair-swap kernel, or TPL_E_ALIAS */
};

/* Kernel families a GFX950 plan can pick. */
enum {
    TPL_KERNEL_NONE = 0,   /* nothing to do (empty tensor) or a PAGES32 plan */
    TPL_KERNEL_GATHER = 1, /* element-wise gather/scatter, any layout */
    TPL_KERNEL_QUAD = 2,   /* 4x4 dword blocks transposed in registers across lanes (DPP,
                              permlane16 swap); 1-, 2- and 4-byte elements, a destination-
                              contiguous extent of 4 (or 4-row blocks of records) */
    TPL_KERNEL_LDS = 3,    /* tiled 2-D transpose staged through LDS with XOR-ordered phases */
    TPL_KERNEL_REG16 = 4,  /* 16-byte elements: 8x8 element blocks, pure lane remap */
    TPL_KERNEL_COPY = 5,   /* both sides contiguous along one mode: vector copy of runs */
    TPL_KERNEL_SWAP = 6,   /* in-place square transpose: mirrored tile pairs swapped through LDS */
    TPL_KERNEL_REC = 7,    /* records of any size to field rows or back: the dense side as one
                              contiguous block through LDS */
    TPL_KERNEL_ETILE = 8   /* 2-D tiles through LDS for layouts whose bases, row pitches or
                              swizzle granules rule out 16-byte vectors: the aligned 16-byte
                              chunks covering each row (plain operands of 1-4 bytes), else one
                              element per access */
};

/*
 * XOR swizzle of an operand (buffers page, "Pool sugar": alloc_mma builds
 * MMA-compatible tiles as a plain layout composed with a swizzle; the pages
 * leave its form to the allocator).  The usual XOR function of the layout
 * offset m, in elements:
 *
 *   swz(m) = m XOR (((m >> (base + shift)) mod 2^bits) << base)
 *
 * It acts on a side's layout offset with the batch as the outermost mode,
 * before the element offset is added:
 *   address = off + swz(b * span + sum_i c_i * stride_i).
 * bits = 0 is the plain layout; otherwise 1 <= bits <= 16, base >= 0,
 * shift >= bits (so swz is its own inverse), base + shift + bits <= 48.
 */
typedef struct {
    int32_t bits, base, shift;
} tpl_swizzle;

#define TPL_MAX_RANK 8
#define TPL_MAX_SHARD 10

typedef struct {
    int32_t status;                 /* tpl_status of the planning */
    int32_t rank;                   /* modes in the shard (batch folded in as a mode) */
    int64_t extent[TPL_MAX_SHARD];  /* shard extents, outermost first */
    int64_t src_str[TPL_MAX_SHARD]; /* shard source strides (elements) */
    int64_t dst_str[TPL_MAX_SHARD]; /* shard destination strides (elements) */
    int64_t P;                      /* elements staged per lane per phase */
    int32_t k, shift, mask;         /* XOR swizzle j = r ^ ((lane >> shift) & mask) of the
                                       exchange's read phase (PAGES32: of both phases) */
    int32_t k_w, shift_w, mask_w;   /* GFX950 LDS kernel: XOR of the LDS write phase */
    int32_t kernel;                 /* TPL_KERNEL_* (GFX950 only) */
    int32_t tile[2];                /* tile extents in elements along (b, a), the destination-
                                       and the source-contiguous mode: LDS, SWAP, QUAD, REC and
                                       ETILE kernels (ETILE: the width's tile or its tall tile) */
    int32_t chunks_per_thread;      /* 16-byte source chunks each thread loads, LDS kernel */
    int32_t lds_pitch;              /* LDS row pitch in bytes: LDS, SWAP and ETILE kernels */
    int64_t grid, block;            /* launch shape of the main kernel */
} tpl_plan_info;

/*
 * Enqueue the permutation on `stream` and return without waiting.
 *
 * src, dst      device pointers (caller-owned; the library never allocates).
 * dtype_bytes   element width shared by both sides.
 * rank          number of modes, 1..8; extents/src_strides/dst_strides have
 *               `rank` entries each (host arrays, borrowed for the call).
 * elem_offsets  host array {src offset, dst offset} in elements (may be NULL
 *               for {0, 0}).
 * batch         number of contiguous batch items (>= 0; 0 does nothing).
 * stream        HIP stream (NULL = the null stream).
 *
 * Source and destination may be the same memory (equal pointers after the
 * offsets) when either every work unit's source footprint equals its
 * destination footprint (e.g. a batch of small in-place transposes), or the
 * permutation is a square transpose (equal extents and row pitch on the two
 * transposed modes, batch modes with equal strides on both sides and
 * disjoint items): then pairs of mirrored tiles are swapped, each pair by one
 * workgroup that reads both tiles before writing either.  Any other overlap
 * returns TPL_E_ALIAS.
 *
 * Memory touched: only destination bytes of elements in the layout are
 * written.  Reads stay between the source layout's first and last byte,
 * except that a 2-D transpose whose source rows do not start on 16 bytes
 * (TPL_KERNEL_ETILE, elements of 1-4 bytes) reads each row piece as the
 * aligned 16-byte blocks covering it: up to 15 bytes before and after a
 * piece, never outside those aligned blocks (so never on another page),
 * and never stored.
 * Returns a tpl_status; thread-safe.
 */
int tpl_permute(const void *src, void *dst, int dtype_bytes, int rank,
                const int64_t *extents, const int64_t *src_strides,
                const int64_t *dst_strides, const int64_t *elem_offsets,
                int64_t batch, hipStream_t stream);

/*
 * tpl_permute with either side (or both) swizzled (NULL = plain).  Every
 * element still lands bit for bit at swz_dst(...) of its coordinate.  The
 * vector kernels are used where each 16-byte access stays inside one
 * swizzle granule (2^base elements of at least 16 bytes); otherwise the
 * element-wise kernel runs.  In place (src == dst) only when both layouts
 * and both swizzles are equal (nothing moves); any other overlap returns
 * TPL_E_ALIAS.  An invalid swizzle returns TPL_E_ARG.
 */
int tpl_permute_swizzled(const void *src, void *dst, int dtype_bytes, int rank,
                         const int64_t *extents, const int64_t *src_strides,
                         const int64_t *dst_strides, const int64_t *elem_offsets,
                         int64_t batch, const tpl_swizzle *src_swizzle,
                         const tpl_swizzle *dst_swizzle, hipStream_t stream);

/*
 * Host-only planning, no device needed (permute_layout page, "Algorithm"
 * steps 1 and 2: align the two layouts into one shard, then pick the XOR
 * swizzle).  With TPL_GEOM_PAGES32 it runs the pages' method on one warp
 * region: shard, P = elements / 32, and the smallest k whose XOR swizzle
 * makes the read and the write phase bank-conflict-free (declines with
 * TPL_E_NO_K otherwise; a region of more than 4096 elements per lane
 * declines with TPL_E_LAYOUT, since the search simulates every step).  With TPL_GEOM_GFX950 it returns the plan
 * tpl_permute would launch (assuming 256-byte aligned base pointers), with
 * TPL_GEOM_GFX950_INPLACE the plan it would launch with src == dst.
 *
 * Arguments are those of tpl_permute without the pointers and the stream.
 * elem_offsets ({src, dst} in elements, NULL for {0, 0}) is taken because
 * the device plan depends on it: the offsets set the alignment of both
 * bases, which decides whether 16-byte vectors apply on each side.  `out`
 * (caller-owned, may be NULL) is filled on every return, with out->status
 * equal to the return value; on a non-OK return tpl_last_error() gives the
 * reason.  Nothing is allocated or launched.
 */
int tpl_plan(int dtype_bytes, int rank, const int64_t *extents,
             const int64_t *src_strides, const int64_t *dst_strides,
             const int64_t *elem_offsets, int64_t batch, int geometry,
             tpl_plan_info *out);

/* tpl_plan for swizzled operands (NULL = plain); for PAGES32 and
 * GFX950_HALFWAVE the bank model sees the swizzled addresses. */
int tpl_plan_swizzled(int dtype_bytes, int rank, const int64_t *extents,
                      const int64_t *src_strides, const int64_t *dst_strides,
                      const int64_t *elem_offsets, int64_t batch,
                      const tpl_swizzle *src_swizzle, const tpl_swizzle *dst_swizzle,
                      int geometry, tpl_plan_info *out);

/*
 * The same operation as tpl_permute, executed the way the pages' warp
 * primitive is (permute_layout page, "Algorithm"): every batch item is moved
 * by one 32-lane half-wave, which copies the item's source footprint into
 * LDS, permutes it LDS to LDS with the register-staged, XOR-swizzled
 * program of tpl_wave.h, and copies the destination footprint back.
 *
 * Extra operand rules: prod(extents) = 32 * P with P in {1, 2, 4, 8, 16, 32};
 * each item's destination footprint is dense (its offsets, swizzled, are
 * exactly 0 .. prod(extents) - 1) and both footprints fit 8 KiB; with
 * batch > 1 a swizzled side's item span is a multiple of the swizzle period
 * 2^(base + shift + bits); otherwise TPL_E_LAYOUT.  Swizzles (NULL = plain)
 * are applied to the LDS addresses of the program's two phases, and the
 * bank model plans k on the swizzled addresses.  xor_k < 0 takes the
 * smallest conflict-free k of the half-wave bank model (TPL_E_NO_K if none);
 * xor_k >= 0 forces that k (shift = 5 - k), which lets a caller measure the
 * unswizzled program.  Source and destination must not overlap.
 */
int tpl_permute_staged(const void *src, void *dst, int dtype_bytes, int rank,
                       const int64_t *extents, const int64_t *src_strides,
                       const int64_t *dst_strides, const int64_t *elem_offsets,
                       int64_t batch, const tpl_swizzle *src_swizzle,
                       const tpl_swizzle *dst_swizzle, int xor_k, hipStream_t stream);

/*
 * Static text of a status code, one phrase per reason the permute_layout
 * page gives for declining a call ("What it accepts": dtype mismatch, extent
 * mismatch, unsupported dtype byte width, layouts that do not slice or
 * canonicalise, no conflict-free swizzle), plus this library's argument,
 * aliasing and HIP errors.  Unknown codes give "unknown status".  The
 * string is owned by the library and never freed.
 */
const char *tpl_status_string(int status);

/*
 * Reason text of this thread's last non-OK return from any entry point
 * (the status phrase of the page's "What it accepts" list, with the detail
 * that failed), or an empty string if none.  The buffer is thread-local,
 * owned by the library, and valid until the next failing call on the same
 * thread.
 */
const char *tpl_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* TPL_H */
