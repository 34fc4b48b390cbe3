// planner.hpp -- host-side steps of permute_layout: validation, canonical
// shard, bank simulation and XOR-k choice, kernel selection, plan cache.
#pragma once

#include <stdint.h>
#include <string>

#include "common.hpp"
#include "../../include/tpl.h"

namespace tpl {

struct Mode {
    int64_t e, s, d;   // extent, source stride, destination stride (elements)
};

struct Shard {
    int rank = 0;
    Mode m[kMaxShard];
};

// One LDS access phase as the bank simulator sees it.
struct Geometry {
    int lanes;          // lanes per wave
    int bank_bytes;     // bytes per bank
    bool same_word_ok;  // lanes touching the same word do not conflict
    // banks and lanes per pass for an access of `bytes` bytes (read or write)
    int banks_read[5], pass_read[5];    // index: log2(bytes) - 0 (1,2,4,8,16)
    int banks_write[5], pass_write[5];
    // how lanes are grouped into passes: 0 = consecutive runs of pass_* lanes;
    // 1 = by (lane bit 5, parity of lane bits 2..4), four passes of 16 lanes
    int group_read[5], group_write[5];
};

const Geometry& geometry_pages32();
const Geometry& geometry_gfx950();

// Does one unrolled step (one access per lane) run without bank conflicts?
// `addr` holds each lane's byte address, `bytes` the access width; lanes with
// active[l] == false do not take part.
bool step_conflict_free(const Geometry& g, bool is_write, int bytes, const int64_t* addr,
                        const bool* active, int lanes);

// An operand swizzle as the caller gives it, in elements: bits [base,
// base + bits) of the layout offset are XORed with bits [base + shift,
// base + shift + bits).  bits == 0: plain layout.
struct SwzSpec {
    int bits = 0, base = 0, shift = 0;
};

bool swz_valid(const SwzSpec& z);
Swz swz_bytes(const SwzSpec& z, int w);   // the same swizzle on byte offsets

struct Plan {
    int status = TPL_OK;
    SwzSpec zs, zd;         // operand swizzles
    std::string reason;
    Shard shard;            // canonical shard, batch folded in
    int w = 0;
    int kernel = TPL_KERNEL_NONE;
    int64_t P = 0;
    int k = 0, shift = 0, mask = 0;        // read phase (PAGES32: both phases)
    int k_w = 0, shift_w = 0, mask_w = 0;  // LDS write phase
    int tile_b = 0, tile_a = 0, cpt = 0, pitch = 0, ww = 0;
    int64_t grid = 0, block = 0;
    int lds_bytes = 0;
    bool big = false;       // 64-bit index math needed
    bool unit_is_item = false;  // each batch item is moved by one work unit (reads before writes)
    int mode_a = -1, mode_b = -1;          // shard indices of the two contiguous modes
    int batch_modes = 0;                   // modes the kernel decomposes as batch
    int64_t src_off_bytes = 0, dst_off_bytes = 0;
    // kernel arguments (pointers filled at launch)
    GatherArgs gather{};
    CopyArgs copy{};
    QuadArgs quad{};
    LdsArgs lds{};
    Reg16Args reg16{};
    RecArgs rec{};
    bool rec_dense_src = false;
};

// Full planning for the device path.  src_align / dst_align: alignment in
// bytes of the base pointers (after elem_offsets are applied).
Plan plan_gfx950(int w, int rank, const int64_t* ext, const int64_t* ss, const int64_t* ds,
                 const int64_t* offs, int64_t batch, int src_align, int dst_align,
                 const SwzSpec& zs = SwzSpec(), const SwzSpec& zd = SwzSpec());

// The plan for src == dst: the device plan when each of its work units reads
// its whole footprint before writing it; else the pair-swap plan of a square
// transpose; else TPL_E_ALIAS.
Plan plan_inplace(int w, int rank, const int64_t* ext, const int64_t* ss, const int64_t* ds,
                  const int64_t* offs, int64_t batch, int src_align, int dst_align,
                  const SwzSpec& zs = SwzSpec(), const SwzSpec& zd = SwzSpec());

// Does the device plan move every batch item with one read-before-write unit,
// so that it may run with src == dst?
bool inplace_by_unit(const Plan& p);

const LdsShape* swap_shapes(int* n);

// The element-tile shape for width w (nullptr for other widths).
const EtileShape* etile_shape(int w);
const EtileShape* etile_tall_shape(int w);   // nullptr for widths without one

// The pages' method on one warp region (32 lanes, 32 banks).
Plan plan_pages32(int w, int rank, const int64_t* ext, const int64_t* ss, const int64_t* ds,
                  int64_t batch, const SwzSpec& zs = SwzSpec(), const SwzSpec& zd = SwzSpec());

// The same 32-lane program run by one gfx950 half-wave on LDS, with the
// measured gfx950 bank model.
Plan plan_halfwave(int w, int rank, const int64_t* ext, const int64_t* ss, const int64_t* ds,
                   int64_t batch, const SwzSpec& zs = SwzSpec(), const SwzSpec& zd = SwzSpec());

Plan plan_warp32(const Geometry& g, int w, int rank, const int64_t* ext, const int64_t* ss,
                 const int64_t* ds, int64_t batch, const SwzSpec& zs = SwzSpec(), const SwzSpec& zd = SwzSpec());

// Canonical shard (unit modes dropped, neighbours merged where both sides merge).
Shard make_shard(int rank, const int64_t* ext, const int64_t* ss, const int64_t* ds,
                 int64_t batch);

bool dst_injective(const Shard& sh);

// Element count batch * prod(ext); false on overflow past 2^62.
bool count_elements(int rank, const int64_t* ext, int64_t batch, int64_t* out);

void fill_info(const Plan& p, tpl_plan_info* out);

}  // namespace tpl
