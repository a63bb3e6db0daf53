// hk_grid.hpp -- workgroup id -> output tile map, shared by host and device.
//
// "How to make AMD GPUs go brrr" (section "Inter-processor scheduling:
// chiplet-aware approach") observes that MI355X deals thread blocks to its 8
// chiplets (XCDs, each with a private L2) round-robin, that a plain row-major
// order of output tiles therefore reuses L2 poorly, and that grouping
// workgroups into adjacent regions of the output serves both the per-chiplet
// L2 and the shared last-level cache.  The pages give no formula; this is
// ours:
//
//  1. Window.  Workgroups are dispatched in id order, so ids
//     [n*W, (n+1)*W) run together when W is the number of co-resident
//     workgroups (one per CU here).  Within a window, id r goes to chiplet
//     x = r % X (X = 8).  We renumber slots so each chiplet owns a
//     consecutive run: slot = x*q + min(x, rem) + r / X, where q and rem
//     are the quotient and remainder of the window size by X.  This is a
//     bijection on the window, also for a short last window.
//  2. Grouped order.  Slot l (over the whole grid) walks the tiles in groups
//     of group_m tile rows, column by column inside a group.  A chiplet's run
//     of W/X consecutive slots is then a group_m x (W/X/group_m) block (L2),
//     and a window is a group_m x (W/group_m) band (last-level cache).
//
// ROW_MAJOR keeps the identity order for comparison.
#pragma once

#include <stdint.h>

#ifndef HK_HD
#define HK_HD __host__ __device__ __forceinline__
#endif

namespace hk {

enum GridOrder : int32_t { kGridRowMajor = 1, kGridXcd = 2 };

struct GridParams {
    int32_t order;
    int32_t tiles_m;
    int32_t tiles_n;
    int32_t group_m;  // >= 1
    int32_t window;   // >= 1
    int32_t nxcd;     // >= 1
};

// Step 1: hardware workgroup id -> logical slot.
HK_HD uint32_t xcd_slot(uint32_t w, uint32_t total, uint32_t window, uint32_t nxcd) {
    const uint32_t n = w / window;
    const uint32_t base = n * window;
    const uint32_t r = w - base;
    const uint32_t wsize = (total - base < window) ? (total - base) : window;
    const uint32_t q = wsize / nxcd;
    const uint32_t rem = wsize - q * nxcd;
    const uint32_t x = r % nxcd;
    const uint32_t i = r / nxcd;
    return base + x * q + (x < rem ? x : rem) + i;
}

// Step 2: logical slot -> (tm, tn), grouped column-major within group_m rows.
HK_HD void grouped_tile(uint32_t l, uint32_t tiles_m, uint32_t tiles_n, uint32_t group_m,
                        uint32_t* tm, uint32_t* tn) {
    const uint32_t per_group = group_m * tiles_n;
    const uint32_t g = l / per_group;
    const uint32_t first_m = g * group_m;
    const uint32_t rows = (tiles_m - first_m < group_m) ? (tiles_m - first_m) : group_m;
    const uint32_t in = l - g * per_group;
    *tm = first_m + in % rows;
    *tn = in / rows;
}

HK_HD void tile_of(uint32_t w, const GridParams& p, uint32_t* tm, uint32_t* tn) {
    const uint32_t tiles_n = (uint32_t)p.tiles_n;
    if (p.order == kGridRowMajor) {
        *tm = w / tiles_n;
        *tn = w - (w / tiles_n) * tiles_n;
        return;
    }
    const uint32_t total = (uint32_t)p.tiles_m * tiles_n;
    const uint32_t l = xcd_slot(w, total, (uint32_t)p.window, (uint32_t)p.nxcd);
    grouped_tile(l, (uint32_t)p.tiles_m, tiles_n, (uint32_t)p.group_m, tm, tn);
}

}  // namespace hk
