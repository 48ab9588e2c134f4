// gdn_plan.hpp -- host-only planning of a call of the gated-delta-rule and block-causal
// entries: argument checks on the dims, the frames-per-group choice, window size and the
// workspace layout.  Plain C++ with no HIP dependency, so that it can also be built on its
// own (the CPU test tier builds it with address and undefined-behaviour sanitizers).
#pragma once
#include <stddef.h>
#include <stdint.h>

#include "gdn.h"

namespace gdn {

constexpr long long kMaxUnits = 8192;  // default (b, h, frame) units per window

// bytes of the workspace regions of the gated-delta-rule path: per unit (afr, bfr, xexp),
// per group (agr, bgr, sgrp)
struct GdnRegions {
    size_t afr, bfr, xexp, agr, bgr, sgrp;
};
GdnRegions gdn_region_bytes(int nd, int esize);
// block-causal per-frame regions: the frame sums (part) and the prefix operands (pack)
size_t bc_unit_bytes(int nd, int esize, size_t* part, size_t* pack);

// Plan of one call: window size and workspace offsets.
struct Plan {
    long long BH = 0, T = 0;
    int nd = 0, es = 0, nfw = 0, nwin = 0, G = 1;
    // block-causal: off_a per-frame sums, off_c prefix operands; gated delta rule: the
    // regions of GdnRegions
    size_t off_a = 0, off_b = 0, off_x = 0, off_ga = 0, off_gb = 0, off_c = 0, off_carry = 0, total = 0;
};

int nd_of(int d);
// Frames per group for B*H pairs on `cus` compute units (see the definition).
int group_frames(long long BH, int n_frames, int frame_len, int cus);
// Checks dims for `entry` and fills the plan; `cus` is the device's compute-unit count.
// Returns GDN_OK or a negative gdn_status_t.
int check_dims(const gdn_dims_t* d, int entry, Plan* p, int cus);
bool misaligned(const void* ptr);
bool overlap(const void* a, size_t na, const void* b, size_t nb);

}  // namespace gdn
