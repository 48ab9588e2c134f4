// gdn_plan.cpp -- host-only planning of the gated-delta-rule and block-causal calls (see
// gdn_plan.hpp).  No device code and no HIP calls: everything here is arithmetic on the
// caller's dims.
#include "gdn_plan.hpp"

#include <stdint.h>

namespace gdn {

namespace {
constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
int esize_of(int dtype) { return dtype == GDN_BF16 ? 2 : 4; }
}  // namespace

int nd_of(int d) {
    switch (d) {
        case 16: return 1;
        case 32: return 2;
        case 64: return 4;
        case 112: return 7;
        case 128: return 8;
        default: return 0;
    }
}

GdnRegions gdn_region_bytes(int nd, int esize) {
    const size_t frag = (size_t)nd * ((nd + 1) / 2) * 64 * 8;  // elements of one set of A fragments
    const size_t tiles = (size_t)nd * nd * 256;                // elements of the B tiles
    const bool bf = esize == 2;
    GdnRegions r;
    r.afr = frag * (bf ? 2 : 4);         // fp16 (bf16 inputs) or fp32
    r.bfr = tiles * (bf ? 2 : 4);
    r.xexp = bf ? 16 * sizeof(int) : 0;
    r.agr = frag * esize * (bf ? 2 : 1);  // bf16 operands are stored as hi + lo
    r.bgr = tiles * 4;
    r.sgrp = (size_t)16 * nd * 16 * nd * 4;  // a d x d fp32 state
    return r;
}

size_t bc_unit_bytes(int nd, int esize, size_t* part, size_t* pack) {
    const int kb = (nd + 1) / 2;
    const int nsplit = esize == 2 ? 2 : 1;  // bf16 operands are stored as hi + lo
    *part = (size_t)nd * (nd + 1) * 256 * 4;
    *pack = (size_t)nsplit * (nd + 1) * kb * 64 * 8 * esize;
    return *part + *pack;
}

// Frames per group of the gated-delta-rule path.  The frame-map kernel runs one
// workgroup per (b, h, group) and one workgroup per CU (its LDS footprint), so its time
// goes as (rounds of workgroups over the device's CUs) x (frames per group); the serial
// chain takes one step per group.  G minimises the sum of the two, with about 0.051 us
// per token of a frame in the frame-map kernel and 1 us per chain step (measured at
// d = 112 on MI355X).  Windows hold whole groups.
int group_frames(long long BH, int n_frames, int frame_len, int cus) {
    const long long ncu = cus > 0 ? cus : 256;
    const double per_frame = 0.051 * frame_len, per_step = 1.0;
    int best = 1;
    double best_cost = 1e300;
    for (int G = 1; G <= n_frames && G <= 64; ++G) {
        const long long groups = (n_frames + G - 1) / G;
        const long long rounds = (BH * groups + ncu - 1) / ncu;
        const double cost = rounds * G * per_frame + groups * per_step;
        if (cost < best_cost * (1 - 1e-9)) {
            best_cost = cost;
            best = G;
        }
    }
    return best;
}

int check_dims(const gdn_dims_t* d, int entry, Plan* p, int cus) {
    if (!d) return GDN_ERR_NULL;
    if (d->dtype != GDN_BF16 && d->dtype != GDN_F32) return GDN_ERR_DTYPE;
    if (d->B < 0 || d->H < 0 || d->n_frames < 0 || d->frame_len < 1) return GDN_ERR_DIMS;
    if (d->window_units < 0 || d->group_frames < 0) return GDN_ERR_DIMS;
    if (d->d_k != d->d_v || nd_of(d->d_k) == 0) return GDN_ERR_UNSUPPORTED;
    const uint32_t allowed = (entry == GDN_ENTRY_BLOCK_CAUSAL)
                                 ? (uint32_t)(GDN_F_RELU_QK | GDN_F_OUT_F32)
                                 : (uint32_t)(GDN_F_NORMALIZE_K | GDN_F_ADDITIVE | GDN_F_OUT_F32 |
                                              GDN_F_GATE_LOGITS | GDN_F_ROPE_QK);
    if (d->flags & ~allowed) return GDN_ERR_UNSUPPORTED;
    if (d->flags & GDN_F_ROPE_QK) {  // rotary embedding on the gated-delta-rule entries' load path
        if (entry != GDN_ENTRY_FORWARD && entry != GDN_ENTRY_READONLY && entry != GDN_ENTRY_TOKEN)
            return GDN_ERR_UNSUPPORTED;
        const int dw = d->d_k - d->rope_d_t - d->rope_d_h;
        if (d->rope_d_t < 0 || d->rope_d_h < 0 || dw < 0 || d->rope_grid_w < 1 || d->rope_frame_offset < 0 ||
            !(d->rope_base > 0.f) || d->frame_len % d->rope_grid_w != 0 ||
            (long long)d->rope_frame_offset + d->n_frames > (1LL << 24))
            return GDN_ERR_DIMS;
        if ((d->rope_d_t | d->rope_d_h | dw) & 1) return GDN_ERR_UNSUPPORTED;  // rotations act on pairs
    }
    p->BH = (long long)d->B * d->H;
    p->T = (long long)d->n_frames * d->frame_len;
    if (p->BH > 65535) return GDN_ERR_DIMS;  // grid y extent
    p->nd = nd_of(d->d_k);
    p->es = esize_of(d->dtype);
    // element count of q must fit comfortably in 63 bits
    if (p->T > ((long long)1 << 40) / (p->BH ? p->BH : 1) / d->d_k) return GDN_ERR_DIMS;
    if (p->BH == 0 || d->n_frames == 0) return GDN_OK;
    const bool bc = entry == GDN_ENTRY_BLOCK_CAUSAL;
    if (!bc) {
        p->G = d->group_frames > 0 ? (d->group_frames < d->n_frames ? d->group_frames : d->n_frames)
                                   : group_frames(p->BH, d->n_frames, d->frame_len, cus);
    }
    const long long G = p->G;
    const long long wu = d->window_units > 0 ? d->window_units : kMaxUnits;
    long long nfw = wu / p->BH / G * G;  // whole groups per window
    if (nfw < G) nfw = G;
    if (nfw > d->n_frames) nfw = d->n_frames;
    p->nfw = (int)nfw;
    p->nwin = (int)((d->n_frames + nfw - 1) / nfw);
    const size_t units = (size_t)p->BH * (size_t)nfw;
    size_t carry = 0;
    GdnRegions r{0, 0, 0, 0, 0, 0};
    size_t groups = 0;
    if (bc) {
        bc_unit_bytes(p->nd, p->es, &r.afr, &r.sgrp);
        carry = (size_t)p->BH * p->nd * (p->nd + 1) * 256 * 4;
        groups = units;
    } else {
        r = gdn_region_bytes(p->nd, p->es);
        carry = (size_t)p->BH * d->d_k * d->d_v * 4;
        groups = (size_t)p->BH * ((p->nfw + p->G - 1) / p->G);
    }
    p->off_a = 0;
    p->off_b = align_up(units * r.afr);
    p->off_x = p->off_b + align_up(units * r.bfr);
    p->off_ga = p->off_x + align_up(units * r.xexp);
    p->off_gb = p->off_ga + align_up(groups * r.agr);
    p->off_c = p->off_gb + align_up(groups * r.bgr);
    p->off_carry = p->off_c + align_up(groups * r.sgrp);
    p->total = p->off_carry + (p->nwin > 1 ? align_up(carry) : 0);
    return GDN_OK;
}

bool misaligned(const void* ptr) { return ptr && ((uintptr_t)ptr & 15u) != 0; }

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + nb && b0 < a0 + na;
}

}  // namespace gdn
