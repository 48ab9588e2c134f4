// gdn_kernels.hpp -- argument blocks and launcher declarations shared by the kernel
// sources and the C ABI layer.  Workspace formats (per (b, h, frame) "unit", frames of
// one window stored contiguously per (b, h); per (b, h, group) likewise):
//   Afr    per unit, the frame's A map for the readout: A_f^T as K32 A-operand
//          fragments, PAIR slot map over k_in, ND x KB fragments of 64 lanes x 8
//          elements.  fp32 inputs: fp32.  bf16 inputs: fp16, row slice w of A (rows
//          16w..16w+15, the k_in of the map) scaled by 2^-Xexp[w] so that its largest
//          magnitude lies in [2^14, 2^15).
//   Bfr    per unit, the frame's B map for the readout as accumulator tiles: ND slices x
//          ND tiles x 64 lanes x 4 values.  fp32 inputs: fp32.  bf16 inputs: fp16, row
//          slice w scaled by 2^-Xexp[8 + w] like Afr.
//   Xexp   per unit (bf16 inputs), 16 ints: the slice exponents of Afr, then of Bfr.
//   (A_f, B_f) of a frame is the partial map of its group up to that frame's end.
//   Agr    per group, the group's whole map A for the chain over groups: the fragments of
//          Afr in the dtype of the inputs; for bf16 a hi set then a lo set.
//   Bgr    per group, the group's whole map B for the chain: the tiles of Bfr in fp32.
//   Sgrp   per group, the state before the group, fp32 [d_v][d_k] row-major.
//   BCpart block-causal per-frame sums phi(K)^T [V | 1]: ND x (ND+1) accumulator tiles.
//   BCpack block-causal S_f^T and z_f as K32 A-operand fragments: (ND+1) x KB fragments
//          (bf16: hi set then lo set).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>

#include "gdn_plan.hpp"

namespace gdn {

// 3D rotary position embedding on the load path (GDN_F_ROPE_QK): pair j of a token row
// (elements 2j, 2j+1) turns by pos * freq_j, pos being the token's frame (pairs below p1),
// latent row (pairs below p2) or latent column; freq_j / 2 pi is given as float hi + lo
// (rounded from double) so that late frames keep the angle's full precision.
constexpr int kRopePairs = 64;  // d <= 128
struct RopeArgs {
    int on;
    int p1, p2;          // first pair of the row part and of the column part
    int grid_w;          // latent columns: token t of a frame sits at (t / grid_w, t % grid_w)
    int frame0;          // absolute frame index of the call's first frame
    float ghi[kRopePairs], glo[kRopePairs];
};

struct P1Args {
    const void* k;
    const void* v;
    const float* alpha;
    const float* beta;
    long long T;        // tokens per (b, h)
    int frame_len;
    int f0;             // first frame of the window
    int nf;             // frames in the window
    int G;              // frames per group
    int BH;
    unsigned flags;     // bit 0: normalise k, bit 1: additive
    void* Agr;          // whole-group maps A and B (chain operands)
    float* Bgr;
    int emit_all;       // maps at every frame end (else only at each group's last frame)
    // per-token readout pass only:
    const void* q;
    void* out;
    const float* Sgrp;  // state before each group of the window [BH, groups, d, d], or NULL
    int out_f32;
    // one-group calls: the start state is Sgrp (state_in, or NULL = zero), the frame maps
    // pass runs in true-start mode, and the state after the group goes to state_out
    int true_start;
    float* state_out;
    // frame mode: the readout's per-frame maps and, for bf16, their slice exponents
    void* Afr;
    void* Bfr;
    int* Xexp;
    RopeArgs rope;      // k rotated as it is loaded (frame maps pass)
};

struct P2Args {
    const void* Agr;
    const float* Bgr;
    const float* state_src;  // [BH, d, d] or NULL (zero state)
    float* state_dst;        // [BH, d, d] or NULL
    float* Sgrp;             // [BH, groups, d, d]: state before each group
    int nf;
    int G;
};

struct P3Args {
    const void* q;
    void* out;
    const void* Afr;
    const void* Bfr;
    const int* Xexp;
    const float* Sgrp;  // state before each group, or NULL for a zero state
    long long T;
    int frame_len;
    int f0;
    int nf;
    int G;
    int out_f32;        // out is float32 (else the input dtype)
    int b_is_state;     // the B maps are the true states (true-start frame maps): no compose
    int parts;          // workgroups per frame, each over a range of its 64-token chunks (set
                        // by the launcher)
    RopeArgs rope;      // q rotated as it is loaded
};

struct BC1Args {
    const void* k;
    const void* v;
    long long T;
    int frame_len;
    int f0;
    int nf;
    unsigned relu;
    float* part;
};

struct BC2Args {
    const float* part;
    const float* s_in;   // [BH, d_k, d_v] or NULL (window 0 only)
    const float* z_in;   // [BH, d_k] or NULL
    const float* carry_in;  // tile-layout carry from the previous window or NULL
    float* carry_out;       // tile-layout carry for the next window or NULL
    float* s_out;        // [BH, d_k, d_v] or NULL (last window only)
    float* z_out;        // [BH, d_k] or NULL
    void* pack;
    int nf;
};

struct BC3Args {
    const void* q;
    void* out;
    const void* pack;
    long long T;
    int frame_len;
    int f0;
    int nf;
    unsigned relu;
    float eps;
    int out_f32;
    int parts;  // workgroups per frame (set by the launcher)
};

// Launchers.  ev: NULL, or the 6 events of one window -- recorded before and after each
// of the window's three launches, on the stream that launch goes to.
// phase 0: frame maps (P1Args), 1: chain over groups (P2Args), 2: readout (P3Args),
// 3: per-token readout (P1Args; recorded in the third launch's event slots).
template <typename E, int ND>
hipError_t launch_gdn_phase(int phase, const void* args, int BH, hipStream_t st, void* const* ev);
// the variants with the 3D rotary embedding on load (gdn_frame_rope.hip): phase 0 the frame
// maps in `mode` (bit 0 normalise, bit 1 additive, bit 2 true start), phase 2 the readout,
// phase 3 the per-token readout (mode bits 0 and 1)
template <typename E, int ND>
hipError_t launch_gdn_rope(int phase, unsigned mode, const void* args, int BH, hipStream_t st);
template <typename E, int ND>
hipError_t launch_bc_window(const BC1Args&, const BC2Args&, const BC3Args&, int BH, hipStream_t,
                            void* const* ev);

inline hipError_t record(void* const* ev, int i, hipStream_t st) {
    return ev ? hipEventRecord((hipEvent_t)ev[i], st) : hipSuccess;
}


}  // namespace gdn
