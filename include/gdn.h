/*
 * gdn.h -- C ABI of the MI355X (gfx950) frame-wise recurrent linear attention library
 * (libgdn_mi355x.so).
 *
 * What is computed (definitions restated from the sources; see the oracle for the
 * plain reference implementation):
 *
 *  Frame-wise gated delta rule.  "SANA-WM ... 720p video" news summary
 *  (vi.news.hada.io, topic 29572), section "hybrid architecture for long rollouts":
 *  the token mixer is a frame-wise Gated DeltaNet; "How NVIDIA SANA-WM generates
 *  60-second 720p video on one GPU" (dothoosh.com), technical-specification paragraph:
 *  its recurrent state keeps a fixed size whatever the video length.  The update is the
 *  published gated delta rule (Yang, Kautz & Hatamizadeh, "Gated Delta Networks",
 *  ICLR 2025), per (batch b, head h), with S of shape d_v x d_k:
 *      k^_t = k_t / sqrt(max(|k_t|^2, 1e-12))          (GDN_F_NORMALIZE_K)
 *      S    <- a_t S (I - b_t k^_t k^_t^T) + b_t v_t k^_t^T,  a_t = max(alpha_t, FLT_MIN)
 *  Readout is frame-wise ("SANA-Video ... Block Linear Diffusion Transformer" talk,
 *  block-KV-cache segment: block i reads the state that already holds its own
 *  contribution): every token t of frame f gets o_t = S_f q_t, S_f being the state
 *  after frame f's last token.  Tokens of a frame are consumed in memory order.
 *  With GDN_F_ADDITIVE the update is S <- S + v_t k_t^T (gate 1, no delta term), the
 *  reduction to block-causal linear attention.
 *
 *  Block-causal linear attention (same talk, same segment), ReLU feature map phi:
 *      S_f = S_in + sum_{g<=f} phi(K_g)^T V_g   (d_k x d_v),   z_f = z_in + sum phi(k)
 *      o_t = phi(q_t)^T S_f / (phi(q_t) . z_f + 1e-6)
 *
 *  Frame-block-causal softmax attention (the softmax layers interleaved with the
 *  Gated DeltaNet in the hybrid mixer; see softmax_attn_block_causal below): exact
 *  softmax over the keys of the query's own and earlier frames.
 *
 *  Causal temporal convolution with a block carry (the causal FFN's temporal
 *  convolution; see temporal_conv_block below) and the 3D rotary position embedding of
 *  q and k (rope3d_apply).
 *
 * Conventions shared by every entry point
 *  - Tensor pointers are DEVICE pointers owned by the caller; `dims` is a HOST pointer.
 *  - Layouts are contiguous row-major: q, k, out [B, H, T, d]; v [B, H, T, d_v];
 *    alpha, beta [B, H, T] (float32); GDN state [B, H, d_v, d_k] (float32);
 *    block-causal state [B, H, d_k, d_v] and normaliser [B, H, d_k] (float32);
 *    T = n_frames * frame_len.
 *  - dtype (GDN_BF16 or GDN_F32) is the type of q, k, v and, unless GDN_F_OUT_F32 is
 *    set, of out.  bf16 inputs are contracted on bf16 matrix cores with float32
 *    accumulation and a float32 state; operands that carry the state are split into
 *    bf16 hi + lo pairs so they keep ~16 significant bits (the readout's composition
 *    with the fp16 per-frame maps runs on fp16 matrix cores, the state as an fp16
 *    hi + lo pair under a power-of-two scale).  float32 inputs run on
 *    float32 matrix cores.  A bf16 out is the round-to-nearest-even of the float32
 *    result that GDN_F_OUT_F32 returns.
 *  - Supported: d_k == d_v in {16, 32, 64, 112, 128}; frame_len >= 1; every pointer
 *    16-byte aligned.  B, H or n_frames may be 0 (nothing to compute; a forward call
 *    with n_frames == 0 copies state_in, or zeros, to state_out).
 *  - workspace: caller-owned device scratch of at least gdn_workspace_bytes(dims,
 *    entry) bytes.  Its size grows with B*H but never with n_frames: frames are
 *    processed in windows of at most 8192 (b, h, frame) units (dims->window_units
 *    overrides that bound).  Contents need no initialisation and are garbage afterwards.
 *    Two calls in flight at once need two workspaces.
 *  - stream: a hipStream_t (NULL = the default stream) of the current device.  Every
 *    launch is enqueued on it, asynchronously; the library never allocates, frees or
 *    synchronises.  The first call on each device sets the kernels' shared-memory
 *    attributes there (once per device, safe from several host threads).  Calls with
 *    distinct workspaces and outputs may run concurrently from several threads and
 *    streams.
 *  - Errors: every check runs on the host before anything is enqueued and returns a
 *    negative gdn_status_t; nothing is launched then.  A failed launch returns
 *    GDN_ERR_HIP.  Device faults surface at the caller's next synchronisation.
 *  - Aliasing: state_out may equal state_in (updated in place).  out must not overlap
 *    any input, state or the workspace; overlaps the library can see (pointer ranges)
 *    return GDN_ERR_ALIAS, others are undefined behaviour.
 *  - Results are deterministic: no atomics, fixed reduction order.
 */
#ifndef GDN_MI355X_H
#define GDN_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_ABI_VERSION 9

typedef enum {
    GDN_OK = 0,
    GDN_ERR_NULL = -1,        /* a required pointer is NULL                              */
    GDN_ERR_DIMS = -2,        /* negative or inconsistent sizes, or size overflow         */
    GDN_ERR_DTYPE = -3,       /* dtype not GDN_BF16 / GDN_F32                             */
    GDN_ERR_ALIGN = -4,       /* a pointer is not 16-byte aligned                         */
    GDN_ERR_ALIAS = -5,       /* out overlaps an input, a state or the workspace          */
    GDN_ERR_WORKSPACE = -6,   /* workspace NULL or smaller than gdn_workspace_bytes()     */
    GDN_ERR_UNSUPPORTED = -7, /* d_k != d_v, d not in {16,32,64,112,128}, or a bad flag   */
    GDN_ERR_HIP = -8          /* a HIP launch failed                                      */
} gdn_status_t;

enum { GDN_BF16 = 0, GDN_F32 = 1 };

enum {
    GDN_F_NORMALIZE_K = 1u << 0, /* L2-normalise k inside the kernel (float32)            */
    GDN_F_ADDITIVE = 1u << 1,    /* gated delta rule entries: S <- S + v k^T              */
    GDN_F_RELU_QK = 1u << 2,     /* block-causal entry: phi = ReLU on q and k (else id)  */
    GDN_F_OUT_F32 = 1u << 3,     /* out is float32 whatever dtype is (all entries)        */
    GDN_F_GATE_LOGITS = 1u << 4, /* gated delta rule entries: alpha and beta hold logits a,
                                    b; the gates are alpha = exp(-softplus(a)) (clamped
                                    below at FLT_MIN) and beta = 1 / (1 + e^-b), formed in
                                    float32 inside the kernels                            */
    GDN_F_ROPE_QK = 1u << 5      /* gdn_frame_forward(_readonly, _noalloc) and
                                    gdn_token_forward: q and k are
                                    rotated by the 3D rotary position embedding of
                                    rope3d_apply (parameters in dims->rope_*) as the kernels
                                    load them; the tensors in memory are not changed      */
};

enum { GDN_ENTRY_FORWARD = 0, GDN_ENTRY_READONLY = 1, GDN_ENTRY_BLOCK_CAUSAL = 2, GDN_ENTRY_TOKEN = 3 };

typedef struct gdn_dims {
    int32_t B, H;                 /* batch (independent rollouts) and heads              */
    int32_t n_frames, frame_len;  /* T = n_frames * frame_len tokens per (b, h)          */
    int32_t d_k, d_v;             /* head dimensions (equal)                             */
    int32_t dtype;                /* GDN_BF16 or GDN_F32: q, k, v, out                   */
    uint32_t flags;               /* GDN_F_* bits                                        */
    void* workspace;              /* device scratch, >= gdn_workspace_bytes() bytes      */
    size_t workspace_bytes;
    void* const* phase_events;    /* optional, may be NULL: 6 * phase_windows caller-created
                                     hipEvent_t.  For window w < phase_windows, events 6w+2i
                                     and 6w+2i+1 are recorded just before and just after the
                                     window's i-th launch (i = 0, 1, 2), on the stream that
                                     launch goes to; for per-kernel timing only           */
    int32_t phase_windows;        /* windows covered by phase_events (see gdn_window_count) */
    /* Plan overrides, for tests and tuning; 0 = the library's choice.  They change how the
     * work is cut (and the workspace size), not the result beyond rounding. */
    int32_t window_units;         /* (b, h, frame) units per window (default 8192)        */
    int32_t group_frames;         /* gated delta rule: frames per group of the frame-map
                                     kernel (default: chosen from B*H, n_frames, frame_len
                                     and the device's compute units)                     */
    /* 3D rotary position embedding with GDN_F_ROPE_QK ("SANA-Video ... Block Linear
     * Diffusion Transformer" talk, segment on temporal modelling; the axial reading of
     * rope3d_apply): d is cut into parts of rope_d_t, rope_d_h and d - rope_d_t - rope_d_h
     * dimensions (all even) rotated by the token's frame, latent row and latent column;
     * in a part of n dimensions the pair (2i, 2i+1) turns by pos * rope_base^(-2i/n).
     * frame_len = grid_h * rope_grid_w; token t of frame f sits at frame rope_frame_offset
     * + f, row (t / rope_grid_w), column t mod rope_grid_w; rope_frame_offset + n_frames
     * <= 2^24.  Ignored without the flag. */
    int32_t rope_d_t, rope_d_h, rope_grid_w, rope_frame_offset;
    float rope_base;
} gdn_dims_t;

/*
 * Frame-wise gated delta rule, forward over n_frames frames, carrying the state.
 *  q, k      [B,H,T,d_k] dtype      v, out [B,H,T,d_v] dtype
 *  alpha     [B,H,T] float32 gate in (0,1] (clamped below at FLT_MIN); may be NULL
 *            only with GDN_F_ADDITIVE.  beta [B,H,T] float32 in [0,1]; same rule.
 *            With GDN_F_GATE_LOGITS both hold logits instead (any finite value).
 *  state_in  [B,H,d_v,d_k] float32, NULL = zero state.  Read only.
 *  state_out [B,H,d_v,d_k] float32, the state after the last frame; NULL = not
 *            written; may equal state_in.
 *  out       o_t = S_f q_t for every token of every frame.
 */
int gdn_frame_forward(const void* q, const void* k, const void* v,
                      const float* alpha, const float* beta,
                      const float* state_in, float* state_out, void* out,
                      const gdn_dims_t* dims, void* stream);

/*
 * gdn_frame_forward for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same computation,
 * arguments and results, with the scratch taken from a static device array of
 * gdn_noalloc_scratch_bytes() bytes (64 MiB) that each device holds until the process
 * ends, instead of dims->workspace (ignored).  The entry and the kernels it launches
 * allocate nothing.  A call whose workspace (gdn_workspace_bytes(dims, GDN_ENTRY_FORWARD))
 * exceeds the array returns GDN_ERR_WORKSPACE before anything is enqueued; a smaller
 * dims->window_units makes large calls fit.  All calls on one device share its array:
 * calls that may run at the same time on one device (other streams, other host threads)
 * race and must be serialised by the caller.  The array needs no initialisation and keeps
 * the last call's garbage.
 */
int gdn_frame_forward_noalloc(const void* q, const void* k, const void* v,
                              const float* alpha, const float* beta,
                              const float* state_in, float* state_out, void* out,
                              const gdn_dims_t* dims, void* stream);

/* Size in bytes of the static scratch array of gdn_frame_forward_noalloc. */
size_t gdn_noalloc_scratch_bytes(void);

/*
 * Read-only-state variant for the denoising steps inside a frame ("SANA-Video" talk,
 * opening: video is generated block by block causally and diffused within the block;
 * the cached state is only updated once the block is final).  Same outputs as
 * gdn_frame_forward (each frame attends to the carried state advanced through its own
 * tokens); state_in is never written and no state is returned.
 */
int gdn_frame_forward_readonly(const void* q, const void* k, const void* v,
                               const float* alpha, const float* beta,
                               const float* state_in, void* out,
                               const gdn_dims_t* dims, void* stream);

/*
 * Gated delta rule with a per-token causal readout: the general Gated DeltaNet that the
 * frame-wise mixer specialises ("SANA-WM ... 720p video" news summary, section "hybrid
 * architecture for long rollouts"; update as in Gated Delta Networks).  Every token t
 * reads the state after its own update,  o_t = S_t q_t  -- the same as gdn_frame_forward
 * with one-token frames.  Arguments, layouts, state semantics, flags and errors are those
 * of gdn_frame_forward; n_frames and frame_len only set how T = n_frames * frame_len
 * tokens are cut into chunks and windows (the result does not depend on them beyond
 * rounding), and, with GDN_F_ROPE_QK, the tokens' rotary positions.
 */
int gdn_token_forward(const void* q, const void* k, const void* v,
                      const float* alpha, const float* beta,
                      const float* state_in, float* state_out, void* out,
                      const gdn_dims_t* dims, void* stream);

/*
 * Block-causal linear attention (bidirectional inside a frame, causal across frames).
 *  q, k [B,H,T,d_k], v, out [B,H,T,d_v] dtype.  phi = ReLU when GDN_F_RELU_QK is set.
 *  state_in [B,H,d_k,d_v], z_in [B,H,d_k] float32 (NULL = zero); state_out, z_out
 *  (NULL = not written; may equal state_in / z_in).
 */
int linear_attn_block_causal(const void* q, const void* k, const void* v,
                             const float* state_in, const float* z_in,
                             float* state_out, float* z_out, void* out,
                             const gdn_dims_t* dims, void* stream);

/*
 * Frame-block-causal softmax attention: the softmax layers that the hybrid mixer
 * interleaves with the frame-wise Gated DeltaNet ("SANA-WM: one-minute 720p world
 * model", hn.hoangyell.com, "Hybrid Linear Attention" among its four technical decisions;
 * "SANA-WM ... 720p video" news summary, section "hybrid architecture for long rollouts").
 * The pages fix neither the mask nor the window; this entry computes, exactly, attention
 * in which query i of global frame f_i = (kv_frames - n_frames) + i / frame_len sees
 * every key of frames <= f_i:
 *     o_i = sum_j exp(s q_i.k_j) v_j / sum_j exp(s q_i.k_j),  j < (f_i + 1) frame_len,
 *     s = 1 / sqrt(d_k).
 *  q, out [B,H,n_frames*frame_len,d] dtype (out float32 with GDN_F_OUT_F32);
 *  k, v   [B,H,kv_frames*frame_len,d] dtype, kv_frames >= n_frames: the last n_frames
 *         frames are the queries' own, earlier ones cached frames (the window is the
 *         caller's choice of which earlier frames to pass).
 *  Allowed flags: GDN_F_OUT_F32 only.  No workspace is used (dims->workspace ignored).
 *  phase_events, if phase_windows >= 1: events 0 and 1 are recorded just before and just
 *  after the single launch.  bf16 inputs: logits and softmax in float32, probabilities
 *  rounded to bf16 for the product with V, float32 accumulation.  out must not overlap
 *  q, k or v (GDN_ERR_ALIAS).  Returns GDN_ERR_DIMS when kv_frames < n_frames.
 */
int softmax_attn_block_causal(const void* q, const void* k, const void* v, void* out,
                              int32_t kv_frames, const gdn_dims_t* dims, void* stream);

/*
 * Causal temporal convolution of one block of frames, with the carry between blocks: the
 * temporal convolution of the causal FFN ("SANA-Video ... Block Linear Diffusion
 * Transformer" talk, segment on a causal FFN with temporal convolution: a zero token
 * follows each block in training, so a block never sees the next one, and the previous
 * block's last token is cached as its first, so it sees the one before).  The pages fix
 * neither kernel size nor weights; this entry computes a depthwise, three-tap convolution
 * along frames, per (b, position p, channel c), for the block's frames f = 0..F-1:
 *     y[f] = w[0][c] prev(f) + w[1][c] x[f] + w[2][c] next(f) + bias[c]
 *     prev(0) = carry_in (0 when NULL),  next(F-1) = 0,  carry_out = x[F-1]
 *  x, y      [B, F, P, C] dtype (y float32 with GDN_F_OUT_F32), F = n_frames, P = frame_len
 *  carry_in  [B, P, C] dtype or NULL;  carry_out [B, P, C] dtype or NULL, may equal
 *            carry_in (with F = 0 it receives carry_in, or zeros)
 *  weight    [3, C] float32 (taps for the previous, the same and the next frame);
 *            bias [C] float32 or NULL
 *  C must be a multiple of 8 (bf16) or 4 (float32).  events (may be NULL): two hipEvent_t
 *  recorded just before and after the single launch.  Allowed flags: GDN_F_OUT_F32.
 *  y must not overlap x or the carries (GDN_ERR_ALIAS).
 */
int temporal_conv_block(const void* x, const void* carry_in, const float* weight,
                        const float* bias, void* y, void* carry_out, int32_t B,
                        int32_t n_frames, int32_t frame_len, int32_t channels,
                        int32_t dtype, uint32_t flags, void* const* events, void* stream);

/*
 * 3D rotary position embedding of q or k, in place ("SANA-Video ... Block Linear Diffusion
 * Transformer" talk, segment on temporal modelling: a 3D RoPE for the linear attention).
 * The pages fix neither the frequency layout nor the split of d nor the base; this entry
 * computes the axial form with those from the caller: d is cut into contiguous parts of
 * d_t, d_h and d_w = d - d_t - d_h dimensions (all even), rotated by the token's frame,
 * latent row and latent column; in a part of n dimensions the pair (2i, 2i+1) turns by
 * pos * base^(-2i/n).
 *  x [B, H, T, d] dtype, T = n_frames * grid_h * grid_w; token t sits at frame
 *    frame_offset + t / (grid_h grid_w), row (t mod grid_h grid_w) / grid_w, column
 *    t mod grid_w.  d must be a multiple of 8 (bf16) or 4 (float32), at most 256;
 *    frame_offset + n_frames <= 2^24.  A stand-alone pass (not fused into the attention kernels).
 *  events (may be NULL): two hipEvent_t recorded around the single launch.
 */
int rope3d_apply(void* x, int32_t B, int32_t H, int32_t n_frames, int32_t grid_h,
                 int32_t grid_w, int32_t d, int32_t d_t, int32_t d_h, int32_t frame_offset,
                 float base, int32_t dtype, void* const* events, void* stream);

/* Bytes of workspace the entry (GDN_ENTRY_*) needs for these dims; 0 on invalid dims.
 * Bounded independently of n_frames. */
size_t gdn_workspace_bytes(const gdn_dims_t* dims, int entry);

/* Number of windows (each: three launches) a call with these dims makes, >= 0, or a
 * negative gdn_status_t for invalid dims. */
int gdn_window_count(const gdn_dims_t* dims, int entry);

/* Static, human-readable text for a gdn_status_t value. */
const char* gdn_status_str(int status);

/* GDN_ABI_VERSION of the built library. */
int gdn_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* GDN_MI355X_H */
