/*
 * oracle_gdn.c -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, obviously-correct CPU reference for the frame-wise recurrent
 * linear attention computed by the HIP library in this repository.  Only the
 * test suite, the smoke check and the CPU-baseline leg of the benchmark may
 * load this file's shared object.  It shares no code, header, table or helper
 * with the GPU path: everything below is written out from the definitions.
 *
 * Accumulation is in double precision.  Inputs arrive as float32 arrays; bf16
 * tensors widen to float32 exactly, so the oracle sees the very values the
 * GPU sees.
 *
 * Sources of the definitions (cited by page title and section):
 *  [V]  "SANA-Video: Efficient Video Generation with Block Linear Diffusion
 *       Transformer" (ICLR 2026 oral, talk transcript), block-KV-cache segment:
 *       the linear-attention state has a fixed D x D shape whatever the
 *       sequence length; block i's state is block i-1's cached state plus
 *       block i's own key-value contribution; blocks are generated causally.
 *  [W]  "SANA-WM ... 720p video" news summary (vi.news.hada.io, topic 29572),
 *       section "core design and generation pipeline" / "hybrid architecture
 *       for long rollouts": the token mixer is a frame-wise Gated DeltaNet.
 *  [P4] "How NVIDIA SANA-WM generates 60-second 720p video on one GPU"
 *       (dothoosh.com), technical-specification paragraph: the Gated DeltaNet
 *       recurrent state has a fixed size regardless of video length.
 *  [GDN] The pages name the gated delta rule but do not print it.  Its update
 *       is the published one (Yang, Kautz & Hatamizadeh, "Gated Delta
 *       Networks: Improving Mamba2 with Delta Rule", ICLR 2025, the gated
 *       delta rule recurrence):  S_t = a_t S_{t-1} (I - b_t k_t k_t^T)
 *       + b_t v_t k_t^T, with S of shape d_v x d_k and L2-normalised k.
 *
 * Readings taken where the pages are silent:
 *  - frame-wise readout: every token of frame f reads o_t = S_f q_t where S_f
 *    is the state after frame f's last token (bidirectional inside a frame,
 *    causal across frames), which is what [V]'s "block i uses S_i = S_{i-1} +
 *    block i's contribution" gives when the gate is 1 and the delta term off;
 *  - tokens of a frame are consumed in memory order;
 *  - k is normalised as k / sqrt(max(sum k^2, 1e-12));
 *  - a_t is clamped below at FLT_MIN so that it stays in (0, 1];
 *  - no scaling of q;
 *  - block-causal ReLU attention: o_t = phi(q_t)^T S_f / (phi(q_t).z_f + eps)
 *    with phi = ReLU, S_f = sum over frames g <= f of phi(K_g)^T V_g and
 *    z_f = sum of phi(k) (plus optional carried S_in, z_in).
 *
 * Layouts: q, k, out [B, H, T, d] (T = n_frames * frame_len), alpha and beta
 * [B, H, T], GDN state [B, H, d_v, d_k], block-causal state [B, H, d_k, d_v]
 * and normaliser [B, H, d_k]; all row-major.
 */
#include <float.h>
#include <math.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_NORMALIZE_K 1u /* L2-normalise k before use                  */
#define ORACLE_ADDITIVE    2u /* S += v k^T: no gate, no beta, no delta term */
#define ORACLE_GATE_LOGITS 4u /* alpha, beta hold logits a, b: alpha = exp(-softplus(a)),
                                 beta = 1 / (1 + exp(-b))                            */

int oracle_abi_version(void) { return 1; }

/*
 * Frame-wise gated delta rule, one token at a time ([W] frame-wise Gated
 * DeltaNet with the [GDN] update, [V] frame-boundary readout).
 *   a = max(alpha_t, FLT_MIN)
 *   S <- a S (I - b k k^T) + b v k^T
 * expanded without forming d x d matrices:  with s = S k,
 *   S <- a S + b (v - a s) k^T.
 * With ORACLE_ADDITIVE:  S <- S + v k^T.
 * With ORACLE_GATE_LOGITS the gate arrays hold logits (the parameterisation the
 * synthetic workloads draw the gates from): a = exp(-softplus(alpha_t)), with
 * softplus(x) = log(1 + e^x) evaluated without overflow, clamped below at FLT_MIN
 * as above; b = 1 / (1 + e^{-beta_t}).
 * After a frame's last token, o_t = S q_t for every token t of the frame.
 *
 * state_in may be NULL (zero state); state_out may be NULL.
 * Returns 0, or -1 on bad sizes / allocation failure.
 */
int oracle_gdn_forward(const float* q, const float* k, const float* v,
                       const float* alpha, const float* beta,
                       const float* state_in, double* state_out, double* out,
                       int B, int H, int n_frames, int frame_len, int dk, int dv,
                       unsigned flags, int n_threads)
{
    if (B < 0 || H < 0 || n_frames < 0 || frame_len < 0 || dk <= 0 || dv <= 0) return -1;
    const long long T = (long long)n_frames * frame_len;
    const int BH = B * H;
    int failed = 0;
#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
#pragma omp parallel for schedule(dynamic, 1) reduction(| : failed)
#endif
    for (int bh = 0; bh < BH; ++bh) {
        double* S = (double*)malloc(sizeof(double) * (size_t)dv * dk);  /* d_v x d_k */
        double* kk = (double*)malloc(sizeof(double) * (size_t)dk);
        double* s = (double*)malloc(sizeof(double) * (size_t)dv);
        if (!S || !kk || !s) { free(S); free(kk); free(s); failed = 1; continue; }
        if (state_in) {
            for (long long i = 0; i < (long long)dv * dk; ++i)
                S[i] = (double)state_in[(size_t)bh * dv * dk + i];
        } else {
            memset(S, 0, sizeof(double) * (size_t)dv * dk);
        }
        const float* qh = q + (size_t)bh * T * dk;
        const float* kh = k + (size_t)bh * T * dk;
        const float* vh = v + (size_t)bh * T * dv;
        const float* ah = alpha ? alpha + (size_t)bh * T : NULL;
        const float* bth = beta ? beta + (size_t)bh * T : NULL;
        double* oh = out + (size_t)bh * T * dv;

        for (int f = 0; f < n_frames; ++f) {
            const long long t0 = (long long)f * frame_len;
            /* recurrence over the frame's tokens, in memory order */
            for (long long t = t0; t < t0 + frame_len; ++t) {
                double nrm2 = 0.0;
                for (int j = 0; j < dk; ++j) {
                    kk[j] = (double)kh[t * dk + j];
                    nrm2 += kk[j] * kk[j];
                }
                if (flags & ORACLE_NORMALIZE_K) {
                    const double inv = 1.0 / sqrt(nrm2 > 1e-12 ? nrm2 : 1e-12);
                    for (int j = 0; j < dk; ++j) kk[j] *= inv;
                }
                const float* vt = vh + t * dv;
                if (flags & ORACLE_ADDITIVE) {
                    for (int i = 0; i < dv; ++i)
                        for (int j = 0; j < dk; ++j)
                            S[(size_t)i * dk + j] += (double)vt[i] * kk[j];
                } else {
                    double a, b;
                    if (flags & ORACLE_GATE_LOGITS) {
                        const double x = (double)ah[t], y = (double)bth[t];
                        const double sp = x > 0.0 ? x + log1p(exp(-x)) : log1p(exp(x));
                        a = exp(-sp);
                        if (a < (double)FLT_MIN) a = (double)FLT_MIN;
                        b = 1.0 / (1.0 + exp(-y));
                    } else {
                        a = (double)(ah[t] > FLT_MIN ? ah[t] : FLT_MIN);
                        b = (double)bth[t];
                    }
                    for (int i = 0; i < dv; ++i) {
                        double acc = 0.0;
                        for (int j = 0; j < dk; ++j) acc += S[(size_t)i * dk + j] * kk[j];
                        s[i] = acc;
                    }
                    for (int i = 0; i < dv; ++i) {
                        const double coef = b * ((double)vt[i] - a * s[i]);
                        for (int j = 0; j < dk; ++j)
                            S[(size_t)i * dk + j] = a * S[(size_t)i * dk + j] + coef * kk[j];
                    }
                }
            }
            /* readout from the state after the frame's last token */
            for (long long t = t0; t < t0 + frame_len; ++t) {
                for (int i = 0; i < dv; ++i) {
                    double acc = 0.0;
                    for (int j = 0; j < dk; ++j) acc += S[(size_t)i * dk + j] * (double)qh[t * dk + j];
                    oh[t * dv + i] = acc;
                }
            }
        }
        if (state_out)
            memcpy(state_out + (size_t)bh * dv * dk, S, sizeof(double) * (size_t)dv * dk);
        free(S); free(kk); free(s);
    }
    return failed ? -1 : 0;
}

/*
 * Block-causal linear attention with a ReLU feature map ([V], block-KV-cache
 * segment: the state is a fixed D x D sum, updated additively block by block,
 * and each block reads the state that already includes its own contribution).
 *   S_f = S_in + sum_{g <= f} phi(K_g)^T V_g        (d_k x d_v)
 *   z_f = z_in + sum_{g <= f} sum_{t in g} phi(k_t) (d_k)
 *   o_t = phi(q_t)^T S_f / (phi(q_t) . z_f + eps)
 * state_in, z_in, state_out, z_out may be NULL.
 */
int oracle_linear_attn_block_causal(const float* q, const float* k, const float* v,
                                    const float* state_in, const float* z_in,
                                    double* state_out, double* z_out, double* out,
                                    int B, int H, int n_frames, int frame_len,
                                    int dk, int dv, double eps, int n_threads)
{
    if (B < 0 || H < 0 || n_frames < 0 || frame_len < 0 || dk <= 0 || dv <= 0) return -1;
    const long long T = (long long)n_frames * frame_len;
    const int BH = B * H;
    int failed = 0;
#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
#pragma omp parallel for schedule(dynamic, 1) reduction(| : failed)
#endif
    for (int bh = 0; bh < BH; ++bh) {
        double* S = (double*)malloc(sizeof(double) * (size_t)dk * dv);  /* d_k x d_v */
        double* z = (double*)malloc(sizeof(double) * (size_t)dk);
        double* ph = (double*)malloc(sizeof(double) * (size_t)dk);
        if (!S || !z || !ph) { free(S); free(z); free(ph); failed = 1; continue; }
        for (long long i = 0; i < (long long)dk * dv; ++i)
            S[i] = state_in ? (double)state_in[(size_t)bh * dk * dv + i] : 0.0;
        for (int i = 0; i < dk; ++i) z[i] = z_in ? (double)z_in[(size_t)bh * dk + i] : 0.0;
        const float* qh = q + (size_t)bh * T * dk;
        const float* kh = k + (size_t)bh * T * dk;
        const float* vh = v + (size_t)bh * T * dv;
        double* oh = out + (size_t)bh * T * dv;
        for (int f = 0; f < n_frames; ++f) {
            const long long t0 = (long long)f * frame_len;
            for (long long t = t0; t < t0 + frame_len; ++t) {
                for (int i = 0; i < dk; ++i) {
                    const double x = (double)kh[t * dk + i];
                    ph[i] = x > 0.0 ? x : 0.0;
                    z[i] += ph[i];
                }
                for (int i = 0; i < dk; ++i)
                    for (int j = 0; j < dv; ++j)
                        S[(size_t)i * dv + j] += ph[i] * (double)vh[t * dv + j];
            }
            for (long long t = t0; t < t0 + frame_len; ++t) {
                double den = 0.0;
                for (int i = 0; i < dk; ++i) {
                    const double x = (double)qh[t * dk + i];
                    ph[i] = x > 0.0 ? x : 0.0;
                    den += ph[i] * z[i];
                }
                den += eps;
                for (int j = 0; j < dv; ++j) {
                    double num = 0.0;
                    for (int i = 0; i < dk; ++i) num += ph[i] * S[(size_t)i * dv + j];
                    oh[t * dv + j] = num / den;
                }
            }
        }
        if (state_out) memcpy(state_out + (size_t)bh * dk * dv, S, sizeof(double) * (size_t)dk * dv);
        if (z_out) memcpy(z_out + (size_t)bh * dk, z, sizeof(double) * (size_t)dk);
        free(S); free(z); free(ph);
    }
    return failed ? -1 : 0;
}

/*
 * Frame-block-causal softmax attention: the softmax layers of the hybrid mixer.
 * [W] section "hybrid architecture for long rollouts", with "SANA-WM: one-minute
 * 720p world model" (hn.hoangyell.com), "Hybrid Linear Attention" among its four
 * technical decisions, and the Turkish summary of the same news topic
 * (tr.news.hada.io, topic 29572), first bullet: the frame-wise Gated DeltaNet covers
 * most of the sequence and is interleaved with periodic softmax attention over
 * windows of frames.  The pages give neither the mask nor the window.  Reading taken:
 * a query token sees, through an exact softmax, every key of its own frame and of
 * earlier frames -- the same frame-level visibility as the linear layers' frame-end
 * readout -- among the kv_frames frames the caller passes (the caller's choice of
 * earlier frames is the window; the last n_frames of them are the queries' frames).
 *
 *   f_i   = (kv_frames - n_frames) + i / frame_len       (global frame of query i)
 *   l_ij  = scale * (q_i . k_j)   for keys j < (f_i + 1) * frame_len
 *   o_i   = sum_j exp(l_ij) v_j / sum_j exp(l_ij)
 *
 * written with the row maximum subtracted from every l_ij before exp (an exact
 * identity that keeps exp in range).  scale <= 0 selects 1 / sqrt(dk).
 * q, out [B, H, n_frames * frame_len, dk | dv]; k, v [B, H, kv_frames * frame_len, dk | dv].
 * Returns 0, or -1 on bad sizes / allocation failure.
 */
int oracle_softmax_attn_block_causal(const float* q, const float* k, const float* v,
                                     double* out, int B, int H, int n_frames, int kv_frames,
                                     int frame_len, int dk, int dv, double scale, int n_threads)
{
    if (B < 0 || H < 0 || n_frames < 0 || kv_frames < n_frames || frame_len < 1 || dk <= 0 || dv <= 0)
        return -1;
    if (scale <= 0.0) scale = 1.0 / sqrt((double)dk);
    const long long Tq = (long long)n_frames * frame_len, Tk = (long long)kv_frames * frame_len;
    const long long rows = (long long)B * H * Tq;
    const int off = kv_frames - n_frames;
    int failed = 0;
#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
#pragma omp parallel reduction(| : failed)
#endif
    {
        double* lg = (double*)malloc(sizeof(double) * (size_t)(Tk > 0 ? Tk : 1));
        if (!lg) failed = 1;
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 64)
#endif
        for (long long r = 0; r < rows; ++r) {
            if (!lg) continue;
            const long long bh = r / Tq, i = r - bh * Tq;
            const long long nvis = ((long long)off + i / frame_len + 1) * frame_len;
            const float* qi = q + (size_t)r * dk;
            const float* kh = k + (size_t)bh * Tk * dk;
            const float* vh = v + (size_t)bh * Tk * dv;
            double m = -HUGE_VAL;
            for (long long j = 0; j < nvis; ++j) {
                double s = 0.0;
                for (int c = 0; c < dk; ++c) s += (double)qi[c] * (double)kh[j * dk + c];
                lg[j] = scale * s;
                if (lg[j] > m) m = lg[j];
            }
            double den = 0.0;
            double* oi = out + (size_t)r * dv;
            for (int c = 0; c < dv; ++c) oi[c] = 0.0;
            for (long long j = 0; j < nvis; ++j) {
                const double p = exp(lg[j] - m);
                den += p;
                for (int c = 0; c < dv; ++c) oi[c] += p * (double)vh[j * dv + c];
            }
            for (int c = 0; c < dv; ++c) oi[c] /= den;
        }
        free(lg);
    }
    return failed ? -1 : 0;
}

/*
 * Causal temporal convolution with a block carry: the temporal convolution of the
 * causal FFN ("SANA-Video ... Block Linear Diffusion Transformer" talk, the segment on
 * a causal FFN with temporal convolution, two-block example).  During training a zero
 * token is padded between consecutive blocks, so a block never sees the next one, and
 * the last token of block i-1 is cached as block i's first token, so a block does see
 * the one before it.  The pages give neither the kernel size nor the weights.  Reading
 * taken: a depthwise convolution along the frame axis with three taps centred on the
 * frame (the zero token and the cached token are each one frame wide), weights w[3][C]
 * and bias[C] given by the caller.  For a block of F frames, per (b, position p,
 * channel c):
 *   prev(f) = f > 0 ? x[f-1] : carry_in (zero when there is none)
 *   next(f) = f < F-1 ? x[f+1] : 0       (the zero token after the block)
 *   y[f]    = w[0][c] prev(f) + w[1][c] x[f] + w[2][c] next(f) + bias[c]
 *   carry_out = x[F-1]                    (the next block's cached token)
 * x, y [B, F, P, C]; carry_in, carry_out [B, P, C]; bias may be NULL.
 * Returns 0, or -1 on bad sizes.
 */
int oracle_temporal_conv_block(const float* x, const float* carry_in, const float* w,
                               const float* bias, double* y, double* carry_out,
                               int B, int F, int P, int C)
{
    if (B < 0 || F < 0 || P < 0 || C < 0) return -1;
    const size_t frame = (size_t)P * C;
    for (int b = 0; b < B; ++b) {
        const float* xb = x + (size_t)b * F * frame;
        double* yb = y + (size_t)b * F * frame;
        for (size_t e = 0; e < frame; ++e) {
            const int c = (int)(e % (size_t)C);
            for (int f = 0; f < F; ++f) {
                const double prev = f > 0 ? (double)xb[(size_t)(f - 1) * frame + e]
                                          : (carry_in ? (double)carry_in[(size_t)b * frame + e] : 0.0);
                const double next = f < F - 1 ? (double)xb[(size_t)(f + 1) * frame + e] : 0.0;
                yb[(size_t)f * frame + e] = (double)w[c] * prev + (double)w[C + c] * (double)xb[(size_t)f * frame + e]
                                          + (double)w[2 * C + c] * next + (bias ? (double)bias[c] : 0.0);
            }
            if (carry_out && F > 0) carry_out[(size_t)b * frame + e] = (double)xb[(size_t)(F - 1) * frame + e];
        }
    }
    return 0;
}

/*
 * 3D rotary position embedding on q or k: "SANA-Video ... Block Linear Diffusion
 * Transformer" talk, the segment on temporal modelling (a 3D RoPE for the linear
 * attention).  The pages give no frequency layout, split of the head dimension or base.
 * Reading taken: the axial form -- the head dimension is cut into three contiguous
 * parts of d_t, d_h and d_w = d - d_t - d_h dimensions (all even, given by the caller),
 * rotated by the token's frame index, latent row and latent column respectively; inside
 * a part of size n, the pair (2i, 2i+1) turns by the angle pos * base^(-2i/n):
 *   (x_{2i}, x_{2i+1}) <- (x_{2i} cos a - x_{2i+1} sin a,  x_{2i} sin a + x_{2i+1} cos a).
 * Token t of a [B, H, T, d] tensor, T = n_frames * grid_h * grid_w, sits at frame
 * frame_offset + t / (grid_h grid_w), row (t mod grid_h grid_w) / grid_w, column t mod
 * grid_w.  Returns 0, or -1 on bad sizes.
 */
int oracle_rope3d(const float* x, double* y, int B, int H, int n_frames, int grid_h, int grid_w,
                  int d, int d_t, int d_h, int frame_offset, double base)
{
    const int d_w = d - d_t - d_h;
    if (B < 0 || H < 0 || n_frames < 0 || grid_h < 1 || grid_w < 1 || d_t < 0 || d_h < 0 || d_w < 0 ||
        (d_t | d_h | d_w) & 1 || base <= 0.0)
        return -1;
    const long long per_frame = (long long)grid_h * grid_w, T = (long long)n_frames * per_frame;
    for (long long r = 0; r < (long long)B * H * T; ++r) {
        const long long t = r % T;
        const long long pos[3] = {frame_offset + t / per_frame, (t % per_frame) / grid_w, t % grid_w};
        const int start[3] = {0, d_t, d_t + d_h}, size[3] = {d_t, d_h, d_w};
        const float* xr = x + r * d;
        double* yr = y + r * d;
        for (int ax = 0; ax < 3; ++ax) {
            for (int i = 0; 2 * i < size[ax]; ++i) {
                const double ang = (double)pos[ax] * pow(base, -2.0 * i / size[ax]);
                const double x0 = xr[start[ax] + 2 * i], x1 = xr[start[ax] + 2 * i + 1];
                yr[start[ax] + 2 * i] = x0 * cos(ang) - x1 * sin(ang);
                yr[start[ax] + 2 * i + 1] = x0 * sin(ang) + x1 * cos(ang);
            }
        }
    }
    return 0;
}
