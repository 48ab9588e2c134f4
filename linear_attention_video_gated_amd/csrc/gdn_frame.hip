// gdn_frame.hip -- frame-wise gated delta rule on gfx950.
//
// Method: the gated delta rule of Gated DeltaNet (named as the frame-wise token mixer in
// the SANA-WM news summary, section "hybrid architecture for long rollouts"; update as
// published by Yang, Kautz & Hatamizadeh, 2025), read out at frame boundaries (SANA-Video
// talk, block-KV-cache segment).  Per (b, h), state S is d_v x d_k, fp32.
//
// Organisation (three launches per window of frames):
//  1. gdn_frame_affine  -- one workgroup per (b, h, frame), all frames in parallel.  The
//     frame is cut into chunks of 64 tokens; each chunk is turned into its WY/UT factors
//     (Gram matrix K K^T, unit-lower-triangular inverse T = (I + L)^-1, W and U), all on
//     bf16 matrix cores with fp32 accumulation.  The chunks are applied, in order, to a
//     stacked state [I ; 0], which yields the frame's affine map
//          S_f = S_{f-1} A_f + B_f      (A_f: d_k x d_k, B_f: d_v x d_k)
//     since the readout needs only the state at frame ends.
//  2. gdn_frame_chain   -- one wave per (b, h, 16-row slice of S): the serial part, one
//     d x d matrix product per frame.  Writes each S_f as readout operand fragments and
//     the final state.
//  3. gdn_frame_readout -- one workgroup per (b, h, frame): O_f = Q_f S_f^T, streaming Q in
//     and O out.
// Chunk algebra (derivation from the recurrence, restated; G_t = sum_{i<=t} log a_i in
// the chunk, k^ the normalised keys):
//   L_ti = b_t e^{G_t - G_i} k^_t.k^_i (i < t),  T = (I + L)^-1,
//   U = T diag(b) V,  W = T diag(b e^G) K^,  Kt = diag(e^{G_C - G}) K^,
//   S <- e^{G_C} S + (U - W S^T)^T Kt.
// Rows of S never mix, which is what lets the state be split into 16-row slices.
//
// Precision (bf16 inputs).  Inputs q, k, v are exact bf16 operands.  Quantities that carry
// the state (the chunk innovation Kt-scaled (U - W S^T), the frame maps A_f and the
// states S_{f-1}, S_f) are sent to the matrix cores as bf16 hi + lo pairs, which keeps
// ~16 significant bits; W and U are formed in correction form, X = R + Y with
// Y = (T_II - I) R_I - T_II sum_J L_IJ X_J, so only the small correction Y is rounded.
#include "common.hpp"
#include "gdn_kernels.hpp"
#include <float.h>

namespace gdn {

// -------------------------------------------------------------------------------------
// Phase 1: per-frame affine maps
// -------------------------------------------------------------------------------------
template <typename E, int ND> struct P1 {
    using G = Geo<E, ND>;
    static constexpr int NW = ND;                 // waves per workgroup
    static constexpr int NT = 64 * NW;
    static constexpr int KR_P = G::DP + G::EPV;   // sKrow pitch (elements)
    static constexpr int VR_P = G::D + G::EPV;    // sVrow pitch
    static constexpr int KT_P = 64 + G::EPV;      // sKt pitch (tokens)
    static constexpr int L_P = 68;                // sL pitch (floats)
    static constexpr int TD_P = 20;               // sTd pitch (floats)
    static constexpr int KROW_B = 64 * KR_P * (int)sizeof(E);
    static constexpr int L_B = 64 * L_P * 4;
    static constexpr int U1_B = ((KROW_B > L_B ? KROW_B : L_B) + 255) / 256 * 256;
    static constexpr int VROW_B = (64 * VR_P * (int)sizeof(E) + 255) / 256 * 256;
    static constexpr int KT_B = (G::D * KT_P * (int)sizeof(E) + 255) / 256 * 256;
    static constexpr int TD_B = 4 * 16 * TD_P * 4;
    static constexpr int W_B = 4 * G::KB * G::FRAG * (int)sizeof(E);
    static constexpr int APK_E = G::ND * G::KB * G::FRAG;  // A_f fragments (elements)
    static constexpr int OFF_VROW = U1_B;
    static constexpr int OFF_KT = OFF_VROW + VROW_B;
    static constexpr int OFF_TD = OFF_KT + KT_B;
    static constexpr int OFF_W = OFF_TD + TD_B;
    static constexpr int OFF_SC = OFF_W + W_B;
    static constexpr int LDS_B = OFF_SC + 6 * 64 * 4 + 64;
    static_assert(APK_E * (int)sizeof(E) <= OFF_KT, "A_f staging must fit in sKrow+sVrow");
    static_assert(LDS_B <= 160 * 1024, "LDS budget");
};

__constant__ int kTriI[10] = {0, 1, 1, 2, 2, 2, 3, 3, 3, 3};
__constant__ int kTriJ[10] = {0, 0, 1, 0, 1, 2, 0, 1, 2, 3};

template <typename E, int ND>
__global__ __launch_bounds__(64 * ND, 1) void gdn_frame_affine(P1Args a) {
    using L = P1<E, ND>;
    using O = Ops<E>;
    using F8 = typename O::F8;
    using F4 = typename O::F4;
    using V16 = typename O::V16;
    constexpr int D = L::G::D, KB = L::G::KB, DP = L::G::DP, EPV = L::G::EPV;
    extern __shared__ __attribute__((aligned(256))) unsigned char smem[];
    E* sKrow = (E*)smem;
    float* sL = (float*)smem;           // aliases sKrow once the Gram matrix is built
    E* sVrow = (E*)(smem + L::OFF_VROW);
    E* sKt = (E*)(smem + L::OFF_KT);
    float* sTd = (float*)(smem + L::OFF_TD);
    E* sW = (E*)(smem + L::OFF_W);
    float* sBeta = (float*)(smem + L::OFF_SC);
    float* sWs = sBeta + 64;
    float* sKts = sBeta + 128;
    float* sN = sBeta + 192;
    float* sG = sBeta + 256;
    float* sGam = sBeta + 320;
    float* sAlp = sBeta + 336;

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int c = lane & 15, g = lane >> 4;
    const int fw = blockIdx.x, bh = blockIdx.y;
    const int N = a.frame_len;
    const long long tok0 = (long long)bh * a.T + (long long)(a.f0 + fw) * N;
    const E* kp = (const E*)a.k + tok0 * D;
    const E* vp = (const E*)a.v + tok0 * D;
    const bool additive = (a.flags & 2u) != 0;
    const bool normalize = (a.flags & 1u) != 0;

    // stacked state [A-slice ; B-slice] rows 16w..16w+15, kept transposed as
    // accumulator tiles: XA[t] lane (c,g) = A[16w + c][16t + 4g + i]
    f32x4 XA[ND], XB[ND];
#pragma unroll
    for (int t = 0; t < ND; ++t) {
#pragma unroll
        for (int i = 0; i < 4; ++i) XA[t][i] = (16 * w + c == 16 * t + 4 * g + i) ? 1.f : 0.f;
        XB[t] = zero4();
    }

    // Chunk loads: thread (p = tid % 32, colblock cb) owns token rows 2p and 2p+1 of a
    // 16-byte column block; the next chunk is fetched into registers while this one is
    // being computed.  Row pairs let the transposed copy use one 4-byte (bf16) store per
    // element pair.
    constexpr int CB = D / EPV;                 // 16-byte column blocks per row
    constexpr int NCB = L::NT / 32;             // column blocks covered per pass
    constexpr int NPASS = (CB + NCB - 1) / NCB;
    const int pr = tid & 31, cb0 = tid >> 5;
    V16 rk[NPASS][2], rv[NPASS][2];
    float ra = 0.f, rb = 0.f;
    auto fetch = [&](int c0, int Cc) {
#pragma unroll
        for (int ps = 0; ps < NPASS; ++ps) {
            const int cb = cb0 + ps * NCB;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int row = 2 * pr + h;
                if (cb < CB && row < Cc) {
                    rk[ps][h] = *(const V16*)(kp + (long long)(c0 + row) * D + cb * EPV);
                    rv[ps][h] = *(const V16*)(vp + (long long)(c0 + row) * D + cb * EPV);
                } else {
#pragma unroll
                    for (int j = 0; j < EPV; ++j) rk[ps][h][j] = rv[ps][h][j] = (E)0.f;
                }
            }
        }
        if (tid < 64 && tid < Cc && !additive) {
            ra = a.alpha[tok0 + c0 + tid];
            rb = a.beta[tok0 + c0 + tid];
        }
    };

    const int nch = (N + 63) / 64;
    fetch(0, min(64, N));
    for (int ch = 0; ch < nch; ++ch) {
        const int c0 = ch * 64;
        const int Cc = min(64, N - c0);
        __syncthreads();  // readers of the previous chunk are done
        // ---- registers -> LDS: K row-major and transposed, V row-major; zero padding
        {
#pragma unroll
            for (int ps = 0; ps < NPASS; ++ps) {
                const int cb = cb0 + ps * NCB;
                if (cb < CB) {
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        *(V16*)(sKrow + (2 * pr + h) * L::KR_P + cb * EPV) = rk[ps][h];
                        *(V16*)(sVrow + (2 * pr + h) * L::VR_P + cb * EPV) = rv[ps][h];
                    }
#pragma unroll
                    for (int j = 0; j < EPV; ++j) {
                        O::st2(sKt + (cb * EPV + j) * L::KT_P + 2 * pr, rk[ps][0][j], rk[ps][1][j]);
                    }
                }
            }
            // zero the padded columns D..DP-1 of sKrow (sL overwrote them)
            constexpr int PADV = (DP - D) / EPV;
            if (PADV > 0) {
                V16 z;
#pragma unroll
                for (int j = 0; j < EPV; ++j) z[j] = (E)0.f;
                for (int u = tid; u < 64 * PADV; u += L::NT)
                    *(V16*)(sKrow + (u / PADV) * L::KR_P + D + (u % PADV) * EPV) = z;
            }
            if (tid < 64) {
                sAlp[tid] = ra;
                sBeta[tid] = rb;
            }
        }
        __syncthreads();
        if (ch + 1 < nch) fetch(c0 + 64, min(64, N - c0 - 64));  // overlaps this chunk's compute
        // ---- per-token scalars: key norm, log-gate prefix, derived scales (wave 0)
        if (w == 0) {
            const int t = lane;
            const bool valid = t < Cc;
            float n2 = 0.f;
#pragma unroll
            for (int j = 0; j < D; j += EPV) {
                V16 x = *(const V16*)(sKrow + t * L::KR_P + j);
#pragma unroll
                for (int e = 0; e < EPV; ++e) n2 += (float)x[e] * (float)x[e];
            }
            const float nrm = valid ? (normalize ? rsqrtf(fmaxf(n2, 1e-12f)) : 1.f) : 0.f;
            float gl = 0.f, be = 0.f;
            if (valid) {
                if (additive) {
                    be = 1.f;
                } else {
                    gl = log2f(fmaxf(sAlp[t], FLT_MIN));
                    be = sBeta[t];
                }
            }
            float Gs = gl;  // inclusive prefix sum over the chunk (log2 units)
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float o = __shfl_up(Gs, off, 64);
                if (lane >= off) Gs += o;
            }
            const float GC = __shfl(Gs, 63, 64);
            sBeta[t] = be;
            sN[t] = nrm;
            sG[t] = Gs;
            sWs[t] = additive ? 0.f : be * exp2f(Gs) * nrm;
            sKts[t] = exp2f(GC - Gs) * nrm;
            if (lane == 0) sGam[0] = exp2f(GC);
        }
        __syncthreads();
        // ---- Gram matrix of the chunk's keys -> L (strictly lower, scaled)
        constexpr int NQ = (10 + L::NW - 1) / L::NW;
        f32x4 Lt[NQ];
#pragma unroll
        for (int qi = 0; qi < NQ; ++qi) {
            const int q = w + qi * L::NW;
            Lt[qi] = zero4();
            if (q < 10 && !additive) {
                const int it = kTriI[q], jt = kTriJ[q];
                f32x4 acc = zero4();
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) {
                    F8 fa = O::ld8(sKrow + (16 * it + c) * L::KR_P + 32 * kb + 8 * g);
                    F8 fb = O::ld8(sKrow + (16 * jt + c) * L::KR_P + 32 * kb + 8 * g);
                    acc = O::mma32(fa, fb, acc);
                }
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) {
                    const int i = 16 * it + 4 * g + ii, j = 16 * jt + c;
                    acc[ii] = (i > j) ? sBeta[i] * sN[i] * sN[j] * exp2f(sG[i] - sG[j]) * acc[ii] : 0.f;
                }
                Lt[qi] = acc;
            }
        }
        __syncthreads();  // sKrow no longer read: its space becomes sL
#pragma unroll
        for (int qi = 0; qi < NQ; ++qi) {
            const int q = w + qi * L::NW;
            if (q < 10) {
                const int it = kTriI[q], jt = kTriJ[q];
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) sL[(16 * it + 4 * g + ii) * L::L_P + 16 * jt + c] = Lt[qi][ii];
            }
        }
        __syncthreads();
        // ---- inverses of the four 16x16 diagonal blocks of (I + L), forward substitution
        if (w == 0) {
            const int bb = lane >> 4, j = lane & 15;
            float tc[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float acc = 0.f;
#pragma unroll
                for (int kk = 0; kk < i; ++kk) acc += sL[(16 * bb + i) * L::L_P + 16 * bb + kk] * tc[kk];
                tc[i] = (i == j) ? 1.f : (i > j ? -acc : 0.f);
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) sTd[(16 * bb + i) * L::TD_P + j] = tc[i];
        }
        __syncthreads();
        // ---- block forward substitution, correction form: X_I = R_I + Y_I with
        //      Y_I = (T_II - I) R_I - T_II sum_{J<I} L_IJ X_J,  R = diag(b e^G n) K or diag(b) V
        f32x4 Ur[4];
        {
            f32x4 XW[4];
#pragma unroll
            for (int I = 0; I < 4; ++I) {
                f32x4 rw, ru;
                const f32x4 kcol = O::ld4f(sKt + (16 * w + c) * L::KT_P + 16 * I + 4 * g);
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) {
                    const int t = 16 * I + 4 * g + ii;
                    rw[ii] = sWs[t] * kcol[ii];
                    ru[ii] = sBeta[t] * tof(sVrow[t * L::VR_P + 16 * w + c]);
                }
                f32x4 aw = zero4(), au = zero4();
#pragma unroll
                for (int J = 0; J < I; ++J) {
                    const F4 lf = O::pack4(*(const f32x4*)(sL + (16 * I + c) * L::L_P + 16 * J + 4 * g));
                    aw = O::mma16(lf, O::pack4(XW[J]), aw);
                    au = O::mma16(lf, O::pack4(Ur[J]), au);
                }
                f32x4 tr = *(const f32x4*)(sTd + (16 * I + c) * L::TD_P + 4 * g);
                const F4 ntf = O::pack4(-tr);
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) tr[ii] -= (c == 4 * g + ii) ? 1.f : 0.f;
                const F4 tmi = O::pack4(tr);
                f32x4 yw = O::mma16(tmi, O::pack4(rw), zero4());
                f32x4 yu = O::mma16(tmi, O::pack4(ru), zero4());
                if (I > 0) {
                    yw = O::mma16(ntf, O::pack4(aw), yw);
                    yu = O::mma16(ntf, O::pack4(au), yu);
                }
                XW[I] = rw + yw;
                Ur[I] = ru + yu;
            }
            // scatter W (tokens x d_k) into A-operand fragments (PAIR slot map over d_k)
            const int kbw = w >> 1, jb = (w & 1) * 4 + (c & 3);
#pragma unroll
            for (int I = 0; I < 4; ++I) {
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) {
                    const int lp = 4 * g + ii + 16 * (c >> 2);
                    E* fr = sW + ((I * KB + kbw) * 64 + lp) * 8;
                    fr[jb] = O::cvt(XW[I][ii]);
                    if ((ND & 1) && w == ND - 1) fr[4 + (c & 3)] = (E)0.f;
                }
            }
        }
        __syncthreads();
        // ---- apply the chunk to both state slices:  X <- g_C X + Kt^T (Z - W X^T)
        {
            const float gam = sGam[0];
            F8 xa[KB], xb[KB];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                const f32x4 hiA = (2 * kb + 1 < ND) ? XA[(2 * kb + 1) % ND] : zero4();
                const f32x4 hiB = (2 * kb + 1 < ND) ? XB[(2 * kb + 1) % ND] : zero4();
                xa[kb] = O::pack8(XA[2 * kb], hiA);
                xb[kb] = O::pack8(XB[2 * kb], hiB);
            }
            f32x4 PA[4], PB[4];
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                PA[tt] = zero4();
                PB[tt] = zero4();
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) {
                    const F8 wf = O::ld8(sW + ((tt * KB + kb) * 64 + lane) * 8);
                    PA[tt] = O::mma32(wf, xa[kb], PA[tt]);
                    PB[tt] = O::mma32(wf, xb[kb], PB[tt]);
                }
            }
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                const f32x4 s = *(const f32x4*)(sKts + 16 * tt + 4 * g);
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) {
                    PA[tt][ii] = -PA[tt][ii] * s[ii];
                    PB[tt][ii] = (Ur[tt][ii] - PB[tt][ii]) * s[ii];
                }
            }
            F8 dAh[2], dAl[2], dBh[2], dBl[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                O::split8(PA[2 * h], PA[2 * h + 1], dAh[h], dAl[h]);
                O::split8(PB[2 * h], PB[2 * h + 1], dBh[h], dBl[h]);
            }
#pragma unroll
            for (int m = 0; m < ND; ++m) {
                const E* kr = sKt + (16 * m + c) * L::KT_P + 4 * g;
                f32x4 xa2 = XA[m] * gam, xb2 = XB[m] * gam;
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const F8 kf = O::ld44(kr + 32 * h, kr + 32 * h + 16);
                    xa2 = O::mma32(kf, dAh[h], xa2);
                    xb2 = O::mma32(kf, dBh[h], xb2);
                    if (O::kSplit) {
                        xa2 = O::mma32(kf, dAl[h], xa2);
                        xb2 = O::mma32(kf, dBl[h], xb2);
                    }
                }
                XA[m] = xa2;
                XB[m] = xb2;
            }
        }
    }

    // ---- frame end: B_f tiles straight out; A_f through LDS into operand fragments
    const long long unit = (long long)bh * a.nf + fw;
    {
        float* bt = a.Bt + unit * (ND * ND * 256) + (long long)w * ND * 256;
#pragma unroll
        for (int t = 0; t < ND; ++t) *(f32x4*)(bt + t * 256 + lane * 4) = XB[t];
    }
    E* sAp = (E*)smem;  // sKrow/sL and sVrow are no longer read by any wave
    constexpr int NS = SplitCount<E>::N;
#pragma unroll
    for (int part = 0; part < NS; ++part) {
        if (part) __syncthreads();  // the previous part has been copied out
        const int kbw = w >> 1, jb = (w & 1) * 4 + (c & 3);
#pragma unroll
        for (int t = 0; t < ND; ++t) {
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
                const int lp = 4 * g + ii + 16 * (c >> 2);
                E* fr = sAp + ((t * KB + kbw) * 64 + lp) * 8;
                const float x = XA[t][ii];
                fr[jb] = O::cvt(part ? O::lo_of(x) : x);
                if ((ND & 1) && w == ND - 1) fr[4 + (c & 3)] = (E)0.f;
            }
        }
        __syncthreads();
        E* dst = (E*)a.Apack + (unit * NS + part) * L::APK_E;
        constexpr int NV = L::APK_E / EPV;
        for (int u = tid; u < NV; u += L::NT) *(V16*)(dst + u * EPV) = *(const V16*)(sAp + u * EPV);
    }
}

// -------------------------------------------------------------------------------------
// Phase 2: the serial chain over frames, S_f = S_{f-1} A_f + B_f, one 16-row slice per wave
// -------------------------------------------------------------------------------------
template <typename E, int ND>
__global__ __launch_bounds__(64) void gdn_frame_chain(P2Args a) {
    using O = Ops<E>;
    using F8 = typename O::F8;
    using Gm = Geo<E, ND>;
    constexpr int D = Gm::D, KB = Gm::KB;
    constexpr int APK_E = ND * KB * Gm::FRAG;
    constexpr int NS = SplitCount<E>::N;
    const int lane = threadIdx.x, c = lane & 15, g = lane >> 4;
    const int s = blockIdx.x, bh = blockIdx.y;

    // state tiles: X[t] lane (c,g) = S[16s + c][16t + 4g + i]
    f32x4 X[ND];
    const long long srow = (long long)bh * D * D + (long long)(16 * s + c) * D;
#pragma unroll
    for (int t = 0; t < ND; ++t)
        X[t] = a.state_src ? *(const f32x4*)(a.state_src + srow + 16 * t + 4 * g) : zero4();

    for (int fw = 0; fw < a.nf; ++fw) {
        const long long unit = (long long)bh * a.nf + fw;
        const E* ah = (const E*)a.Apack + unit * NS * APK_E;
        const E* al = ah + APK_E;
        const float* bt = a.Bt + unit * (ND * ND * 256) + (long long)s * ND * 256;
        // issue every load of the frame before the first use
        F8 fh[ND][KB], fl[ND][KB];
        f32x4 acc[ND];
#pragma unroll
        for (int t = 0; t < ND; ++t) {
            acc[t] = *(const f32x4*)(bt + t * 256 + lane * 4);
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                const int off = ((t * KB + kb) * 64 + lane) * 8;
                fh[t][kb] = O::ld8(ah + off);
                fl[t][kb] = O::kSplit ? O::ld8(al + off) : O::zero8();
            }
        }
        F8 xh[KB], xl[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
            O::split8(X[2 * kb], (2 * kb + 1 < ND) ? X[(2 * kb + 1) % ND] : zero4(), xh[kb], xl[kb]);
#pragma unroll
        for (int t = 0; t < ND; ++t) {
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                acc[t] = O::mma32(fh[t][kb], xh[kb], acc[t]);
                if (O::kSplit) {
                    acc[t] = O::mma32(fl[t][kb], xh[kb], acc[t]);
                    acc[t] = O::mma32(fh[t][kb], xl[kb], acc[t]);
                }
            }
            X[t] = acc[t];
        }
        // S_f as readout operand (hi, then lo for bf16): fragment (n = s, kb = t/2),
        // lane c + 16 (2 (t%2) + g/2), elements 4 (g%2) .. +3  (IDENT slot map over d_k)
        E* sp = (E*)a.Spack + unit * NS * APK_E;
#pragma unroll
        for (int part = 0; part < NS; ++part) {
            E* spp = sp + part * APK_E;
#pragma unroll
            for (int t = 0; t < ND; ++t) {
                const int lp = c + 16 * (2 * (t & 1) + (g >> 1));
                f32x4 v = X[t];
                if (part) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) v[i] = O::lo_of(v[i]);
                }
                O::st4(spp + ((s * KB + (t >> 1)) * 64 + lp) * 8 + 4 * (g & 1), v);
            }
            if (ND & 1) {
                const int lp = c + 16 * (2 + (g >> 1));
                O::st4(spp + ((s * KB + KB - 1) * 64 + lp) * 8 + 4 * (g & 1), zero4());
            }
        }
    }
    if (a.state_dst) {
#pragma unroll
        for (int t = 0; t < ND; ++t) *(f32x4*)(a.state_dst + srow + 16 * t + 4 * g) = X[t];
    }
}

// -------------------------------------------------------------------------------------
// Phase 3: readout O_f = Q_f S_f^T (as O^T = S_f Q^T so each lane owns 4 outputs of a token)
// -------------------------------------------------------------------------------------
template <typename E, int ND>
__global__ __launch_bounds__(256) void gdn_frame_readout(P3Args a) {
    using O = Ops<E>;
    using F8 = typename O::F8;
    using Gm = Geo<E, ND>;
    constexpr int D = Gm::D, KB = Gm::KB;
    constexpr int APK_E = ND * KB * Gm::FRAG;
    constexpr int NS = SplitCount<E>::N;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int c = lane & 15, g = lane >> 4;
    const int fw = blockIdx.x, bh = blockIdx.y;
    const int N = a.frame_len;
    const long long unit = (long long)bh * a.nf + fw;
    const E* sp = (const E*)a.Spack + unit * NS * APK_E;
    F8 sh[ND][KB], sl[ND][KB];
#pragma unroll
    for (int n = 0; n < ND; ++n)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            sh[n][kb] = O::ld8(sp + ((n * KB + kb) * 64 + lane) * 8);
            sl[n][kb] = O::kSplit ? O::ld8(sp + APK_E + ((n * KB + kb) * 64 + lane) * 8) : O::zero8();
        }

    const long long tok0 = (long long)bh * a.T + (long long)(a.f0 + fw) * N;
    const E* qp = (const E*)a.q + tok0 * D;
    const int ntile = (N + 15) / 16;
    for (int tt = w; tt < ntile; tt += 4) {
        const int t = 16 * tt + c;
        const bool valid = t < N;
        F8 qb[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            const int col = 32 * kb + 8 * g;
            qb[kb] = (valid && col < D) ? O::ld8(qp + (long long)t * D + col) : O::zero8();
        }
#pragma unroll
        for (int n = 0; n < ND; ++n) {
            f32x4 acc = zero4();
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                acc = O::mma32(sh[n][kb], qb[kb], acc);
                if (O::kSplit) acc = O::mma32(sl[n][kb], qb[kb], acc);
            }
            if (valid) {
                const long long o = (tok0 + t) * D + 16 * n + 4 * g;
                if (a.out_f32) *(f32x4*)((float*)a.out + o) = acc;
                else O::st4((E*)a.out + o, acc);
            }
        }
    }
}

// -------------------------------------------------------------------------------------
// launchers
// -------------------------------------------------------------------------------------
template <typename E, int ND>
hipError_t launch_gdn_window(const P1Args& p1, const P2Args& p2, const P3Args& p3, hipStream_t st,
                             void* const* ev) {
    using L = P1<E, ND>;
    static bool attr_done = false;
    if (!attr_done) {
        hipError_t e = hipFuncSetAttribute((const void*)gdn_frame_affine<E, ND>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, L::LDS_B);
        if (e != hipSuccess) return e;
        attr_done = true;
    }
    const int BH = p1.BH;
    hipError_t e = record(ev, 0, st);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((gdn_frame_affine<E, ND>), dim3(p1.nf, BH), dim3(L::NT), L::LDS_B, st, p1);
    if ((e = hipGetLastError()) != hipSuccess || (e = record(ev, 1, st)) != hipSuccess) return e;
    hipLaunchKernelGGL((gdn_frame_chain<E, ND>), dim3(ND, BH), dim3(64), 0, st, p2);
    if ((e = hipGetLastError()) != hipSuccess || (e = record(ev, 2, st)) != hipSuccess) return e;
    hipLaunchKernelGGL((gdn_frame_readout<E, ND>), dim3(p3.nf, BH), dim3(256), 0, st, p3);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    return record(ev, 3, st);
}

#define GDN_INST(E, ND) \
    template hipError_t launch_gdn_window<E, ND>(const P1Args&, const P2Args&, const P3Args&, hipStream_t, \
                                                 void* const*);
GDN_INST(bf16, 1) GDN_INST(bf16, 2) GDN_INST(bf16, 4) GDN_INST(bf16, 7) GDN_INST(bf16, 8)
GDN_INST(float, 1) GDN_INST(float, 2) GDN_INST(float, 4) GDN_INST(float, 7) GDN_INST(float, 8)

size_t gdn_unit_bytes(int nd, int esize, size_t* apack, size_t* bt, size_t* spack) {
    const int kb = (nd + 1) / 2;
    const int nsplit = esize == 2 ? 2 : 1;  // bf16 operands are stored as hi + lo
    *apack = (size_t)nsplit * nd * kb * 64 * 8 * esize;
    *bt = (size_t)nd * nd * 256 * 4;
    *spack = *apack;
    return *apack + *bt + *spack;
}

}  // namespace gdn
