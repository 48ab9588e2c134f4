// gdn_frame.hpp -- frame-wise gated delta rule on gfx950: the kernels (their launchers are
// in gdn_frame.hip; the rotary-embedding instantiations in gdn_frame_rope.hip).
//
// Method: the gated delta rule of Gated DeltaNet (named as the frame-wise token mixer in
// the SANA-WM news summary, section "hybrid architecture for long rollouts"; update as
// published by Yang, Kautz & Hatamizadeh, 2025), read out at frame boundaries (SANA-Video
// talk, block-KV-cache segment).  Per (b, h), state S is d_v x d_k, fp32.
//
// The readout needs the state only at frame ends, and over any run of tokens the state
// map is affine:  S_end = S_start A + B.  Three launches per window of frames:
//  1. gdn_frame_affine  -- one workgroup per (b, h, group of G consecutive frames), all
//     groups in parallel.  Each frame is cut into chunks of 64 tokens; each chunk becomes
//     its WY/UT factors (Gram matrix K K^T, unit-lower-triangular inverse T = (I + L)^-1,
//     W and U) on bf16 matrix cores with fp32 accumulation, and is applied to a stacked
//     state [A ; B] that starts at [I ; 0] at the group start.  At every frame end the
//     partial map (A_{g,<=f}, B_{g,<=f}) of the group so far is written out.  With a
//     single group per (b, h) the start state is known and the pass runs from it (true
//     start: B only, the B maps are the states).
//  2. gdn_frame_chain   -- one workgroup per (b, h, 16-row slice of S): the serial part,
//     one product per GROUP:  S_g = S_{g-1} A_g + B_g.  Writes the state before every
//     group and the final state.
//  3. gdn_frame_readout -- one workgroup per (b, h, frame), or per part of a frame's
//     chunks when a call has few frames: composes S_f = S_{g-1} A_{g,<=f} + B_{g,<=f},
//     then streams Q in and O = Q S_f^T out.
//     For the per-token readout the third launch is gdn_token_readout instead: the same
//     chunk pipeline rerun from each group's true start state, writing o_t = S_t q_t.
// Chunk algebra (derivation from the recurrence, restated; G_t = sum_{i<=t} log a_i in
// the chunk, k^ the normalised keys):
//   L_ti = b_t e^{G_t - G_i} k^_t.k^_i (i < t),  T = (I + L)^-1,
//   U = T diag(b) V,  W = T diag(b e^G) K^,  Kt = diag(e^{G_C - G}) K^,
//   S <- e^{G_C} S + (U - W S^T)^T Kt.
// Rows of S never mix, which is what lets the state be split into 16-row slices.
//
// Precision (bf16 inputs).  Inputs q, k, v are exact bf16 operands.  Quantities that carry
// the state (the chunk innovation Kt-scaled (U - W S^T), the maps A and the states S) are
// sent to the matrix cores as bf16 hi + lo pairs, which keeps ~16 significant bits; W and
// U are formed block by block as X_I = Z_I + (T_II - I) Z_I with Z_I = R_I - sum_{J<I}
// L_IJ X_J kept in fp32, so only the operand of the correction (T_II - I) Z_I is rounded.
// The per-frame maps that only the readout composes with are kept in fp16 with a power
// of two per 16-row slice (11 significant bits, below the rounding of the bf16 output;
// the readout takes A to the fp16 matrix cores as stored, against S as an fp16 hi + lo pair);
// the group maps that the chain carries keep the hi + lo pair (A) and fp32 (B).
#pragma once
#include "common.hpp"
#include "gdn_kernels.hpp"
#include <float.h>
#include <type_traits>

namespace gdn {

// -------------------------------------------------------------------------------------
// Phase 1: per-frame partial affine maps of each group of frames
// -------------------------------------------------------------------------------------
// Workgroup = ND "chain" waves + "prep" waves, software-pipelined: chain wave w owns the
// 16-row slices w of A and of B; per chunk it runs the block substitution for W column
// tile w and U column tile w, then the state update.  The prep waves prepare chunks
// ahead: key norms, gate prefix, Gram matrix, scaled L, inverses of the 16x16 diagonal
// blocks of (I + L), and the bf16 operand fragments the substitution consumes.
//  - OV (bf16 where the buffers fit in LDS): two prep waves and one barrier per chunk
//    (schedule at the main loop); the global -> LDS copies are issued by the prep waves
//    and the first four chain waves.
//  - otherwise one prep wave and two barriers per chunk (bf16, d = 128), or the same
//    stages one after the other on single buffers (fp32 inputs, whose buffers do not fit
//    twice in LDS at d >= 112).
template <int V> struct RoleC {
    static constexpr int value = V;
};

// TOK: the per-token readout pass (see gdn_token_readout below); otherwise the frame maps.
// RP: keys rotated by the 3D rotary embedding as they are loaded (GDN_F_ROPE_QK).
template <typename E, int ND, bool TOK = false, bool RP = false> struct P1 {
    using G = Geo<E, ND>;
    static constexpr bool BF = sizeof(E) == 2;
    static constexpr int al(int b) { return (b + 255) / 256 * 256; }
    static constexpr int RB = G::D * (int)sizeof(E);  // bytes of one K, V or Q row
    // LDS row pitch of bf16 tiles: a multiple of 32 bytes with an odd count of 32-byte
    // units, so that the transposed reads (8 consecutive rows x 32 bytes per half-wave) hit
    // distinct banks.  fp32 tiles are read with plain loads and keep their length.
    static constexpr int pitch(int rb) {
        return !BF ? rb : ((rb + 31) / 32 % 2 == 1) ? (rb + 31) / 32 * 32 : (rb + 31) / 32 * 32 + 32;
    }
    static constexpr int KPB = pitch(RB);
    static constexpr int KG = KPB / 16;           // 16-byte granules per LDS row
    static constexpr int DG = RB / 16;            // granules that hold data
    // W staged transposed (row = a d_k column of W, 64 tokens per row)
    static constexpr int WRB = 64 * (int)sizeof(E);
    static constexpr int WPB = pitch(WRB);
    static constexpr int LD_P = 20;               // diagonal L blocks: row pitch (floats)
    // block stride: 16 rows plus 4 floats, so that the inverse's broadcast reads of the
    // four blocks (one address per block, 16 lanes each) fall in different banks
    static constexpr int LD_BS = 16 * LD_P + 4;
    static constexpr int NFR = 10;                // fragments: 6 L_IJ, 4 (T_II - I)
    static constexpr int FR_E = NFR * 64 * 4;     // elements per fragment set
    static constexpr int KV_B = al(64 * KPB);
    static constexpr int RAW_B = al(2 * 64 * 4);
    // per-token scalars: [0,64) b e^G n, [64,128) b, [128,192) e^{G_C - G} n, [192] gamma_C;
    // TOK adds [208,272) G (log2, inclusive), [272,336) n, [336,400) e^G and, for fp32
    // inputs, [400,464) the low part of G (G = hi + lo, see wave_incl_scan2)
    static constexpr int SC_N = TOK ? (BF ? 400 : 464) : 208;
    static constexpr int SC_B = al(SC_N * 4);
    static constexpr int FR_B = al(FR_E * (int)sizeof(E));
    static constexpr int W_B = al(G::D * WPB);
    // TOK: the 10 lower-triangle 16x16 tiles of the decay-masked (K Q^T), hi (+ lo) fragments
    static constexpr int AQ_B = TOK ? al(10 * SplitCount<E>::N * 64 * 4 * (int)sizeof(E)) : 0;
    static constexpr int LD_B = al(4 * LD_BS * 4);
    // prep wave's per-token scalars: [0,64) G, [64,128) n, [128,192) b n, [192,256) the
    // within-block decay, [256,448) the cross-block decays; fp32 inputs add [448,512) the
    // low part of G
    static constexpr int TKN = BF ? 7 : 8;
    static constexpr int TK_B = al(TKN * 64 * 4);
    // Buffer counts.  OV (overlapped): the chain waves run the state update of chunk q
    // together with the substitution of chunk q+1, the prep wave prepares chunk q+2 and
    // copies of chunk q+3 are in flight -- K for chunks q..q+3, V and gates for q+1..q+3,
    // scalars for q..q+2, fragments and W for two chunks.  Used where it fits in LDS.
    static constexpr int ov_bytes() {
        return 4 * KV_B + 3 * KV_B + 3 * RAW_B + 3 * SC_B + 2 * FR_B + 2 * W_B + LD_B + 2 * TK_B;
    }
    // TOK, two barriers per chunk: K and gates for chunks q..q+2, V and Q for q..q+1
    static constexpr int tok_bytes() {
        return 3 * KV_B + 4 * KV_B + 3 * RAW_B + 2 * SC_B + 2 * FR_B + W_B + AQ_B + LD_B + TK_B;
    }
    static constexpr bool OV = !TOK && BF && ov_bytes() <= 160 * 1024;
    static constexpr bool PIPE = BF && (!TOK || tok_bytes() <= 160 * 1024);
    static constexpr int NPW = OV ? 2 : 1;        // prep waves
    // helper waves at d = 112 (OV, and the per-token pass's two-barrier schedule): they form
    // the chunk's W column tiles, which the chain waves would otherwise substitute beside
    // their U tiles (and, in the per-token pass, the intra-chunk weight tiles past the
    // chain waves' one each).  Twelve waves are three per SIMD: at most 168 registers.
    static constexpr int NH = ((OV || (TOK && PIPE)) && ND == 7) ? 3 : 0;
    static constexpr int NW = ND + NPW + NH;      // chain waves + prep waves + helper waves
    static constexpr int NT = 64 * NW;
    static constexpr int NB = PIPE ? 2 : 1;       // fragment sets
    static constexpr int NBK = OV ? 4 : (!PIPE ? 1 : 3);                 // K chunk buffers
    static constexpr int NBV = OV ? 3 : (TOK ? (PIPE ? 2 : 1) : NBK);    // V chunk buffers
    static constexpr int NBQ = TOK ? (PIPE ? 2 : 1) : 0;                 // Q chunk buffers
    static constexpr int NBR = OV ? 3 : NBK;      // gate buffers
    static constexpr int NBS = OV ? 3 : NB;       // per-token scalar sets
    static constexpr int NBW = OV ? 2 : 1;        // W staging buffers
    static constexpr int PD = PIPE ? (OV ? 3 : NBK - 1) : 0;  // chunks the K copies run ahead
    static constexpr int OFF_K = 0;                        // [NBK] row-major K chunk
    static constexpr int OFF_V = OFF_K + NBK * KV_B;       // [NBV] row-major V chunk
    static constexpr int OFF_Q = OFF_V + NBV * KV_B;       // [NBQ] row-major Q chunk (TOK)
    static constexpr int OFF_RAW = OFF_Q + NBQ * KV_B;     // [NBR] alpha[64], beta[64]
    static constexpr int OFF_SC = OFF_RAW + NBR * RAW_B;   // [NBS] per-token scalars
    static constexpr int OFF_FR = OFF_SC + NBS * SC_B;     // [NB] substitution fragments
    static constexpr int OFF_W = OFF_FR + NB * FR_B;       // [NBW] W staging (chain waves)
    static constexpr int OFF_AQ = OFF_W + NBW * W_B;       // masked (K Q^T) fragments (TOK)
    static constexpr int OFF_LD = OFF_AQ + AQ_B;           // diagonal blocks of L (prep wave)
    static constexpr int OFF_TK = OFF_LD + LD_B;           // [NPW] per-token scalars (prep waves)
    static constexpr int OFF_RP = OFF_TK + NPW * TK_B;     // rotary frequencies (hi, lo)
    static constexpr int RP_B = RP ? 2 * kRopePairs * 4 : 0;
    static constexpr int LDS_B = OFF_RP + RP_B;
    static_assert(LDS_B <= 160 * 1024, "LDS budget");
    static_assert(RB % 16 == 0, "rows are whole 16-byte granules");
    static constexpr int APK_E = G::ND * G::KB * G::FRAG;  // A fragments (elements)
};


// fragment index of L_IJ (I > J) in a fragment set
__host__ __device__ constexpr int frL(int I, int J) { return I * (I - 1) / 2 + J; }
__host__ __device__ constexpr int frTm(int I) { return 6 + I; }

// MODE = the call's GDN_F_NORMALIZE_K (bit 0) and GDN_F_ADDITIVE (bit 1) flags, true-start
// mode (bit 2) and the rotary embedding of k (bit 3), fixed at compile time so that the
// per-tile choices they make are not branches and calls without rotation carry none of it.
template <typename E, int ND, int MODE, bool TOK>
__device__ __forceinline__ void affine_body(P1Args a) {
    constexpr bool ROPE = (MODE & 8) != 0;
    using L = P1<E, ND, TOK, ROPE>;
    using O = Ops<E>;
    using F8 = typename O::F8;
    using F4 = typename O::F4;
    using V16 = typename O::V16;
    constexpr int D = L::G::D, KB = L::G::KB;
    constexpr int NS = SplitCount<E>::N;
    extern __shared__ __attribute__((aligned(256))) unsigned char smem[];
    float* const sSC0 = (float*)(smem + L::OFF_SC);
    E* const sFR0 = (E*)(smem + L::OFF_FR);
    float* const sLD = (float*)(smem + L::OFF_LD);
    float* const sTK0 = (float*)(smem + L::OFF_TK);
    constexpr int BM = L::NB - 1;
    auto KB_ = [&](int p) { return (E*)(smem + L::OFF_K + (p % L::NBK) * L::KV_B); };
    auto VB_ = [&](int p) { return (E*)(smem + L::OFF_V + (p % L::NBV) * L::KV_B); };
    auto RAW = [&](int p) { return (float*)(smem + L::OFF_RAW + (p % L::NBR) * L::RAW_B); };
    constexpr int NBQ1 = L::NBQ ? L::NBQ : 1;
    auto QB_ = [&](int p) { return (E*)(smem + L::OFF_Q + (p % NBQ1) * L::KV_B); };
    auto SC = [&](int p) { return (float*)((unsigned char*)sSC0 + (p % L::NBS) * L::SC_B); };
    auto FR = [&](int p) { return (E*)((unsigned char*)sFR0 + (p & BM) * L::FR_B); };
    auto WB_ = [&](int p) { return (E*)(smem + L::OFF_W + (p % L::NBW) * L::W_B); };
    // SC layout: [0,64) ws = b e^G n, [64,128) b, [128,192) kts = e^{G_C - G} n, [192] gamma_C

    const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c = lane & 15, g = lane >> 4;
    const bool prep = (w >= ND) && (w < ND + L::NPW);
    const bool helper = w >= ND + L::NPW;  // (L::NH > 0 only)
    const int gi = blockIdx.x, bh = blockIdx.y;
    const int N = a.frame_len;
    const int fw0 = gi * a.G;                              // first frame (in window) of the group
    const int nfg = min(a.G, a.nf - fw0);                  // frames in this group
    const long long tok0 = (long long)bh * a.T + (long long)(a.f0 + fw0) * N;
    const E* kp = (const E*)a.k + tok0 * D;
    const E* vp = (const E*)a.v + tok0 * D;
    const E* qp = TOK ? (const E*)a.q + tok0 * D : nullptr;
    constexpr bool additive = (MODE & 2) != 0;
    constexpr bool normalize = (MODE & 1) != 0;
    // TS (true start, frame maps only): the call has one group per (b, h), so the state at
    // the group start is known -- the B part starts from it, the A part is not formed,
    // every frame end writes the true state S_f as its B map, and state_out is written here.
    constexpr bool TS = !TOK && (MODE & 4) != 0;
    const int nch = (N + 63) / 64;
    const int nq = nfg * nch;                   // chunks of the group, frame by frame
    auto chunk_t0 = [&](int q) { const int f = q / nch; return (long long)f * N + (q - f * nch) * 64; };
    auto chunk_len = [&](int q) { const int f = q / nch; return min(64, N - (q - f * nch) * 64); };

    // ---- chunk loads: global -> LDS copies with no register staging.  K and V land
    //      row-major (pitch KPB); each copy instruction moves 64 granules of 16 bytes and
    //      instructions are dealt round-robin to all waves.  Rows past the chunk's end and
    //      padding granules copy a valid in-bounds granule instead (their values are
    //      finite and multiplied by zero scale factors, never used as data).
    // copy instructions dealt round-robin to the waves whose bits are set in `mask`
    // Copies of chunk p for the tiles tf .. tf+nt-1 of (K, V, Q) and, with `gates`, of
    // alpha and beta.  Instruction i copies 1 KB row block i / nt of tile tf + i % nt (the
    // tiles alternate), and the instructions are dealt round-robin to the waves whose bits
    // are set in `mask`: the copies in flight together then read neighbouring bytes.
    // (Giving each wave a contiguous range of a tile instead was measured 1.7x slower at
    // d = 112; alternating the tiles or not made no measurable difference.)
    auto dma_tiles = [&](int p, int tf, int nt, bool gates, unsigned mask) {
        if (!((mask >> w) & 1u)) return;
        const int wi = __builtin_popcount(mask & ((1u << w) - 1u)), nw = __builtin_popcount(mask);
        const long long t0 = chunk_t0(p);
        const int Cc = chunk_len(p);
        for (int i = wi; i < nt * L::KG; i += nw) {
            const int ts = tf + i % nt, ii = i / nt;
            const int gidx = ii * 64 + lane, row = gidx / L::KG, piece = gidx - row * L::KG;
            const long long el = (t0 + min(row, Cc - 1)) * D + min(piece, L::DG - 1) * (16 / (int)sizeof(E));
            auto cp = [&](const E* src, int dst) {
                if constexpr (L::PIPE) dma16(src + el, smem + dst + ii * 1024);
                else *(u32x4*)(smem + dst + ii * 1024 + 16 * lane) = *(const u32x4*)(src + el);  // same, synchronous
            };
            if (ts == 0) cp(kp, L::OFF_K + (p % L::NBK) * L::KV_B);
            else if (ts == 1) cp(vp, L::OFF_V + (p % L::NBV) * L::KV_B);
            else cp(qp, L::OFF_Q + (p % NBQ1) * L::KV_B);
        }
        if (gates && !additive && wi == (nt * L::KG) % nw) {
            const long long tt = tok0 + t0 + min(lane, Cc - 1);
            const int dst = L::OFF_RAW + (p % L::NBR) * L::RAW_B;
            if constexpr (L::PIPE) {
                dma4(a.alpha + tt, smem + dst);
                dma4(a.beta + tt, smem + dst + 256);
            } else {
                ((float*)(smem + dst))[lane] = a.alpha[tt];
                ((float*)(smem + dst + 256))[lane] = a.beta[tt];
            }
        }
    };
    // With the rotary embedding the copying waves also rotate the keys they copied, so the
    // key rows are dealt round-robin over the copying waves on their own (and the value rows
    // likewise, starting half-way round): every copying wave gets about the same share of
    // the rotation.  Key row block ii goes to wave number ii mod nw of the mask.
    auto dma_chunk_rp = [&](int p, unsigned mask) {
        if (!((mask >> w) & 1u)) return;
        const int wi = __builtin_popcount(mask & ((1u << w) - 1u)), nw = __builtin_popcount(mask);
        const long long t0 = chunk_t0(p);
        const int Cc = chunk_len(p);
        for (int ts = 0; ts < 2; ++ts)
            for (int ii = (wi + nw - ts * (nw / 2)) % nw; ii < L::KG; ii += nw) {
                const int gidx = ii * 64 + lane, row = gidx / L::KG, piece = gidx - row * L::KG;
                const long long el = (t0 + min(row, Cc - 1)) * D + min(piece, L::DG - 1) * (16 / (int)sizeof(E));
                const int dst = ts == 0 ? L::OFF_K + (p % L::NBK) * L::KV_B : L::OFF_V + (p % L::NBV) * L::KV_B;
                if constexpr (L::PIPE) {
                    dma16((ts == 0 ? kp : vp) + el, smem + dst + ii * 1024);
                } else {  // same, synchronous
                    *(u32x4*)(smem + dst + ii * 1024 + 16 * lane) = *(const u32x4*)((ts == 0 ? kp : vp) + el);
                }
            }
        if (!additive && wi == nw - 1) {
            const long long tt = tok0 + t0 + min(lane, Cc - 1);
            const int dst = L::OFF_RAW + (p % L::NBR) * L::RAW_B;
            if constexpr (L::PIPE) {
                dma4(a.alpha + tt, smem + dst);
                dma4(a.beta + tt, smem + dst + 256);
            } else {
                ((float*)(smem + dst))[lane] = a.alpha[tt];
                ((float*)(smem + dst + 256))[lane] = a.beta[tt];
            }
        }
    };
    auto dma_chunk = [&](int p, unsigned mask) {
        if constexpr (ROPE && !TOK) dma_chunk_rp(p, mask);
        else dma_tiles(p, 0, 2, true, mask);
    };

    // At the end of iteration q chunk q+2 must have landed (the prep wave reads it next)
    // while the copies of chunks q+3 .. q+PD may still be in flight: wait until at most
    // that many of this wave's copy instructions are outstanding (they complete in
    // issue order).
    constexpr unsigned kAll = (1u << L::NW) - 1u;
    // Waves that issue the copies in the overlapped schedule's loop: chain waves 0..3 and
    // both prep waves, five or so copy instructions each.  Measured at d = 112: a wave
    // keeps only a few global -> LDS copies in flight and stalls at issue beyond that, so
    // one or two issuing waves are far too slow, while all waves stall every chain wave;
    // chain waves 0..3 are the first of the two chain waves on their SIMD and finish their
    // chunk early, which hides their stall.
    // (at d = 16 the workgroup has three waves: the mask keeps to the waves that exist)
    constexpr unsigned kCopy = L::OV ? ((0xFu | (3u << ND)) & kAll) : kAll;
    // the per-token pass's loop likewise: chain waves 0..3 and the prep wave (the second
    // chain wave on each SIMD finishes last and was measured stalling ~1,500 cycles per
    // chunk on its share of the copies)
    constexpr unsigned kCopyT = (TOK && L::PIPE) ? ((0xFu | (1u << ND)) & kAll) : kAll;
    int ncopy = 0;  // copy instructions this wave issues per chunk (with all waves copying)
    if constexpr (ROPE && !TOK) {
        for (int ii = w; ii < L::KG; ii += L::NW) ++ncopy;
        for (int ii = (w + L::NW - L::NW / 2) % L::NW; ii < L::KG; ii += L::NW) ++ncopy;
        if (!additive && w == L::NW - 1) ncopy += 2;
    } else {
        for (int i = w; i < 2 * L::KG; i += L::NW) ++ncopy;
        if (!additive && w == (2 * L::KG) % L::NW) ncopy += 2;
    }
    // GDN_F_ROPE_QK: keys (and, in the per-token pass, queries) are rotated by the 3D rotary
    // embedding in LDS, in place.  Each wave rotates the granules it copied itself for
    // chunk p (dma_chunk_rp; dma_tiles in the per-token pass), once its own copies of that
    // chunk have completed and before the barrier that publishes the chunk, so every
    // reader sees rotated values and no wave waits for another.  Rows past the chunk's end
    // hold copies of a valid row and are rotated harmlessly (their scale factors are 0).
    // (the frequencies are read from LDS, copied there at the kernel's start)
    const float* const sRP = (const float*)(smem + L::OFF_RP);
    const float rinv_w = ROPE ? 1.f / (float)a.rope.grid_w : 0.f;
    // rotates the granule that copy lane `lane` of row block ii of chunk p's tile `buf` holds
    auto rotate_granule = [&](E* buf, int p, int ii) {
        const int fl = p / nch, cq = p - fl * nch;
        const float pf = (float)(a.rope.frame0 + a.f0 + fw0 + fl);
        const int gidx = ii * 64 + lane, row = gidx / L::KG, piece = gidx - row * L::KG;
        if (piece >= L::DG) return;  // padding granule
        const int t = cq * 64 + row, hr = rope_div(t, a.rope.grid_w, rinv_w);
        V16* g16 = (V16*)((unsigned char*)buf + row * L::KPB + piece * 16);
        *g16 = rope_rotate<E>(*g16, piece * (L::G::EPV / 2), pf, (float)hr, (float)(t - hr * a.rope.grid_w),
                              a.rope.p1, a.rope.p2, sRP, sRP + kRopePairs);
    };
    auto rotate_own = [&](int p, unsigned mask) {
        if constexpr (!ROPE || TOK) return;
        if (!((mask >> w) & 1u)) return;
        const int wi = __builtin_popcount(mask & ((1u << w) - 1u)), nw = __builtin_popcount(mask);
        for (int ii = wi; ii < L::KG; ii += nw) rotate_granule(KB_(p), p, ii);  // this wave's key row blocks (dma_chunk_rp)
    };
    // the per-token pass: the K and Q row blocks this wave copied with dma_tiles(p, tf, nt, ., mask)
    auto rotate_tiles = [&](int p, int tf, int nt, unsigned mask) {
        if constexpr (!ROPE || !TOK) return;
        if (!((mask >> w) & 1u)) return;
        const int wi = __builtin_popcount(mask & ((1u << w) - 1u)), nw = __builtin_popcount(mask);
        for (int i = wi; i < nt * L::KG; i += nw) {
            const int ts = tf + i % nt;
            if (ts != 1) rotate_granule(ts == 0 ? KB_(p) : QB_(p), p, i / nt);  // V is not rotated
        }
    };
    auto wait_dma_behind = [&](int q) {
        const int ahead = min(L::PD - 2, nq - 3 - q);  // chunks q+3 .. issued and not needed yet
        const int n = ahead > 0 ? ahead * ncopy : 0;
        switch (n < 15 ? n : 15) {
#define GDN_W(N) case N: __builtin_amdgcn_s_waitcnt(0x0F70 | N); break;
            GDN_W(0) GDN_W(1) GDN_W(2) GDN_W(3) GDN_W(4) GDN_W(5) GDN_W(6) GDN_W(7)
            GDN_W(8) GDN_W(9) GDN_W(10) GDN_W(11) GDN_W(12) GDN_W(13) GDN_W(14) GDN_W(15)
#undef GDN_W
        }
    };

    // Prep roles: with two prep waves, role 0 takes the diagonal blocks of L (and their
    // inverses, prep3) and the per-token scalars the chain waves read, role 1 the
    // off-diagonal blocks; each computes the key norms and gate prefix it needs itself.
    // A single prep wave (role 2) does all of it.
    auto has_diag = [](auto R) { return R.value != 1; };
    auto has_off = [](auto R) { return R.value != 0; };
    // ---- prep, first part: Gram matrix on the matrix cores and the key norms
    auto prep1 = [&](int p, f32x4 (&gr)[10], auto R) {
        float* const sTK = sTK0 + (R.value == 1 ? L::TKN * 64 : 0);
        const int Cc = chunk_len(p);
        const int t = lane;
        const bool valid = t < Cc;
        // Gram tiles computed transposed, K_J K_I^T: lane (c, g) then holds row 16I + c,
        // columns 16J + 4g .. +3 of K K^T -- the row layout of the K16 A operand.  Each
        // 16-token row block of K is read from LDS once, as fragments kf[X][kb].
        {
            F8 kf[4][KB];
#pragma unroll
            for (int X = 0; X < 4; ++X)
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)  // d_k columns past D are zero
                    kf[X][kb] = (32 * kb + 8 * g < D)
                                    ? O::ld8((const E*)((const char*)KB_(p) + (16 * X + c) * L::KPB) + 32 * kb + 8 * g)
                                    : O::zero8();
#pragma unroll
            for (int q = 0; q < 10; ++q) {
                const int I = q < 1 ? 0 : q < 3 ? 1 : q < 6 ? 2 : 3;  // lower-triangle tile (I, J)
                const int J = q - I * (I + 1) / 2;
                gr[q] = zero4();
                if (I != J && !has_off(R)) continue;  // (diagonal tiles give the norms)
                if (!additive || (normalize && I == J)) {
#pragma unroll
                    for (int kb = 0; kb < KB; ++kb) gr[q] = O::mma32(kf[J][kb], kf[I][kb], gr[q]);
                }
            }
        }
        // key norm of token t from the Gram diagonal: lane (c, c/4) of diagonal tile I holds
        // k_i.k_i for i = 16I + c, in element c % 4
        float n2 = 0.f;
        {
            const int src = (t & 15) + 16 * ((t & 15) >> 2), e = c & 3;
#pragma unroll
            for (int I = 0; I < 4; ++I) {
                const f32x4 x = gr[I * (I + 3) / 2];
                float d = x[0];  // x[e], as selects
                d = e == 1 ? x[1] : d;
                d = e == 2 ? x[2] : d;
                d = e == 3 ? x[3] : d;
                const float v = __shfl(d, src);
                n2 = (t >> 4) == I ? v : n2;
            }
        }
        const float nrm = valid ? (normalize ? hw_rsq(fmaxf(n2, 1e-12f)) : 1.f) : 0.f;
        sTK[64 + t] = nrm;
    };
    // ---- prep, second part: gate prefix and per-token scalars, L from the Gram tiles, its
    //      off-diagonal blocks as operand fragments, its diagonal blocks to LDS
    auto prep2 = [&](int p, f32x4 (&gr)[10], auto R) {
        float* const sTK = sTK0 + (R.value == 1 ? L::TKN * 64 : 0);
        E* fr = FR(p);
        const int Cc = chunk_len(p);
        float* sc = SC(p);
        const int t = lane;
        const bool valid = t < Cc;
        const float nrm = sTK[64 + t];
        // (rows past the chunk's end hold finite copies: read them, then select)
        float gl = 0.f, be = 0.f;
        if constexpr (additive) {
            be = valid ? 1.f : 0.f;
        } else {
            const float al = RAW(p)[t], bl = RAW(p)[64 + t];
            float l2a, bb;
            if (a.flags & 16u) {
                // gates given as logits: log2 alpha = -softplus(al) log2(e), beta = sigmoid(bl);
                // softplus(x) = max(x, 0) + log(1 + e^{-|x|}); clamped as alpha >= FLT_MIN is
                constexpr float kLog2e = 1.4426950408889634f;
                const float sp2 = fmaxf(al, 0.f) * kLog2e + hw_log2(1.f + hw_exp2(-fabsf(al) * kLog2e));
                l2a = fmaxf(-sp2, -126.f);
                bb = 1.f / (1.f + hw_exp2(-bl * kLog2e));
            } else {
                l2a = hw_log2(fmaxf(al, FLT_MIN));
                bb = bl;
            }
            gl = valid ? l2a : 0.f;
            be = valid ? bb : 0.f;
        }
        // inclusive prefix over the chunk (log2 units).  Only differences of it and values
        // near the chunk's start are used; for fp32 inputs it is carried as hi + lo so
        // that a difference stays accurate after a run of near-zero gates (whose prefix
        // can reach thousands, where fp32 keeps ~1e-4 absolute); bf16 inputs keep hi only
        // (the bf16 rounding of the operands dominates there)
        float Gl = 0.f;
        const float Gs = L::BF ? wave_incl_scan(gl) : wave_incl_scan2(gl, Gl);
        // (the lane-read builtins are integer-typed: move the bits, not the value)
        auto lane_of = [](float x, int l) {
            return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l));
        };
        // G_x - G_y from (hi, lo) pairs
        auto gdif = [](float xh, float xl, float yh, float yl) { return L::BF ? xh - yh : (xh - yh) + (xl - yl); };
        const float GC = lane_of(Gs, 63), GCl = L::BF ? 0.f : lane_of(Gl, 63);
        if (has_diag(R)) {
            sc[t] = additive ? 0.f : be * hw_exp2(Gs + Gl) * nrm;
            sc[64 + t] = be;
            sc[128 + t] = hw_exp2(gdif(GC, GCl, Gs, Gl)) * nrm;
            if (t == 0) sc[192] = hw_exp2(GC + GCl);
            if constexpr (TOK) {
                sc[208 + t] = Gs;
                sc[272 + t] = nrm;
                sc[336 + t] = hw_exp2(Gs + Gl);
                if constexpr (!L::BF) sc[400 + t] = Gl;
            }
        }
        // decay factors of L split at the end of 16-token block J (both factors <= 1):
        // e^{G_i - G_j} = e^{G_i - G_end(J)} e^{G_end(J) - G_j} for i in a later block
        const int Jt = t >> 4;
        auto blk_end = [&](float x) {
            return lane_of(x, 15) * (Jt == 0) + lane_of(x, 31) * (Jt == 1) + lane_of(x, 47) * (Jt == 2) +
                   lane_of(x, 63) * (Jt == 3);
        };
        const float Gend = blk_end(Gs), Gendl = L::BF ? 0.f : blk_end(Gl);
        sTK[t] = Gs;
        if constexpr (!L::BF) sTK[448 + t] = Gl;
        sTK[128 + t] = be * nrm;
        sTK[192 + t] = nrm * hw_exp2(gdif(Gend, Gendl, Gs, Gl));
#pragma unroll
        for (int J = 0; J < 3; ++J)
            sTK[256 + 64 * J + t] =
                J < Jt ? be * nrm *
                             hw_exp2(gdif(Gs, Gl, lane_of(Gs, 16 * J + 15), L::BF ? 0.f : lane_of(Gl, 16 * J + 15)))
                       : 0.f;
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");  // sTK written by other lanes
        // every per-token factor first (reads only), then the scaling, then the writes
        f32x4 cf[3], gj[4], nj[4], gjl[4];
        float rf[6], si[4], gi_[4], gil[4];
#pragma unroll
        for (int J = 0; J < 4; ++J) {
            if (J < 3) cf[J] = *(const f32x4*)(sTK + 192 + 16 * J + 4 * g);
            gj[J] = *(const f32x4*)(sTK + 16 * J + 4 * g);
            nj[J] = *(const f32x4*)(sTK + 64 + 16 * J + 4 * g);
            si[J] = sTK[128 + 16 * J + c];
            gi_[J] = sTK[16 * J + c];
            gjl[J] = L::BF ? zero4() : *(const f32x4*)(sTK + 448 + 16 * J + 4 * g);
            gil[J] = L::BF ? 0.f : sTK[448 + 16 * J + c];
        }
#pragma unroll
        for (int q = 0; q < 10; ++q) {
            const int I = q < 1 ? 0 : q < 3 ? 1 : q < 6 ? 2 : 3;
            const int J = q - I * (I + 1) / 2;
            if (I != J) rf[frL(I, J)] = sTK[256 + 64 * J + 16 * I + c];
        }
#pragma unroll
        for (int q = 0; q < 10; ++q) {
            const int I = q < 1 ? 0 : q < 3 ? 1 : q < 6 ? 2 : 3;
            const int J = q - I * (I + 1) / 2;
            const int i = 16 * I + c;
            f32x4& acc = gr[q];
            if (I != J ? !has_off(R) : !has_diag(R)) continue;
            if (additive) {
                acc = zero4();
            } else if (I != J) {
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) acc[ii] *= rf[frL(I, J)] * cf[J][ii];
            } else {
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) {
                    const int j = 16 * J + 4 * g + ii;
                    acc[ii] = (i > j) ? si[I] * nj[J][ii] * hw_exp2(gdif(gi_[I], gil[I], gj[J][ii], gjl[J][ii])) *
                                            acc[ii]
                                      : 0.f;
                }
            }
        }
#pragma unroll
        for (int q = 0; q < 10; ++q) {
            const int I = q < 1 ? 0 : q < 3 ? 1 : q < 6 ? 2 : 3;
            const int J = q - I * (I + 1) / 2;
            if (I != J) {
                if (has_off(R)) *(F4*)(fr + (frL(I, J) * 64 + lane) * 4) = O::pack4(gr[q]);
            } else {
                if (has_diag(R)) *(f32x4*)(sLD + I * L::LD_BS + c * L::LD_P + 4 * g) = gr[q];
            }
        }
    };
    // ---- prep, third part (role 0 or 2): inverses of the diagonal blocks of (I + L) ->
    //      (T_II - I) fragments
    auto prep3 = [&](int p) {
        E* fr = FR(p);
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");  // sLD written by other lanes
        // lane (bb, r): row r of T_bb = (I + L_bb)^-1, from T (I + L) = I read backwards:
        // T[r][j] = [r == j] - sum_{k > j} T[r][k] L[k][j].  Each solved entry updates all
        // earlier columns (independent FMAs) with row k of the block.
        const int bb = lane >> 4, r = lane & 15;
        const float* lb = sLD + bb * L::LD_BS;
        // rows 15..PRE are read up front, the others when the solve gets there (registers)
        constexpr int PRE = L::OV ? 8 : 16;
        f32x4 lr[16][4];
#pragma unroll
        for (int k = PRE; k < 16; ++k)
#pragma unroll
            for (int k4 = 0; k4 < (k + 3) / 4; ++k4) lr[k][k4] = *(const f32x4*)(lb + k * L::LD_P + 4 * k4);
        float acc[16], tr[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) acc[k] = 0.f;
#pragma unroll
        for (int k = 15; k >= 0; --k) {
            tr[k] = (k == r) ? 1.f : (k < r ? -acc[k] : 0.f);
#pragma unroll
            for (int k4 = 0; k4 < (k + 3) / 4; ++k4) {
                const f32x4 x = k >= PRE ? lr[k][k4] : *(const f32x4*)(lb + k * L::LD_P + 4 * k4);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (4 * k4 + e < k) acc[4 * k4 + e] += tr[k] * x[e];
            }
        }
        // (T_II - I) as K16 A operand: fragment lane (r, g) holds row r, columns 4g..4g+3.
        // -T_II = -(T_II - I) - I is formed by its users (exact, T's diagonal being 1).
        E* tm = fr + (frTm(bb) * 64) * 4;
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) {
            f32x4 x;
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = (4 * gg + e == r) ? 0.f : tr[4 * gg + e];
            O::st4(tm + (r + 16 * gg) * 4, x);
        }
    };

    // ---- chain waves: state slices XA, XB (declared in the chain waves' branch below),
    //      kept transposed as accumulator tiles: XA[t] lane (c,g) = A[16w + c][16t + 4g + i]
    // block forward substitution, correction form: with A_I = sum_{J<I} L_IJ X_J and
    // Z_I = R_I - A_I (both fp32),  X_I = T_II Z_I = Z_I + (T_II - I) Z_I,  where only the
    // correction's operand Z_I is rounded to bf16.  R = diag(b e^G n) K  or  diag(b) V.
    // W goes to LDS pre-scaled by -kts and U stays in registers scaled by kts, so that the
    // state update's innovation is U~ + W~ X^T straight off the matrix cores.
    // column tile cw of W (to LDS, transposed) and/or of U (to Ur, this wave's own)
    // PART: 0 both, 1 U only, 2 W only
    auto subst_part = [&](int q, f32x4 (&Ur)[4], int cw, auto PART) {
        constexpr int P = decltype(PART)::value;
        constexpr bool DW = P != 1, DU = P != 2;
        const float* sc = SC(q);
        const E* fr = FR(q);
        const E* kb = KB_(q);
        const E* vb = VB_(q);
        f32x4 XW[4];
        F4 pw[4], pu[4];
#pragma unroll
        for (int I = 0; I < 4; ++I) {
            // lane (c, g): tokens 16I + 4g + i, column 16cw + c
            f32x4 zw, zu;
            if constexpr (DW) {
                const f32x4 kcol = __builtin_convertvector(O::ldtr(kb, L::KPB, 16 * I, 16 * cw, lane), f32x4);
                zw = *(const f32x4*)(sc + 16 * I + 4 * g) * kcol;
            }
            if constexpr (DU) {
                const f32x4 vcol = __builtin_convertvector(O::ldtr(vb, L::KPB, 16 * I, 16 * cw, lane), f32x4);
                zu = *(const f32x4*)(sc + 64 + 16 * I + 4 * g) * vcol;
            }
            if (I > 0) {
                f32x4 aw = zero4(), au = zero4();
#pragma unroll
                for (int J = 0; J < I; ++J) {
                    const F4 lf = *(const F4*)(fr + (frL(I, J) * 64 + lane) * 4);
                    if constexpr (DW) aw = O::mma16(lf, pw[J], aw);
                    if constexpr (DU) au = O::mma16(lf, pu[J], au);
                }
                if constexpr (DW) zw -= aw;
                if constexpr (DU) zu -= au;
            }
            const F4 tmf = *(const F4*)(fr + (frTm(I) * 64 + lane) * 4);
            if constexpr (DW) {
                XW[I] = O::mma16(tmf, O::pack4(zw), zw);
                pw[I] = O::pack4(XW[I]);
            }
            if constexpr (DU) {
                Ur[I] = O::mma16(tmf, O::pack4(zu), zu);
                pu[I] = O::pack4(Ur[I]);
            }
        }
        // W^T row 16cw + c, tokens 16I + 4g .. +3: one 8-byte piece per lane and block
        E* const wt = (E*)((char*)WB_(q) + (16 * cw + c) * L::WPB) + 4 * g;
#pragma unroll
        for (int I = 0; I < 4; ++I) {
            f32x4 wv;
            if constexpr (TOK) {  // unscaled: the readout needs v' = U - W S0^T itself
                wv = -XW[I];
            } else {
                const f32x4 s = *(const f32x4*)(sc + 128 + 16 * I + 4 * g);
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) {
                    if constexpr (DW) wv[ii] = -s[ii] * XW[I][ii];
                    if constexpr (DU) Ur[I][ii] *= s[ii];
                }
            }
            if constexpr (DW) O::st4(wt + 16 * I, wv);
        }
    };
    // the chain waves' substitution: both tiles of column w, or only U's where helper
    // waves form W
    auto subst = [&](int q, f32x4 (&Ur)[4]) {
        if constexpr (L::NH > 0) subst_part(q, Ur, w, std::integral_constant<int, 1>{});
        else subst_part(q, Ur, w, std::integral_constant<int, 0>{});
    };
    // helper wave h: W column tiles h, h + NH, ...
    auto subst_helper = [&](int q) {
        f32x4 unused[4];
        for (int cw = w - ND - L::NPW; cw < ND; cw += (L::NH > 0 ? L::NH : ND))
            subst_part(q, unused, cw, std::integral_constant<int, 2>{});
    };

    // Operand fragment of the row-major chunk tile `buf` (K or Q, pitch KPB): lane (c, g)
    // gets row r0 + c, columns 32kb + 4g + j and 32kb + 16 + 4g + j (j < 4); columns past
    // d_k are zero (the PAIR slot map of the K32 products).
    auto rowfrag = [&](const E* buf, int r0, int kb) {
        const E* r = (const E*)((const char*)buf + (r0 + c) * L::KPB) + 32 * kb + 4 * g;
        F8 f;
        if (2 * kb + 1 < ND) {
            f = O::ld44(r, r + 16);
        } else {
            f = O::ld44(r, r);
#pragma unroll
            for (int j = 4; j < 8; ++j) f[j] = (E)0.f;
        }
        return f;
    };

    // ---- TOK, beside the substitution: the ten lower-triangle tiles (tile T
    //      of query tokens, tile J of key tokens, J <= T) of the intra-chunk weights
    //          Aqk[t][i] = e^{G_t - G_i} n_i (q_t . k_i)   (i <= t, else 0),
    //      computed as (K Q^T) so that lane (c, g) holds Aqk[16T + c][16J + 4g + i]: the B
    //      operand of the readout's K16 product over key tokens.  Decay factors as in L:
    //      one exp2 of a difference inside a block, split at the key block's end across
    //      blocks (both factors <= 1).  Each chain wave takes one tile, the prep wave the
    //      rest.
    // Tiles x in [x0, 10) with x = x0 (mod xs) go to the calling wave.
    auto aqk = [&](int q, int x0, int xs) {
        const float* sc = SC(q);
        E* const aq = (E*)(smem + L::OFF_AQ);
        for (int x = x0; x < 10; x += xs) {
            const int T = x < 1 ? 0 : x < 3 ? 1 : x < 6 ? 2 : 3;
            const int J = x - T * (T + 1) / 2;
            f32x4 a4 = zero4();
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) a4 = O::mma32(rowfrag(KB_(q), 16 * J, kb), rowfrag(QB_(q), 16 * T, kb), a4);
            const float gt = sc[208 + 16 * T + c];
            const f32x4 gi4 = *(const f32x4*)(sc + 208 + 16 * J + 4 * g);
            const f32x4 ni4 = *(const f32x4*)(sc + 272 + 16 * J + 4 * g);
            // fp32 inputs: G = hi + lo (differences stay accurate after near-zero gates)
            const float gtl = L::BF ? 0.f : sc[400 + 16 * T + c];
            const f32x4 gi4l = L::BF ? zero4() : *(const f32x4*)(sc + 400 + 16 * J + 4 * g);
            auto gdif = [](float xh, float xl, float yh, float yl) { return L::BF ? xh - yh : (xh - yh) + (xl - yl); };
            if (T == J) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    a4[i] = (4 * g + i <= c) ? a4[i] * ni4[i] * hw_exp2(gdif(gt, gtl, gi4[i], gi4l[i])) : 0.f;
            } else {
                const float ge = sc[208 + 16 * J + 15], gel = L::BF ? 0.f : sc[400 + 16 * J + 15];
                const float rowf = hw_exp2(gdif(gt, gtl, ge, gel));
#pragma unroll
                for (int i = 0; i < 4; ++i) a4[i] *= rowf * ni4[i] * hw_exp2(gdif(ge, gel, gi4[i], gi4l[i]));
            }
            F4 hi, lo;
            O::split4(a4, hi, lo);
            *(F4*)(aq + ((x * NS) * 64 + lane) * 4) = hi;
            if constexpr (NS > 1) *(F4*)(aq + ((x * NS + 1) * 64 + lane) * 4) = lo;
        }
    };

    // ---- TOK, chain waves: chunk q from its true start state S0 (slice XB), B part only.
    //      v' = U - W S0^T (fp32), the state update with D' = diag(e^{G_C - G} n) v', and the
    //      outputs of the chunk's tokens for this wave's 16 state rows, as O^T tiles:
    //          O^T[r][t] = e^{G_t} (S0 q_t)[r] + sum_{i <= t} v'[i][r] Aqk[t][i]
    //      (lane (c, g) of tile T: token 16T + c, rows 16w + 4g .. +3 -- 4 consecutive
    //      outputs).  S0, v' and Aqk go to the matrix cores as hi + lo pairs.
    auto chain_tok = [&](int q, f32x4 (&XB)[ND], const f32x4 (&Ur)[4]) {
        const float* sc = SC(q);
        const E* kbuf = KB_(q);
        const float gam = sc[192];
        F8 xh[KB], xl[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
            O::split8(XB[2 * kb], (2 * kb + 1 < ND) ? XB[(2 * kb + 1) % ND] : zero4(), xh[kb], xl[kb]);
        F4 vh[4], vl[4];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            f32x4 PB[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int tt = 2 * h + u;
                PB[u] = Ur[tt];
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) {
                    const auto w0 = O::ldtr(WB_(q), L::WPB, 32 * kb, 16 * tt, lane);
                    F8 wf;
                    if (2 * kb + 1 < ND) {
                        wf = __builtin_shufflevector(w0, O::ldtr(WB_(q), L::WPB, 32 * kb + 16, 16 * tt, lane), 0, 1,
                                                     2, 3, 4, 5, 6, 7);
                    } else {
                        wf = __builtin_shufflevector(w0, w0, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
                        for (int j = 4; j < 8; ++j) wf[j] = (E)0.f;
                    }
                    PB[u] = O::mma32(wf, xh[kb], PB[u]);
                }
                O::split4(PB[u], vh[tt], vl[tt]);  // v' tile tt (rows 16w.., tokens 16tt..)
                const f32x4 s = *(const f32x4*)(sc + 128 + 16 * tt + 4 * g);
                PB[u] *= s;
            }
            F8 dBh, dBl;
            O::split8(PB[0], PB[1], dBh, dBl);
#pragma unroll
            for (int m = 0; m < ND; ++m) {
                const F8 kf = __builtin_shufflevector(O::ldtr(kbuf, L::KPB, 32 * h, 16 * m, lane),
                                                      O::ldtr(kbuf, L::KPB, 32 * h + 16, 16 * m, lane), 0, 1, 2, 3,
                                                      4, 5, 6, 7);
                f32x4 xb2 = h == 0 ? XB[m] * gam : XB[m];
                xb2 = O::mma32(kf, dBh, xb2);
                if (O::kSplit) xb2 = O::mma32(kf, dBl, xb2);
                XB[m] = xb2;
            }
        }
        // outputs
        const E* const aq = (const E*)(smem + L::OFF_AQ);
        const int Cc = chunk_len(q);
        const long long trow = tok0 + chunk_t0(q);
#pragma unroll
        for (int T = 0; T < 4; ++T) {
            f32x4 o = zero4();
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                const F8 qf = rowfrag(QB_(q), 16 * T, kb);
                o = O::mma32(xh[kb], qf, o);
                if (O::kSplit) o = O::mma32(xl[kb], qf, o);
            }
            o *= sc[336 + 16 * T + c];
#pragma unroll
            for (int J = 0; J <= T; ++J) {
                const int x = T * (T + 1) / 2 + J;
                const F4 ah = *(const F4*)(aq + ((x * NS) * 64 + lane) * 4);
                o = O::mma16(vh[J], ah, o);
                if constexpr (NS > 1) {
                    const F4 al = *(const F4*)(aq + ((x * NS + 1) * 64 + lane) * 4);
                    o = O::mma16(vl[J], ah, o);
                    o = O::mma16(vh[J], al, o);
                }
            }
            if (16 * T + c < Cc) {
                const long long off = (trow + 16 * T + c) * D + 16 * w + 4 * g;
                if (a.out_f32) *(f32x4*)((float*)a.out + off) = o;
                else O::st4((E*)a.out + off, o);
            }
        }
    };

    // apply the chunk to both slices:  X <- g_C X + K^T D',  D' = U~ + W~ X^T (chunk-start X)
    auto chain = [&](int q, f32x4 (&XA)[ND], f32x4 (&XB)[ND], const f32x4 (&Ur)[4]) {
        const float* sc = SC(q);
        const E* kb = KB_(q);
        const float gam = sc[192];
        F8 xa[KB], xb[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            const f32x4 hiA = (2 * kb + 1 < ND) ? XA[(2 * kb + 1) % ND] : zero4();
            const f32x4 hiB = (2 * kb + 1 < ND) ? XB[(2 * kb + 1) % ND] : zero4();
            if constexpr (!TS) xa[kb] = O::pack8(XA[2 * kb], hiA);
            xb[kb] = O::pack8(XB[2 * kb], hiB);
        }
        // token halves h = 0, 1: innovation D' for the half's two token tiles, then
        // X += K^T D' (xa / xb keep the chunk-start state)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            f32x4 PA[2], PB[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int tt = 2 * h + u;
                PA[u] = zero4();
                PB[u] = Ur[tt];
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) {
                    // lane (c, g): W[16tt + c][32kb + 4g + j] and [32kb + 16 + 4g + j], j < 4
                    const auto w0 = O::ldtr(WB_(q), L::WPB, 32 * kb, 16 * tt, lane);
                    F8 wf;
                    if (2 * kb + 1 < ND) {
                        wf = __builtin_shufflevector(w0, O::ldtr(WB_(q), L::WPB, 32 * kb + 16, 16 * tt, lane), 0, 1,
                                                     2, 3, 4, 5, 6, 7);
                    } else {  // d_k columns 32kb+16.. do not exist: zero half
                        wf = __builtin_shufflevector(w0, w0, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
                        for (int j = 4; j < 8; ++j) wf[j] = (E)0.f;
                    }
                    if constexpr (!TS) PA[u] = O::mma32(wf, xa[kb], PA[u]);
                    PB[u] = O::mma32(wf, xb[kb], PB[u]);
                }
            }
            // the B part carries the state and gets a hi + lo innovation; the A part,
            // which only maps a carried state, a single bf16 one
            F8 dA;
            if constexpr (!TS) dA = O::pack8(PA[0], PA[1]);
            F8 dBh, dBl;
            O::split8(PB[0], PB[1], dBh, dBl);
#pragma unroll
            for (int m = 0; m < ND; ++m) {
                // K^T operand, PAIR slot map over the half's 32 tokens
                const F8 kf = __builtin_shufflevector(O::ldtr(kb, L::KPB, 32 * h, 16 * m, lane),
                                                      O::ldtr(kb, L::KPB, 32 * h + 16, 16 * m, lane), 0, 1, 2, 3,
                                                      4, 5, 6, 7);
                f32x4 xb2 = h == 0 ? XB[m] * gam : XB[m];
                if constexpr (!TS) {
                    f32x4 xa2 = h == 0 ? XA[m] * gam : XA[m];
                    XA[m] = O::mma32(kf, dA, xa2);
                }
                xb2 = O::mma32(kf, dBh, xb2);
                if (O::kSplit) xb2 = O::mma32(kf, dBl, xb2);
                XB[m] = xb2;
            }
        }
    };

    // frame end: the partial map of the group so far, in two copies -- every frame's, for
    // the readout, and the group's last one, for the chain over groups.  The readout's
    // copy is fp32 for fp32 inputs; for bf16 inputs it is fp16, this wave's rows (of A and
    // of B) scaled by a power of two that puts their largest magnitude in [2^14, 2^15),
    // the exponent stored beside.  The chain's copy is fp32 for B and the operand dtype
    // for A (bf16 as hi and lo).  B goes out as accumulator tiles, A as the A operand of
    // the map application (PAIR slot map over A's rows); that needs A's tiles
    // transposed, which one K16 product with the identity does exactly (an operand times
    // 1, accumulated in fp32): it turns lane (c, g) into the owner of A[16w + 4g + i][16t
    // + c], i.e. of 4 consecutive slots of its own fragment lane, written as one piece.
    auto slice_exp = [&](const f32x4 (&X)[ND]) {  // exponent e: max |X 2^-e| in [2^14, 2^15)
        float m = 0.f;
#pragma unroll
        for (int t = 0; t < ND; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) m = fmaxf(m, fabsf(X[t][i]));
        m = wave_max(m);
        return m > 0.f ? __builtin_amdgcn_frexp_expf(m) - 15 : 0;
    };
    auto emit = [&](int fl, const f32x4 (&XA)[ND], const f32x4 (&XB)[ND]) {
        const long long unit = (long long)bh * a.nf + fw0 + fl;
        const long long grp = (long long)bh * ((a.nf + a.G - 1) / a.G) + gi;
        const bool last = fl == nfg - 1 && !TS;  // the group's map, for the chain
        const int bso = w * ND * 256;            // this wave's B tiles (elements)
        if (a.emit_all) {
            if constexpr (L::BF) {
                const int e = slice_exp(XB);
                const auto r = buf_rsrc((_Float16*)a.Bfr + unit * (ND * ND * 256));
#pragma unroll
                for (int t = 0; t < ND; ++t) {
                    f32x4 x;
#pragma unroll
                    for (int i = 0; i < 4; ++i) x[i] = __builtin_amdgcn_ldexpf(XB[t][i], -e);
                    buf_st(to_f16x4(x), r, lane * 8, (bso + t * 256) * 2);
                }
                if (lane == 0) a.Xexp[unit * 16 + 8 + w] = e;
            } else {
                const auto r = buf_rsrc((float*)a.Bfr + unit * (ND * ND * 256));
#pragma unroll
                for (int t = 0; t < ND; ++t) buf_st(XB[t], r, lane * 16, (bso + t * 256) * 4);
            }
        }
        if (last) {
            const auto r = buf_rsrc(a.Bgr + grp * (ND * ND * 256));
#pragma unroll
            for (int t = 0; t < ND; ++t) buf_st(XB[t], r, lane * 16, (bso + t * 256) * 4);
        }
        if constexpr (TS) return;  // B is the true state: no A map
        f32x4 eye;
#pragma unroll
        for (int i = 0; i < 4; ++i) eye[i] = (4 * g + i == c) ? 1.f : 0.f;
        const int kbw = w >> 1, half = w & 1;
        // this lane's piece of fragment (t, kbw): element offset (t KB + kbw) 512 + fo
        const int fo = lane * 8 + 4 * half;
        const bool pad = (ND & 1) && w == ND - 1;  // also zero the slots of rows past d_k
        auto put = [&](E* ap, int part) {          // part 1: the lo set of a bf16 split
            const F4 eyef = O::pack4(eye);
            const auto r = buf_rsrc(ap);
#pragma unroll
            for (int t = 0; t < ND; ++t) {
                f32x4 x = XA[t];
                if (part) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) x[i] = O::lo_of(x[i]);
                }
                const f32x4 xt = O::mma16(O::pack4(x), eyef, zero4());
                const int so = (t * KB + kbw) * 512 * (int)sizeof(E);
                buf_st(O::pack4(xt), r, fo * (int)sizeof(E), so);
                if (pad) buf_st(O::pack4(zero4()), r, (fo + 4) * (int)sizeof(E), so);
            }
        };
        if (a.emit_all) {
            if constexpr (L::BF) {
                const int e = slice_exp(XA);
                const f16x4 eyeh = to_f16x4(eye);
                const auto r = buf_rsrc((_Float16*)a.Afr + unit * L::APK_E);
#pragma unroll
                for (int t = 0; t < ND; ++t) {
                    f32x4 x;
#pragma unroll
                    for (int i = 0; i < 4; ++i) x[i] = __builtin_amdgcn_ldexpf(XA[t][i], -e);
                    const f32x4 xt = __builtin_amdgcn_mfma_f32_16x16x16f16(to_f16x4(x), eyeh, zero4(), 0, 0, 0);
                    const int so = (t * KB + kbw) * 512 * 2;
                    buf_st(to_f16x4(xt), r, fo * 2, so);
                    if (pad) buf_st(to_f16x4(zero4()), r, (fo + 4) * 2, so);
                }
                if (lane == 0) a.Xexp[unit * 16 + w] = e;
            } else {
                put((E*)a.Afr + unit * L::APK_E, 0);
            }
        }
        if (last) {
#pragma unroll
            for (int part = 0; part < NS; ++part) put((E*)a.Agr + (grp * NS + part) * L::APK_E, part);
        }
    };

    // rotary frequencies to LDS, read there by rotate_granule
    if constexpr (ROPE) {
        if (tid < 2 * kRopePairs)
            ((float*)(smem + L::OFF_RP))[tid] = tid < kRopePairs ? a.rope.ghi[tid] : a.rope.glo[tid - kRopePairs];
        lds_barrier();
    }

    // The prep wave and the chain waves run separate loops with the same barriers, so
    // that neither keeps the other's registers live.
    //
    // Overlapped schedule (OV), one barrier per chunk.  Iteration q:
    //      chain waves: state update of q, then substitution of q+1
    //      prep waves:  (role 1) issue the copies of chunk q+3; Gram, norms, gates, L
    //                   and diagonal inverses of q+2; wait for the copies of chunk q+3
    //   B
    //
    // Two-phase schedule (where the OV buffers do not fit), iteration q (copies of chunk
    // q+PD are issued at its start):
    //      | chain waves: substitution of q   | prep: Gram and norms of q+1
    //   B2 | chain waves: state update of q   | prep: gates, L, inverses of q+1
    //      (wait for the copies of chunk q+2)
    //   B3
    if (prep) {
        f32x4 gr[10];  // Gram tiles of the chunk being prepared
        if constexpr (TOK && L::PIPE) {
            // K and gates run two chunks ahead, V and Q one
            constexpr RoleC<2> R{};
            dma_tiles(0, 0, 1, true, kAll);
            dma_tiles(0, 1, 2, false, kAll);
            if (nq > 1) dma_tiles(1, 0, 1, true, kAll);
            wait_vmem();
            rotate_tiles(0, 0, 1, kAll);
            rotate_tiles(0, 1, 2, kAll);
            if (nq > 1) rotate_tiles(1, 0, 1, kAll);
            lds_barrier();  // chunk 0 and chunk 1's K in LDS
            prep1(0, gr, R);
            prep2(0, gr, R);
            prep3(0);
            lds_barrier();  // chunk 0 prepared
            for (int q = 0; q < nq; ++q) {
                if (q + 2 < nq) dma_tiles(q + 2, 0, 1, true, kCopyT);
                if (q + 1 < nq) {
                    dma_tiles(q + 1, 1, 2, false, kCopyT);
                    prep1(q + 1, gr, R);
                }
                if constexpr (L::NH == 0) aqk(q, ND, 1);  // the tiles past the chain waves' one each
                lds_barrier();  // B2: W and the intra-chunk weights of chunk q staged
                if (q + 1 < nq) {
                    prep2(q + 1, gr, R);
                    prep3(q + 1);
                }
                wait_vmem();
                if (q + 2 < nq) rotate_tiles(q + 2, 0, 1, kCopyT);
                if (q + 1 < nq) rotate_tiles(q + 1, 1, 2, kCopyT);
                lds_barrier();  // B3: chunk q+1 prepared and in LDS, chunk q+2's K in LDS
            }
        } else if constexpr (TOK) {
            constexpr RoleC<2> R{};
            for (int q = 0; q < nq; ++q) {
                dma_tiles(q, 0, 3, true, kAll);
                wait_vmem();
                rotate_tiles(q, 0, 3, kAll);
                lds_barrier();
                prep1(q, gr, R);
                lds_barrier();
                prep2(q, gr, R);
                prep3(q);
                lds_barrier();
                aqk(q, ND, 1);
                lds_barrier();
                lds_barrier();
            }
        } else if constexpr (L::OV) {
            auto run = [&](auto R) {
                auto prep_all = [&](int p) {
                    prep1(p, gr, R);
                    prep2(p, gr, R);
                    if (has_diag(R)) prep3(p);
                };
                dma_chunk(0, kAll);
                if (nq > 1) dma_chunk(1, kAll);
                wait_vmem();
                rotate_own(0, kAll);
                if (nq > 1) rotate_own(1, kAll);
                if (nq > 2) dma_chunk(2, kAll);
                lds_barrier();  // chunks 0 and 1 in LDS
                prep_all(0);
                lds_barrier();  // chunk 0 prepared
                if (nq > 1) prep_all(1);
                wait_vmem();
                if (nq > 2) rotate_own(2, kAll);
                lds_barrier();  // chunk 1 prepared, chunk 0 substituted, chunk 2 in LDS
                for (int q = 0; q < nq; ++q) {
                    // one wave issues every copy: global -> LDS copies from several waves of
                    // a workgroup at once were measured to move far less data per second
                    if (q + 3 < nq) dma_chunk(q + 3, kCopy);
                    if (q + 2 < nq) prep_all(q + 2);
                    wait_vmem();
                    if (q + 3 < nq) rotate_own(q + 3, kCopy);
                    lds_barrier();  // chunk q+2 prepared, q+1 substituted, q+3 in LDS
                }
            };
            if (w == ND) run(RoleC<0>{});
            else run(RoleC<1>{});
        } else if constexpr (L::PIPE) {
            constexpr RoleC<2> R{};
            dma_chunk(0, kAll);
            if (nq > 1) dma_chunk(1, kAll);
            wait_vmem();
            rotate_own(0, kAll);
            if (nq > 1) rotate_own(1, kAll);
            for (int c2 = 2; c2 < L::PD && c2 < nq; ++c2) dma_chunk(c2, kAll);
            lds_barrier();  // chunks 0 and 1 in LDS
            prep1(0, gr, R);
            prep2(0, gr, R);
            prep3(0);
            lds_barrier();  // chunk 0 prepared
            for (int q = 0; q < nq; ++q) {
                const bool more = q + 1 < nq;
                if (q + L::PD < nq) dma_chunk(q + L::PD, kAll);
                if (more) prep1(q + 1, gr, R);
                lds_barrier();  // B2: W of chunk q staged by the chain waves
                if (more) {
                    prep2(q + 1, gr, R);
                    prep3(q + 1);
                }
                wait_dma_behind(q);
                if (q + 2 < nq) rotate_own(q + 2, kAll);
                lds_barrier();  // B3: chunk q+1 prepared, chunk q+2 in LDS, chunk q's buffers free
            }
        } else {
            constexpr RoleC<2> R{};
            for (int q = 0; q < nq; ++q) {
                dma_chunk(q, kAll);
                wait_vmem();
                rotate_own(q, kAll);
                lds_barrier();
                prep1(q, gr, R);
                lds_barrier();
                prep2(q, gr, R);
                prep3(q);
                lds_barrier();
                lds_barrier();
                lds_barrier();
            }
        }
    } else if (helper) {
        // helper waves, with the chain waves' barriers.  Per-token pass: the W column tiles
        // of chunk q and intra-chunk weight tile ND + h beside the chain waves'
        // substitution; OV: the W column tiles of chunk q+1 beside the state update of q.
        if constexpr (TOK && L::NH > 0) {
            dma_tiles(0, 0, 1, true, kAll);
            dma_tiles(0, 1, 2, false, kAll);
            if (nq > 1) dma_tiles(1, 0, 1, true, kAll);
            wait_vmem();
            rotate_tiles(0, 0, 1, kAll);
            rotate_tiles(0, 1, 2, kAll);
            if (nq > 1) rotate_tiles(1, 0, 1, kAll);
            lds_barrier();
            lds_barrier();
            for (int q = 0; q < nq; ++q) {
                subst_helper(q);
                aqk(q, w - L::NPW, 10);  // tile ND + h
                lds_barrier();  // B2
                lds_barrier();  // B3
            }
        } else if constexpr (L::NH > 0) {
            dma_chunk(0, kAll);
            if (nq > 1) dma_chunk(1, kAll);
            wait_vmem();
            rotate_own(0, kAll);
            if (nq > 1) rotate_own(1, kAll);
            if (nq > 2) dma_chunk(2, kAll);
            lds_barrier();
            lds_barrier();
            subst_helper(0);
            wait_vmem();
            if (nq > 2) rotate_own(2, kAll);
            lds_barrier();
            for (int q = 0; q < nq; ++q) {
                if (q + 1 < nq) subst_helper(q + 1);
                lds_barrier();
            }
        }
    } else {
        f32x4 XA[ND], XB[ND];
#pragma unroll
        for (int t = 0; t < ND; ++t) {
#pragma unroll
            for (int i = 0; i < 4; ++i) XA[t][i] = (16 * w + c == 16 * t + 4 * g + i) ? 1.f : 0.f;
            XB[t] = zero4();
        }
        f32x4 Ur[4];  // U column tile w of the chunk to be applied next, pre-scaled by kts
        if constexpr (TOK || TS) {
            // the true state at the group start: S_before rows 16w.. (zero when NULL)
            const int ngw = (a.nf + a.G - 1) / a.G;
            const float* sg = a.Sgrp ? a.Sgrp + ((long long)bh * ngw + gi) * D * D + (long long)(16 * w + c) * D
                                     : nullptr;
#pragma unroll
            for (int t = 0; t < ND; ++t) XB[t] = sg ? *(const f32x4*)(sg + 16 * t + 4 * g) : zero4();
        }
        if constexpr (TOK) {
            if constexpr (L::PIPE) {
                dma_tiles(0, 0, 1, true, kAll);
                dma_tiles(0, 1, 2, false, kAll);
                if (nq > 1) dma_tiles(1, 0, 1, true, kAll);
                wait_vmem();
                rotate_tiles(0, 0, 1, kAll);
                rotate_tiles(0, 1, 2, kAll);
                if (nq > 1) rotate_tiles(1, 0, 1, kAll);
                lds_barrier();
                lds_barrier();
                for (int q = 0; q < nq; ++q) {
                    if (q + 2 < nq) dma_tiles(q + 2, 0, 1, true, kCopyT);
                    if (q + 1 < nq) dma_tiles(q + 1, 1, 2, false, kCopyT);
                    subst(q, Ur);
                    aqk(q, w, 10);
                    lds_barrier();  // B2
                    chain_tok(q, XB, Ur);
                    wait_vmem();
                    if (q + 2 < nq) rotate_tiles(q + 2, 0, 1, kCopyT);
                    if (q + 1 < nq) rotate_tiles(q + 1, 1, 2, kCopyT);
                    lds_barrier();  // B3
                }
            } else {
                for (int q = 0; q < nq; ++q) {
                    dma_tiles(q, 0, 3, true, kAll);
                    wait_vmem();
                    rotate_tiles(q, 0, 3, kAll);
                    lds_barrier();
                    lds_barrier();
                    lds_barrier();
                    subst(q, Ur);
                    aqk(q, w, 10);
                    lds_barrier();
                    chain_tok(q, XB, Ur);
                    lds_barrier();
                }
            }
        } else if constexpr (L::OV) {
            dma_chunk(0, kAll);
            if (nq > 1) dma_chunk(1, kAll);
            wait_vmem();
            rotate_own(0, kAll);
            if (nq > 1) rotate_own(1, kAll);
            if (nq > 2) dma_chunk(2, kAll);
            lds_barrier();
            lds_barrier();
            subst(0, Ur);
            wait_vmem();
            if (nq > 2) rotate_own(2, kAll);
            lds_barrier();
            // (no copies here: the prep waves issue them and wait for them)
            for (int q = 0; q < nq; ++q) {
                if (q + 3 < nq) dma_chunk(q + 3, kCopy);
                chain(q, XA, XB, Ur);
                const int fl = q / nch;
                if (q - fl * nch == nch - 1 && (a.emit_all || fl == nfg - 1)) emit(fl, XA, XB);
                if (q + 1 < nq) subst(q + 1, Ur);
                if ((kCopy >> w) & 1u) wait_vmem();
                if (q + 3 < nq) rotate_own(q + 3, kCopy);
                lds_barrier();
            }
        } else {
            if constexpr (L::PIPE) {
                dma_chunk(0, kAll);
                if (nq > 1) dma_chunk(1, kAll);
                wait_vmem();
                rotate_own(0, kAll);
                if (nq > 1) rotate_own(1, kAll);
                for (int c2 = 2; c2 < L::PD && c2 < nq; ++c2) dma_chunk(c2, kAll);
                lds_barrier();
                lds_barrier();
            }
            for (int q = 0; q < nq; ++q) {
                if constexpr (L::PIPE) {
                    if (q + L::PD < nq) dma_chunk(q + L::PD, kAll);
                    subst(q, Ur);
                    lds_barrier();  // B2
                } else {
                    dma_chunk(q, kAll);
                    wait_vmem();
                    rotate_own(q, kAll);
                    lds_barrier();
                    lds_barrier();
                    lds_barrier();
                    subst(q, Ur);
                    lds_barrier();
                }
                chain(q, XA, XB, Ur);
                const int fl = q / nch;
                if (q - fl * nch == nch - 1 && (a.emit_all || fl == nfg - 1)) emit(fl, XA, XB);
                if constexpr (L::PIPE) {
                    wait_dma_behind(q);
                    if (q + 2 < nq) rotate_own(q + 2, kAll);
                }
                lds_barrier();  // B3
            }
        }
        // the state after the group's last token (one-group calls only)
        if constexpr (TOK || TS) {
            if (a.state_out) {
                float* so = a.state_out + (long long)bh * D * D + (long long)(16 * w + c) * D;
#pragma unroll
                for (int t = 0; t < ND; ++t) *(f32x4*)(so + 16 * t + 4 * g) = XB[t];
            }
        }
    }
}

template <typename E, int ND, int MODE>
__global__ __launch_bounds__((P1<E, ND, false, (MODE & 8) != 0>::NT), 1) void gdn_frame_affine(P1Args a) {
    affine_body<E, ND, MODE, false>(a);
}

// Per-token readout pass: the same chunk pipeline run from each group's true start state
// (the state before the group, from the chain), B part only, writing o_t = S_t q_t for
// every token (TOK branches of the body above).
template <typename E, int ND, int MODE>
__global__ __launch_bounds__((P1<E, ND, true, (MODE & 8) != 0>::NT), 1) void gdn_token_readout(P1Args a) {
    affine_body<E, ND, MODE, true>(a);
}

// -------------------------------------------------------------------------------------
// Phase 2: the serial chain over groups, S_g = S_{g-1} A_g + B_g
// -------------------------------------------------------------------------------------
// Rows of S never mix, so each 16-row slice runs its own chain: one workgroup of ND
// waves per (b, h, slice), wave t computing output column tile t of the slice.  A step
// is short (KB x 3 dependent products per wave), so it is the latency of fetching the
// group maps that bounds the chain: each wave streams only its own column tile of A
// (KB fragments per part) and its tile of B, straight into registers, PD groups ahead
// of the step that uses them.  The slice's state tiles meet in LDS once per step
// (double-buffered, one barrier) so that every wave holds the full rows as B operands.
// Workgroups are numbered so that the ND slices of one (b, h) share an XCD (workgroup i
// goes to XCD i mod 8) and so its L2: the ND-fold reads of a map come from there.
template <typename E, int ND> struct P2 {
    static constexpr int KB = (ND + 1) / 2;
    static constexpr int NS = SplitCount<E>::N;
    static constexpr int APK_E = ND * KB * 64 * 8;  // one part of A (elements)
    static constexpr int PD = 3;                     // groups in flight ahead of the step
    static constexpr int NT = 64 * ND;
    static constexpr int LDS_B = 2 * ND * 64 * 16;   // two sets of the slice's state tiles
    // workgroups for BH (b, h) pairs: 8 XCDs x ceil(BH / 8) pairs x ND slices
    static int grid(int BH) { return 8 * ((BH + 7) / 8) * ND; }
};

template <typename E, int ND>
__global__ __launch_bounds__((P2<E, ND>::NT), 1) void gdn_frame_chain(P2Args a, int BH) {
    using O = Ops<E>;
    using F8 = typename O::F8;
    using P = P2<E, ND>;
    constexpr int D = 16 * ND, KB = P::KB, APK_E = P::APK_E, PD = P::PD;
    extern __shared__ __attribute__((aligned(256))) unsigned char smem[];
    f32x4* const sX = (f32x4*)smem;  // [2][ND tiles][64 lanes]
    const int lane = threadIdx.x & 63, t = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int c = lane & 15, g = lane >> 4;
    // workgroup i: XCD x = i % 8, its k-th workgroup there is slice k % ND of pair
    // x + 8 (k / ND)
    const int wg = blockIdx.x, k = wg >> 3;
    const int bh = (wg & 7) + 8 * (k / ND), s = k % ND;
    if (bh >= BH) return;  // whole workgroup: no barrier is reached
    const int ngw = (a.nf + a.G - 1) / a.G;

    // prefetch ring: slot j holds group gi = j (mod PD)
    F8 ah[PD][KB], al[PD][KB];
    f32x4 bt[PD];
    const E* const abase = (const E*)a.Agr + (long long)bh * ngw * P::NS * APK_E + (t * KB * 64 + lane) * 8;
    const float* const bbase = a.Bgr + (long long)bh * ngw * (ND * ND * 256) + (s * ND + t) * 256 + lane * 4;
#define GDN_CHAIN_LOAD(J, GI)                                                                  \
    {                                                                                          \
        const E* src = abase + (long long)(GI) * P::NS * APK_E;                                \
        _Pragma("unroll") for (int kb = 0; kb < KB; ++kb) {                                    \
            ah[J][kb] = O::ld8(src + kb * 512);                                                \
            if (O::kSplit) al[J][kb] = O::ld8(src + APK_E + kb * 512);                         \
        }                                                                                      \
        bt[J] = *(const f32x4*)(bbase + (long long)(GI) * (ND * ND * 256));                    \
    }
    // this wave's tile of the state: lane (c, g) = S[16 s + c][16 t + 4 g + i]
    const long long srow = (long long)(16 * s + c) * D + 16 * t + 4 * g;
    f32x4 X = a.state_src ? *(const f32x4*)(a.state_src + (long long)bh * D * D + srow) : zero4();
    // The steps of a full run of PD groups issue the same memory operations whatever the
    // data (prefetch indices clamped to the last group), so the wait before each step's
    // products counts only the loads it needs; a run of groups that varies would make it
    // wait for every load in flight.
#pragma unroll
    for (int j = 0; j < PD; ++j) GDN_CHAIN_LOAD(j, j < ngw ? j : ngw - 1)
#define GDN_CHAIN_STEP(J, GI, PREFETCH)                                                        \
    {                                                                                          \
        const int gi_ = (GI);                                                                  \
        /* state before the group, for the readout */                                         \
        *(f32x4*)(a.Sgrp + ((long long)bh * ngw + gi_) * D * D + srow) = X;                    \
        f32x4* const xs = sX + (gi_ & 1) * ND * 64;                                            \
        xs[t * 64 + lane] = X;                                                                 \
        lds_barrier();                                                                         \
        /* X <- B + A^T X over the whole rows of the slice */                                 \
        f32x4 acc = bt[J];                                                                     \
        _Pragma("unroll") for (int kb = 0; kb < KB; ++kb) {                                    \
            F8 xh, xl;                                                                         \
            O::split8(xs[2 * kb * 64 + lane], (2 * kb + 1 < ND) ? xs[(2 * kb + 1) * 64 + lane] \
                                                                : zero4(), xh, xl);            \
            acc = O::mma32(ah[J][kb], xh, acc);                                                \
            if (O::kSplit) {                                                                   \
                acc = O::mma32(al[J][kb], xh, acc);                                            \
                acc = O::mma32(ah[J][kb], xl, acc);                                            \
            }                                                                                  \
        }                                                                                      \
        /* the slot's next loads stay behind its last products: they reuse its registers */ \
        asm volatile("" : "+v"(acc)::"memory");                                               \
        X = acc;                                                                               \
        if (PREFETCH) GDN_CHAIN_LOAD(J, gi_ + PD < ngw ? gi_ + PD : ngw - 1)                   \
    }
    int g0 = 0;
    for (; g0 + PD <= ngw; g0 += PD) {
#pragma unroll
        for (int j = 0; j < PD; ++j) GDN_CHAIN_STEP(j, g0 + j, true)
    }
#pragma unroll
    for (int j = 0; j < PD - 1; ++j)
        if (g0 + j < ngw) GDN_CHAIN_STEP(j, g0 + j, false)
#undef GDN_CHAIN_STEP
#undef GDN_CHAIN_LOAD
    if (a.state_dst) *(f32x4*)(a.state_dst + (long long)bh * D * D + srow) = X;
}

// -------------------------------------------------------------------------------------
// Phase 3: S_f = S_{g-1} A_{g,<=f} + B_{g,<=f}, then O_f = Q_f S_f^T, computed as
// O^T = S_f Q^T so that each lane owns 4 outputs of one token.  One workgroup of 4 waves
// per (b, h, frame); wave w owns the 16-row slices w and w + 4 of S_f: it composes them
// in registers, and the composed accumulator tiles are, as they stand, the A operand
// fragments (PAIR slot map over d_k) of its output columns -- no data movement.  Q is
// then read with the same slot map.
// -------------------------------------------------------------------------------------
// LDS of the readout: two 64-token Q chunks (row pitch d + 8), then (ROPE: q rotated by the
// 3D rotary embedding as it is loaded) the rotary frequencies
template <typename E, int ND, bool ROPE = false> struct P3 {
    // bf16 inputs: one 64-token chunk of O staged after the Q buffers, written out as whole rows
    static constexpr int OFF_O = 2 * 64 * (16 * ND + 8) * (int)sizeof(E);
    static constexpr int OFF_RP = OFF_O + (sizeof(E) == 2 ? 64 * (16 * ND + 8) * 2 : 0);
    static constexpr int LDS_B = OFF_RP + (ROPE ? 2 * kRopePairs * 4 : 0);
};

template <typename E, int ND, bool ROPE>
__global__ __launch_bounds__(256, 2) void gdn_frame_readout(P3Args a) {
    using O = Ops<E>;
    using F8 = typename O::F8;
    constexpr int D = 16 * ND, KB = (ND + 1) / 2;
    constexpr int APK_E = ND * KB * 64 * 8;
    constexpr int NS = SplitCount<E>::N;
    constexpr int NSL = (ND + 3) / 4;  // slices per wave (at most 2)
    const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c = lane & 15, g = lane >> 4;
    const int fw = blockIdx.x / a.parts, part = blockIdx.x - fw * a.parts, bh = blockIdx.y;
    const int N = a.frame_len;
    // this workgroup's chunks of the frame: [c0, c1)
    const int nch_all = (N + 63) / 64, cpp = (nch_all + a.parts - 1) / a.parts;
    const int c0 = part * cpp, c1 = min(nch_all, c0 + cpp);
    if (c0 >= c1) return;
    extern __shared__ __attribute__((aligned(256))) unsigned char smem[];
    const int ngw = (a.nf + a.G - 1) / a.G;
    const int gi = fw / a.G;
    const long long unit = (long long)bh * a.nf + fw;
    bool own[NSL];
#pragma unroll
    for (int u = 0; u < NSL; ++u) own[u] = w + 4 * u < ND;

    // ---- compose: X_u = Sgrp slice (w + 4u) A + B slice, A streamed tile by tile (or,
    //      after a true-start frame-maps pass, X_u = B slice: the B map is the state).
    //      bf16 inputs: the stored maps are fp16 with each row slice scaled by 2^-e (A's
    //      exponents in Xexp[0..8), B's in Xexp[8..16)).
    const int* ex = O::kSplit ? a.Xexp + unit * 16 : nullptr;
    auto ldB = [&](int sl, int t) -> f32x4 {  // tile t of row slice sl of B
        const long long o = unit * (ND * ND * 256) + ((long long)sl * ND + t) * 256 + lane * 4;
        if constexpr (O::kSplit) {
            const f32x4 x = __builtin_convertvector(*(const f16x4*)((const _Float16*)a.Bfr + o), f32x4);
            const int e = ex[8 + sl];
            return f32x4{__builtin_amdgcn_ldexpf(x[0], e), __builtin_amdgcn_ldexpf(x[1], e),
                         __builtin_amdgcn_ldexpf(x[2], e), __builtin_amdgcn_ldexpf(x[3], e)};
        } else {
            return *(const f32x4*)((const float*)a.Bfr + o);
        }
    };
    f32x4 X[NSL][ND];
    if (a.b_is_state) {
#pragma unroll
        for (int u = 0; u < NSL; ++u) {
            const int sl = own[u] ? w + 4 * u : 0;
#pragma unroll
            for (int t = 0; t < ND; ++t) X[u][t] = ldB(sl, t);
        }
    } else {
#pragma unroll
    for (int u = 0; u < NSL; ++u) {
        const int sl = own[u] ? w + 4 * u : 0;
        const float* sg = a.Sgrp + ((long long)bh * ngw + gi) * D * D + (long long)(16 * sl + c) * D;
#pragma unroll
        for (int t = 0; t < ND; ++t) X[u][t] = a.Sgrp ? *(const f32x4*)(sg + 16 * t + 4 * g) : zero4();
    }
    if constexpr (O::kSplit) {
        // bf16 inputs: the stored A is fp16, row slice t (A's rows 16t..) scaled by 2^-e_t,
        // and goes to the fp16 matrix cores as it is.  The columns 16t.. of S (the same
        // k_in) take 2^e_t, and the whole of this wave's rows one more power of two 2^sc
        // that puts their largest magnitude below 2^14 (exponents added, so nothing
        // underflows on the way); S is then an fp16 hi + lo pair (22 significant bits).
        // The product is formed from zero in that scale, scaled back by 2^-sc and added
        // to B (a decayed A can make 2^sc large: B itself is never scaled).
        int emax = -100000;
#pragma unroll
        for (int t = 0; t < ND; ++t) {
            float mt = 0.f;
#pragma unroll
            for (int u = 0; u < NSL; ++u)
#pragma unroll
                for (int i = 0; i < 4; ++i) mt = fmaxf(mt, fabsf(X[u][t][i]));
            if (mt > 0.f) emax = max(emax, __builtin_amdgcn_frexp_expf(mt) + ex[t]);
        }
        // the frame's A map (the same for every wave) staged once in the Q buffers, which
        // the compose runs before: one coalesced copy instead of four waves each reading
        // it from L2
        static_assert(APK_E * 2 <= P3<E, ND, ROPE>::OFF_RP, "the A map fits in the Q buffers");
        _Float16* const sA = (_Float16*)smem;
        {
            const u32x4* src = (const u32x4*)((const _Float16*)a.Afr + unit * APK_E);
            for (int i = tid; i < APK_E / 8; i += 256) ((u32x4*)sA)[i] = src[i];
        }
        emax = (int)wave_max((float)emax);
        const int sc = emax > -100000 ? 14 - emax : 0;
        f16x8 sh16[NSL][KB], sl16[NSL][KB];
#pragma unroll
        for (int u = 0; u < NSL; ++u)
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                f32x4 lo4 = X[u][2 * kb], hi4 = (2 * kb + 1 < ND) ? X[u][(2 * kb + 1) % ND] : zero4();
                const int e0 = ex[2 * kb] + sc, e1 = (2 * kb + 1 < ND) ? ex[(2 * kb + 1) % ND] + sc : 0;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    lo4[i] = __builtin_amdgcn_ldexpf(lo4[i], e0);
                    hi4[i] = __builtin_amdgcn_ldexpf(hi4[i], e1);
                }
                const f16x4 h0 = to_f16x4(lo4), h1 = to_f16x4(hi4);
                const f16x4 l0 = to_f16x4(lo4 - __builtin_convertvector(h0, f32x4));
                const f16x4 l1 = to_f16x4(hi4 - __builtin_convertvector(h1, f32x4));
                sh16[u][kb] = __builtin_shufflevector(h0, h1, 0, 1, 2, 3, 4, 5, 6, 7);
                sl16[u][kb] = __builtin_shufflevector(l0, l1, 0, 1, 2, 3, 4, 5, 6, 7);
            }
        lds_barrier();  // the A map in LDS
#pragma unroll
        for (int t = 0; t < ND; ++t) {
            f16x8 fa[KB];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) fa[kb] = *(const f16x8*)(sA + ((t * KB + kb) * 64 + lane) * 8);
#pragma unroll
            for (int u = 0; u < NSL; ++u) {
                f32x4 acc = zero4();
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) {
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(fa[kb], sh16[u][kb], acc, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(fa[kb], sl16[u][kb], acc, 0, 0, 0);
                }
                const f32x4 bt = ldB(own[u] ? w + 4 * u : 0, t);
#pragma unroll
                for (int i = 0; i < 4; ++i) X[u][t][i] = __builtin_amdgcn_ldexpf(acc[i], -sc) + bt[i];
            }
        }
        lds_barrier();  // every wave has read the A map: the Q buffers are free
    } else {
        // fp32 inputs: maps and states in fp32 on the fp32 matrix cores
        F8 xf[NSL][KB];
#pragma unroll
        for (int u = 0; u < NSL; ++u)
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) xf[u][kb] = O::pack8(X[u][2 * kb], (2 * kb + 1 < ND) ? X[u][(2 * kb + 1) % ND] : zero4());
#pragma unroll
        for (int t = 0; t < ND; ++t) {
            F8 fa[KB];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) fa[kb] = O::ld8((const E*)a.Afr + unit * APK_E + ((t * KB + kb) * 64 + lane) * 8);
#pragma unroll
            for (int u = 0; u < NSL; ++u) {
                f32x4 acc = ldB(own[u] ? w + 4 * u : 0, t);
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) acc = O::mma32(fa[kb], xf[u][kb], acc);
                X[u][t] = acc;
            }
        }
    }
    }
    // S_f slices as readout A fragments (hi, lo): slot (g, j) of k block kb holds
    // S[16 s + c][32 kb + 4g + j] (j < 4), S[16 s + c][32 kb + 16 + 4g + j - 4] (j >= 4)
    F8 sh[NSL][KB], sl_[NSL][KB];
#pragma unroll
    for (int u = 0; u < NSL; ++u)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
            O::split8(X[u][2 * kb], (2 * kb + 1 < ND) ? X[u][(2 * kb + 1) % ND] : zero4(), sh[u][kb], sl_[u][kb]);

    // ---- readout: Q goes through LDS in chunks of 64 tokens (double-buffered, the next
    //      chunk's global loads in flight while this one is computed); every wave reads
    //      every token tile from LDS for its own output columns
    constexpr int QP = D + 8;                              // LDS row pitch (elements)
    constexpr int EPV = Ops<E>::EPV;
    constexpr int CBQ = D / EPV;                           // 16-byte pieces per token row
    constexpr int QV = (64 * CBQ + 255) / 256;             // pieces per thread per chunk
    E* const sQ = (E*)smem;                                // [2][64][QP]
    E* const sO = (E*)(smem + P3<E, ND, ROPE>::OFF_O);     // [64][QP] (bf16 output)
    using V16 = typename Ops<E>::V16;
    const long long tok0 = (long long)bh * a.T + (long long)(a.f0 + fw) * N;
    const E* qp = (const E*)a.q + tok0 * D;
    V16 qr[QV];
    auto qload = [&](int ch) {
#pragma unroll
        for (int k = 0; k < QV; ++k) {
            const int v = tid + 256 * k, row = v / CBQ, cb = v - row * CBQ;
            if (v < 64 * CBQ && 64 * ch + row < N) qr[k] = *(const V16*)(qp + (long long)(64 * ch + row) * D + cb * EPV);
            else {
#pragma unroll
                for (int e = 0; e < EPV; ++e) qr[k][e] = (E)0.f;
            }
        }
    };
    // GDN_F_ROPE_QK: q is rotated by the 3D rotary embedding between its load and its LDS
    // store (rows past the frame's end are zeros and stay zeros)
    const float* const sRP = (const float*)(smem + P3<E, ND, ROPE>::OFF_RP);
    const float rinv_w = ROPE ? 1.f / (float)a.rope.grid_w : 0.f;
    if constexpr (ROPE) {
        if (tid < 2 * kRopePairs)
            ((float*)(smem + P3<E, ND, ROPE>::OFF_RP))[tid] = tid < kRopePairs ? a.rope.ghi[tid] : a.rope.glo[tid - kRopePairs];
        lds_barrier();
    }
    auto qstore = [&](int buf, int ch) {
        const float pf = (float)(a.rope.frame0 + a.f0 + fw);
#pragma unroll
        for (int k = 0; k < QV; ++k) {
            const int v = tid + 256 * k, row = v / CBQ, cb = v - row * CBQ;
            if (v < 64 * CBQ) {
                if constexpr (ROPE) {
                    const int t = 64 * ch + row, hr = rope_div(t, a.rope.grid_w, rinv_w);
                    qr[k] = rope_rotate<E>(qr[k], cb * (EPV / 2), pf, (float)hr, (float)(t - hr * a.rope.grid_w),
                                           a.rope.p1, a.rope.p2, sRP, sRP + kRopePairs);
                }
                *(V16*)(sQ + (buf * 64 + row) * QP + cb * EPV) = qr[k];
            }
        }
    };
    qload(c0);
    qstore(0, c0);
    if (c0 + 1 < c1) qload(c0 + 1);
    lds_barrier();
    for (int ch = c0; ch < c1; ++ch) {
        const E* qb0 = sQ + ((ch - c0) & 1) * 64 * QP;
#pragma unroll
        for (int tl = 0; tl < 4; ++tl) {
            const int t = 64 * ch + 16 * tl + c;
            F8 qb[KB];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                const E* r = qb0 + (16 * tl + c) * QP + 32 * kb + 4 * g;
                if (32 * kb + 16 < D) {
                    qb[kb] = O::ld44(r, r + 16);
                } else {  // d_k columns 32kb + 16.. do not exist
                    qb[kb] = O::ld44(r, r);
#pragma unroll
                    for (int j = 4; j < 8; ++j) qb[kb][j] = (E)0.f;
                }
            }
#pragma unroll
            for (int u = 0; u < NSL; ++u) {
                if (!own[u]) continue;
                f32x4 acc = zero4();
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) {
                    acc = O::mma32(sh[u][kb], qb[kb], acc);
                    if (O::kSplit) acc = O::mma32(sl_[u][kb], qb[kb], acc);
                }
                if (O::kSplit && !a.out_f32) {  // staged: lane (c, g) holds 4 outputs of token 16 tl + c
                    O::st4(sO + (16 * tl + c) * QP + 16 * (w + 4 * u) + 4 * g, acc);
                } else if (t < N) {
                    const long long o = (tok0 + t) * D + 16 * (w + 4 * u) + 4 * g;
                    if (a.out_f32) *(f32x4*)((float*)a.out + o) = acc;
                    else O::st4((E*)a.out + o, acc);
                }
            }
        }
        if (O::kSplit && !a.out_f32) {
            lds_barrier();  // the chunk's O rows complete in LDS
            for (int v = tid; v < 64 * CBQ; v += 256) {
                const int row = v / CBQ, cb = v - row * CBQ;
                if (64 * ch + row < N)
                    *(V16*)((E*)a.out + (tok0 + 64 * ch + row) * D + cb * EPV) = *(const V16*)(sO + row * QP + cb * EPV);
            }
        }
        if (ch + 1 < c1) {
            qstore((ch + 1 - c0) & 1, ch + 1);
            if (ch + 2 < c1) qload(ch + 2);
        }
        lds_barrier();
    }
}

}  // namespace gdn
