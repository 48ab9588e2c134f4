// softmax_attn.hip -- frame-block-causal softmax attention on gfx950: the softmax layers
// that the hybrid mixer interleaves with the frame-wise gated delta rule ("SANA-WM:
// one-minute 720p world model", hn.hoangyell.com, "Hybrid Linear Attention" among its four
// technical decisions; the news summaries of the same topic, section on the hybrid
// architecture for long rollouts).  The pages give neither mask nor window; the reading
// here: a query of global frame f sees, through an exact softmax, every key of frames
// <= f among the kv_frames frames passed (the last n_frames of them are the queries' own
// frames, the earlier ones a cache -- which earlier frames to pass is the window):
//   o_i = sum_j exp(s q_i.k_j) v_j / sum_j exp(s q_i.k_j),   j < (f_i + 1) N,  s = 1/sqrt(d)
//
// One launch.  A workgroup (8 waves for bf16, 4 for float32) takes 32 consecutive queries
// of one (b, h) per wave and streams the keys it needs -- those up to the end of its last
// query's frame -- in blocks of 64 through LDS (global -> LDS copies one block ahead).
// Software-pipelined: a block's scores are formed while the previous block's exponentials
// are taken, in one scheduling region.  Per block and wave, on the matrix cores:
//   S^T = K Q^T   (4 key tiles x 2 query tiles, k = d; K rows read as 16-byte pieces):
//                 the accumulator gives each lane one query column, 16 of its keys, so
//                 the row maximum needs two lane exchanges;
//   O^T += V^T P^T (d tiles x 2 query tiles, k = the 64 keys): the probabilities enter
//                 as the B operand straight from the S^T registers (PAIR slot map), V^T
//                 comes from transposed LDS reads.
// Online softmax in base 2 (logits scaled by s log2 e), in float32, with a reference point
// that moves only when a score exceeds it by more than 2^8 (weights <= 256); P is rounded
// to the operand type (bf16 for bf16 inputs) before the product, and the row sums are
// taken on the matrix cores from the same rounded weights.  Blocks
// past every query of a wave are skipped (the mask's own structure, not the data), and
// only blocks that straddle a query's frame end are masked element by element.
// Workgroups are dispatched heaviest first: the last query tiles of every head, which
// see the most keys, lead the grid.
#include "gdn.h"
#include "common.hpp"
#include <math.h>
#include <stdint.h>

#define SA_API extern "C" __attribute__((visibility("default")))

namespace gdn {
namespace {

struct SAArgs {
    const void* q;
    const void* k;
    const void* v;
    void* out;
    long long Tq, Tk;  // tokens per (b, h): queries / keys
    int frame_len;
    int off;           // kv_frames - n_frames: global frame of the first query frame
    int ntiles;        // query tiles (one workgroup each) per (b, h)
    int BH;
    float sl2e;        // softmax scale * log2(e)
    int out_f32;
};

// LDS layout: K and V blocks of 64 keys, row-major with the row pitch rule of the other
// kernels (bf16 rows span an odd number of 32-byte units: conflict-free transposed
// reads), two buffers of each (the block in use, the next block's copies).  One
// workgroup per CU (launch bound one): bf16's eight waves take the register file at two
// waves per SIMD, float32's blocks most of the LDS.
template <typename E, int ND> struct SAL {
    static constexpr bool BF = sizeof(E) == 2;
    static constexpr int RB = 16 * ND * (int)sizeof(E);
    static constexpr int KPB = !BF ? RB : ((RB + 31) / 32 % 2 == 1) ? (RB + 31) / 32 * 32 : (RB + 31) / 32 * 32 + 32;
    static constexpr int KG = KPB / 16, DG = RB / 16;  // 16-byte granules per row / with data
    static constexpr int BLK_B = 64 * KPB;             // one K or V block
    static constexpr int NI = BLK_B / 1024;            // 1 KB copy instructions per K or V block
    // bf16: 8 waves (256 queries share each key block's copy); float32: 4 waves (register
    // budget).  Two K slots and two V slots: a block's scores are formed one step before
    // its PV product, and the copies of the next K and V land one step ahead
    static constexpr int NWV = BF ? 8 : 4;
    static constexpr int NT = 64 * NWV;
    static constexpr int QT = 32 * NWV;                // queries per workgroup
    // K slots carry 64 zero bytes after their last row: the score operand reads 32 bytes
    // per lane from column 32 kb + 8 g, which runs past d on the last row
    static constexpr int PADB = 64;
    static constexpr int KSLOT = BLK_B + PADB;
    static constexpr int LDS_B = 2 * KSLOT + 2 * BLK_B;  // K slots 0, 1, then V slots 0, 1
    static_assert(BLK_B % 1024 == 0, "blocks are whole 1 KB copies");
    static_assert(LDS_B <= 160 * 1024, "LDS budget");
};

// op over the lanes l, l^16, l^32 and l^48 -- the four row groups g of one accumulator
// column -- with the gfx950 lane swaps (v_permlane32_swap: lanes 32..63 of the first
// register trade places with lanes 0..31 of the second; v_permlane16_swap: the odd rows of
// 16 lanes of the first with the even rows of the second).  Given two copies of x, each
// lane ends up holding its own value and its partner's.  Written as one instruction with
// two in/out registers (wait states before and after): the builtins' two results get
// folded into one by the compiler.
__device__ __forceinline__ float across_g_max(float x) {
    float y = x;
    __asm__ volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(x), "+v"(y));
    x = fmaxf(x, y);
    y = x;
    __asm__ volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(x), "+v"(y));
    return fmaxf(x, y);
}

template <typename E, int ND>
__global__ __launch_bounds__((SAL<E, ND>::NT), 1) void sa_fwd(SAArgs a) {
    using O = Ops<E>;
    using F8 = typename O::F8;
    using L = SAL<E, ND>;
    constexpr int D = 16 * ND, KB = (ND + 1) / 2;
    extern __shared__ __attribute__((aligned(256))) unsigned char smem[];
    const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c = lane & 15, g = lane >> 4;
    const int rank = blockIdx.x / a.BH;
    const int bh = blockIdx.x - rank * a.BH;
    const int tile = a.ntiles - 1 - rank;
    const long long N = a.frame_len;
    const long long q0 = (long long)tile * L::QT;
    const long long qlast = min(q0 + L::QT - 1, a.Tq - 1);
    // keys this workgroup needs: through the end of its last query's frame (<= Tk)
    const long long kend_wg = ((long long)a.off + qlast / N + 1) * N;
    const int nblk = (int)((kend_wg + 63) / 64);
    const E* kp = (const E*)a.k + (long long)bh * a.Tk * D;
    const E* vp = (const E*)a.v + (long long)bh * a.Tk * D;
    const E* qp = (const E*)a.q + (long long)bh * a.Tq * D;

    // Copies of a K or V block: instruction ii = w + NWV u moves 1 KB; lane l's 16 bytes are
    // granule ii * 64 + l of the block (row, piece), the same for every block, so each lane
    // keeps its element offsets; rows past the keys copy the last key (finite values;
    // their weights are masked to zero).  K of block b lands in K slot b % 2, V in V slot
    // b % 2 (LDS: K slots 0, 1 then V slots 0, 1).
    constexpr int NUK = (L::NI + L::NWV - 1) / L::NWV;
    int roff[NUK], prow[NUK];
#pragma unroll
    for (int u = 0; u < NUK; ++u) {
        const int ii = w + L::NWV * u;
        const int gidx = ii * 64 + lane, row = gidx / L::KG, piece = gidx - row * L::KG;
        prow[u] = row;
        roff[u] = row * D + min(piece, L::DG - 1) * (16 / (int)sizeof(E));
    }
    auto copy = [&](const E* src, int b, int boff) {
        unsigned char* dst = smem + boff;
        const bool tail = 64LL * (b + 1) > a.Tk;  // the last block of the keys may be ragged
#pragma unroll
        for (int u = 0; u < NUK; ++u) {
            const int ii = w + L::NWV * u;
            if (ii >= L::NI) break;
            int off = roff[u];
            if (tail) off += (int)(min(64LL * b + prow[u], a.Tk - 1) - 64LL * b - prow[u]) * D;
            dma16(src + 64LL * b * D + off, dst + ii * 1024);
        }
    };
    auto copyK = [&](int b) { copy(kp, b, (b & 1) * L::KSLOT); };
    auto copyV = [&](int b) { copy(vp, b, 2 * L::KSLOT + (b & 1) * L::BLK_B); };

    // this wave's queries: q0 + 32w + 16qt + c (qt = 0, 1); those past Tq compute on the
    // last query's values and are not stored
    const long long qw0 = q0 + 32 * w;
    const bool active = qw0 < a.Tq;
    const long long qwl = min(qw0 + 31, a.Tq - 1);
    const long long kmax_w = ((long long)a.off + qwl / N + 1) * N;                 // keys any query sees
    const long long kmin_w = ((long long)a.off + min(qw0, a.Tq - 1) / N + 1) * N;  // keys every query sees
    long long kend[2];
    F8 qf[2][KB];  // Q^T operands, IDENT slot map over d: lane (c, g) holds d 32kb + 8g ..
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
        const long long qi = min(qw0 + 16 * qt + c, a.Tq - 1);
        kend[qt] = ((long long)a.off + qi / N + 1) * N;
        const E* r = qp + qi * D;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            const int col = 32 * kb + 8 * g;
            qf[qt][kb] = col < D ? O::ld8(r + col) : O::zero8();
        }
    }
    // Software pipeline over key blocks: iteration b forms the scores of block b + 1 on
    // the matrix cores beside block b's exponentials on the vector units, then block b's
    // PV product.  Iteration b reads K of b + 1 and V of b, while K of b + 2 and V of b + 1
    // are copied into the slots that K of b and V of b - 1 have left.  The first copies go
    // out after the Q loads: the wait before block 0 then covers both.
    copyK(0);
    copyV(0);
    if (nblk > 1) copyK(1);
    f32x4 acc[2][ND];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt)
#pragma unroll
        for (int t = 0; t < ND; ++t) acc[qt][t] = zero4();
    float m[2] = {-INFINITY, -INFINITY};
    // row sums on the matrix cores: a ones operand times the same (rounded) probabilities
    // that enter the PV product; every row of lsum[qt] holds query c's sum
    f32x4 lsum[2] = {zero4(), zero4()};
    F8 ones;
#pragma unroll
    for (int j = 0; j < 8; ++j) ones[j] = (E)1.f;
    // S^T tiles of block bb: sc[qt][kt] lane (c, g) = q(16qt + c) . k(64bb + 16kt + 4g + i)
    auto scores = [&](int bb, f32x4 (&sc)[2][4]) {
        const unsigned char* kbuf = smem + (bb & 1) * L::KSLOT;
#pragma unroll
        for (int qt = 0; qt < 2; ++qt)
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) sc[qt][kt] = zero4();
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                // IDENT slot map: key row 16kt + c, d 32kb + 8g .. +7.  Past d the piece
                // holds the next row's (or, after row 63, the next slot's) finite values,
                // which meet zero slots of Q
                const F8 kf = O::ld8((const E*)(kbuf + (16 * kt + c) * L::KPB) + 32 * kb + 8 * g);
#pragma unroll
                for (int qt = 0; qt < 2; ++qt) sc[qt][kt] = O::mma32(kf, qf[qt][kb], sc[qt][kt]);
            }
        }
    };
    constexpr int PADF = L::PADB / 4;  // floats of one K slot's zero tail
    if (tid < 2 * PADF) ((float*)(smem + (tid / PADF) * L::KSLOT + L::BLK_B))[tid % PADF] = 0.f;
    f32x4 s[2][4], sn[2][4];
    wait_vmem_le(0);
    lds_barrier();
    if (active) scores(0, s);  // key 0 is seen by every query
    for (int b = 0; b < nblk; ++b) {
        wait_vmem_le(0);  // this wave's copies of K of b + 1 and V of b done
        lds_barrier();    // every wave's copies visible; iteration b - 1's slots free
        if (b + 2 < nblk) copyK(b + 2);
        if (b + 1 < nblk) copyV(b + 1);
        if (!active || 64LL * b >= kmax_w) continue;  // no query of this wave sees block b
        const E* vbuf = (const E*)(smem + 2 * L::KSLOT + (b & 1) * L::BLK_B);
        if (64LL * (b + 1) > kmin_w) {  // some query of the wave misses some key of the block
#pragma unroll
            for (int qt = 0; qt < 2; ++qt) {
                const int rel = (int)max(-1LL, min(64LL, kend[qt] - 64LL * b));  // keys it sees here
#pragma unroll
                for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (16 * kt + 4 * g + i >= rel) s[qt][kt][i] = -INFINITY;
            }
        }
        // the maxima of the raw scores; the scale (s log2 e > 0) commutes with them
        float mc[2];
        bool move[2];
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
            float mx = -INFINITY;
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[qt][kt][i]);
            mc[qt] = across_g_max(mx) * a.sl2e;
            move[qt] = __builtin_amdgcn_ballot_w64(mc[qt] > m[qt] + 8.f) != 0;
        }
        // The reference point m of the exponentials moves only when some query of the
        // wave sees a score more than 2^8 above it (always in block 0, whose key 0 every
        // query sees, so m is finite from then on): the weights stay <= 256 and the
        // rescaling of the accumulators is skipped for most blocks; the quotient is the
        // same softmax whatever the reference point.
        if (move[0] || move[1]) {
#pragma unroll
            for (int qt = 0; qt < 2; ++qt) {
                if (!move[qt]) continue;
                const float mn = fmaxf(m[qt], mc[qt]);
                const float corr = hw_exp2(m[qt] - mn);
                m[qt] = mn;
                lsum[qt] *= corr;
#pragma unroll
                for (int t = 0; t < ND; ++t) acc[qt][t] *= corr;
            }
        }
        // one scheduling region: block b + 1's scores (formed whether or not the wave
        // uses them: its K slot holds finite keys) beside block b's exponentials
        scores(b + 1 < nblk ? b + 1 : b, sn);
        F8 pf[2][2];
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
            const float mn = m[qt];
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                for (int i = 0; i < 4; ++i) s[qt][kt][i] = hw_exp2(__builtin_fmaf(s[qt][kt][i], a.sl2e, -mn));
            pf[qt][0] = O::pack8(s[qt][0], s[qt][1]);
            pf[qt][1] = O::pack8(s[qt][2], s[qt][3]);
        }
        // O^T[d tile t] += V^T P^T over the block's 64 keys, PAIR slot map over keys
#pragma unroll
        for (int t = 0; t < ND; ++t) {
#pragma unroll
            for (int st = 0; st < 2; ++st) {
                const F8 vf = __builtin_shufflevector(O::ldtr(vbuf, L::KPB, 32 * st, 16 * t, lane),
                                                      O::ldtr(vbuf, L::KPB, 32 * st + 16, 16 * t, lane), 0, 1, 2, 3,
                                                      4, 5, 6, 7);
#pragma unroll
                for (int qt = 0; qt < 2; ++qt) acc[qt][t] = O::mma32(vf, pf[qt][st], acc[qt][t]);
            }
        }
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int qt = 0; qt < 2; ++qt) lsum[qt] = O::mma32(ones, pf[qt][st], lsum[qt]);
#pragma unroll
        for (int qt = 0; qt < 2; ++qt)
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) s[qt][kt] = sn[qt][kt];
    }
    if (!active) return;
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
        const float inv = 1.f / lsum[qt][0];
        const long long qi = qw0 + 16 * qt + c;
        if (qi >= a.Tq) continue;
        const long long o = ((long long)bh * a.Tq + qi) * D + 4 * g;
#pragma unroll
        for (int t = 0; t < ND; ++t) {
            if (a.out_f32) *(f32x4*)((float*)a.out + o + 16 * t) = acc[qt][t] * inv;
            else O::st4((E*)a.out + o + 16 * t, acc[qt][t] * inv);
        }
    }
}

template <typename E, int ND>
hipError_t launch_sa(const SAArgs& a, hipStream_t st, void* const* ev) {
    static PerDeviceOnce attr;  // per instantiation
    hipError_t e = attr.run([] {
        return hipFuncSetAttribute((const void*)sa_fwd<E, ND>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                   SAL<E, ND>::LDS_B);
    });
    if (e != hipSuccess) return e;
    if (ev && (e = hipEventRecord((hipEvent_t)ev[0], st)) != hipSuccess) return e;
    constexpr int lds = SAL<E, ND>::LDS_B;
    SAArgs r = a;
    r.ntiles = (int)((a.Tq + SAL<E, ND>::QT - 1) / SAL<E, ND>::QT);
    const long long nwg = (long long)r.ntiles * a.BH;
    constexpr int nt = SAL<E, ND>::NT;
    hipLaunchKernelGGL((sa_fwd<E, ND>), dim3((unsigned)nwg), dim3(nt), lds, st, r);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    return ev ? hipEventRecord((hipEvent_t)ev[1], st) : hipSuccess;
}

int nd_of_d(int d) {
    switch (d) {
        case 16: return 1;
        case 32: return 2;
        case 64: return 4;
        case 112: return 7;
        case 128: return 8;
        default: return 0;
    }
}

bool misaligned16(const void* p) { return p && ((uintptr_t)p & 15u) != 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + nb && b0 < a0 + na;
}

}  // namespace
}  // namespace gdn

using namespace gdn;

SA_API int softmax_attn_block_causal(const void* q, const void* k, const void* v, void* out, int32_t kv_frames,
                                     const gdn_dims_t* d, void* stream) {
    if (!d) return GDN_ERR_NULL;
    if (d->dtype != GDN_BF16 && d->dtype != GDN_F32) return GDN_ERR_DTYPE;
    if (d->B < 0 || d->H < 0 || d->n_frames < 0 || d->frame_len < 1 || kv_frames < d->n_frames)
        return GDN_ERR_DIMS;
    const int nd = nd_of_d(d->d_k);
    if (d->d_k != d->d_v || nd == 0) return GDN_ERR_UNSUPPORTED;
    if (d->flags & ~(uint32_t)GDN_F_OUT_F32) return GDN_ERR_UNSUPPORTED;
    const long long BH = (long long)d->B * d->H;
    const long long Tq = (long long)d->n_frames * d->frame_len, Tk = (long long)kv_frames * d->frame_len;
    if (BH == 0 || Tq == 0) return GDN_OK;
    // element counts of k and v must fit comfortably in 63 bits; the grid in 31
    if (Tk > ((long long)1 << 40) / BH / d->d_k) return GDN_ERR_DIMS;
    if ((Tq + 127) / 128 * BH >= ((long long)1 << 31)) return GDN_ERR_DIMS;  // grid (>= 128 queries a workgroup)
    if (!q || !k || !v || !out) return GDN_ERR_NULL;
    if (misaligned16(q) || misaligned16(k) || misaligned16(v) || misaligned16(out)) return GDN_ERR_ALIGN;
    const int es = d->dtype == GDN_BF16 ? 2 : 4;
    const size_t qbytes = (size_t)(BH * Tq * d->d_k) * es, kbytes = (size_t)(BH * Tk * d->d_k) * es;
    const size_t obytes = (size_t)(BH * Tq * d->d_v) * ((d->flags & GDN_F_OUT_F32) ? 4 : es);
    if (overlaps(out, obytes, q, qbytes) || overlaps(out, obytes, k, kbytes) || overlaps(out, obytes, v, kbytes))
        return GDN_ERR_ALIAS;
    SAArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.out = out;
    a.Tq = Tq;
    a.Tk = Tk;
    a.frame_len = d->frame_len;
    a.off = kv_frames - d->n_frames;
    a.ntiles = 0;  // set per instantiation (queries per workgroup)
    a.BH = (int)BH;
    a.sl2e = (float)(1.4426950408889634 / sqrt((double)d->d_k));
    a.out_f32 = (d->flags & GDN_F_OUT_F32) != 0;
    void* const* ev = (d->phase_events && d->phase_windows >= 1) ? d->phase_events : nullptr;
    hipStream_t st = (hipStream_t)stream;
    hipError_t e = hipErrorInvalidValue;
    if (d->dtype == GDN_BF16) {
        switch (nd) {
            case 1: e = launch_sa<bf16, 1>(a, st, ev); break;
            case 2: e = launch_sa<bf16, 2>(a, st, ev); break;
            case 4: e = launch_sa<bf16, 4>(a, st, ev); break;
            case 7: e = launch_sa<bf16, 7>(a, st, ev); break;
            case 8: e = launch_sa<bf16, 8>(a, st, ev); break;
        }
    } else {
        switch (nd) {
            case 1: e = launch_sa<float, 1>(a, st, ev); break;
            case 2: e = launch_sa<float, 2>(a, st, ev); break;
            case 4: e = launch_sa<float, 4>(a, st, ev); break;
            case 7: e = launch_sa<float, 7>(a, st, ev); break;
            case 8: e = launch_sa<float, 8>(a, st, ev); break;
        }
    }
    return e == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}
