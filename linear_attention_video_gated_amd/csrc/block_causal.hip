// block_causal.hip -- block-causal linear attention with a ReLU feature map on gfx950.
//
// SANA-Video talk (ICLR 2026 oral transcript), block-KV-cache segment: the state is a
// fixed D x D matrix, updated additively block by block, and block i reads the state
// that includes its own contribution (bidirectional inside a frame, causal across frames).
//   S_f = S_in + sum_{g<=f} phi(K_g)^T V_g,   z_f = z_in + sum_{g<=f} sum_t phi(k_t)
//   o_t = phi(q_t)^T S_f / (phi(q_t) . z_f + eps)
// Three launches per window of frames:
//   bc_partial  -- one workgroup per (b, h, frame): phi(K_f)^T [V_f | 1] on bf16 matrix
//                  cores (the extra ones-column yields the key sums that form z); K and
//                  V copied global -> LDS in 32-token sub-chunks, four in flight, operands
//                  taken with transposed LDS reads.
//   bc_scan     -- one wave per (b, h, 16x16 tile): running sum over frames in fp32,
//                  written as readout operand fragments.
//   bc_readout  -- one workgroup per (b, h, frame) or part of one: Q chunks copied
//                  global -> LDS one chunk ahead; each wave owns output column slices and
//                  reads every token tile; the denominator is one more product with z (an
//                  extra row of the operand), then the division.
#include "common.hpp"
#include "gdn_kernels.hpp"

namespace gdn {

// Row layout of K, V (bc_partial) and Q (bc_readout) tiles in LDS: bf16 rows span an odd
// number of 32-byte units (conflict-free transposed reads); the global -> LDS copies fill
// padding granules with a copy of a data granule.
template <typename E, int ND> struct BCP {
    static constexpr bool BF = sizeof(E) == 2;
    static constexpr int RB = 16 * ND * (int)sizeof(E);  // bytes of one K, V or Q row
    static constexpr int KPB = !BF ? RB : ((RB + 31) / 32 % 2 == 1) ? (RB + 31) / 32 * 32 : (RB + 31) / 32 * 32 + 32;
    static constexpr int KG = KPB / 16, DG = RB / 16;    // granules per LDS row / with data
    static constexpr int TILE_B = 64 * KPB;              // 64 rows (a bc_readout Q chunk)
    // bc_partial: K and V in 32-token sub-chunks, NB buffers, NB - 1 sub-chunks in flight
    static constexpr int SUB_B = 32 * KPB;               // one K or V sub-chunk
    static constexpr int NB = BF ? 5 : 4;
    static constexpr int NI = 2 * SUB_B / 1024;          // 1 KB copy instructions per sub-chunk
    static constexpr int LDS_B = NB * 2 * SUB_B;
};

template <typename E, int ND>
__global__ __launch_bounds__(256, 2) void bc_partial(BC1Args a) {
    using O = Ops<E>;
    using F8 = typename O::F8;
    using L = BCP<E, ND>;
    constexpr int D = 16 * ND;
    constexpr int MW = (ND + 3) / 4;  // row slices (features of K) per wave: w, w + 4
    extern __shared__ __attribute__((aligned(256))) unsigned char smem[];
    const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c = lane & 15, g = lane >> 4;
    const int fw = blockIdx.x, bh = blockIdx.y;
    const int N = a.frame_len, nsub = (N + 31) / 32;
    const long long tok0 = (long long)bh * a.T + (long long)(a.f0 + fw) * N;
    const E* kp = (const E*)a.k + tok0 * D;
    const E* vp = (const E*)a.v + tok0 * D;
    auto buf = [&](int sc, int which) { return smem + ((sc % L::NB) * 2 + which) * L::SUB_B; };
    // copies of sub-chunk sc: instruction i moves 1 KB row block i / 2 of K (i even) or V;
    // rows past the frame copy its last row (finite values, masked out of the sums)
    auto copy = [&](int sc) {
        const int r0 = 32 * sc, Cc = min(32, N - r0);
        for (int i = w; i < L::NI; i += 4) {
            const int which = i & 1, ii = i >> 1;
            const int gidx = ii * 64 + lane, row = gidx / L::KG, piece = gidx - row * L::KG;
            const E* src = (which ? vp : kp) + (long long)(r0 + min(row, Cc - 1)) * D +
                           min(piece, L::DG - 1) * (16 / (int)sizeof(E));
            dma16(src, buf(sc, which) + ii * 1024);
        }
    };
    const int ncp = (L::NI - w + 3) / 4;  // this wave's copy instructions per sub-chunk
    // acc[u][n]: rows 16(w + 4u) + 4g + i (features of phi(K)), columns 16n + c of [V | 1]
    f32x4 acc[MW][ND + 1];
#pragma unroll
    for (int u = 0; u < MW; ++u)
#pragma unroll
        for (int n = 0; n <= ND; ++n) acc[u][n] = zero4();
    for (int sc = 0; sc < L::NB - 1 && sc < nsub; ++sc) copy(sc);
    for (int sc = 0; sc < nsub; ++sc) {
        // this wave's copies of sub-chunk sc done; those of the next ones may be in flight
        wait_vmem_le(ncp * min(L::NB - 2, nsub - 1 - sc));
        lds_barrier();  // every wave's copies visible; sub-chunk sc-1's buffer free
        if (sc + L::NB - 1 < nsub) copy(sc + L::NB - 1);
        const E* kb = (const E*)buf(sc, 0);
        const E* vb = (const E*)buf(sc, 1);
        const int Cc = min(32, N - 32 * sc);
        // K32 operands over the sub-chunk's 32 tokens, PAIR slot map: slot (g, j) is token
        // 4g + j (j < 4) or 16 + 4g + j - 4
        F8 kf[MW];
#pragma unroll
        for (int u = 0; u < MW; ++u) {
            const int m = min(w + 4 * u, ND - 1);
            kf[u] = __builtin_shufflevector(O::ldtr(kb, L::KPB, 0, 16 * m, lane), O::ldtr(kb, L::KPB, 16, 16 * m, lane),
                                            0, 1, 2, 3, 4, 5, 6, 7);
            if (a.relu) kf[u] = O::relu8(kf[u]);
            if (Cc < 32) {  // tokens past the frame's end
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    if ((j < 4 ? 4 * g + j : 16 + 4 * g + j - 4) >= Cc) kf[u][j] = (E)0.f;
            }
        }
#pragma unroll
        for (int n = 0; n < ND; ++n) {
            const F8 vf = __builtin_shufflevector(O::ldtr(vb, L::KPB, 0, 16 * n, lane),
                                                  O::ldtr(vb, L::KPB, 16, 16 * n, lane), 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
            for (int u = 0; u < MW; ++u) acc[u][n] = O::mma32(kf[u], vf, acc[u][n]);
        }
        F8 of;  // the ones column (column 0 of block ND): key sums
#pragma unroll
        for (int j = 0; j < 8; ++j) of[j] = (E)(c == 0 ? 1.f : 0.f);
#pragma unroll
        for (int u = 0; u < MW; ++u) acc[u][ND] = O::mma32(kf[u], of, acc[u][ND]);
    }
    const long long unit = (long long)bh * a.nf + fw;
    float* pp = a.part + unit * (ND * (ND + 1) * 256);
#pragma unroll
    for (int u = 0; u < MW; ++u) {
        const int m = w + 4 * u;
        if (m >= ND) continue;
#pragma unroll
        for (int n = 0; n <= ND; ++n) *(f32x4*)(pp + (m * (ND + 1) + n) * 256 + lane * 4) = acc[u][n];
    }
}

template <typename E, int ND>
__global__ __launch_bounds__(64) void bc_scan(BC2Args a) {
    using O = Ops<E>;
    constexpr int D = 16 * ND, KB = (ND + 1) / 2, NTL = ND * (ND + 1);
    constexpr int PK_E = (ND + 1) * KB * 64 * 8;
    constexpr int NS = SplitCount<E>::N;
    const int lane = threadIdx.x, c = lane & 15, g = lane >> 4;
    const int q = blockIdx.x, bh = blockIdx.y;
    const int m = q / (ND + 1), n = q % (ND + 1);
    f32x4 acc = zero4();
    if (a.carry_in) {
        acc = *(const f32x4*)(a.carry_in + ((long long)bh * NTL + q) * 256 + lane * 4);
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int kr = 16 * m + 4 * g + i;
            if (n < ND) acc[i] = a.s_in ? a.s_in[(long long)bh * D * D + (long long)kr * D + 16 * n + c] : 0.f;
            else acc[i] = (a.z_in && c == 0) ? a.z_in[(long long)bh * D + kr] : 0.f;
        }
    }
    // frames in batches of eight: the batch's sums are all loaded before any is used, so
    // one load latency is paid per batch rather than per frame
    constexpr int BT = 8;
    for (int f0 = 0; f0 < a.nf; f0 += BT) {
        f32x4 pb[BT];
#pragma unroll
        for (int i = 0; i < BT; ++i)
            pb[i] = f0 + i < a.nf ? *(const f32x4*)(a.part + (((long long)bh * a.nf + f0 + i) * NTL + q) * 256 + lane * 4)
                                  : zero4();
#pragma unroll
        for (int i = 0; i < BT; ++i) {
            const int fw = f0 + i;
            if (fw >= a.nf) break;
            const long long unit = (long long)bh * a.nf + fw;
            acc += pb[i];
#pragma unroll
            for (int part = 0; part < NS; ++part) {
                E* pk = (E*)a.pack + (unit * NS + part) * PK_E;
                f32x4 v = acc;
                if (part) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) v[j] = O::lo_of(v[j]);
                }
                const int lp = c + 16 * (2 * (m & 1) + (g >> 1));
                O::st4(pk + ((n * KB + (m >> 1)) * 64 + lp) * 8 + 4 * (g & 1), v);
                if ((ND & 1) && m == ND - 1) {
                    const int lp2 = c + 16 * (2 + (g >> 1));
                    O::st4(pk + ((n * KB + KB - 1) * 64 + lp2) * 8 + 4 * (g & 1), zero4());
                }
            }
        }
    }
    if (a.carry_out) *(f32x4*)(a.carry_out + ((long long)bh * NTL + q) * 256 + lane * 4) = acc;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int kr = 16 * m + 4 * g + i;
        if (n < ND) {
            if (a.s_out) a.s_out[(long long)bh * D * D + (long long)kr * D + 16 * n + c] = acc[i];
        } else if (a.z_out && c == 0) {
            a.z_out[(long long)bh * D + kr] = acc[i];
        }
    }
}

template <typename E, int ND>
__global__ __launch_bounds__(256) void bc_readout(BC3Args a) {
    using O = Ops<E>;
    using F8 = typename O::F8;
    using L = BCP<E, ND>;  // Q chunks use bc_partial's row layout
    constexpr int D = 16 * ND, KB = (ND + 1) / 2;
    constexpr int PK_E = (ND + 1) * KB * 64 * 8;
    constexpr int NS = SplitCount<E>::N;
    constexpr int NSL = (ND + 3) / 4;  // output column slices per wave (w, w + 4)
    extern __shared__ __attribute__((aligned(256))) unsigned char smem[];
    const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c = lane & 15, g = lane >> 4;
    const int fw = blockIdx.x / a.parts, part = blockIdx.x - fw * a.parts, bh = blockIdx.y;
    const int N = a.frame_len;
    // this workgroup's 64-token chunks of the frame: [c0, c1)
    const int nch = (N + 63) / 64, cpp = (nch + a.parts - 1) / a.parts;
    const int c0 = part * cpp, c1 = min(nch, c0 + cpp);
    if (c0 >= c1) return;
    const long long unit = (long long)bh * a.nf + fw;
    const E* pk = (const E*)a.pack + unit * NS * PK_E;
    // operand fragments of the z row (n = ND) and of this wave's column slices of S_f
    auto frag = [&](int n, int kb, int sp) { return O::ld8(pk + sp * PK_E + ((n * KB + kb) * 64 + lane) * 8); };
    F8 zf[KB], zl[KB], sf[NSL][KB], sl[NSL][KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
        zf[kb] = frag(ND, kb, 0);
        zl[kb] = O::kSplit ? frag(ND, kb, 1) : O::zero8();
#pragma unroll
        for (int u = 0; u < NSL; ++u) {
            const int n = min(w + 4 * u, ND - 1);
            sf[u][kb] = frag(n, kb, 0);
            sl[u][kb] = O::kSplit ? frag(n, kb, 1) : O::zero8();
        }
    }
    const long long tok0 = (long long)bh * a.T + (long long)(a.f0 + fw) * N;
    const E* qp = (const E*)a.q + tok0 * D;
    // Q chunks copied global -> LDS one chunk ahead (double-buffered); every wave reads
    // every token tile of a chunk for its own output columns
    auto copy = [&](int ch) {
        const int r0 = 64 * ch, Cc = min(64, N - r0);
        unsigned char* dst = smem + ((ch - c0) & 1) * L::TILE_B;
        for (int i = w; i < L::KG; i += 4) {
            const int gidx = i * 64 + lane, row = gidx / L::KG, piece = gidx - row * L::KG;
            dma16(qp + (long long)(r0 + min(row, Cc - 1)) * D + min(piece, L::DG - 1) * (16 / (int)sizeof(E)),
                  dst + i * 1024);
        }
    };
    const int nown = (w < ND) + (NSL > 1 && w + 4 < ND);  // output slices of this wave
    int nst = 0;  // output stores issued after the copies of the next chunk
    copy(c0);
    for (int ch = c0; ch < c1; ++ch) {
        wait_vmem_le(nst);  // this wave's copies of chunk ch (the previous chunk's stores may still be in flight)
        lds_barrier();      // every wave's copies visible; the previous chunk's buffer free
        if (ch + 1 < c1) copy(ch + 1);
        const unsigned char* qb0 = smem + ((ch - c0) & 1) * L::TILE_B;
        const int ntl = (min(64, N - 64 * ch) + 15) / 16;
        nst = ntl * nown;
        for (int tl = 0; tl < ntl; ++tl) {
            const int t = 64 * ch + 16 * tl + c;
            F8 qb[KB];  // IDENT slot map: token 16 tl + c, features 32 kb + 8 g + j
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                const int col = 32 * kb + 8 * g;
                qb[kb] = col < D ? O::ld8((const E*)(qb0 + (16 * tl + c) * L::KPB) + col) : O::zero8();
                if (a.relu) qb[kb] = O::relu8(qb[kb]);
            }
            f32x4 den = zero4();
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                den = O::mma32(zf[kb], qb[kb], den);
                if (O::kSplit) den = O::mma32(zl[kb], qb[kb], den);
            }
            const float dn = __shfl(den[0], c, 64) + a.eps;  // row 0 of the z tile, token c
            const float inv = __builtin_amdgcn_rcpf(dn);  // hardware reciprocal, about 1 ulp
#pragma unroll
            for (int u = 0; u < NSL; ++u) {
                if (w + 4 * u >= ND) continue;
                f32x4 acc = zero4();
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) {
                    acc = O::mma32(sf[u][kb], qb[kb], acc);
                    if (O::kSplit) acc = O::mma32(sl[u][kb], qb[kb], acc);
                }
                if (t < N) {
                    const long long o = (tok0 + t) * D + 16 * (w + 4 * u) + 4 * g;
                    if (a.out_f32) *(f32x4*)((float*)a.out + o) = acc * inv;
                    else O::st4((E*)a.out + o, acc * inv);
                }
            }
        }
    }
}

template <typename E, int ND>
hipError_t launch_bc_window(const BC1Args& a1, const BC2Args& a2, const BC3Args& a3, int BH, hipStream_t st,
                            void* const* ev) {
    hipError_t e = record(ev, 0, st);
    if (e != hipSuccess) return e;
    static PerDeviceOnce attr;  // per instantiation
    e = attr.run([] {
        hipError_t r = hipFuncSetAttribute((const void*)bc_partial<E, ND>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                           BCP<E, ND>::LDS_B);
        if (r != hipSuccess) return r;
        return hipFuncSetAttribute((const void*)bc_readout<E, ND>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                   2 * BCP<E, ND>::TILE_B);
    });
    if (e != hipSuccess) return e;
    constexpr int lds1 = BCP<E, ND>::LDS_B;
    hipLaunchKernelGGL((bc_partial<E, ND>), dim3(a1.nf, BH), dim3(256), lds1, st, a1);
    if ((e = hipGetLastError()) != hipSuccess || (e = record(ev, 1, st)) != hipSuccess ||
        (e = record(ev, 2, st)) != hipSuccess)
        return e;
    hipLaunchKernelGGL((bc_scan<E, ND>), dim3(ND * (ND + 1), BH), dim3(64), 0, st, a2);
    if ((e = hipGetLastError()) != hipSuccess || (e = record(ev, 3, st)) != hipSuccess ||
        (e = record(ev, 4, st)) != hipSuccess)
        return e;
    // few frames: split each frame's chunks over several workgroups (each loads the frame's
    // S_f fragments itself; measured at 420 frames of 390 tokens, one per frame was best)
    BC3Args r = a3;
    const long long frames = (long long)a3.nf * BH;
    long long parts = 768 / (frames > 0 ? frames : 1);
    const int nch = (a3.frame_len + 63) / 64;
    r.parts = (int)(parts < 1 ? 1 : parts > nch ? nch : parts);
    constexpr int lds3 = 2 * BCP<E, ND>::TILE_B;
    hipLaunchKernelGGL((bc_readout<E, ND>), dim3(a3.nf * r.parts, BH), dim3(256), lds3, st, r);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    return record(ev, 5, st);
}

#define BC_INST(E, ND)                                                                                     \
    template hipError_t launch_bc_window<E, ND>(const BC1Args&, const BC2Args&, const BC3Args&, int, hipStream_t, \
                                                void* const*);
BC_INST(bf16, 1) BC_INST(bf16, 2) BC_INST(bf16, 4) BC_INST(bf16, 7) BC_INST(bf16, 8)
BC_INST(float, 1) BC_INST(float, 2) BC_INST(float, 4) BC_INST(float, 7) BC_INST(float, 8)


}  // namespace gdn
