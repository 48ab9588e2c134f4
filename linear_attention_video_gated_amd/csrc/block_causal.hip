// block_causal.hip -- block-causal linear attention with a ReLU feature map on gfx950.
//
// SANA-Video talk (ICLR 2026 oral transcript), block-KV-cache segment: the state is a
// fixed D x D matrix, updated additively block by block, and block i reads the state
// that includes its own contribution (bidirectional inside a frame, causal across frames).
//   S_f = S_in + sum_{g<=f} phi(K_g)^T V_g,   z_f = z_in + sum_{g<=f} sum_t phi(k_t)
//   o_t = phi(q_t)^T S_f / (phi(q_t) . z_f + eps)
// Three launches per window of frames:
//   bc_partial  -- one workgroup per (b, h, frame): phi(K_f)^T [V_f | 1] on bf16 matrix
//                  cores (the extra ones-column yields the key sums that form z).
//   bc_scan     -- one wave per (b, h, 16x16 tile): running sum over frames in fp32,
//                  written as readout operand fragments.
//   bc_readout  -- one workgroup per (b, h, frame): numerator and denominator in one
//                  contraction (z is an extra row of the operand), then the division.
#include "common.hpp"
#include "gdn_kernels.hpp"

namespace gdn {

template <typename E, int ND>
__global__ __launch_bounds__(256) void bc_partial(BC1Args a) {
    using O = Ops<E>;
    using F8 = typename O::F8;
    using V16 = typename O::V16;
    constexpr int D = 16 * ND, EPV = O::EPV;
    constexpr int P = 64 + EPV;          // transposed pitch (tokens)
    constexpr int NTL = ND * (ND + 1);
    constexpr int NQ = (NTL + 3) / 4;
    __shared__ __attribute__((aligned(16))) E sKt[D * P];
    __shared__ __attribute__((aligned(16))) E sVt[D * P];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int c = lane & 15, g = lane >> 4;
    const int fw = blockIdx.x, bh = blockIdx.y;
    const int N = a.frame_len;
    const long long tok0 = (long long)bh * a.T + (long long)(a.f0 + fw) * N;
    const E* kp = (const E*)a.k + tok0 * D;
    const E* vp = (const E*)a.v + tok0 * D;

    f32x4 acc[NQ];
#pragma unroll
    for (int qi = 0; qi < NQ; ++qi) acc[qi] = zero4();

    for (int c0 = 0; c0 < N; c0 += 64) {
        const int Cc = min(64, N - c0);
        lds_barrier();
        constexpr int UPR = D / EPV;
        for (int u = tid; u < 64 * UPR; u += 256) {
            const int row = u / UPR, col = (u % UPR) * EPV;
            V16 kv, vv;
            if (row < Cc) {
                kv = *(const V16*)(kp + (long long)(c0 + row) * D + col);
                vv = *(const V16*)(vp + (long long)(c0 + row) * D + col);
            } else {
#pragma unroll
                for (int j = 0; j < EPV; ++j) kv[j] = vv[j] = (E)0.f;
            }
#pragma unroll
            for (int j = 0; j < EPV; ++j) {
                E kx = kv[j];
                if (a.relu && !((float)kx > 0.f)) kx = (E)0.f;
                sKt[(col + j) * P + row] = kx;
                sVt[(col + j) * P + row] = vv[j];
            }
        }
        lds_barrier();
#pragma unroll
        for (int qi = 0; qi < NQ; ++qi) {
            const int q = w + 4 * qi;
            if (q < NTL) {
                const int m = q / (ND + 1), n = q % (ND + 1);
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const F8 fa = O::ld8(sKt + (16 * m + c) * P + 32 * kb + 8 * g);
                    F8 fb;
                    if (n < ND) {
                        fb = O::ld8(sVt + (16 * n + c) * P + 32 * kb + 8 * g);
                    } else {
#pragma unroll
                        for (int j = 0; j < 8; ++j) fb[j] = (c == 0 && 32 * kb + 8 * g + j < Cc) ? (E)1.f : (E)0.f;
                    }
                    acc[qi] = O::mma32(fa, fb, acc[qi]);
                }
            }
        }
    }
    const long long unit = (long long)bh * a.nf + fw;
    float* pp = a.part + unit * (NTL * 256);
#pragma unroll
    for (int qi = 0; qi < NQ; ++qi) {
        const int q = w + 4 * qi;
        if (q < NTL) *(f32x4*)(pp + q * 256 + lane * 4) = acc[qi];
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
    for (int fw = 0; fw < a.nf; ++fw) {
        const long long unit = (long long)bh * a.nf + fw;
        acc += *(const f32x4*)(a.part + (unit * NTL + q) * 256 + lane * 4);
#pragma unroll
        for (int part = 0; part < NS; ++part) {
            E* pk = (E*)a.pack + (unit * NS + part) * PK_E;
            f32x4 v = acc;
            if (part) {
#pragma unroll
                for (int i = 0; i < 4; ++i) v[i] = O::lo_of(v[i]);
            }
            const int lp = c + 16 * (2 * (m & 1) + (g >> 1));
            O::st4(pk + ((n * KB + (m >> 1)) * 64 + lp) * 8 + 4 * (g & 1), v);
            if ((ND & 1) && m == ND - 1) {
                const int lp2 = c + 16 * (2 + (g >> 1));
                O::st4(pk + ((n * KB + KB - 1) * 64 + lp2) * 8 + 4 * (g & 1), zero4());
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
    constexpr int D = 16 * ND, KB = (ND + 1) / 2;
    constexpr int PK_E = (ND + 1) * KB * 64 * 8;
    constexpr int NS = SplitCount<E>::N;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int c = lane & 15, g = lane >> 4;
    const int fw = blockIdx.x, bh = blockIdx.y;
    const int N = a.frame_len;
    const long long unit = (long long)bh * a.nf + fw;
    const E* pk = (const E*)a.pack + unit * NS * PK_E;
    F8 sf[ND + 1][KB], sl[ND + 1][KB];
#pragma unroll
    for (int n = 0; n <= ND; ++n)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            sf[n][kb] = O::ld8(pk + ((n * KB + kb) * 64 + lane) * 8);
            sl[n][kb] = O::kSplit ? O::ld8(pk + PK_E + ((n * KB + kb) * 64 + lane) * 8) : O::zero8();
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
            if (a.relu) {
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    if (!((float)qb[kb][j] > 0.f)) qb[kb][j] = 0.f;
            }
        }
        f32x4 den = zero4();
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            den = O::mma32(sf[ND][kb], qb[kb], den);
            if (O::kSplit) den = O::mma32(sl[ND][kb], qb[kb], den);
        }
        const float dn = __shfl(den[0], c, 64) + a.eps;  // row 0 of the z tile, token c
        const float inv = 1.f / dn;
#pragma unroll
        for (int n = 0; n < ND; ++n) {
            f32x4 acc = zero4();
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                acc = O::mma32(sf[n][kb], qb[kb], acc);
                if (O::kSplit) acc = O::mma32(sl[n][kb], qb[kb], acc);
            }
            if (valid) {
                const long long o = (tok0 + t) * D + 16 * n + 4 * g;
                if (a.out_f32) *(f32x4*)((float*)a.out + o) = acc * inv;
                else O::st4((E*)a.out + o, acc * inv);
            }
        }
    }
}

template <typename E, int ND>
hipError_t launch_bc_window(const BC1Args& a1, const BC2Args& a2, const BC3Args& a3, int BH, hipStream_t st,
                            void* const* ev) {
    hipError_t e = record(ev, 0, st);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bc_partial<E, ND>), dim3(a1.nf, BH), dim3(256), 0, st, a1);
    if ((e = hipGetLastError()) != hipSuccess || (e = record(ev, 1, st)) != hipSuccess ||
        (e = record(ev, 2, st)) != hipSuccess)
        return e;
    hipLaunchKernelGGL((bc_scan<E, ND>), dim3(ND * (ND + 1), BH), dim3(64), 0, st, a2);
    if ((e = hipGetLastError()) != hipSuccess || (e = record(ev, 3, st)) != hipSuccess ||
        (e = record(ev, 4, st)) != hipSuccess)
        return e;
    hipLaunchKernelGGL((bc_readout<E, ND>), dim3(a3.nf, BH), dim3(256), 0, st, a3);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    return record(ev, 5, st);
}

#define BC_INST(E, ND)                                                                                     \
    template hipError_t launch_bc_window<E, ND>(const BC1Args&, const BC2Args&, const BC3Args&, int, hipStream_t, \
                                                void* const*);
BC_INST(bf16, 1) BC_INST(bf16, 2) BC_INST(bf16, 4) BC_INST(bf16, 7) BC_INST(bf16, 8)
BC_INST(float, 1) BC_INST(float, 2) BC_INST(float, 4) BC_INST(float, 7) BC_INST(float, 8)

size_t bc_unit_bytes(int nd, int esize, size_t* part, size_t* pack) {
    const int kb = (nd + 1) / 2;
    const int nsplit = esize == 2 ? 2 : 1;  // bf16 operands are stored as hi + lo
    *part = (size_t)nd * (nd + 1) * 256 * 4;
    *pack = (size_t)nsplit * (nd + 1) * kb * 64 * 8 * esize;
    return *part + *pack;
}

}  // namespace gdn
