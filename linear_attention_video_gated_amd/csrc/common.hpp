// common.hpp -- gfx950 (CDNA4) building blocks shared by the kernels of this library:
// element types, matrix-core (MFMA) wrappers and the register "fragment" layouts.
//
// Fragment layouts (wave64, 16x16 output tiles).  Lane l is split into c = l % 16 and
// g = l / 16.
//   K32 step (v_mfma_f32_16x16x32_bf16, or eight v_mfma_f32_16x16x4_f32):
//     A operand: lane (c, g) holds A[row c][slot (g, j)], j = 0..7
//     B operand: lane (c, g) holds B[slot (g, j)][col c]
//     The hardware pairs A's and B's slot (g, j); which logical k a slot stands for
//     is the loader's choice, as long as A and B agree.  Two slot maps are used:
//       IDENT: slot (g, j) -> k = 8g + j
//       PAIR : slot (g, j) -> k = 4g + j (j < 4), 16 + 4g + (j - 4) (j >= 4)
//   K16 step (v_mfma_f32_16x16x16_bf16, or four v_mfma_f32_16x16x4_f32):
//     lane (c, g) holds 4 values, slot (g, i) -> k = 4g + i.
//   Accumulator D (16x16 fp32): lane (c, g) holds D[4g + i][c], i = 0..3.
// PAIR exists so that two accumulator tiles stacked along rows (rows 0..15 and
// 16..31) become, without any data movement, the B operand of the next contraction
// over those 32 rows; likewise one accumulator tile is a K16 B operand.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

namespace gdn {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short short4_ __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }
__device__ __forceinline__ f16x4 to_f16x4(f32x4 x) { return __builtin_convertvector(x, f16x4); }  // RNE

// Stores through a raw buffer resource: address = base + soffset + voffset with base and
// soffset uniform (SGPRs) and voffset the lane's byte offset, so that a run of stores to
// different places shares one per-lane VGPR instead of a 64-bit address each.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(void* base) {
    return __builtin_amdgcn_make_buffer_rsrc(base, 0, 0x7fffffff, 0x00020000);
}
template <typename V> __device__ __forceinline__ void buf_st(V x, __amdgpu_buffer_rsrc_t r, int voff, int soff) {
    if constexpr (sizeof(V) == 8) __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, x), r, voff, soff, 0);
    else __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), r, voff, soff, 0);
}

// Maximum over the 64 lanes of a wave, returned to every lane: DPP row rotations by 8, 4, 2
// and 1 give each lane its 16-lane row's maximum; row_bcast:15 and row_bcast:31 carry it
// across the four rows into the last one (lanes of the rows a step does not write keep
// their value), and lane 63's value is read out.  (Shuffles through LDS, one per step, made
// the frame-map kernel about 1% slower.)
__device__ __forceinline__ float wave_max(float x) {
#define GDN_DPPMAX(CTRL, ROWMASK)                                                                      \
    {                                                                                                  \
        const int b = __builtin_bit_cast(int, x);                                                      \
        x = fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(b, b, CTRL, ROWMASK, 0xf, false))); \
    }
    GDN_DPPMAX(0x128, 0xf)
    GDN_DPPMAX(0x124, 0xf)
    GDN_DPPMAX(0x122, 0xf)
    GDN_DPPMAX(0x121, 0xf)
    GDN_DPPMAX(0x142, 0xa)
    GDN_DPPMAX(0x143, 0xc)
#undef GDN_DPPMAX
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
}

template <typename E> struct Ops;

// bf16 inputs: bf16 operands, fp32 accumulation.
template <> struct Ops<bf16> {
    using F8 = bf16x8;   // K32 fragment, 16 B per lane
    using F4 = bf16x4;   // K16 fragment, 8 B per lane
    using V16 = bf16x8;  // 16-byte vector of elements
    static constexpr int EPV = 8;
    static __device__ __forceinline__ f32x4 mma32(F8 a, F8 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ f32x4 mma16(F4 a, F4 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(short4_, a),
                                                         __builtin_bit_cast(short4_, b), c, 0, 0, 0);
    }
    static __device__ __forceinline__ bf16 cvt(float x) { return (bf16)x; }
    // conversions written pairwise, so that each v_cvt_pk_bf16_f32 rounds two values (RNE)
    static __device__ __forceinline__ unsigned pk2(float a, float b) {
        return __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{a, b}, bf16x2));
    }
    static __device__ __forceinline__ F8 pack8(f32x4 lo, f32x4 hi) {
        const u32x4 w = {pk2(lo[0], lo[1]), pk2(lo[2], lo[3]), pk2(hi[0], hi[1]), pk2(hi[2], hi[3])};
        return __builtin_bit_cast(F8, w);
    }
    static __device__ __forceinline__ F4 pack4(f32x4 x) {
        const u32x2 w = {pk2(x[0], x[1]), pk2(x[2], x[3])};
        return __builtin_bit_cast(F4, w);
    }
    // 8 consecutive elements from LDS / global (16-byte aligned)
    static __device__ __forceinline__ F8 ld8(const bf16* p) { return *(const F8*)p; }
    // elements [p0, p0+4) then [p1, p1+4)  (PAIR slot map from two 8-byte pieces)
    static __device__ __forceinline__ F8 ld44(const bf16* p0, const bf16* p1) {
        bf16x4 a = *(const bf16x4*)p0, b = *(const bf16x4*)p1;
        return F8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    }
    static __device__ __forceinline__ F4 ld4(const bf16* p) { return *(const F4*)p; }
    static __device__ __forceinline__ void st8(bf16* p, F8 x) { *(F8*)p = x; }
    static __device__ __forceinline__ void st2(bf16* p, bf16 a, bf16 b) { *(bf16x2*)p = bf16x2{a, b}; }
    static __device__ __forceinline__ void st4(bf16* p, f32x4 x) { *(F4*)p = pack4(x); }
    static __device__ __forceinline__ f32x4 ld4f(const bf16* p) { return __builtin_convertvector(*(const F4*)p, f32x4); }
    static __device__ __forceinline__ F8 zero8() {
        F8 r;
        for (int j = 0; j < 8; ++j) r[j] = (bf16)0.f;
        return r;
    }
    // x = hi + lo + O(2^-16 |x|): hi = RNE(x), lo = RNE(x - hi)
    static constexpr bool kSplit = true;
    static __device__ __forceinline__ void split8(f32x4 a, f32x4 b, F8& hi, F8& lo) {
        hi = pack8(a, b);
        lo = pack8(a - __builtin_convertvector(__builtin_shufflevector(hi, hi, 0, 1, 2, 3), f32x4),
                   b - __builtin_convertvector(__builtin_shufflevector(hi, hi, 4, 5, 6, 7), f32x4));
    }
    static __device__ __forceinline__ void split4(f32x4 a, F4& hi, F4& lo) {
        hi = pack4(a);
        lo = pack4(a - __builtin_convertvector(hi, f32x4));
    }
    static __device__ __forceinline__ float lo_of(float x) { return x - (float)(bf16)x; }
    // ReLU of 8 values: a bf16 is sign-magnitude, so max(x, 0) is the signed 16-bit
    // integer max of its bits with 0 (negative values and -0 become +0), two per
    // v_pk_max_i16
    static __device__ __forceinline__ F8 relu8(F8 x) {
        typedef short s16x8 __attribute__((ext_vector_type(8)));
        const s16x8 v = __builtin_bit_cast(s16x8, x);
        return __builtin_bit_cast(F8, __builtin_elementwise_max(v, s16x8{0, 0, 0, 0, 0, 0, 0, 0}));
    }
    // LDS transpose load (ds_read_b64_tr_b16): from a row-major 16-bit matrix M in LDS
    // (row pitch pb bytes), lane (c, g) receives M[r0 + 4g + i][c0 + c], i = 0..3 -- a K16
    // operand fragment whose k runs along M's rows.  In each 16-lane group, source lane s
    // points at row r0 + 4g + s/4, columns c0 + 4(s%4) .. +3 (layout checked on gfx950).
    static __device__ __forceinline__ F4 ldtr(const bf16* m, int pb, int r0, int c0, int lane) {
        const int s = lane & 15, g = lane >> 4;
        const bf16* p = (const bf16*)((const char*)m + (r0 + 4 * g + (s >> 2)) * pb) + c0 + 4 * (s & 3);
        return __builtin_bit_cast(F4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) short4_*)(p)));
    }
};

// fp32 inputs: fp32 matrix cores (v_mfma_f32_16x16x4_f32), fp32 throughout.
template <> struct Ops<float> {
    using F8 = f32x8;
    using F4 = f32x4;
    using V16 = f32x4;
    static constexpr int EPV = 4;
    static __device__ __forceinline__ f32x4 mma32(F8 a, F8 b, f32x4 c) {
#pragma unroll
        for (int j = 0; j < 8; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], b[j], c, 0, 0, 0);
        return c;
    }
    static __device__ __forceinline__ f32x4 mma16(F4 a, F4 b, f32x4 c) {
#pragma unroll
        for (int j = 0; j < 4; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], b[j], c, 0, 0, 0);
        return c;
    }
    static __device__ __forceinline__ float cvt(float x) { return x; }
    static __device__ __forceinline__ F8 pack8(f32x4 lo, f32x4 hi) {
        return F8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
    static __device__ __forceinline__ F4 pack4(f32x4 x) { return x; }
    static __device__ __forceinline__ F8 ld8(const float* p) {
        f32x4 a = *(const f32x4*)p, b = *(const f32x4*)(p + 4);
        return F8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    }
    static __device__ __forceinline__ F8 ld44(const float* p0, const float* p1) {
        f32x4 a = *(const f32x4*)p0, b = *(const f32x4*)p1;
        return F8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    }
    static __device__ __forceinline__ F4 ld4(const float* p) { return *(const F4*)p; }
    static __device__ __forceinline__ void st8(float* p, F8 x) {
        *(f32x4*)p = f32x4{x[0], x[1], x[2], x[3]};
        *(f32x4*)(p + 4) = f32x4{x[4], x[5], x[6], x[7]};
    }
    static __device__ __forceinline__ void st4(float* p, f32x4 x) { *(f32x4*)p = x; }
    static __device__ __forceinline__ void st2(float* p, float a, float b) { *(f32x2*)p = f32x2{a, b}; }
    static __device__ __forceinline__ f32x4 ld4f(const float* p) { return *(const f32x4*)p; }
    static __device__ __forceinline__ F8 zero8() { return F8{0, 0, 0, 0, 0, 0, 0, 0}; }
    // fp32 operands need no split: lo is identically zero and never used
    static constexpr bool kSplit = false;
    static __device__ __forceinline__ void split8(f32x4 a, f32x4 b, F8& hi, F8& lo) {
        hi = pack8(a, b);
        lo = zero8();
    }
    static __device__ __forceinline__ void split4(f32x4 a, F4& hi, F4& lo) {
        hi = a;
        lo = zero4();
    }
    static __device__ __forceinline__ float lo_of(float) { return 0.f; }
    static __device__ __forceinline__ F8 relu8(F8 x) {
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = x[j] > 0.f ? x[j] : 0.f;
        return x;
    }
    // lane (c, g) receives M[r0 + 4g + i][c0 + c], i = 0..3 (plain loads for 32-bit data)
    static __device__ __forceinline__ F4 ldtr(const float* m, int pb, int r0, int c0, int lane) {
        const int c = lane & 15, g = lane >> 4;
        const float* p = (const float*)((const char*)m + (r0 + 4 * g) * pb) + c0 + c;
        return F4{p[0], *(const float*)((const char*)p + pb), *(const float*)((const char*)p + 2 * pb),
                  *(const float*)((const char*)p + 3 * pb)};
    }
};

template <typename E> __device__ __forceinline__ float tof(E x) { return (float)x; }

// Hardware transcendentals (v_exp_f32, v_log_f32, v_rsq_f32; about 1 ulp).  exp2 of
// arguments below -126 may flush to zero, which is the correct limit for a decay.
__device__ __forceinline__ float hw_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float hw_log2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float hw_rsq(float x) { return __builtin_amdgcn_rsqf(x); }

// Asynchronous global -> LDS copies (global_load_lds): lane l's `bytes` (4 or 16) from its
// own global address land at lds_base + l * bytes; lanes with exec off write nothing.
// Completion is counted by vmcnt, like a load.
__device__ __forceinline__ void dma16(const void* gsrc, void* lds_base) {
    __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)gsrc,
                                     (__attribute__((address_space(3))) void*)lds_base, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void* gsrc, void* lds_base) {
    __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)gsrc,
                                     (__attribute__((address_space(3))) void*)lds_base, 4, 0, 0);
}
// s_waitcnt vmcnt(0), other counters untouched (gfx9 encoding: expcnt 7, lgkmcnt 15)
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// s_waitcnt vmcnt(n): wait until at most n of the wave's vector memory operations are
// outstanding (they complete in issue order); n wave-uniform, clamped to [0, 31]
// (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt and lgkmcnt left at their maximum)
__device__ __forceinline__ void wait_vmem_le(int n) {
    switch (n < 0 ? 0 : n > 31 ? 31 : n) {
#define GDN_WV(N) case N: __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14)); break;
        GDN_WV(0) GDN_WV(1) GDN_WV(2) GDN_WV(3) GDN_WV(4) GDN_WV(5) GDN_WV(6) GDN_WV(7)
        GDN_WV(8) GDN_WV(9) GDN_WV(10) GDN_WV(11) GDN_WV(12) GDN_WV(13) GDN_WV(14) GDN_WV(15)
        GDN_WV(16) GDN_WV(17) GDN_WV(18) GDN_WV(19) GDN_WV(20) GDN_WV(21) GDN_WV(22) GDN_WV(23)
        GDN_WV(24) GDN_WV(25) GDN_WV(26) GDN_WV(27) GDN_WV(28) GDN_WV(29) GDN_WV(30) GDN_WV(31)
#undef GDN_WV
    }
}

// Workgroup barrier that orders LDS accesses only.  __syncthreads() also waits for every
// outstanding global load and store of the wave, which would stall register prefetches
// and write-backs at each barrier; kernels whose waves communicate through LDS alone use
// this instead.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP moves: shifts by 1, 2, 4, 8
// inside each row of 16 lanes, then row broadcasts of lane 15 and lane 31.
__device__ __forceinline__ float wave_incl_scan(float x) {
#define GDN_DPP(CTRL, ROWMASK)                                                                        \
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, \
                                                               ROWMASK, 0xf, false))
    GDN_DPP(0x111, 0xf);  // row_shr:1
    GDN_DPP(0x112, 0xf);  // row_shr:2
    GDN_DPP(0x114, 0xf);  // row_shr:4
    GDN_DPP(0x118, 0xf);  // row_shr:8
    GDN_DPP(0x142, 0xa);  // row_bcast:15 into rows 1 and 3
    GDN_DPP(0x143, 0xc);  // row_bcast:31 into rows 2 and 3
#undef GDN_DPP
    return x;
}

// The same inclusive prefix carried as an unevaluated sum hi + lo (hi = the rounded
// prefix, lo = the rounding error of every addition, each addition an error-free
// two-sum).  A difference of two prefixes, (hi_t - hi_i) + (lo_t - lo_i), is then accurate
// to about 2^-24 of the difference itself, however large the two prefixes are (a run of
// near-zero gates before both tokens cancels exactly).
__device__ __forceinline__ float wave_incl_scan2(float x, float& lo_out) {
#pragma clang fp contract(off)  // the two-sums must round each operation as written
    float hi = x, lo = 0.f;
#define GDN_DPP2(CTRL, ROWMASK)                                                                                 \
    {                                                                                                           \
        const float bh = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, hi), \
                                                                               CTRL, ROWMASK, 0xf, false));    \
        const float bl = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, lo), \
                                                                               CTRL, ROWMASK, 0xf, false));    \
        const float s = hi + bh, bb = s - hi, e = (hi - (s - bb)) + (bh - bb);                                  \
        hi = s;                                                                                                 \
        lo = lo + (bl + e);                                                                                     \
    }
    GDN_DPP2(0x111, 0xf)
    GDN_DPP2(0x112, 0xf)
    GDN_DPP2(0x114, 0xf)
    GDN_DPP2(0x118, 0xf)
    GDN_DPP2(0x142, 0xa)
    GDN_DPP2(0x143, 0xc)
#undef GDN_DPP2
    lo_out = lo;
    return hi;
}

// Rotary embedding angle in revolutions of position pos (an integer below 2^24, exact in
// float) at frequency / 2 pi = gh + gl (double split into two floats): the fraction of the
// rounded product (an exact subtraction) plus the product's exact remainder and the low
// part.  Contraction is off: fusing the product into the subtraction would count its
// remainder twice.
__device__ __forceinline__ float rope_rev(float pos, float gh, float gl) {
#pragma clang fp contract(off)
    const float rh = pos * gh;
    return (rh - __builtin_floorf(rh)) + (__builtin_fmaf(pos, gh, -rh) + pos * gl);
}

// t / w for 0 <= t < 2^24, w >= 1, from a float reciprocal rinv ~ 1 / w with an exact
// correction of the quotient (the float estimate is within one of it)
__device__ __forceinline__ int rope_div(int t, int w, float rinv) {
    int h = (int)((float)t * rinv);
    h -= (h * w > t) ? 1 : 0;
    h += ((h + 1) * w <= t) ? 1 : 0;
    return h;
}

// Rotates the pairs of a 16-byte vector of one token row (elements 2j0 .. 2j0 + 2n - 1):
// pair j turns by pos[axis(j)] * freq_j, axis 0 below pair p1, 1 below p2, else 2; the
// hardware sine and cosine take revolutions.  bf16 results are rounded to nearest even.
template <typename E, typename V>
__device__ __forceinline__ V rope_rotate(V v, int j0, float pos0, float pos1, float pos2, int p1, int p2,
                                         const float* ghi, const float* glo) {
    constexpr int NP = (int)(sizeof(V) / sizeof(E)) / 2;
#pragma unroll
    for (int e = 0; e < NP; ++e) {
        const int j = j0 + e;
        const float ps = j < p1 ? pos0 : (j < p2 ? pos1 : pos2);
        const float fr = rope_rev(ps, ghi[j], glo[j]);
        const float sn = __builtin_amdgcn_sinf(fr), cs = __builtin_amdgcn_cosf(fr);
        const float x0 = (float)v[2 * e], x1 = (float)v[2 * e + 1];
        v[2 * e] = (E)(x0 * cs - x1 * sn);
        v[2 * e + 1] = (E)(x0 * sn + x1 * cs);
    }
    return v;
}

// Split precision: bf16 operands that must carry ~16 significant bits are sent to the
// matrix cores as hi + lo pairs (hi = RNE(x), lo = RNE(x - hi)); a product a*b is then
// a_hi*b_hi + a_lo*b_hi + a_hi*b_lo (the lo*lo term is below fp32 accumulation noise).
// NSPLIT is the number of stored parts of such an operand.
template <typename E> struct SplitCount { static constexpr int N = Ops<E>::kSplit ? 2 : 1; };

// Geometry derived from the head dimension d = 16 * ND.
template <typename E, int ND_> struct Geo {
    static constexpr int ND = ND_;              // 16-wide tiles along d
    static constexpr int D = 16 * ND;
    static constexpr int KB = (ND + 1) / 2;     // 32-wide k steps along d (zero padded)
    static constexpr int DP = 32 * KB;          // padded d
    static constexpr int EPV = Ops<E>::EPV;     // elements per 16-byte vector
    static constexpr int FRAG = 64 * 8;         // elements in one K32 operand fragment
};

// Per-device one-time set-up (kernel attributes): the first call on each device runs f
// there, once, whatever the number of host threads; later calls return its status.
struct PerDeviceOnce {
    static constexpr int kMaxDevices = 64;
    std::once_flag flag[kMaxDevices];
    hipError_t status[kMaxDevices] = {};
    template <typename F>
    hipError_t run(F&& f) {
        int dev = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess) return e;
        if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
        std::call_once(flag[dev], [&] { status[dev] = f(); });
        return status[dev];
    }
};

}  // namespace gdn
