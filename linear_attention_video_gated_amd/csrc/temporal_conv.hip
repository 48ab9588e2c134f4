// temporal_conv.hip -- causal temporal convolution with a block carry on gfx950: the
// temporal convolution of the causal FFN ("SANA-Video: Efficient Video Generation with
// Block Linear Diffusion Transformer" talk, the segment on a causal FFN with temporal
// convolution, two-block example: in training a zero token sits after each block, so a
// block never sees the next one, and the previous block's last token is cached as the
// block's first, so it does see the one before).  The pages give neither kernel size nor
// weights; the reading here: a depthwise convolution along frames with three taps centred
// on the frame, weights w[3][C] and bias[C] from the caller.  For a block of F frames, per
// (b, position p, channel c):
//   y[f] = w[0][c] prev(f) + w[1][c] x[f] + w[2][c] next(f) + bias[c],
//   prev(0) = carry_in (zero without one), next(F-1) = 0,   carry_out = x[F-1].
//
// HBM-bound: each thread owns one 16-byte group of channels at one (b, p) and walks the
// block's frames four at a time with the next four already loading, so x is read once
// and y written once with four loads in flight per thread; consecutive threads take
// consecutive channel groups (coalesced 16-byte accesses), the frame stride is P * C
// elements.  Arithmetic in float32.
#include "gdn.h"
#include "common.hpp"
#include <stdint.h>

#define TC_API extern "C" __attribute__((visibility("default")))

namespace gdn {
namespace {

struct TCArgs {
    const void* x;
    const void* carry_in;  // may be NULL (zero)
    const float* w;        // [3][C]
    const float* bias;     // [C] or NULL
    void* y;
    void* carry_out;       // may be NULL; may equal carry_in
    long long cols;        // 16-byte groups per frame of one batch entry: P * C / EPV
    long long ngrp;        // B * cols
    int F, C, out_f32;
};

template <typename E>
__global__ __launch_bounds__(256) void tconv_block(TCArgs a) {
    constexpr int EPV = 16 / (int)sizeof(E);
    typedef E V __attribute__((ext_vector_type(EPV)));
    const long long gid = (long long)blockIdx.x * 256 + threadIdx.x;
    if (gid >= a.ngrp) return;
    const long long b = gid / a.cols, e = gid - b * a.cols;
    const int c0 = (int)((e * EPV) % a.C);
    const V* x = (const V*)a.x + b * a.F * a.cols + e;
    const long long ce = b * a.cols + e;  // this group in carry_in / carry_out
    V prev;
    if (a.carry_in) {
        prev = ((const V*)a.carry_in)[ce];
    } else {
#pragma unroll
        for (int j = 0; j < EPV; ++j) prev[j] = (E)0.f;
    }
    if (a.F == 0) {  // an empty block passes the carry through
        if (a.carry_out) ((V*)a.carry_out)[ce] = prev;
        return;
    }
    float w0[EPV], w1[EPV], w2[EPV], bs[EPV];
#pragma unroll
    for (int j = 0; j < EPV; ++j) {
        w0[j] = a.w[c0 + j];
        w1[j] = a.w[a.C + c0 + j];
        w2[j] = a.w[2 * a.C + c0 + j];
        bs[j] = a.bias ? a.bias[c0 + j] : 0.f;
    }
    // frames in groups of four: the next group's four loads go out before this group's
    // outputs are formed, so each thread keeps four loads in flight
    auto ld = [&](int f) {
        V v;
        if (f < a.F) {
            v = x[(long long)f * a.cols];
        } else {  // past the block: the zero token
#pragma unroll
            for (int j = 0; j < EPV; ++j) v[j] = (E)0.f;
        }
        return v;
    };
    auto out = [&](int f, const V& p, const V& c, const V& n) {
        if (f >= a.F) return;
        float r[EPV];
#pragma unroll
        for (int j = 0; j < EPV; ++j)
            r[j] = __builtin_fmaf(w0[j], (float)p[j], __builtin_fmaf(w1[j], (float)c[j], __builtin_fmaf(w2[j], (float)n[j], bs[j])));
        const long long o = (b * a.F + f) * a.cols + e;  // in 16-byte groups of the input dtype
        if (a.out_f32) {
            f32x4* dst = (f32x4*)a.y + o * (EPV / 4);
#pragma unroll
            for (int j = 0; j < EPV / 4; ++j) dst[j] = f32x4{r[4 * j], r[4 * j + 1], r[4 * j + 2], r[4 * j + 3]};
        } else {
            V v;
#pragma unroll
            for (int j = 0; j < EPV; ++j) v[j] = (E)r[j];  // round to nearest even
            ((V*)a.y)[o] = v;
        }
        if (f == a.F - 1 && a.carry_out) ((V*)a.carry_out)[ce] = c;  // the next block's carry
    };
    V r0 = ld(0), r1 = ld(1), r2 = ld(2), r3 = ld(3);
    for (int f = 0; f < a.F; f += 4) {
        const V n0 = ld(f + 4), n1 = ld(f + 5), n2 = ld(f + 6), n3 = ld(f + 7);
        out(f, prev, r0, r1);
        out(f + 1, r0, r1, r2);
        out(f + 2, r1, r2, r3);
        out(f + 3, r2, r3, n0);
        prev = r3;
        r0 = n0;
        r1 = n1;
        r2 = n2;
        r3 = n3;
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

TC_API int temporal_conv_block(const void* x, const void* carry_in, const float* weight, const float* bias,
                               void* y, void* carry_out, int32_t B, int32_t n_frames, int32_t frame_len,
                               int32_t channels, int32_t dtype, uint32_t flags, void* const* events,
                               void* stream) {
    if (dtype != GDN_BF16 && dtype != GDN_F32) return GDN_ERR_DTYPE;
    if (B < 0 || n_frames < 0 || frame_len < 0 || channels < 0) return GDN_ERR_DIMS;
    if (flags & ~(uint32_t)GDN_F_OUT_F32) return GDN_ERR_UNSUPPORTED;
    const int es = dtype == GDN_BF16 ? 2 : 4, epv = 16 / es;
    if (channels % epv != 0) return GDN_ERR_UNSUPPORTED;  // whole 16-byte channel groups
    const long long frame = (long long)frame_len * channels;
    if (frame > 0 && ((long long)1 << 40) / frame < (long long)B * (n_frames + 1)) return GDN_ERR_DIMS;
    const long long ngrp = (long long)B * frame / epv;
    if (ngrp == 0) return GDN_OK;
    if ((ngrp + 255) / 256 >= ((long long)1 << 31)) return GDN_ERR_DIMS;
    if (!weight || (n_frames > 0 && (!x || !y))) return GDN_ERR_NULL;
    if (misaligned16(x) || misaligned16(carry_in) || misaligned16(y) || misaligned16(carry_out) ||
        ((uintptr_t)weight & 3u) || ((uintptr_t)bias & 3u))
        return GDN_ERR_ALIGN;
    const bool f32o = (flags & GDN_F_OUT_F32) != 0;
    const long long nx = (long long)B * n_frames * frame, nc = (long long)B * frame;
    const size_t xb = (size_t)nx * es, cb = (size_t)nc * es, yb = (size_t)nx * (f32o ? 4 : es);
    if (overlaps(y, yb, x, xb) || overlaps(y, yb, carry_in, cb) || overlaps(y, yb, carry_out, cb) ||
        overlaps(carry_out, cb, x, xb) || (carry_out != carry_in && overlaps(carry_out, cb, carry_in, cb)))
        return GDN_ERR_ALIAS;
    TCArgs a;
    a.x = x;
    a.carry_in = carry_in;
    a.w = weight;
    a.bias = bias;
    a.y = y;
    a.carry_out = carry_out;
    a.cols = frame / epv;
    a.ngrp = ngrp;
    a.F = n_frames;
    a.C = channels;
    a.out_f32 = f32o;
    hipStream_t st = (hipStream_t)stream;
    if (events && hipEventRecord((hipEvent_t)events[0], st) != hipSuccess) return GDN_ERR_HIP;
    const unsigned grid = (unsigned)((ngrp + 255) / 256);
    if (dtype == GDN_BF16) hipLaunchKernelGGL(tconv_block<bf16>, dim3(grid), dim3(256), 0, st, a);
    else hipLaunchKernelGGL(tconv_block<float>, dim3(grid), dim3(256), 0, st, a);
    if (hipGetLastError() != hipSuccess) return GDN_ERR_HIP;
    if (events && hipEventRecord((hipEvent_t)events[1], st) != hipSuccess) return GDN_ERR_HIP;
    return GDN_OK;
}
