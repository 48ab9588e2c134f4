// rope3d.hip -- 3D rotary position embedding of q or k on gfx950, in place
// ("SANA-Video: Efficient Video Generation with Block Linear Diffusion Transformer" talk,
// the segment on temporal modelling: a 3D RoPE for the linear attention).  The pages give
// no frequency layout, split of the head dimension or base; the reading here is the axial
// form with those three left to the caller: the head dimension is cut into contiguous
// parts of d_t, d_h and d_w = d - d_t - d_h dimensions (even), rotated by the token's
// frame, latent row and latent column; in a part of n dimensions the pair (2i, 2i+1)
// turns by pos * base^(-2i/n).  Token t of [B, H, T, d] (T = n_frames grid_h grid_w)
// sits at frame frame_offset + t / (grid_h grid_w), row (t mod grid_h grid_w) / grid_w,
// column t mod grid_w.
//
// A stand-alone pass (one read and one write of the tensor): each thread rotates the
// pairs of 16-byte groups of token rows, four groups 256 apart at a time (all four loaded
// before any is rotated); consecutive threads take consecutive groups (coalesced).  Index
// arithmetic is 32-bit below 2^31 groups.  Frequencies / 2 pi come from the host in
// double as float hi + lo pairs, kept in LDS;
// the angle in revolutions is reduced exactly to its fraction (late frames keep full
// precision) and fed to the hardware sine and cosine; rotation in float32; a bf16 result
// is rounded to nearest even.
#include "gdn.h"
#include "common.hpp"
#include <math.h>
#include <stdint.h>

#define RP_API extern "C" __attribute__((visibility("default")))

namespace gdn {
namespace {

constexpr int kMaxPairs = 128;  // d <= 256
// Workgroups of a launch at most: each walks tiles of 256 x RU groups.  At the 5 s grid
// (5.2 M groups) 4,096 measured 29.2 us and 1,024 30.2 us, back to back, against 44.1 us
// for one group per thread and a workgroup per 256 groups.
constexpr long long RP_GRID_CAP = 4096;

struct RPArgs {
    void* x;
    long long ngrp;   // 16-byte groups in the tensor
    long long T;      // tokens per (b, h)
    int gpr;          // groups per token row: d / EPV
    int grid_h, grid_w, frame_offset;
    int start[3], size[3];
    float ghi[kMaxPairs], glo[kMaxPairs];  // frequency / 2 pi of pair j/2 as hi + lo (from double)
};

// Each workgroup walks tiles of 256 x RU groups (RU per thread, all loaded before any is
// rotated); I is the index type (32-bit unless the tensor has 2^31 groups or more).
constexpr int RU = 4;
template <typename E, typename I>
__global__ __launch_bounds__(256) void rope3d_apply_kernel(RPArgs a) {
    constexpr int EPV = 16 / (int)sizeof(E);
    typedef E V __attribute__((ext_vector_type(EPV)));
    __shared__ float sfr[2 * kMaxPairs];  // frequencies / 2 pi: hi, then lo
    for (int i = threadIdx.x; i < 2 * kMaxPairs; i += 256) sfr[i] = i < kMaxPairs ? a.ghi[i] : a.glo[i - kMaxPairs];
    __syncthreads();
    const I ngrp = (I)a.ngrp, T = (I)a.T, gpr = (I)a.gpr, gw = (I)a.grid_w;
    const I per_frame = (I)a.grid_h * gw;
    const I stride = (I)gridDim.x * (256 * RU);
    for (I base = (I)blockIdx.x * (256 * RU) + threadIdx.x; base < ngrp; base += stride) {
        V v[RU];
#pragma unroll
        for (int u = 0; u < RU; ++u) {
            const I gid = base + (I)(256 * u);
            if (gid < ngrp) v[u] = ((const V*)a.x)[gid];
        }
#pragma unroll
        for (int u = 0; u < RU; ++u) {
            const I gid = base + (I)(256 * u);
            if (gid >= ngrp) break;
            const I row = gid / gpr;
            const int j0 = (int)(gid - row * gpr) * EPV;  // first dimension of this group
            const I t = row % T;
            const I tf = t / per_frame, ti = t - tf * per_frame;
            const I hr = ti / gw;
            const float pos[3] = {(float)((I)a.frame_offset + tf), (float)hr, (float)(ti - hr * gw)};
#pragma unroll
            for (int p = 0; p < EPV / 2; ++p) {
                const int j = j0 + 2 * p;
                const int ax = j < a.start[1] ? 0 : (j < a.start[2] ? 1 : 2);
                // the angle in revolutions, reduced exactly (rope_rev); then the hardware sine
                // and cosine of 2 pi times that fraction (v_sin_f32 and v_cos_f32 take revolutions)
                const float fr = rope_rev(pos[ax], sfr[j >> 1], sfr[kMaxPairs + (j >> 1)]);
                const float sn = __builtin_amdgcn_sinf(fr), cs = __builtin_amdgcn_cosf(fr);
                const float x0 = (float)v[u][2 * p], x1 = (float)v[u][2 * p + 1];
                v[u][2 * p] = (E)(x0 * cs - x1 * sn);
                v[u][2 * p + 1] = (E)(x0 * sn + x1 * cs);
            }
            ((V*)a.x)[gid] = v[u];
        }
    }
}

}  // namespace
}  // namespace gdn

using namespace gdn;

RP_API int rope3d_apply(void* x, int32_t B, int32_t H, int32_t n_frames, int32_t grid_h, int32_t grid_w,
                        int32_t d, int32_t d_t, int32_t d_h, int32_t frame_offset, float base, int32_t dtype,
                        void* const* events, void* stream) {
    if (dtype != GDN_BF16 && dtype != GDN_F32) return GDN_ERR_DTYPE;
    const int d_w = d - d_t - d_h;
    if (B < 0 || H < 0 || n_frames < 0 || grid_h < 1 || grid_w < 1 || d < 0 || d_t < 0 || d_h < 0 || d_w < 0 ||
        frame_offset < 0 || !(base > 0.f))
        return GDN_ERR_DIMS;
    if ((d_t | d_h | d_w) & 1) return GDN_ERR_UNSUPPORTED;  // rotations act on pairs
    const int es = dtype == GDN_BF16 ? 2 : 4, epv = 16 / es;
    if (d % epv != 0 || d > 2 * kMaxPairs) return GDN_ERR_UNSUPPORTED;  // whole 16-byte groups per row
    const long long T = (long long)n_frames * grid_h * grid_w;
    if (T > 0 && (long long)frame_offset + n_frames > (1LL << 24)) return GDN_ERR_DIMS;  // exact float positions
    if (T > 0 && ((long long)1 << 40) / T / (d > 0 ? d : 1) < (long long)B * H) return GDN_ERR_DIMS;
    const long long ngrp = (long long)B * H * T * d / epv;
    if (ngrp == 0) return GDN_OK;
    if ((ngrp + 255) / 256 >= ((long long)1 << 31)) return GDN_ERR_DIMS;
    if (!x) return GDN_ERR_NULL;
    if ((uintptr_t)x & 15u) return GDN_ERR_ALIGN;
    RPArgs a;
    a.x = x;
    a.ngrp = ngrp;
    a.T = T;
    a.gpr = d / epv;
    a.grid_h = grid_h;
    a.grid_w = grid_w;
    a.frame_offset = frame_offset;
    a.start[0] = 0;
    a.start[1] = d_t;
    a.start[2] = d_t + d_h;
    a.size[0] = d_t;
    a.size[1] = d_h;
    a.size[2] = d_w;
    for (int ax = 0; ax < 3; ++ax)
        for (int i = 0; 2 * i < a.size[ax]; ++i) {  // frequencies in double, split hi + lo
            const double f = pow((double)base, -2.0 * i / a.size[ax]) / (2.0 * 3.141592653589793);
            const int pr = (a.start[ax] >> 1) + i;
            a.ghi[pr] = (float)f;
            a.glo[pr] = (float)(f - (double)a.ghi[pr]);
        }
    hipStream_t st = (hipStream_t)stream;
    if (events && hipEventRecord((hipEvent_t)events[0], st) != hipSuccess) return GDN_ERR_HIP;
    const long long tiles = (ngrp + 256 * RU - 1) / (256 * RU);
    const unsigned grid = (unsigned)(tiles < RP_GRID_CAP ? tiles : RP_GRID_CAP);
    const bool wide = ngrp >= ((long long)1 << 31);
    if (dtype == GDN_BF16) {
        if (wide) hipLaunchKernelGGL((rope3d_apply_kernel<bf16, long long>), dim3(grid), dim3(256), 0, st, a);
        else hipLaunchKernelGGL((rope3d_apply_kernel<bf16, unsigned>), dim3(grid), dim3(256), 0, st, a);
    } else {
        if (wide) hipLaunchKernelGGL((rope3d_apply_kernel<float, long long>), dim3(grid), dim3(256), 0, st, a);
        else hipLaunchKernelGGL((rope3d_apply_kernel<float, unsigned>), dim3(grid), dim3(256), 0, st, a);
    }
    if (hipGetLastError() != hipSuccess) return GDN_ERR_HIP;
    if (events && hipEventRecord((hipEvent_t)events[1], st) != hipSuccess) return GDN_ERR_HIP;
    return GDN_OK;
}
