// gdn_api.hip -- the C ABI declared in include/gdn.h: argument checks (host only, before
// anything is enqueued; the plan and workspace layout are in gdn_plan.cpp) and dispatch
// over (dtype, d) to the kernel launchers.  Frames are processed in windows of at most
// kMaxUnits (b, h, frame) units so the workspace never grows with the number of frames.
//
// All launches go to the caller's stream, window after window.  (Running the chain and
// the readout of one window on other streams beside the next window's frame maps was
// measured slower on MI355X: the frame-map kernel saturates instruction issue and its
// LDS footprint keeps the chain's workgroups off the busy CUs.)
#include "gdn.h"
#include "common.hpp"
#include "gdn_kernels.hpp"
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define GDN_API extern "C" __attribute__((visibility("default")))

namespace gdn {
namespace {

// Compute units of the current device (the group plan depends on it), queried once per
// device; 256 (MI355X) when the query fails.
int device_cus() {
    static PerDeviceOnce once;
    static int cus[PerDeviceOnce::kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= PerDeviceOnce::kMaxDevices) return 256;
    (void)once.run([&] {
        int n = 0;
        const hipError_t e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
        cus[dev] = (e == hipSuccess && n > 0) ? n : 256;
        return hipSuccess;
    });
    return cus[dev] > 0 ? cus[dev] : 256;
}

int plan_call(const gdn_dims_t* d, int entry, Plan* p) { return check_dims(d, entry, p, device_cus()); }

__global__ void fill_or_copy(const float* src, float* dst, long long n) {
    for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (long long)gridDim.x * blockDim.x)
        dst[i] = src ? src[i] : 0.f;
}

int set_state(const float* src, float* dst, long long n, hipStream_t st) {
    if (!dst || dst == src || n == 0) return GDN_OK;
    long long blocks = (n + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(fill_or_copy, dim3((unsigned)blocks), dim3(256), 0, st, src, dst, n);
    return hipGetLastError() == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

// Rotary-embedding arguments of a call (GDN_F_ROPE_QK): the pair frequencies of each part
// computed in double on the host, over 2 pi, split into float hi + lo.
RopeArgs rope_args(const gdn_dims_t* d) {
    RopeArgs r;
    memset(&r, 0, sizeof r);
    if (!(d->flags & GDN_F_ROPE_QK)) return r;
    r.on = 1;
    r.p1 = d->rope_d_t / 2;
    r.p2 = (d->rope_d_t + d->rope_d_h) / 2;
    r.grid_w = d->rope_grid_w;
    r.frame0 = d->rope_frame_offset;
    const int size[3] = {d->rope_d_t, d->rope_d_h, d->d_k - d->rope_d_t - d->rope_d_h};
    int j = 0;
    for (int ax = 0; ax < 3; ++ax)
        for (int i = 0; 2 * i < size[ax] && j < kRopePairs; ++i, ++j) {
            const double f = pow((double)d->rope_base, -2.0 * i / size[ax]) / (2.0 * 3.141592653589793);
            r.ghi[j] = (float)f;
            r.glo[j] = (float)(f - (double)r.ghi[j]);
        }
    return r;
}

// entry GDN_ENTRY_FORWARD / _READONLY: frame maps, chain, frame-end readout;
// GDN_ENTRY_TOKEN: group-end maps, chain, per-token readout pass.
template <typename E, int ND>
int run_gdn(const void* q, const void* k, const void* v, const float* alpha, const float* beta,
            const float* state_in, float* state_out, void* out, const gdn_dims_t* d,
            const Plan& p, hipStream_t st, int entry) {
    const bool tok = entry == GDN_ENTRY_TOKEN;
    char* ws = (char*)d->workspace;
    float* carry = (float*)(ws + p.off_carry);
    const int BH = (int)p.BH;
    void* afr = ws + p.off_a;
    void* bfr = ws + p.off_b;
    int* xexp = (int*)(ws + p.off_x);
    void* agr = ws + p.off_ga;
    float* bgr = (float*)(ws + p.off_gb);
    float* sgrp = (float*)(ws + p.off_c);
    const RopeArgs rope = rope_args(d);
    for (int wi = 0; wi < p.nwin; ++wi) {
        const int f0 = wi * p.nfw;
        const int nf = (d->n_frames - f0 < p.nfw) ? d->n_frames - f0 : p.nfw;
        const bool last = wi == p.nwin - 1;
        // A call with a single group per (b, h) knows the state at the group start:
        // state_in (its layout is that of the per-group states with one group).  The frame
        // maps then run from it (true start: no A part, the B maps are the states, state_out
        // written by that pass), and there is no chain to run; the per-token readout pass
        // needs neither the maps nor the chain.
        const bool single = p.nwin == 1 && nf <= p.G;
        const float* s_before = single ? state_in : sgrp;
        const int of32 = (d->flags & GDN_F_OUT_F32) ? 1 : 0;
        const P1Args a1{k, v, alpha, beta, p.T, d->frame_len, f0, nf, p.G, BH, d->flags, agr, bgr,
                        tok ? 0 : 1, nullptr, nullptr, single ? state_in : nullptr, 0, single ? 1 : 0,
                        single ? state_out : nullptr, afr, bfr, xexp, rope};
        const P1Args a3t{k, v, alpha, beta, p.T, d->frame_len, f0, nf, p.G, BH, d->flags, nullptr, nullptr,
                         0, q, out, s_before, of32, 0, single ? state_out : nullptr, nullptr, nullptr, nullptr, rope};
        const P2Args a2{agr, bgr, wi == 0 ? state_in : carry, last ? state_out : carry, sgrp, nf, p.G};
        const P3Args a3{q, out, afr, bfr, xexp, single ? nullptr : sgrp, p.T, d->frame_len, f0, nf, p.G, of32,
                        single ? 1 : 0, 0, rope};
        void* const* ev = (d->phase_events && wi < d->phase_windows) ? d->phase_events + 6 * wi : nullptr;
        if (tok && single) {  // the readout pass alone
            if (record(ev, 0, st) != hipSuccess || record(ev, 1, st) != hipSuccess) return GDN_ERR_HIP;
        } else if (launch_gdn_phase<E, ND>(0, &a1, BH, st, ev) != hipSuccess) {
            return GDN_ERR_HIP;
        }
        if (single) {
            if (record(ev, 2, st) != hipSuccess || record(ev, 3, st) != hipSuccess) return GDN_ERR_HIP;
        } else if (launch_gdn_phase<E, ND>(1, &a2, BH, st, ev) != hipSuccess) {
            return GDN_ERR_HIP;
        }
        if ((tok ? launch_gdn_phase<E, ND>(3, &a3t, BH, st, ev) : launch_gdn_phase<E, ND>(2, &a3, BH, st, ev)) !=
            hipSuccess)
            return GDN_ERR_HIP;
    }
    return GDN_OK;
}

template <typename E, int ND>
int run_bc(const void* q, const void* k, const void* v, const float* s_in, const float* z_in,
           float* s_out, float* z_out, void* out, const gdn_dims_t* d, const Plan& p, hipStream_t st) {
    char* ws = (char*)d->workspace;
    float* carry = (float*)(ws + p.off_carry);
    const unsigned relu = (d->flags & GDN_F_RELU_QK) ? 1u : 0u;
    for (int wi = 0; wi < p.nwin; ++wi) {
        const int f0 = wi * p.nfw;
        const int nf = (d->n_frames - f0 < p.nfw) ? d->n_frames - f0 : p.nfw;
        const bool last = wi == p.nwin - 1;
        BC1Args a1{k, v, p.T, d->frame_len, f0, nf, relu, (float*)(ws + p.off_a)};
        BC2Args a2{(const float*)(ws + p.off_a), wi == 0 ? s_in : nullptr, wi == 0 ? z_in : nullptr,
                   wi == 0 ? nullptr : carry, last ? nullptr : carry, last ? s_out : nullptr,
                   last ? z_out : nullptr, ws + p.off_c, nf};
        BC3Args a3{q, out, ws + p.off_c, p.T, d->frame_len, f0, nf, relu, 1e-6f, (d->flags & GDN_F_OUT_F32) ? 1 : 0};
        void* const* ev = (d->phase_events && wi < d->phase_windows) ? d->phase_events + 6 * wi : nullptr;
        if (launch_bc_window<E, ND>(a1, a2, a3, (int)p.BH, st, ev) != hipSuccess)
            return GDN_ERR_HIP;
    }
    return GDN_OK;
}

#define DISPATCH(FN, ...)                                                              \
    do {                                                                               \
        if (d->dtype == GDN_BF16) {                                                    \
            switch (p.nd) {                                                            \
                case 1: return FN<bf16, 1>(__VA_ARGS__);                               \
                case 2: return FN<bf16, 2>(__VA_ARGS__);                               \
                case 4: return FN<bf16, 4>(__VA_ARGS__);                               \
                case 7: return FN<bf16, 7>(__VA_ARGS__);                               \
                case 8: return FN<bf16, 8>(__VA_ARGS__);                               \
            }                                                                          \
        } else {                                                                       \
            switch (p.nd) {                                                            \
                case 1: return FN<float, 1>(__VA_ARGS__);                              \
                case 2: return FN<float, 2>(__VA_ARGS__);                              \
                case 4: return FN<float, 4>(__VA_ARGS__);                              \
                case 7: return FN<float, 7>(__VA_ARGS__);                              \
                case 8: return FN<float, 8>(__VA_ARGS__);                              \
            }                                                                          \
        }                                                                              \
        return GDN_ERR_UNSUPPORTED;                                                    \
    } while (0)

int gdn_common(const void* q, const void* k, const void* v, const float* alpha, const float* beta,
               const float* state_in, float* state_out, void* out, const gdn_dims_t* d, void* stream,
               int entry) {
    Plan p;
    int rc = plan_call(d, entry, &p);
    if (rc != GDN_OK) return rc;
    const long long nstate = p.BH * d->d_k * d->d_v;
    const size_t sbytes = (size_t)nstate * 4;
    hipStream_t st = (hipStream_t)stream;
    if (p.BH == 0) return GDN_OK;
    if (d->n_frames == 0) {
        if (misaligned(state_in) || misaligned(state_out)) return GDN_ERR_ALIGN;
        return entry != GDN_ENTRY_READONLY ? set_state(state_in, state_out, nstate, st) : GDN_OK;
    }
    const bool additive = (d->flags & GDN_F_ADDITIVE) != 0;
    if (!q || !k || !v || !out) return GDN_ERR_NULL;
    if (!additive && (!alpha || !beta)) return GDN_ERR_NULL;
    if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(out) || misaligned(alpha) ||
        misaligned(beta) || misaligned(state_in) || misaligned(state_out) || misaligned(d->workspace))
        return GDN_ERR_ALIGN;
    if (!d->workspace || d->workspace_bytes < p.total) return GDN_ERR_WORKSPACE;
    const size_t tbytes = (size_t)p.BH * p.T * d->d_k * p.es;
    const size_t obytes = (size_t)p.BH * p.T * d->d_k * ((d->flags & GDN_F_OUT_F32) ? 4 : p.es);
    const size_t gbytes = (size_t)p.BH * p.T * 4;
    const void* ins[] = {q, k, v, additive ? nullptr : alpha, additive ? nullptr : beta, state_in, state_out};
    const size_t lens[] = {tbytes, tbytes, tbytes, gbytes, gbytes, sbytes, sbytes};
    for (int i = 0; i < 7; ++i) {
        if (overlap(out, obytes, ins[i], lens[i])) return GDN_ERR_ALIAS;
        if (overlap(d->workspace, p.total, ins[i], lens[i])) return GDN_ERR_ALIAS;
    }
    if (overlap(out, obytes, d->workspace, p.total)) return GDN_ERR_ALIAS;
    if (state_out && state_out != state_in && overlap(state_out, sbytes, state_in, sbytes)) return GDN_ERR_ALIAS;
    for (int i = 0; i < 5; ++i)
        if (overlap(state_out, sbytes, ins[i], lens[i])) return GDN_ERR_ALIAS;
    DISPATCH(run_gdn, q, k, v, alpha, beta, state_in, entry != GDN_ENTRY_READONLY ? state_out : nullptr,
             out, d, p, st, entry);
}

}  // namespace

// Scratch of the allocation-free entry (gdn_frame_forward_noalloc): one array per device,
// held by the device until the process ends.  In host code the name `scratch` is a
// host-side stand-in, never a device address: its device address is looked up once per
// device (scratch_on_device) and only that address is passed to kernels.
constexpr size_t kScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

hipError_t scratch_on_device(void** out) {
    static PerDeviceOnce once;
    static void* addr[PerDeviceOnce::kMaxDevices];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= PerDeviceOnce::kMaxDevices) return hipErrorInvalidDevice;
    e = once.run([&] {
        void* ptr = nullptr;
        const hipError_t r = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        addr[dev] = r == hipSuccess ? ptr : nullptr;
        return r == hipSuccess && !ptr ? hipErrorInvalidSymbol : r;
    });
    if (e != hipSuccess) return e;
    *out = addr[dev];
    return hipSuccess;
}

}  // namespace
}  // namespace gdn

using namespace gdn;

GDN_API int gdn_frame_forward_noalloc(const void* q, const void* k, const void* v, const float* alpha,
                                      const float* beta, const float* state_in, float* state_out, void* out,
                                      const gdn_dims_t* dims, void* stream) {
    if (!dims) return GDN_ERR_NULL;
    gdn_dims_t d = *dims;  // the caller's workspace fields are ignored
    d.workspace = nullptr;
    d.workspace_bytes = 0;
    Plan p;
    const int rc = plan_call(&d, GDN_ENTRY_FORWARD, &p);
    if (rc != GDN_OK) return rc;
    if (p.total > kScratchBytes) return GDN_ERR_WORKSPACE;  // beyond the static scratch
    if (p.total > 0) {
        void* ws = nullptr;
        if (scratch_on_device(&ws) != hipSuccess) return GDN_ERR_HIP;
        d.workspace = ws;
        d.workspace_bytes = kScratchBytes;
    }
    return gdn_common(q, k, v, alpha, beta, state_in, state_out, out, &d, stream, GDN_ENTRY_FORWARD);
}

GDN_API size_t gdn_noalloc_scratch_bytes(void) { return kScratchBytes; }

GDN_API int gdn_frame_forward(const void* q, const void* k, const void* v, const float* alpha,
                              const float* beta, const float* state_in, float* state_out, void* out,
                              const gdn_dims_t* dims, void* stream) {
    return gdn_common(q, k, v, alpha, beta, state_in, state_out, out, dims, stream, GDN_ENTRY_FORWARD);
}

GDN_API int gdn_token_forward(const void* q, const void* k, const void* v, const float* alpha,
                              const float* beta, const float* state_in, float* state_out, void* out,
                              const gdn_dims_t* dims, void* stream) {
    return gdn_common(q, k, v, alpha, beta, state_in, state_out, out, dims, stream, GDN_ENTRY_TOKEN);
}

GDN_API int gdn_frame_forward_readonly(const void* q, const void* k, const void* v, const float* alpha,
                                       const float* beta, const float* state_in, void* out,
                                       const gdn_dims_t* dims, void* stream) {
    return gdn_common(q, k, v, alpha, beta, state_in, nullptr, out, dims, stream, GDN_ENTRY_READONLY);
}

GDN_API int linear_attn_block_causal(const void* q, const void* k, const void* v, const float* state_in,
                                     const float* z_in, float* state_out, float* z_out, void* out,
                                     const gdn_dims_t* dims, void* stream) {
    const gdn_dims_t* d = dims;
    Plan p;
    int rc = plan_call(d, GDN_ENTRY_BLOCK_CAUSAL, &p);
    if (rc != GDN_OK) return rc;
    hipStream_t st = (hipStream_t)stream;
    const long long ns = p.BH * d->d_k * d->d_v, nz = p.BH * d->d_k;
    const size_t sbytes = (size_t)ns * 4, zbytes = (size_t)nz * 4;
    if (p.BH == 0) return GDN_OK;
    if (misaligned(state_in) || misaligned(state_out) || misaligned(z_in) || misaligned(z_out)) return GDN_ERR_ALIGN;
    if (d->n_frames == 0) {
        rc = set_state(state_in, state_out, ns, st);
        return rc != GDN_OK ? rc : set_state(z_in, z_out, nz, st);
    }
    if (!q || !k || !v || !out) return GDN_ERR_NULL;
    if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(out) || misaligned(d->workspace))
        return GDN_ERR_ALIGN;
    if (!d->workspace || d->workspace_bytes < p.total) return GDN_ERR_WORKSPACE;
    const size_t tbytes = (size_t)p.BH * p.T * d->d_k * p.es;
    const size_t obytes = (size_t)p.BH * p.T * d->d_k * ((d->flags & GDN_F_OUT_F32) ? 4 : p.es);
    const void* ins[] = {q, k, v, state_in, z_in, state_out, z_out};
    const size_t lens[] = {tbytes, tbytes, tbytes, sbytes, zbytes, sbytes, zbytes};
    for (int i = 0; i < 7; ++i) {
        if (overlap(out, obytes, ins[i], lens[i])) return GDN_ERR_ALIAS;
        if (overlap(d->workspace, p.total, ins[i], lens[i])) return GDN_ERR_ALIAS;
    }
    if (overlap(out, obytes, d->workspace, p.total)) return GDN_ERR_ALIAS;
    if (state_out && state_out != state_in && overlap(state_out, sbytes, state_in, sbytes)) return GDN_ERR_ALIAS;
    if (z_out && z_out != z_in && overlap(z_out, zbytes, z_in, zbytes)) return GDN_ERR_ALIAS;
    for (int i = 0; i < 3; ++i)
        if (overlap(state_out, sbytes, ins[i], lens[i]) || overlap(z_out, zbytes, ins[i], lens[i]))
            return GDN_ERR_ALIAS;
    DISPATCH(run_bc, q, k, v, state_in, z_in, state_out, z_out, out, d, p, st);
}

GDN_API size_t gdn_workspace_bytes(const gdn_dims_t* dims, int entry) {
    if (entry != GDN_ENTRY_FORWARD && entry != GDN_ENTRY_READONLY && entry != GDN_ENTRY_BLOCK_CAUSAL &&
        entry != GDN_ENTRY_TOKEN)
        return 0;
    Plan p;
    if (plan_call(dims, entry, &p) != GDN_OK) return 0;
    return p.total;
}

GDN_API int gdn_window_count(const gdn_dims_t* dims, int entry) {
    if (entry != GDN_ENTRY_FORWARD && entry != GDN_ENTRY_READONLY && entry != GDN_ENTRY_BLOCK_CAUSAL &&
        entry != GDN_ENTRY_TOKEN)
        return GDN_ERR_UNSUPPORTED;
    Plan p;
    const int rc = plan_call(dims, entry, &p);
    return rc != GDN_OK ? rc : p.nwin;
}

GDN_API const char* gdn_status_str(int status) {
    switch (status) {
        case GDN_OK: return "ok";
        case GDN_ERR_NULL: return "a required pointer is NULL";
        case GDN_ERR_DIMS: return "invalid or inconsistent sizes";
        case GDN_ERR_DTYPE: return "unsupported dtype (expected GDN_BF16 or GDN_F32)";
        case GDN_ERR_ALIGN: return "a pointer is not 16-byte aligned";
        case GDN_ERR_ALIAS: return "output overlaps an input, a state or the workspace";
        case GDN_ERR_WORKSPACE: return "workspace missing or smaller than gdn_workspace_bytes()";
        case GDN_ERR_UNSUPPORTED: return "unsupported head dimension or flag";
        case GDN_ERR_HIP: return "HIP kernel launch failed";
        default: return "unknown status";
    }
}

GDN_API int gdn_abi_version(void) { return GDN_ABI_VERSION; }
