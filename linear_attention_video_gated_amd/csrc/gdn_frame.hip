// gdn_frame.hip -- launchers of the frame-wise gated-delta-rule kernels (gdn_frame.hpp):
// frame maps, chain over groups, frame-end readout and per-token readout.  The variants
// that rotate q and k by the 3D rotary embedding on load are built in gdn_frame_rope.hip
// (a translation unit of their own, compiled in parallel) and reached through
// launch_gdn_rope.
#include "gdn_frame.hpp"

namespace gdn {

// -------------------------------------------------------------------------------------
// launchers
// -------------------------------------------------------------------------------------
template <typename E, int ND>
hipError_t launch_gdn_phase(int phase, const void* args, int BH, hipStream_t st, void* const* ev) {
    using L = P1<E, ND>;
    using LT = P1<E, ND, true>;
    static PerDeviceOnce attr;  // per instantiation
    hipError_t e = attr.run([] {
        const void* aff[8] = {(const void*)gdn_frame_affine<E, ND, 0>, (const void*)gdn_frame_affine<E, ND, 1>,
                              (const void*)gdn_frame_affine<E, ND, 2>, (const void*)gdn_frame_affine<E, ND, 3>,
                              (const void*)gdn_frame_affine<E, ND, 4>, (const void*)gdn_frame_affine<E, ND, 5>,
                              (const void*)gdn_frame_affine<E, ND, 6>, (const void*)gdn_frame_affine<E, ND, 7>};
        const void* tok[4] = {(const void*)gdn_token_readout<E, ND, 0>, (const void*)gdn_token_readout<E, ND, 1>,
                              (const void*)gdn_token_readout<E, ND, 2>, (const void*)gdn_token_readout<E, ND, 3>};
        hipError_t e = hipSuccess;
        for (const void* f : aff)
            if ((e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, L::LDS_B)) != hipSuccess)
                return e;
        for (const void* f : tok)
            if ((e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, LT::LDS_B)) != hipSuccess)
                return e;
        e = hipFuncSetAttribute((const void*)gdn_frame_chain<E, ND>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                P2<E, ND>::LDS_B);
        if (e != hipSuccess) return e;
        return hipFuncSetAttribute((const void*)gdn_frame_readout<E, ND, false>,
                                   hipFuncAttributeMaxDynamicSharedMemorySize, P3<E, ND, false>::LDS_B);
    });
    if (e != hipSuccess) return e;
    const int slot = phase == 3 ? 2 : phase;  // the per-token readout is a window's third launch
    e = record(ev, 2 * slot, st);
    if (e != hipSuccess) return e;
    if (phase == 3) {
        const P1Args& p1 = *(const P1Args*)args;
        const dim3 grid((p1.nf + p1.G - 1) / p1.G, BH);
        if (p1.rope.on) {
            if ((e = launch_gdn_rope<E, ND>(3, p1.flags & 3u, args, BH, st)) != hipSuccess) return e;
        } else {
            switch (p1.flags & 3u) {
#define GDN_TOK(M) case M: hipLaunchKernelGGL((gdn_token_readout<E, ND, M>), grid, dim3(LT::NT), LT::LDS_B, st, p1); break;
                GDN_TOK(0) GDN_TOK(1) GDN_TOK(2) GDN_TOK(3)
#undef GDN_TOK
            }
        }
    } else if (phase == 0) {
        const P1Args& p1 = *(const P1Args*)args;
        const int ngw = (p1.nf + p1.G - 1) / p1.G;
        const dim3 grid(ngw, BH);
        const unsigned mode = (p1.flags & 3u) | (p1.true_start ? 4u : 0u);
        if (p1.rope.on) {
            if ((e = launch_gdn_rope<E, ND>(0, mode, args, BH, st)) != hipSuccess) return e;
        } else {
            switch (mode) {
#define GDN_AFF(M) case M: hipLaunchKernelGGL((gdn_frame_affine<E, ND, M>), grid, dim3(L::NT), L::LDS_B, st, p1); break;
                GDN_AFF(0) GDN_AFF(1) GDN_AFF(2) GDN_AFF(3) GDN_AFF(4) GDN_AFF(5) GDN_AFF(6) GDN_AFF(7)
#undef GDN_AFF
            }
        }
    } else if (phase == 1) {
        using L2 = P2<E, ND>;
        hipLaunchKernelGGL((gdn_frame_chain<E, ND>), dim3(L2::grid(BH)), dim3(L2::NT), L2::LDS_B, st,
                           *(const P2Args*)args, BH);
    } else {
        P3Args p3 = *(const P3Args*)args;

        // few frames: split each frame's chunks over several workgroups, up to about three
        // per CU (each part composes S_f itself, mostly from L2).  Measured: 320 frames
        // (the 16-rollout streaming step) run 10% faster in two parts; 420 frames (the 5 s
        // workload) ran 8% slower in two parts, so the count rounds down.
        const long long frames = (long long)p3.nf * BH;
        const int nch = (p3.frame_len + 63) / 64;
        long long parts = 768 / frames;
        if (parts < 1) parts = 1;
        p3.parts = (int)(parts > nch ? nch : parts);
        if (p3.rope.on) {
            if ((e = launch_gdn_rope<E, ND>(2, 0, &p3, BH, st)) != hipSuccess) return e;
        } else {
            hipLaunchKernelGGL((gdn_frame_readout<E, ND, false>), dim3(p3.nf * p3.parts, BH), dim3(256),
                               (P3<E, ND, false>::LDS_B), st, p3);
        }
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    return record(ev, 2 * slot + 1, st);
}

#define GDN_INST(E, ND) template hipError_t launch_gdn_phase<E, ND>(int, const void*, int, hipStream_t, void* const*);
GDN_INST(bf16, 1) GDN_INST(bf16, 2) GDN_INST(bf16, 4) GDN_INST(bf16, 7) GDN_INST(bf16, 8)
GDN_INST(float, 1) GDN_INST(float, 2) GDN_INST(float, 4) GDN_INST(float, 7) GDN_INST(float, 8)


}  // namespace gdn
