// gdn_frame_rope.hip -- the frame-wise gated-delta-rule kernels that rotate q and k by the
// 3D rotary embedding as they load them (GDN_F_ROPE_QK; the rotation is the axial one of
// rope3d_apply, from the "SANA-Video" talk's segment on temporal modelling), instantiated
// in a translation unit of their own so that they compile beside gdn_frame.hip.  Called by
// launch_gdn_phase with the arguments it has already prepared.
#include "gdn_frame.hpp"

namespace gdn {

// phase 0: frame maps (P1Args) in mode `mode` (normalise, additive, true start); phase 2:
// frame-end readout (P3Args, parts already set); phase 3: per-token readout pass (P1Args,
// mode = normalise, additive).  Sets the kernels' LDS attributes once per device.
template <typename E, int ND>
hipError_t launch_gdn_rope(int phase, unsigned mode, const void* args, int BH, hipStream_t st) {
    using LR = P1<E, ND, false, true>;
    using LT = P1<E, ND, true, true>;
    static PerDeviceOnce attr;  // per instantiation
    hipError_t e = attr.run([] {
        const void* aff[8] = {(const void*)gdn_frame_affine<E, ND, 8>, (const void*)gdn_frame_affine<E, ND, 9>,
                              (const void*)gdn_frame_affine<E, ND, 10>, (const void*)gdn_frame_affine<E, ND, 11>,
                              (const void*)gdn_frame_affine<E, ND, 12>, (const void*)gdn_frame_affine<E, ND, 13>,
                              (const void*)gdn_frame_affine<E, ND, 14>, (const void*)gdn_frame_affine<E, ND, 15>};
        const void* tok[4] = {(const void*)gdn_token_readout<E, ND, 8>, (const void*)gdn_token_readout<E, ND, 9>,
                              (const void*)gdn_token_readout<E, ND, 10>, (const void*)gdn_token_readout<E, ND, 11>};
        hipError_t r = hipSuccess;
        for (const void* f : aff)
            if ((r = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, LR::LDS_B)) != hipSuccess)
                return r;
        for (const void* f : tok)
            if ((r = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, LT::LDS_B)) != hipSuccess)
                return r;
        return hipFuncSetAttribute((const void*)gdn_frame_readout<E, ND, true>,
                                   hipFuncAttributeMaxDynamicSharedMemorySize, P3<E, ND, true>::LDS_B);
    });
    if (e != hipSuccess) return e;
    if (phase == 0) {
        const P1Args& p1 = *(const P1Args*)args;
        const dim3 grid((p1.nf + p1.G - 1) / p1.G, BH);
        switch (mode) {
#define GDN_AFF(M) case M: hipLaunchKernelGGL((gdn_frame_affine<E, ND, 8 + M>), grid, dim3(LR::NT), LR::LDS_B, st, p1); break;
            GDN_AFF(0) GDN_AFF(1) GDN_AFF(2) GDN_AFF(3) GDN_AFF(4) GDN_AFF(5) GDN_AFF(6) GDN_AFF(7)
#undef GDN_AFF
            default: return hipErrorInvalidValue;
        }
    } else if (phase == 3) {
        const P1Args& p1 = *(const P1Args*)args;
        const dim3 grid((p1.nf + p1.G - 1) / p1.G, BH);
        switch (mode) {
#define GDN_TOK(M) case M: hipLaunchKernelGGL((gdn_token_readout<E, ND, 8 + M>), grid, dim3(LT::NT), LT::LDS_B, st, p1); break;
            GDN_TOK(0) GDN_TOK(1) GDN_TOK(2) GDN_TOK(3)
#undef GDN_TOK
            default: return hipErrorInvalidValue;
        }
    } else {
        const P3Args& p3 = *(const P3Args*)args;
        hipLaunchKernelGGL((gdn_frame_readout<E, ND, true>), dim3(p3.nf * p3.parts, BH), dim3(256),
                           (P3<E, ND, true>::LDS_B), st, p3);
    }
    return hipGetLastError();
}

#define RP_INST(E, ND) template hipError_t launch_gdn_rope<E, ND>(int, unsigned, const void*, int, hipStream_t);
RP_INST(bf16, 1) RP_INST(bf16, 2) RP_INST(bf16, 4) RP_INST(bf16, 7) RP_INST(bf16, 8)
RP_INST(float, 1) RP_INST(float, 2) RP_INST(float, 4) RP_INST(float, 7) RP_INST(float, 8)
#undef RP_INST

}  // namespace gdn
