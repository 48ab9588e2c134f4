"""GPU parity of the 3D rotary embedding fused into the gated-delta-rule path
(GDN_F_ROPE_QK, through the C ABI): the kernels rotate k as the frame-map pass loads it
and q as the readout loads it (the per-token entry's readout pass rotates both as it
loads them); the oracle rotates q and k first (oracle.rope3d, float64) and then runs the
plain recurrence (oracle.gdn_forward; one-token frames for the per-token readout).  With bf16 inputs the rotated q
and k are bf16 operands, as the stand-alone bf16 rotation pass writes them: the oracle's
rotated tensors are rounded to bf16 (nearest even) before the recurrence -- the rounding
of q alone moves the heavy-tailed outputs (max ~15 RMS) by up to ~3e-2 RMS, so comparing
against unrounded rotations would measure that rounding, not the kernels.  Tolerances as
for the other parity tests: 2e-2 * RMS for bf16 inputs, 1e-4 * RMS for float32 inputs.
The q and k tensors in memory are left unrotated."""
import sys

import numpy as np
import pytest
import torch

import oracle
from linear_attention_video_gated_amd import gdn
from linear_attention_video_gated_amd.inputs import gdn_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = {torch.bfloat16: 2e-2, torch.float32: 1e-4}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def check(name, got, ref, tol):
    got = got.detach().to("cpu", torch.float64).numpy()
    rms = float(np.sqrt(np.mean(ref ** 2)))
    err = float(np.max(np.abs(got - ref)))
    assert np.all(np.isfinite(got)), name
    assert err <= tol * rms, "%s: max|err| %.3e > %.1e * RMS %.3e (ratio %.3e)" % (name, err, tol, rms, err / rms)
    return err / rms


def run(B, H, F, gh, gw, d, dt, dh, dtype, seed, entry="frame", off=0, base=10000.0, plan=None, state=0.2,
        gates="near_one", flags=gdn.NORMALIZE_K):
    N = gh * gw
    say("case rope fused %s B=%d H=%d F=%d grid=%dx%d d=%d split=(%d,%d) off=%d plan=%s %s" %
        (entry, B, H, F, gh, gw, d, dt, dh, off, plan, dtype))
    inp = gdn_inputs(B, H, F, N, d, dtype=dtype, workload_id=seed, gates=gates, state_std=state)
    dv = {k: (v.to(DEV) if v is not None else None) for k, v in inp.items()}
    q0, k0 = dv["q"].clone(), dv["k"].clone()
    rope = {"d_t": dt, "d_h": dh, "grid_w": gw, "frame_offset": off, "base": base}
    additive = bool(flags & gdn.ADDITIVE)
    a_, b_ = (None, None) if additive else (dv["alpha"], dv["beta"])
    if entry == "token":
        out, st = gdn.token_forward(dv["q"], dv["k"], dv["v"], a_, b_, F, N, state_in=dv["state_in"], flags=flags,
                                    out_dtype=torch.float32, rope=rope, plan=plan)
    elif entry == "readonly":
        out = gdn.frame_forward_readonly(dv["q"], dv["k"], dv["v"], a_, b_, F, N, state_in=dv["state_in"],
                                         flags=flags, out_dtype=torch.float32, rope=rope, plan=plan)
        st = None
    else:
        out, st = gdn.frame_forward(dv["q"], dv["k"], dv["v"], a_, b_, F, N, state_in=dv["state_in"], flags=flags,
                                    out_dtype=torch.float32, rope=rope, plan=plan)
    torch.cuda.synchronize()
    assert torch.equal(dv["q"], q0) and torch.equal(dv["k"], k0), "q or k was changed in memory"
    qr = oracle.rope3d(inp["q"], F, gh, gw, dt, dh, frame_offset=off, base=base)
    kr = oracle.rope3d(inp["k"], F, gh, gw, dt, dh, frame_offset=off, base=base)
    if dtype == torch.bfloat16:  # the operands of the bf16 path are bf16 tensors
        qr = torch.from_numpy(qr).to(torch.bfloat16)
        kr = torch.from_numpy(kr).to(torch.bfloat16)
    oflags = (oracle.NORMALIZE_K if flags & gdn.NORMALIZE_K else 0) | (oracle.ADDITIVE if additive else 0)
    fo, no = (F * N, 1) if entry == "token" else (F, N)
    ro, rs = oracle.gdn_forward(qr, kr, inp["v"], inp["alpha"], inp["beta"], fo, no, state_in=inp["state_in"],
                                flags=oflags)
    r1 = check("out", out, ro, TOL[dtype])
    r2 = check("state", st, rs, TOL[dtype]) if st is not None else 0.0
    say("  out err/rms=%.2e state err/rms=%.2e" % (r1, r2))


@pytest.mark.parametrize("entry", ["frame", "readonly", "token"])
@pytest.mark.parametrize("dtype,d,dt,dh", [(torch.bfloat16, 112, 36, 38), (torch.float32, 64, 20, 22),
                                           (torch.float32, 112, 36, 38), (torch.bfloat16, 128, 40, 44),
                                           (torch.bfloat16, 32, 8, 12)])
@pytest.mark.parametrize("plan", [None, {"group_frames": 1}])
def test_rope_fused_ragged(entry, dtype, d, dt, dh, plan):
    """Frames of a 10 x 15 latent grid (150 tokens: two chunks and a 22-token tail), one
    group per call or one frame per group."""
    run(1, 2, 3, 10, 15, d, dt, dh, dtype, seed=1000 + d, entry=entry, plan=plan)


@pytest.mark.parametrize("entry", ["frame", "readonly"])
@pytest.mark.parametrize("dtype,d,dt,dh", [(torch.bfloat16, 112, 36, 38), (torch.float32, 64, 20, 22),
                                           (torch.bfloat16, 128, 40, 44)])
def test_rope_fused_one_frame(entry, dtype, d, dt, dh):
    """One-frame calls (true-start frame maps, readout from the frame-end state)."""
    run(2, 2, 1, 10, 15, d, dt, dh, dtype, seed=1005 + d, entry=entry)


@pytest.mark.parametrize("entry", ["frame", "token"])
def test_rope_fused_720p_grid(entry):
    """The 22 x 40 latent grid of a 720p frame, d = 112 cut (36, 38, 38), several heads."""
    run(1, 4, 3, 22, 40, 112, 36, 38, torch.bfloat16, seed=1010, gates="config", state=None, entry=entry)


@pytest.mark.parametrize("entry", ["frame", "token"])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_rope_fused_late_frames(dtype, entry):
    """Absolute frame positions just below 2^24 (exact float positions), base 100."""
    run(2, 2, 3, 4, 8, 64, 16, 24, dtype, seed=1020, off=(1 << 24) - 3, base=100.0, entry=entry)


@pytest.mark.parametrize("entry", ["frame", "readonly", "token"])
def test_rope_fused_several_windows(entry):
    """Seven frames in windows of two frames (window_units = 4 over B*H = 2; groups of one
    and of two frames), each window's frames rotated at their absolute positions (offset 5)."""
    run(1, 2, 7, 6, 10, 64, 12, 20, torch.float32, seed=1040, entry=entry, off=5,
        plan={"window_units": 4, "group_frames": 1})
    run(1, 2, 7, 6, 10, 112, 36, 38, torch.bfloat16, seed=1041, entry=entry, off=5,
        plan={"window_units": 4, "group_frames": 2})


def test_rope_fused_parts_and_additive():
    """No temporal part, and the additive (block-causal-like) update."""
    run(1, 2, 4, 5, 20, 112, 0, 56, torch.bfloat16, seed=1030)
    run(1, 2, 4, 5, 20, 112, 40, 0, torch.bfloat16, seed=1031, flags=gdn.ADDITIVE | gdn.NORMALIZE_K)


def test_rope_fused_token_parts_and_additive():
    """The per-token entry with no spatial-row part and with the additive update."""
    run(1, 2, 4, 5, 20, 112, 40, 0, torch.bfloat16, seed=1032, entry="token")
    run(1, 2, 4, 5, 20, 64, 0, 32, torch.float32, seed=1033, entry="token", flags=gdn.ADDITIVE | gdn.NORMALIZE_K)
