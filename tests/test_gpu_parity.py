"""GPU parity: the HIP path (called through the C ABI via the binding) against the CPU
oracle, element by element, on the same seeded inputs.

Tolerances (a comparison fails when max |gpu - ref| > tol * RMS(ref)):
  bf16 inputs: tol = 2e-2 ; float32 inputs: tol = 1e-4.
The same bound is applied to the returned state, against RMS of the reference state.

The computed result is compared in float32 (GDN_F_OUT_F32): a bf16 output adds its own
rounding, up to 2^-9 |o|, and the outputs of these workloads are heavy tailed (products
of near-normal factors, max |o| ~ 15 RMS), so rounding alone can reach 3e-2 RMS.  The
bf16 output is checked separately to be, bit for bit, the round-to-nearest-even of the
float32 result.
"""
import os
import sys

import numpy as np
import pytest
import torch

import oracle
from linear_attention_video_gated_amd import gdn
from linear_attention_video_gated_amd.inputs import block_causal_inputs, gdn_inputs

pytestmark = pytest.mark.gpu

TOL = {torch.bfloat16: 2e-2, torch.float32: 1e-4}
DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def check(name, got, ref, tol):
    got = got.detach().to("cpu", torch.float64).numpy() if hasattr(got, "detach") else np.asarray(got)
    rms = float(np.sqrt(np.mean(ref.astype(np.float64) ** 2)))
    err = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    assert np.all(np.isfinite(got)), name + ": non-finite values"
    assert err <= tol * rms + 1e-30, "%s: max|err| %.3e > %.1e * RMS %.3e (ratio %.3e)" % (name, err, tol, rms, err / max(rms, 1e-300))
    return err / max(rms, 1e-300)


def to_dev(inp):
    return {k: (v.to(DEV) if v is not None else None) for k, v in inp.items()}


def run_gdn_case(B, H, F, N, d, dtype, seed, gates="config", state_std=None, flags=gdn.NORMALIZE_K, plan=None):
    say("case gdn B=%d H=%d F=%d N=%d d=%d %s seed=%d gates=%s state=%s flags=%d plan=%s" %
        (B, H, F, N, d, dtype, seed, gates, state_std, flags, plan))
    inp = gdn_inputs(B, H, F, N, d, dtype=dtype, workload_id=seed, gates=gates, state_std=state_std)
    dv = to_dev(inp)
    additive = bool(flags & gdn.ADDITIVE)
    a_, b_ = (None, None) if additive else (dv["alpha"], dv["beta"])
    out, st = gdn.frame_forward(dv["q"], dv["k"], dv["v"], a_, b_, F, N, state_in=dv["state_in"], flags=flags,
                                out_dtype=torch.float32, plan=plan)
    if dtype == torch.bfloat16:
        ob, sb = gdn.frame_forward(dv["q"], dv["k"], dv["v"], a_, b_, F, N, state_in=dv["state_in"], flags=flags,
                                   plan=plan)
        torch.cuda.synchronize()
        assert torch.equal(ob, out.to(torch.bfloat16)), "bf16 out is not RNE of the float32 result"
        assert torch.equal(sb, st)
    torch.cuda.synchronize()
    oflags = (oracle.NORMALIZE_K if flags & gdn.NORMALIZE_K else 0) | (oracle.ADDITIVE if additive else 0)
    ro, rs = oracle.gdn_forward(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], F, N,
                                state_in=inp["state_in"], flags=oflags)
    r1 = check("out", out, ro, TOL[dtype])
    r2 = check("state", st, rs, TOL[dtype])
    say("  out err/rms=%.2e state err/rms=%.2e" % (r1, r2))
    return inp, dv, out, st


def test_tiny_fp32_workload():
    """B=1, H=2, d=32, 8 frames x 16 tokens, float32 end to end."""
    run_gdn_case(1, 2, 8, 16, 32, torch.float32, seed=0)


@pytest.mark.parametrize("d", [112, 32, 16, 64, 128])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_gdn_ragged_multi_chunk(d, dtype):
    # 150 tokens per frame = 2 full 64-token chunks + a 22-token tail
    run_gdn_case(1, 2, 3, 150, d, dtype, seed=100 + d)


@pytest.mark.parametrize("d", [112, 32, 16, 64, 128])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_gdn_one_frame(d, dtype):
    """One-frame calls (the frame maps pass starts from the known state and writes the
    frame-end state as its map; no chain): a ragged frame (three chunks and a tail), every
    head dimension, bf16 output checked as the RNE of the fp32 one."""
    run_gdn_case(2, 3, 1, 200, d, dtype, seed=150 + d, state_std=0.2, gates="near_one")


@pytest.mark.parametrize("N", [1, 16, 63, 64, 65, 880])
def test_gdn_one_frame_lengths(N):
    """One-frame calls of every length class: shorter than one token tile, one chunk, a
    chunk plus one token, and the 720p frame (14 chunks)."""
    run_gdn_case(2, 2, 1, N, 112, torch.bfloat16, seed=170 + N, state_std=0.1)


def test_gdn_one_frame_additive():
    run_gdn_case(1, 2, 1, 130, 64, torch.float32, seed=190, state_std=0.2,
                 flags=gdn.ADDITIVE | gdn.NORMALIZE_K)


@pytest.mark.parametrize("N", [1, 16, 48, 64, 65, 127, 390, 880])
def test_gdn_frame_lengths_d112(N):
    F = 3 if N >= 390 else 5
    run_gdn_case(1, 3, F, N, 112, torch.bfloat16, seed=200 + N, state_std=0.1)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_gdn_slow_gates_carry_state(dtype):
    """alpha ~ 1: the state carried across frames matters for every output."""
    run_gdn_case(2, 2, 6, 130, 112 if dtype == torch.bfloat16 else 32, dtype, seed=300, gates="near_one",
                 state_std=0.3)


@pytest.mark.parametrize("d,dtype", [(112, torch.bfloat16), (128, torch.bfloat16), (64, torch.bfloat16),
                                     (32, torch.float32), (16, torch.float32)])
def test_gdn_chain_group_counts(d, dtype):
    """The chain over groups at every group count up to 8 (whole runs of its three-group
    prefetch and the tails after them), with (b, h) counts that leave part of its
    eight-way workgroup numbering idle, a carried state in and out, and alpha ~ 1 so that
    every group's map reaches the outputs."""
    for ngw, H in [(1, 3), (2, 3), (3, 9), (4, 1), (5, 9), (6, 3), (7, 11), (8, 2)]:
        run_gdn_case(1, H, ngw, 40, d, dtype, seed=330 + ngw, gates="near_one", state_std=0.2,
                     plan={"group_frames": 1})


@pytest.mark.parametrize("normalize", [True, False])
def test_gdn_additive_reduction(normalize):
    flags = gdn.ADDITIVE | (gdn.NORMALIZE_K if normalize else 0)
    run_gdn_case(1, 2, 4, 100, 112, torch.bfloat16, seed=310, state_std=0.2, flags=flags)


def test_gdn_readonly_matches_forward_and_keeps_state():
    inp, dv, out, st = run_gdn_case(2, 3, 2, 200, 112, torch.bfloat16, seed=320, state_std=0.1)
    s_before = dv["state_in"].clone()
    out_ro = gdn.frame_forward_readonly(dv["q"], dv["k"], dv["v"], dv["alpha"], dv["beta"], 2, 200,
                                        state_in=dv["state_in"], out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(out_ro, out)
    assert torch.equal(dv["state_in"], s_before)


@pytest.mark.parametrize("with_state", [True, False])
def test_gdn_readonly_single_frame(with_state):
    """One frame, read-only: the path that reads state_in directly (no chain launch)."""
    inp = gdn_inputs(3, 2, 1, 300, 112, workload_id=325, state_std=0.3 if with_state else None, gates="near_one")
    dv = to_dev(inp)
    out, st = gdn.frame_forward(dv["q"], dv["k"], dv["v"], dv["alpha"], dv["beta"], 1, 300,
                                state_in=dv["state_in"], out_dtype=torch.float32)
    out_ro = gdn.frame_forward_readonly(dv["q"], dv["k"], dv["v"], dv["alpha"], dv["beta"], 1, 300,
                                        state_in=dv["state_in"], out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(out_ro, out)
    ro, rs = oracle.gdn_forward(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], 1, 300,
                                state_in=inp["state_in"])
    check("out", out_ro, ro, 2e-2)
    check("state", st, rs, 2e-2)


def test_gdn_state_in_place():
    inp = gdn_inputs(1, 2, 3, 70, 112, workload_id=330, state_std=0.2, gates="near_one")
    dv = to_dev(inp)
    s = dv["state_in"].clone()
    out, st = gdn.frame_forward(dv["q"], dv["k"], dv["v"], dv["alpha"], dv["beta"], 3, 70,
                                state_in=s, state_out=s, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ro, rs = oracle.gdn_forward(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], 3, 70,
                                state_in=inp["state_in"])
    check("out", out, ro, 2e-2)
    check("state", s, rs, 2e-2)


def test_gdn_multi_window_equals_single():
    """Frames processed in several windows (state carried through the workspace)."""
    inp = gdn_inputs(1, 2, 7, 90, 112, workload_id=340, state_std=0.2, gates="near_one")
    dv = to_dev(inp)
    o1, s1 = gdn.frame_forward(dv["q"], dv["k"], dv["v"], dv["alpha"], dv["beta"], 7, 90, state_in=dv["state_in"],
                               out_dtype=torch.float32)
    plan = {"window_units": 4}  # 2 frames per window for B*H = 2
    assert gdn.window_count(1, 2, 7, 90, 112, plan=plan) > 1
    o2, s2 = gdn.frame_forward(dv["q"], dv["k"], dv["v"], dv["alpha"], dv["beta"], 7, 90, state_in=dv["state_in"],
                               out_dtype=torch.float32, plan=plan)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
    ro, rs = oracle.gdn_forward(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], 7, 90,
                                state_in=inp["state_in"])
    check("out", o2, ro, 2e-2)
    check("state", s2, rs, 2e-2)


def test_gdn_deterministic_and_workspace_poison_harmless():
    inp = gdn_inputs(1, 4, 3, 200, 112, workload_id=350)
    dv = to_dev(inp)
    o1, s1 = gdn.frame_forward(dv["q"], dv["k"], dv["v"], dv["alpha"], dv["beta"], 3, 200)
    for buf in gdn._ws_cache.values():
        buf.view(torch.float32).fill_(float("nan"))
    o2, s2 = gdn.frame_forward(dv["q"], dv["k"], dv["v"], dv["alpha"], dv["beta"], 3, 200)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


def test_gdn_zero_frames_copies_state():
    s_in = torch.randn(1, 2, 32, 32, device=DEV)
    q = torch.empty(1, 2, 0, 32, device=DEV, dtype=torch.bfloat16)
    out, st = gdn.frame_forward(q, q.clone(), q.clone(), torch.empty(1, 2, 0, device=DEV),
                                torch.empty(1, 2, 0, device=DEV), 0, 16, state_in=s_in)
    torch.cuda.synchronize()
    assert torch.equal(st, s_in)


# ---------------------------------------------------------------- block-causal
def run_bc_case(B, H, F, N, d, dtype, seed, state_std=None):
    say("case block_causal B=%d H=%d F=%d N=%d d=%d %s seed=%d state=%s" % (B, H, F, N, d, dtype, seed, state_std))
    inp = block_causal_inputs(B, H, F, N, d, dtype=dtype, workload_id=seed, state_std=state_std)
    dv = to_dev(inp)
    out, st, z = gdn.linear_attn_block_causal(dv["q"], dv["k"], dv["v"], F, N, state_in=dv["state_in"],
                                              z_in=dv["z_in"], out_dtype=torch.float32)
    if dtype == torch.bfloat16:
        ob, _, _ = gdn.linear_attn_block_causal(dv["q"], dv["k"], dv["v"], F, N, state_in=dv["state_in"],
                                                z_in=dv["z_in"])
        torch.cuda.synchronize()
        assert torch.equal(ob, out.to(torch.bfloat16)), "bf16 out is not RNE of the float32 result"
    torch.cuda.synchronize()
    ro, rs, rz = oracle.linear_attn_block_causal(inp["q"], inp["k"], inp["v"], F, N,
                                                 state_in=inp["state_in"], z_in=inp["z_in"])
    tol = TOL[dtype]
    r1 = check("out", out, ro, tol)
    r2 = check("state", st, rs, tol)
    r3 = check("z", z, rz, tol)
    say("  out %.2e state %.2e z %.2e" % (r1, r2, r3))


@pytest.mark.parametrize("d", [112, 32, 128])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_block_causal_small(d, dtype):
    run_bc_case(1, 2, 4, 70, d, dtype, seed=400 + d)


def test_block_causal_with_state_and_ragged():
    run_bc_case(2, 2, 3, 33, 112, torch.bfloat16, seed=410, state_std=0.5)


def test_block_causal_480p_workload():
    """B=1, H=20, d=112, 21 frames x 390 tokens, bf16: the full 480p-shaped workload."""
    run_bc_case(1, 20, 21, 390, 112, torch.bfloat16, seed=1)


def test_block_causal_multi_window():
    inp = block_causal_inputs(1, 2, 5, 40, 112, workload_id=420, state_std=0.5)
    dv = to_dev(inp)
    o1, s1, z1 = gdn.linear_attn_block_causal(dv["q"], dv["k"], dv["v"], 5, 40, state_in=dv["state_in"], z_in=dv["z_in"])
    o2, s2, z2 = gdn.linear_attn_block_causal(dv["q"], dv["k"], dv["v"], 5, 40, state_in=dv["state_in"], z_in=dv["z_in"],
                                              plan={"window_units": 4})
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2) and torch.equal(z1, z2)


@pytest.mark.parametrize("entry", ["frame", "token"])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_gdn_gate_logits(entry, dtype):
    """GDN_F_GATE_LOGITS: alpha and beta hold logits; the oracle forms the gates in float64."""
    F, N, d = 3, 150, 112 if dtype == torch.bfloat16 else 64
    say("case gate logits entry=%s %s" % (entry, dtype))
    inp = gdn_inputs(1, 2, F, N, d, dtype=dtype, workload_id=360, state_std=0.2)
    g = torch.Generator().manual_seed(360)
    a = (2.0 * torch.randn(1, 2, F * N, generator=g)).contiguous()
    b = (2.0 * torch.randn(1, 2, F * N, generator=g)).contiguous()
    # alpha ~ 1 and a near reset (alpha = e^-8 per token for 20 tokens).  Harder resets
    # inside one 64-token chunk push the chunk's log-gate prefix G past ~500 in magnitude,
    # where fp32 differences G_t - G_i keep ~1e-4 absolute precision: the float32 bound
    # of 1e-4 is then no longer met (bf16 inputs are unaffected).
    a[0, 0, :20] = -30.0
    a[0, 1, :20] = 8.0
    dv = to_dev(inp)
    fn = gdn.token_forward if entry == "token" else gdn.frame_forward
    out, st = fn(dv["q"], dv["k"], dv["v"], a.to(DEV), b.to(DEV), F, N, state_in=dv["state_in"],
                 flags=gdn.NORMALIZE_K | gdn.GATE_LOGITS, out_dtype=torch.float32)
    torch.cuda.synchronize()
    nf, fl = (F * N, 1) if entry == "token" else (F, N)
    ro, rs = oracle.gdn_forward(inp["q"], inp["k"], inp["v"], a, b, nf, fl, state_in=inp["state_in"],
                                flags=oracle.NORMALIZE_K | oracle.GATE_LOGITS)
    r1 = check("out", out, ro, TOL[dtype])
    r2 = check("state", st, rs, TOL[dtype])
    say("  out err/rms=%.2e state err/rms=%.2e" % (r1, r2))


@pytest.mark.parametrize("entry", ["frame", "readonly", "token"])
@pytest.mark.parametrize("group", ["1", "4000"])
@pytest.mark.parametrize("d,dtype", [(112, torch.bfloat16), (16, torch.bfloat16), (32, torch.bfloat16),
                                     (64, torch.bfloat16), (128, torch.bfloat16), (16, torch.float32),
                                     (32, torch.float32), (64, torch.float32), (128, torch.float32)])
def test_gdn_group_paths(entry, group, d, dtype):
    """Both organisations of a call: one frame per group (maps, chain over groups, readout)
    and a single group per (b, h) (maps from the known start state, no chain)."""
    plan = {"group_frames": int(group)}
    F, N = 5, 100
    inp = gdn_inputs(2, 2, F, N, d, dtype=dtype, workload_id=370, state_std=0.2, gates="near_one")
    dv = to_dev(inp)
    say("case groups=%s entry=%s" % (group, entry))
    s = dv["state_in"].clone()
    if entry == "readonly":
        out = gdn.frame_forward_readonly(dv["q"], dv["k"], dv["v"], dv["alpha"], dv["beta"], F, N, state_in=s,
                                         out_dtype=torch.float32, plan=plan)
        st = None
    else:
        fn = gdn.token_forward if entry == "token" else gdn.frame_forward
        out, st = fn(dv["q"], dv["k"], dv["v"], dv["alpha"], dv["beta"], F, N, state_in=s, state_out=s,
                     out_dtype=torch.float32, plan=plan)  # state updated in place
    torch.cuda.synchronize()
    nf, fl = (F * N, 1) if entry == "token" else (F, N)
    ro, rs = oracle.gdn_forward(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], nf, fl,
                                state_in=inp["state_in"])
    check("out", out, ro, TOL[dtype])
    if st is not None:
        check("state", s, rs, TOL[dtype])
    else:
        assert torch.equal(s, dv["state_in"]), "read-only call wrote the state"


def test_gdn_many_heads_several_windows():
    """B*H = 1600 (b, h) pairs: the 8192-unit windows hold whole groups of frames, so a call
    of 12 frames runs several windows; the oracle checks a sample of the heads."""
    B, H, F, N, d = 80, 20, 12, 64, 112
    inp = gdn_inputs(B, H, F, N, d, workload_id=380, state_std=0.1, gates="near_one")
    dv = to_dev(inp)
    assert gdn.window_count(B, H, F, N, d) > 1
    out, st = gdn.frame_forward(dv["q"], dv["k"], dv["v"], dv["alpha"], dv["beta"], F, N, state_in=dv["state_in"],
                                out_dtype=torch.float32)
    torch.cuda.synchronize()
    bsel, hsel = [0, 37, 79], [0, 11, 19]
    sub = lambda x: None if x is None else x[bsel][:, hsel].contiguous()
    ro, rs = oracle.gdn_forward(sub(inp["q"]), sub(inp["k"]), sub(inp["v"]), sub(inp["alpha"]), sub(inp["beta"]),
                                F, N, state_in=sub(inp["state_in"]))
    check("out", out[bsel][:, hsel], ro, 2e-2)
    check("state", st[bsel][:, hsel], rs, 2e-2)
