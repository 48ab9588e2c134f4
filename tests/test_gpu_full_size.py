"""GPU parity at the benchmarked size, frame-wise and per-token readouts: the 720p 60 s
rollout (B=1, H=20, d=112, 240 frames x 880 tokens = 211,200 tokens, bf16 inputs, float32
state), one call in the launch configuration bench.py times.

The oracle runs on two of the twenty heads for every frame (about 6 s of fp64 work); the
outputs of those heads are compared on a sample of tokens (every 7th) from every frame,
and the state after frames 60, 120 and 240 is compared through segmented calls (state
carried between calls) against the oracle run in the same segments.  Tolerance as in
test_gpu_parity: max |err| <= 2e-2 * RMS(ref) over the compared values.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from linear_attention_video_gated_amd import gdn
from linear_attention_video_gated_amd.inputs import gdn_inputs
from linear_attention_video_gated_amd.workloads import WORKLOADS

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
HEADS = [0, 13]
SEGMENTS = [(0, 60), (60, 120), (120, 240)]


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rel_err(got, ref):
    rms = float(np.sqrt(np.mean(ref ** 2)))
    return float(np.max(np.abs(got - ref))) / max(rms, 1e-300)


@pytest.mark.parametrize("gates", ["config", "near_one"])
def test_gdn_720p_60s_full_size_sampled(gates):
    wl = WORKLOADS["gdn_720p_60s"]
    B, H, F, N, d = wl.B, wl.H, wl.n_frames, wl.frame_len, wl.d
    say("case full-size gdn B=%d H=%d F=%d N=%d d=%d gates=%s" % (B, H, F, N, d, gates))
    inp = gdn_inputs(B, H, F, N, d, dtype=torch.bfloat16, workload_id=wl.wid, device=DEV, gates=gates,
                     state_std=wl.state_std)
    q, k, v, a, b = inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"]
    out, st = gdn.frame_forward(q, k, v, a, b, F, N, state_in=inp["state_in"], out_dtype=torch.float32)
    # the same rollout in three calls, the state carried between them
    seg_states = []
    s = inp["state_in"]
    for f0, f1 in SEGMENTS:
        t0, t1 = f0 * N, f1 * N
        _, s = gdn.frame_forward(q[:, :, t0:t1].contiguous(), k[:, :, t0:t1].contiguous(),
                                 v[:, :, t0:t1].contiguous(), a[:, :, t0:t1].contiguous(),
                                 b[:, :, t0:t1].contiguous(), f1 - f0, N, state_in=s, out_dtype=torch.float32)
        seg_states.append(s)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all() and torch.isfinite(st).all()

    host = lambda x: x[:, HEADS].float().cpu().numpy()
    hq, hk, hv, ha, hb = host(q), host(k), host(v), host(a), host(b)
    s_ref = None if inp["state_in"] is None else host(inp["state_in"])
    sample = np.arange(0, N, 7)
    for (f0, f1), s_gpu in zip(SEGMENTS, seg_states):
        t0, t1 = f0 * N, f1 * N
        ro, s_ref = oracle.gdn_forward(hq[:, :, t0:t1], hk[:, :, t0:t1], hv[:, :, t0:t1], ha[:, :, t0:t1],
                                       hb[:, :, t0:t1], f1 - f0, N, state_in=s_ref, n_threads=2)
        rows = (np.arange(f0, f1)[:, None] * N + sample[None, :]).ravel()
        got = out[:, HEADS][:, :, torch.as_tensor(rows, device=DEV)].double().cpu().numpy()
        ref = ro[:, :, rows - t0]
        e_out = rel_err(got, ref)
        e_seg = rel_err(s_gpu[:, HEADS].double().cpu().numpy(), s_ref)
        say("  frames %d..%d: out err/rms %.2e, state after frame %d err/rms %.2e" % (f0, f1, e_out, f1, e_seg))
        assert e_out <= 2e-2, "out, frames %d..%d" % (f0, f1)
        assert e_seg <= 2e-2, "state after frame %d" % f1
        s_ref = s_ref.astype(np.float32)
    e_fin = rel_err(st[:, HEADS].double().cpu().numpy(), s_ref.astype(np.float64))
    say("  one-call state_out err/rms %.2e" % e_fin)
    assert e_fin <= 2e-2


@pytest.mark.parametrize("gates", ["config", "near_one"])
def test_token_readout_720p_60s_full_size_sampled(gates):
    """gdn_token_forward at the same size: every token reads the state after itself; the
    oracle runs with one-token frames on the same two heads and segments."""
    wl = WORKLOADS["gdn_720p_60s"]
    B, H, F, N, d = wl.B, wl.H, wl.n_frames, wl.frame_len, wl.d
    say("case full-size token B=%d H=%d F=%d N=%d d=%d gates=%s" % (B, H, F, N, d, gates))
    inp = gdn_inputs(B, H, F, N, d, dtype=torch.bfloat16, workload_id=wl.wid, device=DEV, gates=gates,
                     state_std=wl.state_std)
    q, k, v, a, b = inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"]
    out, st = gdn.token_forward(q, k, v, a, b, F, N, state_in=inp["state_in"], out_dtype=torch.float32)
    seg_states = []
    s = inp["state_in"]
    for f0, f1 in SEGMENTS:
        t0, t1 = f0 * N, f1 * N
        _, s = gdn.token_forward(q[:, :, t0:t1].contiguous(), k[:, :, t0:t1].contiguous(),
                                 v[:, :, t0:t1].contiguous(), a[:, :, t0:t1].contiguous(),
                                 b[:, :, t0:t1].contiguous(), f1 - f0, N, state_in=s, out_dtype=torch.float32)
        seg_states.append(s)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all() and torch.isfinite(st).all()
    host = lambda x: x[:, HEADS].float().cpu().numpy()
    hq, hk, hv, ha, hb = host(q), host(k), host(v), host(a), host(b)
    s_ref = None if inp["state_in"] is None else host(inp["state_in"])
    for (f0, f1), s_gpu in zip(SEGMENTS, seg_states):
        t0, t1 = f0 * N, f1 * N
        ro, s_ref = oracle.gdn_forward(hq[:, :, t0:t1], hk[:, :, t0:t1], hv[:, :, t0:t1], ha[:, :, t0:t1],
                                       hb[:, :, t0:t1], t1 - t0, 1, state_in=s_ref, n_threads=2)
        rows = np.arange(t0, t1, 7)
        got = out[:, HEADS][:, :, torch.as_tensor(rows, device=DEV)].double().cpu().numpy()
        ref = ro[:, :, rows - t0]
        e_out = rel_err(got, ref)
        e_seg = rel_err(s_gpu[:, HEADS].double().cpu().numpy(), s_ref)
        say("  frames %d..%d: out err/rms %.2e, state after frame %d err/rms %.2e" % (f0, f1, e_out, f1, e_seg))
        assert e_out <= 2e-2, "out, frames %d..%d" % (f0, f1)
        assert e_seg <= 2e-2, "state after frame %d" % f1
        s_ref = s_ref.astype(np.float32)
    e_fin = rel_err(st[:, HEADS].double().cpu().numpy(), s_ref.astype(np.float64))
    say("  one-call state_out err/rms %.2e" % e_fin)
    assert e_fin <= 2e-2
