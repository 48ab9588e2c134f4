"""gdn_frame_forward_noalloc, the allocation-free variant of gdn_frame_forward (static
device scratch instead of a caller workspace), through the C ABI: two calls in a row, the
second smaller, each equal bit for bit to gdn_frame_forward on the same inputs and within
the parity bound of the oracle; a float32 call; a call cut into several windows (the
state carried through the shared scratch)."""
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
    assert err <= tol * rms, "%s: max|err| %.3e > %.1e * RMS %.3e" % (name, err, tol, rms)


def one_case(B, H, F, N, d, dtype, seed, plan=None):
    say("case noalloc B=%d H=%d F=%d N=%d d=%d %s plan=%s" % (B, H, F, N, d, dtype, plan))
    inp = gdn_inputs(B, H, F, N, d, dtype=dtype, workload_id=seed, state_std=0.2, gates="near_one")
    dv = {k: (v.to(DEV) if v is not None else None) for k, v in inp.items()}
    need = gdn.workspace_bytes(B, H, F, N, d, dtype=dtype, plan=plan)
    assert 0 < need <= gdn.lib().gdn_noalloc_scratch_bytes()
    ref_o, ref_s = gdn.frame_forward(dv["q"], dv["k"], dv["v"], dv["alpha"], dv["beta"], F, N,
                                     state_in=dv["state_in"], out_dtype=torch.float32, plan=plan)
    out = torch.empty(dv["q"].shape, dtype=torch.float32, device=DEV)
    st = torch.empty_like(ref_s)
    gdn.frame_forward_noalloc(dv["q"], dv["k"], dv["v"], dv["alpha"], dv["beta"], F, N, out,
                              state_in=dv["state_in"], state_out=st, plan=plan)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_o) and torch.equal(st, ref_s)
    ro, rs = oracle.gdn_forward(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], F, N,
                                state_in=inp["state_in"])
    check("out", out, ro, TOL[dtype])
    check("state", st, rs, TOL[dtype])


def test_noalloc_two_calls_second_smaller():
    one_case(2, 4, 5, 150, 112, torch.bfloat16, seed=800)
    one_case(1, 2, 3, 70, 112, torch.bfloat16, seed=801)


def test_noalloc_float32_and_windows():
    one_case(1, 2, 4, 90, 64, torch.float32, seed=802)
    one_case(1, 2, 7, 90, 112, torch.bfloat16, seed=803, plan={"window_units": 4})
