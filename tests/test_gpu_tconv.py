"""GPU parity of the causal temporal convolution with its block carry
(temporal_conv_block through the C ABI) against the CPU oracle, on the same seeded
inputs.  Float32 arithmetic on both sides of a three-tap sum: the float32 result is
compared at 1e-5 * RMS for bf16 and float32 inputs alike; a bf16 output must be its
round-to-nearest-even bit for bit; the carry out is a copy of the last frame (bitwise)."""
import sys

import numpy as np
import pytest
import torch

import oracle
from linear_attention_video_gated_amd import gdn
from linear_attention_video_gated_amd.inputs import tconv_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def check(got, ref, tol=1e-5):
    got = got.detach().to("cpu", torch.float64).numpy()
    rms = float(np.sqrt(np.mean(ref ** 2))) if ref.size else 0.0
    err = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    assert np.all(np.isfinite(got))
    assert err <= tol * rms + 1e-30, "max|err| %.3e > %.1e * RMS %.3e" % (err, tol, rms)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("shape", [(1, 21, 880, 64), (2, 5, 37, 24), (1, 1, 10, 8), (3, 4, 7, 16)])
@pytest.mark.parametrize("carry", [True, False])
def test_tconv_parity(dtype, shape, carry):
    B, F, P, C = shape
    say("case tconv %s %s carry=%s" % (shape, dtype, carry))
    inp = tconv_inputs(B, F, P, C, dtype=dtype, workload_id=800 + F, carry=carry)
    d = {k: (None if v is None else v.to(DEV)) for k, v in inp.items()}
    y32, c_out = gdn.temporal_conv_block(d["x"], d["w"], d["bias"], carry_in=d["carry_in"], out_dtype=torch.float32)
    y, _ = gdn.temporal_conv_block(d["x"], d["w"], d["bias"], carry_in=d["carry_in"])
    torch.cuda.synchronize()
    ry, rc = oracle.temporal_conv_block(inp["x"], inp["w"], bias=inp["bias"], carry_in=inp["carry_in"])
    check(y32, ry)
    assert torch.equal(y, y32.to(dtype))
    assert torch.equal(c_out, d["x"][:, -1])


def test_tconv_blocks_chain_through_the_carry():
    """Three blocks in a row, each with the previous call's carry, against the oracle run
    the same way; no bias."""
    C, P = 32, 50
    carry_g = carry_r = None
    for i, F in enumerate((3, 1, 5)):
        inp = tconv_inputs(1, F, P, C, dtype=torch.bfloat16, workload_id=820 + i, carry=False)
        x = inp["x"].to(DEV)
        w = tconv_inputs(1, 1, 1, C, dtype=torch.float32, workload_id=830)["w"]
        y, carry_g = gdn.temporal_conv_block(x, w.to(DEV), carry_in=carry_g, out_dtype=torch.float32)
        torch.cuda.synchronize()
        ry, carry_r = oracle.temporal_conv_block(inp["x"], w, carry_in=carry_r)
        check(y, ry)


def test_tconv_empty_block_and_in_place_carry():
    inp = tconv_inputs(2, 4, 9, 16, dtype=torch.bfloat16, workload_id=840)
    x, w, cin = inp["x"].to(DEV), inp["w"].to(DEV), inp["carry_in"].to(DEV)
    # an empty block passes the carry on
    c = torch.empty_like(cin)
    y0, c0 = gdn.temporal_conv_block(x[:, :0].contiguous(), w, carry_in=cin, carry_out=c)
    torch.cuda.synchronize()
    assert y0.shape[1] == 0 and torch.equal(c0, cin)
    # carry_out may be carry_in itself
    ref, _ = gdn.temporal_conv_block(x, w, carry_in=cin.clone(), out_dtype=torch.float32)
    c2 = cin.clone()
    y2, c2o = gdn.temporal_conv_block(x, w, carry_in=c2, carry_out=c2, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(y2, ref) and torch.equal(c2o, x[:, -1])
