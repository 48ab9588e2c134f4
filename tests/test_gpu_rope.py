"""GPU parity of the 3D rotary position embedding (rope3d_apply through the C ABI, in place)
against the CPU oracle on the same inputs.  Float32 angles and rotation: float32 inputs
at 1e-5 * RMS; bf16 inputs round the result to bf16: half an ulp of the largest
outputs (|y| in [4, 8) among millions of N(0,1) values) is 2^-6, so the bar is the
library's bf16 one, 2e-2 * RMS."""
import sys

import numpy as np
import pytest
import torch

import oracle
from linear_attention_video_gated_amd import gdn

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = {torch.bfloat16: 2e-2, torch.float32: 1e-5}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("case", [
    (1, 2, 3, 4, 5, 16, 4, 6, 0),       # parts not aligned with the 16-byte groups
    (1, 20, 21, 22, 40, 112, 36, 38, 0),  # the 720p latent grid, d = 112
    (2, 3, 2, 3, 7, 64, 0, 32, 1000),     # no temporal part; late frames
    (1, 1, 5, 1, 1, 8, 8, 0, 3),          # temporal part only
    (1, 2, 3, 2, 3, 16, 4, 6, (1 << 24) - 3),  # frames up to the largest exact float position
])
def test_rope3d_parity(dtype, case):
    B, H, F, gh, gw, d, dt, dh, off = case
    say("case rope3d %s %s" % (case, dtype))
    g = torch.Generator().manual_seed(900 + d)
    x = torch.randn((B, H, F * gh * gw, d), generator=g).to(dtype)
    xd = x.to(DEV)
    gdn.rope3d_apply(xd, F, gh, gw, dt, dh, frame_offset=off)
    torch.cuda.synchronize()
    ref = oracle.rope3d(x, F, gh, gw, dt, dh, frame_offset=off)
    got = xd.double().cpu().numpy()
    rms = float(np.sqrt((ref ** 2).mean()))
    err = float(np.abs(got - ref).max())
    assert err <= TOL[dtype] * rms, (err, rms)


def test_rope3d_wide_index():
    """A tensor of more than 2^31 16-byte groups (34 GB of bf16), which the pass walks
    with 64-bit indices: frames at its start, middle and end against the oracle."""
    B, H, gh, gw, d, dt, dh = 1, 1, 64, 64, 128, 40, 44
    F = 32800  # 32800 * 4096 tokens * 16 groups > 2^31
    say("case rope3d wide index F=%d grid=%dx%d d=%d" % (F, gh, gw, d))
    g = torch.Generator(device=DEV).manual_seed(950)
    x = torch.randn((B, H, F * gh * gw, d), generator=g, device=DEV, dtype=torch.bfloat16)
    N = gh * gw
    frames = [0, 16001, 32767, F - 1]
    before = {f: x[:, :, f * N:(f + 1) * N].cpu() for f in frames}
    gdn.rope3d_apply(x, F, gh, gw, dt, dh)
    torch.cuda.synchronize()
    for f in frames:
        got = x[:, :, f * N:(f + 1) * N].double().cpu().numpy()
        ref = oracle.rope3d(before[f], 1, gh, gw, dt, dh, frame_offset=f)
        rms = float(np.sqrt((ref ** 2).mean()))
        err = float(np.abs(got - ref).max())
        assert err <= TOL[torch.bfloat16] * rms, (f, err, rms)
    del x
    torch.cuda.empty_cache()
