"""GPU parity of frame-block-causal softmax attention (softmax_attn_block_causal through the
C ABI) against the CPU oracle, element by element on the same seeded inputs.

Tolerance as for the other entries: max |gpu - ref| <= tol * RMS(ref), tol = 2e-2 for bf16
inputs (the probabilities enter the product with V rounded to bf16, 2^-9 relative), 1e-4
for float32 inputs.  The float32 result (GDN_F_OUT_F32) is compared; a bf16 output must be
its round-to-nearest-even bit for bit.

Shapes cover: several 128-query tiles with a ragged last one (whole waves past the end),
frames that do not line up with the 64-key blocks, one-token frames (token-causal
attention), a single frame (no mask), cached earlier frames (kv_frames > n_frames), every
supported head dimension in both dtypes, and the 720p 5 s shape (21 frames x 880 tokens,
20 heads, d = 112) on sampled frames.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from linear_attention_video_gated_amd import gdn
from linear_attention_video_gated_amd.inputs import softmax_inputs

pytestmark = pytest.mark.gpu

TOL = {torch.bfloat16: 2e-2, torch.float32: 1e-4}
DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def check(name, got, ref, tol):
    got = got.detach().to("cpu", torch.float64).numpy()
    rms = float(np.sqrt(np.mean(ref ** 2)))
    err = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    assert np.all(np.isfinite(got)), name + ": non-finite values"
    assert err <= tol * rms + 1e-30, "%s: max|err| %.3e > %.1e * RMS %.3e" % (name, err, tol, rms)
    return err / max(rms, 1e-300)


def run_case(B, H, F, KF, N, d, dtype, seed, qscale=1.0):
    say("case softmax B=%d H=%d F=%d KF=%d N=%d d=%d %s seed=%d qscale=%g" % (B, H, F, KF, N, d, dtype, seed, qscale))
    inp = softmax_inputs(B, H, F, KF, N, d, dtype=dtype, workload_id=seed)
    if qscale != 1.0:
        inp["q"] = (inp["q"].float() * qscale).to(dtype)
    q, k, v = (inp[n].to(DEV) for n in ("q", "k", "v"))
    o32 = gdn.softmax_attn_block_causal(q, k, v, F, KF, N, out_dtype=torch.float32)
    ob = gdn.softmax_attn_block_causal(q, k, v, F, KF, N)
    torch.cuda.synchronize()
    ref = oracle.softmax_attn_block_causal(inp["q"], inp["k"], inp["v"], F, KF, N)
    r = check("out", o32, ref, TOL[dtype])
    assert torch.equal(ob, o32.to(dtype)), "the dtype output is not the rounded float32 result"
    return r


SHAPES = [  # (B, H, F, KF, N)
    (1, 2, 3, 3, 50),     # 150 queries: two tiles, the second with three waves past the end
    (2, 3, 2, 5, 70),     # three cached frames; frame ends inside key blocks
    (1, 2, 1, 1, 300),    # one frame: no mask
    (1, 1, 200, 200, 1),  # one-token frames: token-causal attention
    (1, 2, 4, 4, 128),    # frames of two whole key blocks
    (1, 1, 1, 9, 33),     # one new frame against eight cached ones
]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_softmax_parity_d112(shape, dtype):
    B, H, F, KF, N = shape
    run_case(B, H, F, KF, N, 112, dtype, seed=700 + F * 10 + KF)


@pytest.mark.parametrize("d", [16, 32, 64, 128])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_softmax_parity_head_dims(d, dtype):
    run_case(1, 2, 3, 4, 45, d, dtype, seed=710 + d)


def test_softmax_sharp_logits():
    """q scaled by 6: logits of standard deviation 6, weights spread over many orders of
    magnitude (the running maximum and its corrections do the work)."""
    run_case(1, 2, 3, 3, 100, 112, torch.bfloat16, seed=720, qscale=6.0)
    run_case(1, 2, 3, 3, 100, 112, torch.float32, seed=721, qscale=6.0)


def test_softmax_deterministic():
    inp = softmax_inputs(1, 2, 3, 4, 90, 112, dtype=torch.bfloat16, workload_id=730)
    q, k, v = (inp[n].to(DEV) for n in ("q", "k", "v"))
    a = gdn.softmax_attn_block_causal(q, k, v, 3, 4, 90, out_dtype=torch.float32)
    b = gdn.softmax_attn_block_causal(q, k, v, 3, 4, 90, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_softmax_cached_frames_equal_rows_of_full_call():
    """Queries of the last frames against cached earlier frames give the same rows as one
    call over all frames (to float32 rounding: the query tiles start elsewhere)."""
    KF, N = 5, 96
    inp = softmax_inputs(1, 2, KF, KF, N, 112, dtype=torch.bfloat16, workload_id=740)
    q, k, v = (inp[n].to(DEV) for n in ("q", "k", "v"))
    full = gdn.softmax_attn_block_causal(q, k, v, KF, KF, N, out_dtype=torch.float32)
    for F in (1, 2, 4):
        part = gdn.softmax_attn_block_causal(q[:, :, (KF - F) * N:].contiguous(), k, v, F, KF, N,
                                             out_dtype=torch.float32)
        torch.cuda.synchronize()
        d = (part - full[:, :, (KF - F) * N:]).abs().max().item()
        assert d <= 1e-6 * full.abs().max().item(), (F, d)


def test_softmax_720p_5s_sampled_frames():
    """The 720p 5 s shape (B=1, H=20, 21 frames x 880 tokens, d=112, bf16): the whole call
    runs as benchmarked; frames 0, 10 and 20 of heads 0 and 19 are checked against the
    oracle (each frame's queries against the frames up to it)."""
    F, N, H = 21, 880, 20
    say("case softmax 720p 5s sampled")
    inp = softmax_inputs(1, H, F, F, N, 112, dtype=torch.bfloat16, workload_id=6)
    q, k, v = (inp[n].to(DEV) for n in ("q", "k", "v"))
    out = gdn.softmax_attn_block_causal(q, k, v, F, F, N, out_dtype=torch.float32)
    torch.cuda.synchronize()
    for h in (0, 19):
        for f in (0, 10, 20):
            sl = slice(f * N, (f + 1) * N)
            ref = oracle.softmax_attn_block_causal(inp["q"][:, h:h + 1, sl], inp["k"][:, h:h + 1, :(f + 1) * N],
                                                   inp["v"][:, h:h + 1, :(f + 1) * N], 1, f + 1, N)
            check("h%d f%d" % (h, f), out[:, h:h + 1, sl], ref, TOL[torch.bfloat16])


def test_softmax_empty_calls():
    q = torch.empty((1, 2, 0, 112), dtype=torch.bfloat16, device=DEV)
    k = torch.randn((1, 2, 3 * 16, 112), device=DEV).to(torch.bfloat16)
    out = gdn.softmax_attn_block_causal(q, k, k.clone(), 0, 3, 16)
    torch.cuda.synchronize()
    assert out.shape == q.shape


def test_softmax_many_heads_tiny_frames():
    """A 1-D grid of (query tile, head) pairs with many heads: 1000 heads of 3 frames x 5
    tokens (one partial tile each); sampled heads against the oracle."""
    B, H, F, N = 2, 500, 3, 5
    say("case softmax many heads B=%d H=%d" % (B, H))
    inp = softmax_inputs(B, H, F, F, N, 32, dtype=torch.bfloat16, workload_id=750)
    q, k, v = (inp[n].to(DEV) for n in ("q", "k", "v"))
    out = gdn.softmax_attn_block_causal(q, k, v, F, F, N, out_dtype=torch.float32)
    torch.cuda.synchronize()
    for b, h in ((0, 0), (0, 499), (1, 250), (1, 499)):
        ref = oracle.softmax_attn_block_causal(inp["q"][b:b + 1, h:h + 1], inp["k"][b:b + 1, h:h + 1],
                                               inp["v"][b:b + 1, h:h + 1], F, F, N)
        check("b%d h%d" % (b, h), out[b:b + 1, h:h + 1], ref, TOL[torch.bfloat16])


def test_softmax_long_cache_one_frame():
    """One new frame of 100 tokens against 39 cached ones: a long key stream whose end is
    not a multiple of the 64-key block, in both dtypes."""
    for dtype in (torch.bfloat16, torch.float32):
        run_case(1, 2, 1, 40, 100, 112, dtype, seed=760)


def test_softmax_batch_and_ragged_tiles():
    """B = 3 with 5 frames of 77 tokens: query tiles straddle frames and end mid-tile."""
    run_case(3, 2, 5, 5, 77, 64, torch.bfloat16, seed=770)
