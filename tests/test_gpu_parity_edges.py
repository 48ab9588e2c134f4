"""GPU parity at the edges the other parity files do not reach, through the C ABI:

- raw (not normalised) keys, so the kernels' own key normalisation (GDN_F_NORMALIZE_K)
  is observed, and unnormalised short keys with the flag off;
- hard gates: runs of alpha = 0 (the FLT_MIN clamp) at a chunk start and in mid-chunk,
  and gate logits of +60 (alpha = e^-60) and -30 (alpha ~ 1) inside one chunk, for
  float32 inputs at the float32 bound;
- the exact shapes of the 720p 5 s rollout (B=1, H=20, 21 x 880 tokens) and of the
  16-rollout streaming step (B=16, H=20, one 880-token frame, state_in std 0.1, several
  read-only calls and the commit);
- the readout's split of a frame's chunks over several workgroups where the number of
  parts does not divide the chunk count (one part has no chunks);
- two calls on two streams at once.

Tolerances as in test_gpu_parity.py: max |gpu - ref| <= tol * RMS(ref), tol 2e-2 for
bf16 inputs and 1e-4 for float32 inputs, on the float32 result (GDN_F_OUT_F32).
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from linear_attention_video_gated_amd import gdn
from linear_attention_video_gated_amd.inputs import gdn_inputs

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
    assert err <= tol * rms + 1e-30, "%s: max|err| %.3e > %.1e * RMS %.3e (ratio %.3e)" % (
        name, err, tol, rms, err / max(rms, 1e-300))
    return err / max(rms, 1e-300)


def to_dev(inp):
    return {k: (v.to(DEV) if v is not None else None) for k, v in inp.items()}


def run_entry(entry, dv, F, N, flags, alpha=None, beta=None):
    """One call of `entry` on device inputs; returns (out float32, state or None, state_in
    after the call)."""
    a = dv["alpha"] if alpha is None else alpha
    b = dv["beta"] if beta is None else beta
    s = None if dv["state_in"] is None else dv["state_in"].clone()
    if entry == "readonly":
        out = gdn.frame_forward_readonly(dv["q"], dv["k"], dv["v"], a, b, F, N, state_in=s, flags=flags,
                                         out_dtype=torch.float32)
        st = None
    else:
        fn = gdn.token_forward if entry == "token" else gdn.frame_forward
        out, st = fn(dv["q"], dv["k"], dv["v"], a, b, F, N, state_in=s, flags=flags, out_dtype=torch.float32)
    torch.cuda.synchronize()
    return out, st, s


def oracle_entry(entry, inp, F, N, oflags, alpha=None, beta=None):
    a = inp["alpha"] if alpha is None else alpha
    b = inp["beta"] if beta is None else beta
    nf, fl = (F * N, 1) if entry == "token" else (F, N)
    return oracle.gdn_forward(inp["q"], inp["k"], inp["v"], a, b, nf, fl, state_in=inp["state_in"], flags=oflags)


def compare(entry, dtype, out, st, s_after, inp, ro, rs):
    r1 = check("out", out, ro, TOL[dtype])
    r2 = check("state", st, rs, TOL[dtype]) if st is not None else 0.0
    if entry == "readonly" and inp["state_in"] is not None:
        assert torch.equal(s_after.cpu(), inp["state_in"]), "read-only call wrote the state"
    say("  out err/rms=%.2e state err/rms=%.2e" % (r1, r2))


ENTRIES = ["frame", "readonly", "token"]
DTYPES = [(torch.bfloat16, 112), (torch.float32, 64), (torch.float32, 112)]


# ---------------------------------------------------------------- key normalisation
@pytest.mark.parametrize("entry", ENTRIES)
@pytest.mark.parametrize("dtype,d", DTYPES)
def test_raw_keys_normalised_in_kernel(entry, dtype, d):
    """k ~ N(0,1) scaled per token by 10^U(-2,2) (norms from ~0.1 to ~1000), normalised by
    the kernels; 3 frames of 150 tokens (two chunks and a 22-token tail)."""
    F, N = 3, 150
    say("case raw keys entry=%s %s d=%d" % (entry, dtype, d))
    inp = gdn_inputs(1, 2, F, N, d, dtype=dtype, workload_id=700 + d, gates="near_one", state_std=0.2, keys="raw")
    out, st, s = run_entry(entry, to_dev(inp), F, N, gdn.NORMALIZE_K)
    ro, rs = oracle_entry(entry, inp, F, N, oracle.NORMALIZE_K)
    compare(entry, dtype, out, st, s, inp, ro, rs)


@pytest.mark.parametrize("entry", ENTRIES)
@pytest.mark.parametrize("dtype,d", DTYPES)
def test_short_keys_without_normalisation(entry, dtype, d):
    """Unnormalised keys of norm 0.03 .. 1 with GDN_F_NORMALIZE_K off: the update uses k as
    given (a kernel that normalised anyway would be off by up to 30x)."""
    F, N = 3, 150
    say("case short keys, no normalisation, entry=%s %s d=%d" % (entry, dtype, d))
    inp = gdn_inputs(1, 2, F, N, d, dtype=dtype, workload_id=710 + d, gates="near_one", state_std=0.2,
                     keys="short")
    out, st, s = run_entry(entry, to_dev(inp), F, N, 0)
    ro, rs = oracle_entry(entry, inp, F, N, 0)
    compare(entry, dtype, out, st, s, inp, ro, rs)


@pytest.mark.parametrize("normalize", [True, False])
@pytest.mark.parametrize("dtype,d", DTYPES)
def test_additive_with_unnormalised_keys(normalize, dtype, d):
    """GDN_F_ADDITIVE (S += v k^T) with keys that are not unit vectors, with and without
    the normalisation flag."""
    F, N = 4, 100
    flags = gdn.ADDITIVE | (gdn.NORMALIZE_K if normalize else 0)
    say("case additive normalize=%s %s d=%d" % (normalize, dtype, d))
    inp = gdn_inputs(1, 2, F, N, d, dtype=dtype, workload_id=720 + d, state_std=0.2,
                     keys="raw" if normalize else "short")
    dv = to_dev(inp)
    out, st = gdn.frame_forward(dv["q"], dv["k"], dv["v"], None, None, F, N, state_in=dv["state_in"], flags=flags,
                                out_dtype=torch.float32)
    torch.cuda.synchronize()
    oflags = oracle.ADDITIVE | (oracle.NORMALIZE_K if normalize else 0)
    ro, rs = oracle.gdn_forward(inp["q"], inp["k"], inp["v"], None, None, F, N, state_in=inp["state_in"],
                                flags=oflags)
    check("out", out, ro, TOL[dtype])
    check("state", st, rs, TOL[dtype])


# ---------------------------------------------------------------- hard gates
@pytest.mark.parametrize("entry", ENTRIES)
@pytest.mark.parametrize("dtype,d", DTYPES)
def test_alpha_zero_runs(entry, dtype, d):
    """alpha = 0 (clamped to FLT_MIN: log2 = -126 per token) for runs of 20 tokens at the
    start of a frame's first chunk and 16 tokens in the middle of a chunk, plus isolated
    zeros, among slow gates (alpha ~ 1) that carry the state everywhere else."""
    F, N = 3, 150
    say("case alpha = 0 runs entry=%s %s d=%d" % (entry, dtype, d))
    inp = gdn_inputs(1, 2, F, N, d, dtype=dtype, workload_id=730 + d, gates="near_one", state_std=0.3)
    a = inp["alpha"].clone()
    a[:, :, 150:170] = 0.0           # frame 1, first chunk: its start
    a[:, :, 94:110] = 0.0            # frame 0, second chunk: tokens 30 .. 45 of it
    a[:, 0, [30, 31, 299, 449]] = 0.0  # isolated (the last token of frames 1 and 2)
    inp["alpha"] = a.contiguous()
    out, st, s = run_entry(entry, to_dev(inp), F, N, gdn.NORMALIZE_K)
    ro, rs = oracle_entry(entry, inp, F, N, oracle.NORMALIZE_K)
    compare(entry, dtype, out, st, s, inp, ro, rs)


@pytest.mark.parametrize("entry", ["frame", "token"])
@pytest.mark.parametrize("dtype,d", DTYPES)
def test_gate_logits_hard_resets(entry, dtype, d):
    """GDN_F_GATE_LOGITS with logit +60 (alpha = e^-60) on 20 tokens and -30 (alpha ~ 1)
    on 15 tokens inside one 64-token chunk, a +60 run across a chunk boundary, and
    logits ~ 2 N(0,1) elsewhere."""
    F, N = 3, 150
    say("case hard gate logits entry=%s %s d=%d" % (entry, dtype, d))
    inp = gdn_inputs(1, 2, F, N, d, dtype=dtype, workload_id=740 + d, state_std=0.2)
    g = torch.Generator().manual_seed(740 + d)
    la = (2.0 * torch.randn(1, 2, F * N, generator=g)).contiguous()
    lb = (2.0 * torch.randn(1, 2, F * N, generator=g)).contiguous()
    la[:, :, 5:25] = 60.0       # frame 0, chunk 0
    la[:, :, 30:45] = -30.0     # same chunk, after the reset
    la[:, :, 120:135] = 60.0    # frame 0: chunk 1 into the 22-token tail
    la[:, 1, 300:364] = -30.0   # a whole chunk of alpha ~ 1
    inp["alpha"], inp["beta"] = la, lb
    out, st, s = run_entry(entry, to_dev(inp), F, N, gdn.NORMALIZE_K | gdn.GATE_LOGITS)
    ro, rs = oracle_entry(entry, inp, F, N, oracle.NORMALIZE_K | oracle.GATE_LOGITS)
    compare(entry, dtype, out, st, s, inp, ro, rs)


# ---------------------------------------------------------------- exact workload shapes
def test_720p_5s_exact_shape():
    """The 720p 5 s rollout as specified: B=1, H=20, d=112, 21 frames x 880 tokens, bf16
    q, k, v, graded gates, zero start state; every output and the final state of all 20
    heads against the oracle, and the bf16 output equal to the RNE of the float32 one."""
    B, H, F, N, d = 1, 20, 21, 880, 112
    say("case 720p 5 s exact shape")
    inp = gdn_inputs(B, H, F, N, d, workload_id=2)
    dv = to_dev(inp)
    out, st = gdn.frame_forward(dv["q"], dv["k"], dv["v"], dv["alpha"], dv["beta"], F, N, out_dtype=torch.float32)
    ob, sb = gdn.frame_forward(dv["q"], dv["k"], dv["v"], dv["alpha"], dv["beta"], F, N)
    torch.cuda.synchronize()
    assert torch.equal(ob, out.to(torch.bfloat16)) and torch.equal(sb, st)
    ro, rs = oracle.gdn_forward(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], F, N)
    r1 = check("out", out, ro, 2e-2)
    r2 = check("state", st, rs, 2e-2)
    say("  out err/rms=%.2e state err/rms=%.2e" % (r1, r2))


def test_streaming_step_exact_shape():
    """The streaming denoise step as specified: B=16 rollouts, H=20, d=112, one 880-token
    frame, state_in ~ N(0, 0.1^2); read-only calls with fresh q, k, v, alpha, beta (three
    of the fifty) and the commit with its own fresh inputs.  The kernels run all 320
    (rollout, head) pairs; the oracle checks 9 of them."""
    B, H, N, d = 16, 20, 880, 112
    bsel, hsel = [0, 7, 15], [0, 9, 19]
    sub = lambda x: None if x is None else x[bsel][:, hsel].contiguous()
    say("case streaming step exact shape")
    base = gdn_inputs(B, H, 1, N, d, workload_id=4, step=0, state_std=0.1)
    s_in = base["state_in"].to(DEV)
    s_keep = s_in.clone()
    for step in (0, 1, 49, 50):
        inp = base if step == 0 else gdn_inputs(B, H, 1, N, d, workload_id=4, step=step)
        dv = to_dev(inp)
        say("  step %d (%s)" % (step, "commit" if step == 50 else "read-only"))
        if step < 50:
            out = gdn.frame_forward_readonly(dv["q"], dv["k"], dv["v"], dv["alpha"], dv["beta"], 1, N, state_in=s_in,
                                             out_dtype=torch.float32)
            st = None
        else:
            out, st = gdn.frame_forward(dv["q"], dv["k"], dv["v"], dv["alpha"], dv["beta"], 1, N, state_in=s_in,
                                        out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(s_in, s_keep), "state_in was written"
        ro, rs = oracle.gdn_forward(sub(inp["q"]), sub(inp["k"]), sub(inp["v"]), sub(inp["alpha"]),
                                    sub(inp["beta"]), 1, N, state_in=sub(base["state_in"]))
        check("out", out[bsel][:, hsel], ro, 2e-2)
        if st is not None:
            check("state", st[bsel][:, hsel], rs, 2e-2)


# ---------------------------------------------------------------- readout split
@pytest.mark.parametrize("shape", [(2, 4, 20, 300), (8, 20, 1, 300)])
def test_readout_split_with_an_empty_part(shape):
    """160 (b, h, frame) units of 300 tokens: each frame's 5 chunks are split over 4
    workgroups of 2 chunks, the last of which has none; multi-group (20 frames) and
    single-frame (read-only state) calls."""
    B, H, F, N = shape
    say("case readout split B=%d H=%d F=%d N=%d" % shape)
    inp = gdn_inputs(B, H, F, N, 112, workload_id=750 + F, gates="near_one", state_std=0.1)
    dv = to_dev(inp)
    out, st, _ = run_entry("frame", dv, F, N, gdn.NORMALIZE_K)
    ro_out, _, s = run_entry("readonly", dv, F, N, gdn.NORMALIZE_K)
    assert torch.equal(out, ro_out)
    bsel, hsel = [0, B - 1], [0, H - 1]
    sub = lambda x: None if x is None else x[bsel][:, hsel].contiguous()
    ro, rs = oracle.gdn_forward(sub(inp["q"]), sub(inp["k"]), sub(inp["v"]), sub(inp["alpha"]), sub(inp["beta"]),
                                F, N, state_in=sub(inp["state_in"]))
    check("out", out[bsel][:, hsel], ro, 2e-2)
    check("state", st[bsel][:, hsel], rs, 2e-2)


# ---------------------------------------------------------------- streams
def test_two_streams_at_once():
    """Two calls enqueued on two streams without waiting for each other (each with its own
    scratch buffer and outputs) give bit for bit what the same calls give one after the
    other on the current stream."""
    F, N, d = 4, 200, 112
    sets = [to_dev(gdn_inputs(1, 4, F, N, d, workload_id=760 + i, state_std=0.1)) for i in range(2)]
    ref = [gdn.frame_forward(x["q"], x["k"], x["v"], x["alpha"], x["beta"], F, N, state_in=x["state_in"],
                             out_dtype=torch.float32) for x in sets]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    got = [gdn.frame_forward(x["q"], x["k"], x["v"], x["alpha"], x["beta"], F, N, state_in=x["state_in"],
                             out_dtype=torch.float32, stream=s) for x, s in zip(sets, streams)]
    torch.cuda.synchronize()
    for (o1, s1), (o2, s2) in zip(ref, got):
        assert torch.equal(o1, o2) and torch.equal(s1, s2)
