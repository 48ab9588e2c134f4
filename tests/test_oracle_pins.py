"""Pins of the CPU oracle to things other than itself: hand-derived values, closed
forms, textbook special cases, a different route through the algebra (explicit products
of d x d transition matrices, the chunked WY form) and invariants.  CPU only."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from chunked_ref import gdn_chunked, gdn_chunked_tokens
from linear_attention_video_gated_amd.inputs import block_causal_inputs, gdn_inputs

GOLD = os.path.join(os.path.dirname(__file__), "golden", "handworked_d2.json")


def _np(x):
    return x.detach().to(torch.float32).numpy().astype(np.float64) if hasattr(x, "detach") else x


def _rand_gdn(B=1, H=2, F=3, N=5, d=6, dv=None, seed=7, gates="config", state_std=None):
    inp = gdn_inputs(B, H, F, N, d, dtype=torch.float32, workload_id=seed, gates=gates,
                     state_std=state_std, dv=dv)
    return inp


# ---------------------------------------------------------------- hand-worked values
def test_gdn_handworked_d2():
    g = json.load(open(GOLD))["gdn"]
    arr = lambda x: np.asarray(x, dtype=np.float32)[None, None]
    out, st = oracle.gdn_forward(arr(g["q"]), arr(g["k"]), arr(g["v"]), arr(g["alpha"]),
                                 arr(g["beta"]), g["n_frames"], g["frame_len"])
    np.testing.assert_allclose(out[0, 0], np.asarray(g["out"]), atol=1e-6, rtol=1e-6)
    np.testing.assert_allclose(st[0, 0], np.asarray(g["state_out"]), atol=1e-6, rtol=1e-6)


def test_block_causal_handworked_d2():
    g = json.load(open(GOLD))["block_causal"]
    arr = lambda x: np.asarray(x, dtype=np.float32)[None, None]
    out, st, z = oracle.linear_attn_block_causal(arr(g["q"]), arr(g["k"]), arr(g["v"]),
                                                 g["n_frames"], g["frame_len"], eps=g["eps"])
    num = np.asarray(g["num"], dtype=np.float64)
    den = np.asarray(g["den"], dtype=np.float64) + g["eps"]
    np.testing.assert_allclose(out[0, 0], num / den[:, None], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(st[0, 0], np.asarray(g["state_out"]), rtol=0, atol=1e-12)
    np.testing.assert_allclose(z[0, 0], np.asarray(g["z_out"]), rtol=0, atol=1e-12)


# ---------------------------------------------------------------- textbook special cases
def _frame_mask(F, N):
    fr = np.repeat(np.arange(F), N)
    return (fr[None, :] <= fr[:, None]).astype(np.float64)  # M[t, s] = frame(s) <= frame(t)


@pytest.mark.parametrize("with_state", [False, True])
def test_block_causal_equals_masked_quadratic_form(with_state):
    F, N, d, dv = 4, 3, 5, 4
    inp = block_causal_inputs(1, 2, F, N, d, dtype=torch.float32, workload_id=11,
                              state_std=0.5 if with_state else None, dv=dv)
    out, st, z = oracle.linear_attn_block_causal(inp["q"], inp["k"], inp["v"], F, N,
                                                 state_in=inp["state_in"], z_in=inp["z_in"])
    M = _frame_mask(F, N)
    for h in range(2):
        q, k, v = (_np(inp[n])[0, h] for n in ("q", "k", "v"))
        pq, pk = np.maximum(q, 0), np.maximum(k, 0)
        A = M * (pq @ pk.T)
        num, den = A @ v, A.sum(1)
        s_out, z_out = pk.T @ v, pk.sum(0)
        if with_state:
            S0, z0 = _np(inp["state_in"])[0, h], _np(inp["z_in"])[0, h]
            num, den = num + pq @ S0, den + pq @ z0
            s_out, z_out = s_out + S0, z_out + z0
        np.testing.assert_allclose(out[0, h], num / (den + 1e-6)[:, None], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(st[0, h], s_out, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(z[0, h], z_out, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("normalize", [False, True])
def test_gdn_additive_equals_block_causal_quadratic_form(normalize):
    """gate 1, no delta term: O = (M o Q K^T) V + Q S_in^T (S is d_v x d_k)."""
    F, N, d, dv = 3, 4, 5, 3
    inp = _rand_gdn(F=F, N=N, d=d, dv=dv, seed=12, state_std=0.7)
    flags = oracle.ADDITIVE | (oracle.NORMALIZE_K if normalize else 0)
    out, st = oracle.gdn_forward(inp["q"], inp["k"], inp["v"], None, None, F, N,
                                 state_in=inp["state_in"], flags=flags)
    M = _frame_mask(F, N)
    for h in range(2):
        q, k, v = (_np(inp[n])[0, h] for n in ("q", "k", "v"))
        if normalize:
            k = k / np.linalg.norm(k, axis=1, keepdims=True)
        S0 = _np(inp["state_in"])[0, h]
        np.testing.assert_allclose(out[0, h], (M * (q @ k.T)) @ v + q @ S0.T, rtol=1e-11, atol=1e-11)
        np.testing.assert_allclose(st[0, h], S0 + v.T @ k, rtol=1e-11, atol=1e-11)


# ---------------------------------------------------------------- closed forms
def test_gdn_beta_zero_pure_decay():
    """beta = 0: S_f = (prod_{t <= end of f} a_t) S_0 and O_f = Q_f S_f^T."""
    F, N, d = 4, 3, 6
    inp = _rand_gdn(F=F, N=N, d=d, seed=13, gates="near_one", state_std=1.0)
    beta = torch.zeros_like(inp["beta"])
    out, st = oracle.gdn_forward(inp["q"], inp["k"], inp["v"], inp["alpha"], beta, F, N,
                                 state_in=inp["state_in"])
    a = _np(inp["alpha"])
    for h in range(2):
        S0, q = _np(inp["state_in"])[0, h], _np(inp["q"])[0, h]
        for f in range(F):
            Sf = np.prod(a[0, h, :(f + 1) * N]) * S0
            np.testing.assert_allclose(out[0, h, f * N:(f + 1) * N], q[f * N:(f + 1) * N] @ Sf.T,
                                       rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(st[0, h], np.prod(a[0, h]) * S0, rtol=1e-12)


def test_gdn_alpha_zero_is_clamped_and_forgets():
    """a_t = 0 is clamped to FLT_MIN: the past is wiped except for ~1e-38 of it."""
    F, N, d = 2, 3, 4
    inp = _rand_gdn(F=F, N=N, d=d, seed=14, state_std=1.0)
    alpha = inp["alpha"].clone()
    alpha[..., N] = 0.0  # first token of frame 2
    out, st = oracle.gdn_forward(inp["q"], inp["k"], inp["v"], alpha, inp["beta"], F, N,
                                 state_in=inp["state_in"])
    out2, st2 = oracle.gdn_forward(inp["q"][..., N:, :], inp["k"][..., N:, :], inp["v"][..., N:, :],
                                   alpha[..., N:], inp["beta"][..., N:], 1, N, state_in=None)
    np.testing.assert_allclose(out[..., N:, :], out2, rtol=1e-9, atol=1e-30)
    np.testing.assert_allclose(st, st2, rtol=1e-9, atol=1e-30)


def _unit_keys(inp):
    k = _np(inp["k"])
    return (k / np.linalg.norm(k, axis=-1, keepdims=True)).astype(np.float32)


def test_gdn_beta_one_retrieval():
    """b_t = 1: the delta rule writes v_t exactly, S_t k^_t = v_t, whatever a_t."""
    T, d = 12, 8
    inp = _rand_gdn(F=T, N=1, d=d, seed=15, state_std=1.0)
    kh = _unit_keys(inp)
    out, _ = oracle.gdn_forward(kh, kh, inp["v"], inp["alpha"], torch.ones_like(inp["beta"]),
                                T, 1, state_in=inp["state_in"])
    # q = kh (float32) has norm 1 +- 1e-7; the oracle normalises in float64
    nrm = np.linalg.norm(kh.astype(np.float64), axis=-1, keepdims=True)
    np.testing.assert_allclose(out / nrm, _np(inp["v"]), rtol=1e-12, atol=1e-12)


def test_gdn_delta_rule_defining_property():
    """S_t k^_t = a_t (1 - b_t) S_{t-1} k^_t + b_t v_t, token by token (frame_len 1)."""
    T, d, dv = 16, 7, 5
    inp = _rand_gdn(F=T, N=1, d=d, dv=dv, seed=16, state_std=1.0)
    kh = _unit_keys(inp)
    k_next = np.concatenate([kh[..., 1:, :], kh[..., :1, :]], axis=2)
    o_same, _ = oracle.gdn_forward(kh, kh, inp["v"], inp["alpha"], inp["beta"], T, 1,
                                   state_in=inp["state_in"])          # S_t k^_t
    o_next, _ = oracle.gdn_forward(k_next, kh, inp["v"], inp["alpha"], inp["beta"], T, 1,
                                   state_in=inp["state_in"])          # S_t k^_{t+1}
    a, b, v = _np(inp["alpha"]), _np(inp["beta"]), _np(inp["v"])
    nrm = np.linalg.norm(kh.astype(np.float64), axis=-1, keepdims=True)  # q carries |kh| != 1 exactly
    lhs = (o_same / nrm)[..., 1:, :]
    rhs = (a * (1 - b))[..., 1:, None] * (o_next[..., :-1, :] / nrm[..., 1:, :]) + b[..., 1:, None] * v[..., 1:, :]
    np.testing.assert_allclose(lhs, rhs, rtol=1e-11, atol=1e-12)


def test_gdn_explicit_transition_products():
    """Unrolled closed form with dense d x d transition matrices:
    S_F = S_0 prod_t A_t + sum_t b_t v_t k^_t^T prod_{s>t} A_s,  A_t = a_t (I - b_t k^ k^T)."""
    F, N, d, dv = 2, 4, 5, 3
    inp = _rand_gdn(F=F, N=N, d=d, dv=dv, seed=17, state_std=1.0)
    out, st = oracle.gdn_forward(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], F, N,
                                 state_in=inp["state_in"])
    a, b = _np(inp["alpha"]), _np(inp["beta"])
    for h in range(2):
        k = _np(inp["k"])[0, h]
        kh = k / np.linalg.norm(k, axis=1, keepdims=True)
        v, q, S0 = _np(inp["v"])[0, h], _np(inp["q"])[0, h], _np(inp["state_in"])[0, h]
        A = [a[0, h, t] * (np.eye(d) - b[0, h, t] * np.outer(kh[t], kh[t])) for t in range(F * N)]
        for f in range(F):
            end = (f + 1) * N
            tail = [np.eye(d)] * (end + 1)      # tail[t] = prod_{t <= s < end} A_s
            for t in range(end - 1, -1, -1):
                tail[t] = A[t] @ tail[t + 1]
            Sf = S0 @ tail[0] + sum(b[0, h, t] * np.outer(v[t], kh[t]) @ tail[t + 1] for t in range(end))
            np.testing.assert_allclose(out[0, h, f * N:end], q[f * N:end] @ Sf.T, rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(st[0, h], Sf, rtol=1e-10, atol=1e-12)


# ---------------------------------------------------------------- equivalences / invariants
@pytest.mark.parametrize("chunk", [64, 16, 7, 1])
@pytest.mark.parametrize("affine", [False, True])
def test_chunked_form_equals_sequential(chunk, affine):
    """The WY/UT chunk algebra the kernels implement (with tail chunks) equals the
    token-by-token oracle to float64 round-off."""
    F, N, d, dv = 3, 150, 16, 12  # 150 = 2*64 + 22: a ragged tail chunk
    for gates in ("config", "near_one"):
        inp = _rand_gdn(B=1, H=1, F=F, N=N, d=d, dv=dv, seed=18, gates=gates, state_std=0.5)
        out, st = oracle.gdn_forward(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], F, N,
                                     state_in=inp["state_in"])
        o2, s2 = gdn_chunked(_np(inp["q"])[0, 0], _np(inp["k"])[0, 0], _np(inp["v"])[0, 0],
                             _np(inp["alpha"])[0, 0], _np(inp["beta"])[0, 0], F, N, chunk=chunk,
                             state_in=_np(inp["state_in"])[0, 0], affine=affine)
        scale = np.sqrt(np.mean(out ** 2))
        assert np.max(np.abs(o2 - out[0, 0])) <= 1e-11 * scale
        assert np.max(np.abs(s2 - st[0, 0])) <= 1e-11 * np.sqrt(np.mean(st ** 2))


@pytest.mark.parametrize("chunk", [64, 16, 7])
def test_chunked_token_readout_equals_sequential(chunk):
    """Per-token causal readout (every token reads the state after itself) in chunk form --
    exp(G) Q S0^T plus the decay-masked intra-chunk product with v' = U - W S0^T -- equals
    the token-by-token oracle run with one-token frames."""
    T, d, dv = 150, 16, 12
    for gates in ("config", "near_one"):
        inp = _rand_gdn(B=1, H=1, F=1, N=T, d=d, dv=dv, seed=21, gates=gates, state_std=0.5)
        out, st = oracle.gdn_forward(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], T, 1,
                                     state_in=inp["state_in"])
        o2, s2 = gdn_chunked_tokens(_np(inp["q"])[0, 0], _np(inp["k"])[0, 0], _np(inp["v"])[0, 0],
                                    _np(inp["alpha"])[0, 0], _np(inp["beta"])[0, 0], chunk=chunk,
                                    state_in=_np(inp["state_in"])[0, 0])
        assert np.max(np.abs(o2 - out[0, 0])) <= 1e-11 * np.sqrt(np.mean(out ** 2))
        assert np.max(np.abs(s2 - st[0, 0])) <= 1e-11 * np.sqrt(np.mean(st ** 2))


def test_chunked_additive_equals_sequential():
    F, N, d = 2, 70, 8
    inp = _rand_gdn(B=1, H=1, F=F, N=N, d=d, seed=19, state_std=0.5)
    out, st = oracle.gdn_forward(inp["q"], inp["k"], inp["v"], None, None, F, N,
                                 state_in=inp["state_in"], flags=oracle.ADDITIVE | oracle.NORMALIZE_K)
    o2, s2 = gdn_chunked(_np(inp["q"])[0, 0], _np(inp["k"])[0, 0], _np(inp["v"])[0, 0], None, None,
                         F, N, state_in=_np(inp["state_in"])[0, 0], additive=True)
    np.testing.assert_allclose(o2, out[0, 0], rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(s2, st[0, 0], rtol=1e-11, atol=1e-11)


def test_gdn_segments_compose():
    """Frames [0, F1) then [F1, F) with the state carried equal one call over [0, F)."""
    F, F1, N, d = 6, 2, 5, 8
    inp = _rand_gdn(F=F, N=N, d=d, seed=20, gates="near_one", state_std=0.5)
    full, st = oracle.gdn_forward(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], F, N,
                                  state_in=inp["state_in"])
    c = F1 * N
    o1, s1 = oracle.gdn_forward(inp["q"][..., :c, :], inp["k"][..., :c, :], inp["v"][..., :c, :],
                                inp["alpha"][..., :c], inp["beta"][..., :c], F1, N, state_in=inp["state_in"])
    o2, s2 = oracle.gdn_forward(inp["q"][..., c:, :], inp["k"][..., c:, :], inp["v"][..., c:, :],
                                inp["alpha"][..., c:], inp["beta"][..., c:], F - F1, N,
                                state_in=s1.astype(np.float32))
    # the carried state passes through float32 (what a caller stores); compare accordingly
    np.testing.assert_allclose(np.concatenate([o1, o2], axis=2), full, rtol=1e-6, atol=1e-6)
    np.testing.assert_allclose(s2, st, rtol=1e-6, atol=1e-6)


def test_gdn_linear_in_values_and_state():
    F, N, d = 3, 4, 6
    i1 = _rand_gdn(F=F, N=N, d=d, seed=21, state_std=1.0)
    i2 = _rand_gdn(F=F, N=N, d=d, seed=22, state_std=1.0)
    run = lambda v, s: oracle.gdn_forward(i1["q"], i1["k"], v, i1["alpha"], i1["beta"], F, N, state_in=s)
    o1, s1 = run(i1["v"], i1["state_in"])
    o2, s2 = run(i2["v"], i2["state_in"])
    o3, s3 = run(_np(i1["v"]) + _np(i2["v"]), _np(i1["state_in"]) + _np(i2["state_in"]))
    np.testing.assert_allclose(o3, o1 + o2, rtol=1e-6, atol=1e-6)  # sums rounded to fp32 on input
    np.testing.assert_allclose(s3, s1 + s2, rtol=1e-6, atol=1e-6)


def test_oracle_state_is_constant_size():
    """The carried state is d_v x d_k per (b, h) whatever the sequence length."""
    for F in (1, 7):
        inp = _rand_gdn(F=F, N=3, d=4, dv=3, seed=23)
        _, st = oracle.gdn_forward(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], F, 3)
        assert st.shape == (1, 2, 3, 4)


def test_oracle_threads_do_not_change_results():
    inp = _rand_gdn(B=2, H=3, F=2, N=9, d=8, seed=24)
    o1, s1 = oracle.gdn_forward(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], 2, 9, n_threads=1)
    o4, s4 = oracle.gdn_forward(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], 2, 9, n_threads=4)
    assert np.array_equal(o1, o4) and np.array_equal(s1, s4)


# ---------------------------------------------------------------- gates given as logits
def _np64(x):
    return np.asarray(x, dtype=np.float64)


def test_gate_logits_equal_sigmoid_gates():
    """exp(-softplus(a)) = 1 / (1 + e^a) and beta = 1 / (1 + e^-b): the logit mode equals the
    plain mode fed with those gates (computed here by the other formula, in float64, then
    rounded to float32 -- hence the 1e-5 bound)."""
    T, d = 40, 8
    inp = _rand_gdn(B=1, H=2, F=4, N=10, d=d, seed=31, state_std=0.3)
    rng = np.random.default_rng(31)
    a = rng.normal(0.0, 2.0, size=(1, 2, T)).astype(np.float32)
    b = rng.normal(0.0, 2.0, size=(1, 2, T)).astype(np.float32)
    al = (1.0 / (1.0 + np.exp(_np64(a)))).astype(np.float32)
    be = (1.0 / (1.0 + np.exp(-_np64(b)))).astype(np.float32)
    o1, s1 = oracle.gdn_forward(inp["q"], inp["k"], inp["v"], a, b, 4, 10, state_in=inp["state_in"],
                                flags=oracle.NORMALIZE_K | oracle.GATE_LOGITS)
    o2, s2 = oracle.gdn_forward(inp["q"], inp["k"], inp["v"], al, be, 4, 10, state_in=inp["state_in"])
    assert np.max(np.abs(o1 - o2)) <= 1e-5 * np.sqrt(np.mean(o2 ** 2))
    assert np.max(np.abs(s1 - s2)) <= 1e-5 * np.sqrt(np.mean(s2 ** 2))


def test_gate_logits_limits():
    """a = -60, b = +60: alpha = beta = 1 to float64 precision, so with one-token frames and
    q_t = k^_t every token retrieves its own value exactly (S_t k^_t = v_t).  a = +60: the
    state is wiped at every token (alpha ~ 1e-26), so S_t = v_t k^_t^T and o_t = v_t (k^_t . q_t)."""
    T, d, dv = 12, 6, 5
    rng = np.random.default_rng(32)
    k = rng.normal(size=(1, 1, T, d)).astype(np.float32)
    kh = _np64(k) / np.linalg.norm(_np64(k), axis=-1, keepdims=True)
    q_eq = kh.astype(np.float32)
    v = rng.normal(size=(1, 1, T, dv)).astype(np.float32)
    big = np.full((1, 1, T), 60.0, dtype=np.float32)
    flags = oracle.NORMALIZE_K | oracle.GATE_LOGITS
    out, _ = oracle.gdn_forward(q_eq, k, v, -big, big, T, 1, state_in=0.5 * np.ones((1, 1, dv, d), np.float32),
                                flags=flags)
    # q is k^ rounded to float32: the retrieval error is that rounding, ~1e-7 relative
    np.testing.assert_allclose(out[0, 0], _np64(v[0, 0]), rtol=0, atol=1e-6)
    q = rng.normal(size=(1, 1, T, d)).astype(np.float32)
    out, _ = oracle.gdn_forward(q, k, v, big, big, T, 1, state_in=np.ones((1, 1, dv, d), np.float32), flags=flags)
    ref = _np64(v[0, 0]) * np.sum(kh[0, 0] * _np64(q[0, 0]), axis=-1, keepdims=True)
    np.testing.assert_allclose(out[0, 0], ref, rtol=0, atol=1e-12 + 1e-9 * np.abs(ref).max())


# ---------------------------------------------------------------- softmax attention layers
def _sa_rand(B=1, H=2, F=3, KF=None, N=4, d=8, seed=61):
    from linear_attention_video_gated_amd.inputs import softmax_inputs
    KF = F if KF is None else KF
    inp = softmax_inputs(B, H, F, KF, N, d, dtype=torch.float32, workload_id=seed)
    return {n: inp[n].numpy().astype(np.float64) for n in ("q", "k", "v")}


def _sdpa64(q, k, v, **kw):
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64))
    return torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), **kw).numpy()


def test_softmax_handworked_d2():
    g = json.load(open(GOLD))["softmax"]
    arr = lambda x: np.asarray(x, dtype=np.float32)[None, None]
    out = oracle.softmax_attn_block_causal(arr(g["q"]), arr(g["k"]), arr(g["v"]), g["n_frames"],
                                           g["kv_frames"], g["frame_len"], scale=g["scale"])
    np.testing.assert_allclose(out[0, 0], np.asarray(g["out"]), rtol=1e-13, atol=1e-13)


def test_softmax_one_token_frames_is_causal_attention():
    """frame_len = 1: the frame mask is the token-causal mask of textbook attention."""
    x = _sa_rand(F=13, N=1, d=8)
    ref = _sdpa64(x["q"], x["k"], x["v"], is_causal=True)
    out = oracle.softmax_attn_block_causal(x["q"], x["k"], x["v"], 13, 13, 1)
    np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-12)


def test_softmax_last_frame_sees_everything():
    """The queries of the newest frame see every key passed: plain unmasked attention,
    with or without cached earlier frames."""
    for F, KF in ((1, 1), (1, 4)):
        x = _sa_rand(F=F, KF=KF, N=5, d=8, seed=62 + KF)
        ref = _sdpa64(x["q"], x["k"], x["v"])
        out = oracle.softmax_attn_block_causal(x["q"], x["k"], x["v"], F, KF, 5)
        np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-12)


def test_softmax_equal_keys_average_the_visible_values():
    """Equal keys give equal weights: each query gets the mean of the values of the keys it
    sees, which counts the visible frames (its own included, cached ones included)."""
    F, KF, N = 3, 5, 4
    x = _sa_rand(F=F, KF=KF, N=N, d=6, seed=64)
    k = np.broadcast_to(x["k"][:, :, :1], x["k"].shape).copy()
    out = oracle.softmax_attn_block_causal(x["q"], k, x["v"], F, KF, N)
    for i in range(F * N):
        nvis = (KF - F + i // N + 1) * N
        np.testing.assert_allclose(out[:, :, i], x["v"][:, :, :nvis].mean(axis=2), rtol=1e-10, atol=1e-12)


def test_softmax_frame_causality_and_block_invariance():
    F, N = 4, 5
    x = _sa_rand(F=F, N=N, d=8, seed=65)
    base = oracle.softmax_attn_block_causal(x["q"], x["k"], x["v"], F, F, N)
    rng = np.random.default_rng(3)
    for f in range(F):
        # keys and values of later frames do not reach frame f's queries ...
        k2, v2 = x["k"].copy(), x["v"].copy()
        k2[:, :, (f + 1) * N:] = rng.standard_normal(k2[:, :, (f + 1) * N:].shape)
        v2[:, :, (f + 1) * N:] = rng.standard_normal(v2[:, :, (f + 1) * N:].shape)
        o2 = oracle.softmax_attn_block_causal(x["q"], k2, v2, F, F, N)
        np.testing.assert_array_equal(o2[:, :, :(f + 1) * N], base[:, :, :(f + 1) * N])
        # ... but those of frame f itself do (the mask is inclusive of the own frame)
        v3 = x["v"].copy()
        v3[:, :, f * N + N - 1] += 1.0
        o3 = oracle.softmax_attn_block_causal(x["q"], x["k"], v3, F, F, N)
        assert np.abs(o3[:, :, f * N:(f + 1) * N] - base[:, :, f * N:(f + 1) * N]).min() > 1e-6
    # keys (with their values) permuted inside a frame: same outputs (no order inside a frame)
    perm = np.arange(F * N)
    perm[N:2 * N] = perm[N:2 * N][::-1]
    o4 = oracle.softmax_attn_block_causal(x["q"], x["k"][:, :, perm], x["v"][:, :, perm], F, F, N)
    np.testing.assert_allclose(o4, base, rtol=1e-12, atol=1e-13)


def test_softmax_cached_frames_equal_full_call_rows():
    """Queries of the last frames against cached earlier frames = the same rows of one call
    over all frames."""
    KF, N = 5, 3
    x = _sa_rand(F=KF, N=N, d=8, seed=66)
    full = oracle.softmax_attn_block_causal(x["q"], x["k"], x["v"], KF, KF, N)
    for F in (1, 2, 4):
        part = oracle.softmax_attn_block_causal(x["q"][:, :, (KF - F) * N:], x["k"], x["v"], F, KF, N)
        np.testing.assert_allclose(part, full[:, :, (KF - F) * N:], rtol=1e-13, atol=1e-14)


def test_softmax_shift_scale_and_large_logits():
    F, N = 3, 4
    x = _sa_rand(F=F, N=N, d=8, seed=67)
    x["k"] = np.round(x["k"] * 1024) / 1024  # on a grid where k + u below is exact in float32
    base = oracle.softmax_attn_block_causal(x["q"], x["k"], x["v"], F, F, N)
    # a vector added to every key shifts each query's logits by a constant: no change
    u = np.linspace(-2, 3, 8).round(2) // 0.25 * 0.25
    o1 = oracle.softmax_attn_block_causal(x["q"], x["k"] + u, x["v"], F, F, N)
    np.testing.assert_allclose(o1, base, rtol=1e-10, atol=1e-11)
    # the default scale is 1/sqrt(d_k)
    o2 = oracle.softmax_attn_block_causal(x["q"], x["k"], x["v"], F, F, N, scale=1 / np.sqrt(8))
    np.testing.assert_array_equal(o2, base)
    # logits far beyond exp's range: each query takes the value of its best visible key
    q = 1e4 * x["q"]
    o3 = oracle.softmax_attn_block_causal(q, x["k"], x["v"], F, F, N)
    for i in range(F * N):
        nvis = (i // N + 1) * N
        best = np.argmax(np.einsum("bhd,bhjd->bhj", q[:, :, i], x["k"][:, :, :nvis]), axis=-1)
        want = np.take_along_axis(x["v"][:, :, :nvis], best[..., None, None], axis=2)[:, :, 0]
        np.testing.assert_allclose(o3[:, :, i], want, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- causal temporal convolution
def _tc_rand(B=2, F=4, P=3, C=5, seed=81, carry=True):
    from linear_attention_video_gated_amd.inputs import tconv_inputs
    inp = tconv_inputs(B, F, P, C, dtype=torch.float32, workload_id=seed, carry=carry)
    return {k: (None if v is None else v.numpy().astype(np.float64)) for k, v in inp.items()}


def test_tconv_special_taps():
    x = _tc_rand()
    C = x["x"].shape[-1]
    eye = lambda j: np.stack([np.full(C, 1.0 if i == j else 0.0) for i in range(3)])
    # centre tap: identity; the carry out is the block's last frame
    y, c = oracle.temporal_conv_block(x["x"], eye(1), carry_in=x["carry_in"])
    np.testing.assert_array_equal(y, x["x"])
    np.testing.assert_array_equal(c, x["x"][:, -1])
    # left tap: the previous frame, the carried one for frame 0
    y, _ = oracle.temporal_conv_block(x["x"], eye(0), carry_in=x["carry_in"])
    np.testing.assert_array_equal(y[:, 1:], x["x"][:, :-1])
    np.testing.assert_array_equal(y[:, 0], x["carry_in"])
    y, _ = oracle.temporal_conv_block(x["x"], eye(0))  # no carry: zero before the first block
    np.testing.assert_array_equal(y[:, 0], 0 * x["x"][:, 0])
    # right tap: the next frame, the zero token after the last one
    y, _ = oracle.temporal_conv_block(x["x"], eye(2), carry_in=x["carry_in"])
    np.testing.assert_array_equal(y[:, :-1], x["x"][:, 1:])
    np.testing.assert_array_equal(y[:, -1], 0 * x["x"][:, -1])
    # bias only
    y, _ = oracle.temporal_conv_block(x["x"], 0 * eye(0), bias=x["bias"], carry_in=x["carry_in"])
    np.testing.assert_allclose(y, np.broadcast_to(x["bias"], y.shape), rtol=0, atol=1e-7)


def test_tconv_blocks_equal_the_training_sequence():
    """The talk's training form: blocks concatenated with a zero token after each block and
    the previous block's last token before each later block, one 'same'-padded convolution
    over the whole sequence (scipy's correlate1d, zeros outside), the inserted tokens then
    removed -- equals block-by-block calls that carry the last frame."""
    from scipy.ndimage import correlate1d
    blocks = [_tc_rand(B=1, F=F, P=2, C=3, seed=90 + i, carry=False)["x"] for i, F in enumerate((3, 1, 4))]
    prm = _tc_rand(B=1, F=1, P=2, C=3, seed=99)
    w, bias = prm["w"], prm["bias"]
    seq, keep = [], []
    for i, blk in enumerate(blocks):
        if i > 0:
            seq.append(blocks[i - 1][:, -1:])  # cached last token of the previous block
            keep.append(False)
        seq.append(blk)
        keep += [True] * blk.shape[1]
        seq.append(np.zeros_like(blk[:, :1]))  # zero token after the block
        keep.append(False)
    seq = np.concatenate(seq, axis=1)
    ref = np.stack([correlate1d(seq[..., c], w[:, c], axis=1, mode="constant", cval=0.0) for c in range(3)], -1)
    ref = ref[:, np.array(keep)] + bias
    outs, carry = [], None
    for blk in blocks:
        y, carry = oracle.temporal_conv_block(blk, w, bias=bias, carry_in=carry)
        outs.append(y)
    np.testing.assert_allclose(np.concatenate(outs, axis=1), ref, rtol=1e-6, atol=1e-6)


# ---------------------------------------------------------------- 3D rotary position embedding
def _rope_x(B=1, H=2, F=3, gh=2, gw=3, d=16, seed=95):
    g = np.random.default_rng(seed)
    return g.standard_normal((B, H, F * gh * gw, d)).astype(np.float32).astype(np.float64)


def test_rope3d_rotations():
    F, gh, gw, d, dt, dh = 3, 2, 3, 16, 4, 6
    x = _rope_x(F=F, gh=gh, gw=gw, d=d)
    y = oracle.rope3d(x, F, gh, gw, dt, dh)
    # a rotation of every pair: norms of each pair kept
    pn = lambda z: z[..., 0::2] ** 2 + z[..., 1::2] ** 2
    np.testing.assert_allclose(pn(y), pn(x), rtol=1e-12, atol=1e-12)
    # token 0 of frame 0 sits at the origin: unchanged
    np.testing.assert_allclose(y[:, :, 0], x[:, :, 0], rtol=0, atol=1e-15)
    # pair 0 of each part turns by the position itself (frequency base^0 = 1): token 5 is
    # frame 0, row 1, column 2
    t, pos = 5, {0: 0, dt: 1, dt + dh: 2}
    for s0, p0 in pos.items():
        c, s = np.cos(p0), np.sin(p0)
        x0, x1 = x[:, :, t, s0], x[:, :, t, s0 + 1]
        np.testing.assert_allclose(y[:, :, t, s0], x0 * c - x1 * s, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(y[:, :, t, s0 + 1], x0 * s + x1 * c, rtol=1e-12, atol=1e-12)


def test_rope3d_relative_positions():
    """Scores between rotated q and k depend on the two tokens' position difference only:
    moving every frame by the same offset changes no score."""
    F, gh, gw, d, dt, dh = 4, 2, 2, 12, 4, 4
    q, k = _rope_x(F=F, gh=gh, gw=gw, d=d, seed=96), _rope_x(F=F, gh=gh, gw=gw, d=d, seed=97)
    s0 = np.einsum("bhtd,bhsd->bhts", oracle.rope3d(q, F, gh, gw, dt, dh), oracle.rope3d(k, F, gh, gw, dt, dh))
    s7 = np.einsum("bhtd,bhsd->bhts", oracle.rope3d(q, F, gh, gw, dt, dh, frame_offset=7),
                   oracle.rope3d(k, F, gh, gw, dt, dh, frame_offset=7))
    np.testing.assert_allclose(s7, s0, rtol=1e-10, atol=1e-10)
    # and the offset does change the rotated vectors themselves
    assert np.abs(oracle.rope3d(q, F, gh, gw, dt, dh, frame_offset=7) - oracle.rope3d(q, F, gh, gw, dt, dh)).max() > 1e-3


def test_rope3d_frequency_ladder_handworked():
    """Pairs i >= 1 of each part: angles worked by hand (tests/golden/rope3d_handworked.json)
    from pos * base^(-2i/n).  Every pair of the chosen token gets (1, 0) or (0, 1), so the
    rotated pair is (cos a, sin a) or (-sin a, cos a)."""
    import json
    import math
    spec = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "rope3d_handworked.json")))
    for case in spec["cases"]:
        d, F, gh, gw = case["d"], case["n_frames"], case["grid_h"], case["grid_w"]
        x = _rope_x(F=F, gh=gh, gw=gw, d=d, seed=98)
        t = case["token"]
        x[:, :, t, :] = 0.0
        x[:, :, t, 0::4] = 1.0   # even pairs: (1, 0)
        x[:, :, t, 3::4] = 1.0   # odd pairs: (0, 1)
        y = oracle.rope3d(x, F, gh, gw, case["d_t"], case["d_h"], frame_offset=case["frame_offset"],
                          base=case["base"])
        for p, a in enumerate(case["pair_angles"]):
            want = (math.cos(a), math.sin(a)) if p % 2 == 0 else (-math.sin(a), math.cos(a))
            np.testing.assert_allclose(y[:, :, t, 2 * p], want[0], rtol=0, atol=1e-12, err_msg=case["name"])
            np.testing.assert_allclose(y[:, :, t, 2 * p + 1], want[1], rtol=0, atol=1e-12, err_msg=case["name"])
