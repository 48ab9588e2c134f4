"""Float64 numpy model of the chunked (WY / UT-transform) form of the frame-wise gated
delta rule, organised the way the HIP kernels organise it.  Test helper only: it checks
the algebra the kernels implement against the token-by-token oracle, and shares no code
with either.

Chunk form (the WY representation of products of Householder-like factors, as in Yang
et al., "Parallelizing Linear Transformers with the Delta Rule over Sequence Length",
2024, extended with the gate as in Gated Delta Networks, 2025).  For a chunk of C tokens
starting from state S0 (d_v x d_k), with k^ the normalised keys:
    G_t   = sum_{i<=t} log a_i            (inclusive, within the chunk)
    L_ti  = b_t exp(G_t - G_i) (k^_t . k^_i)   for i < t, else 0
    T     = (I + L)^-1
    U     = T diag(b) V,   W = T diag(b exp(G)) K^,   Kt = diag(exp(G_C - G)) K^
    S_C   = exp(G_C) S0 + (U - W S0^T)^T Kt  =  S0 A_c + B_c,
            A_c = exp(G_C) I - W^T Kt,   B_c = U^T Kt.
A frame's map composes its chunks:  S_f = S_{f-1} A_f + B_f.
"""
import numpy as np


def _norm_keys(k, normalize):
    if not normalize:
        return k
    n2 = (k * k).sum(-1, keepdims=True)
    return k / np.sqrt(np.maximum(n2, 1e-12))


def chunk_factors(kh, v, a, b, additive=False):
    """Return (gamma_C, W, U, Kt) for one chunk (kh already normalised)."""
    C = kh.shape[0]
    if additive:
        return 1.0, np.zeros_like(kh), v.copy(), kh.copy()
    G = np.cumsum(np.log(np.maximum(a, np.finfo(np.float32).tiny)))
    Lm = np.zeros((C, C))
    for t in range(C):
        for i in range(t):
            Lm[t, i] = b[t] * np.exp(G[t] - G[i]) * (kh[t] @ kh[i])
    T = np.linalg.inv(np.eye(C) + Lm)
    U = T @ (b[:, None] * v)
    W = T @ ((b * np.exp(G))[:, None] * kh)
    Kt = np.exp(G[-1] - G)[:, None] * kh
    return np.exp(G[-1]), W, U, Kt


def gdn_chunked(q, k, v, alpha, beta, n_frames, frame_len, chunk=64, state_in=None,
                normalize=True, additive=False, affine=True):
    """q,k,v: [T, d] for ONE head (float64). Returns (out [T, d_v], state [d_v, d_k]).

    affine=True builds each frame's (A_f, B_f) from the identity / zero states and then
    chains frames, the three-phase organisation of the HIP path; affine=False carries the
    state chunk to chunk."""
    T, dk = k.shape
    dv = v.shape[1]
    kh = _norm_keys(k.astype(np.float64), normalize)
    S = np.zeros((dv, dk)) if state_in is None else state_in.astype(np.float64).copy()
    out = np.zeros((T, dv))
    for f in range(n_frames):
        t0 = f * frame_len
        if affine:
            A = np.eye(dk)
            Bm = np.zeros((dv, dk))
        for c0 in range(t0, t0 + frame_len, chunk):
            c1 = min(c0 + chunk, t0 + frame_len)
            g, W, U, Kt = chunk_factors(kh[c0:c1], v[c0:c1].astype(np.float64),
                                        None if additive else alpha[c0:c1].astype(np.float64),
                                        None if additive else beta[c0:c1].astype(np.float64),
                                        additive)
            if affine:
                A = g * A + (-(W @ A.T)).T @ Kt
                Bm = g * Bm + (U - W @ Bm.T).T @ Kt
            else:
                S = g * S + (U - W @ S.T).T @ Kt
        if affine:
            S = S @ A + Bm
        out[t0:t0 + frame_len] = q[t0:t0 + frame_len].astype(np.float64) @ S.T
    return out, S


def gdn_chunked_tokens(q, k, v, alpha, beta, chunk=64, state_in=None, normalize=True, additive=False):
    """Per-token causal readout o_t = S_t q_t (S_t the state after token t) in chunk form,
    for ONE head (float64).  Inside a chunk with start state S0 the prefix of the chunk is
    itself a chunk whose factors are the prefix rows of U and W (T is lower triangular), so
        S_t = exp(G_t) S0 + sum_{i<=t} exp(G_t - G_i) v'_i k^_i^T,   v'_i = U_i - W_i S0^T
    and  O = diag(exp(G)) Q S0^T + (M * (Q K^^T)) V',  M_ti = exp(G_t - G_i) for i <= t.
    Returns (out [T, d_v], final state)."""
    T, dk = k.shape
    dv = v.shape[1]
    kh = _norm_keys(k.astype(np.float64), normalize)
    S = np.zeros((dv, dk)) if state_in is None else state_in.astype(np.float64).copy()
    out = np.zeros((T, dv))
    for c0 in range(0, T, chunk):
        c1 = min(c0 + chunk, T)
        C = c1 - c0
        g, W, U, Kt = chunk_factors(kh[c0:c1], v[c0:c1].astype(np.float64),
                                    None if additive else alpha[c0:c1].astype(np.float64),
                                    None if additive else beta[c0:c1].astype(np.float64), additive)
        G = np.zeros(C) if additive else np.cumsum(np.log(np.maximum(alpha[c0:c1].astype(np.float64),
                                                                      np.finfo(np.float32).tiny)))
        Vp = U - W @ S.T
        M = np.tril(np.exp(G[:, None] - G[None, :]))
        qc = q[c0:c1].astype(np.float64)
        out[c0:c1] = np.exp(G)[:, None] * (qc @ S.T) + (M * (qc @ kh[c0:c1].T)) @ Vp
        S = g * S + Vp.T @ Kt
    return out, S
