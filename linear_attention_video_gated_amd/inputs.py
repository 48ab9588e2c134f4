"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds only input synthesis (random draws and the distributions the
workloads prescribe); it contains none of the method's arithmetic.  Both the HIP path
and the CPU oracle receive the very tensors built here.

Seeds: every tensor is drawn from its own stream, keyed by (workload id, tensor id,
step) through ``numpy.random.SeedSequence``.  Tensors are drawn with torch's generator
on the device they are requested on; the CPU and GPU generators are different streams,
so a test that compares two sides always hands both the same tensor (copied).

Distributions (per token, per head):
  q, v ~ N(0, 1); k ~ N(0, 1) then divided by its L2 norm (in fp32); then rounded
  (round-to-nearest-even) to the input dtype.
  beta = sigmoid(N(0, 1)); alpha = exp(-softplus(N(0, 1))), both fp32.
  "near_one" gates: alpha = exp(-1e-3 * softplus(N(0, 1))), a slow decay that keeps
  the carried state alive across many frames.
  state_in (when requested) ~ N(0, std^2) in fp32.
  keys="raw": k ~ N(0, 1) times a per-token scale 10^U(-2, 2), not normalised (the
  kernels' own L2 normalisation then does real work); keys="short": k ~ N(0, 1) / sqrt(d)
  times 10^U(-1, 0) per token, |k| below about 1 (unnormalised keys that keep the delta
  rule contractive, for calls without normalisation).
"""
from __future__ import annotations

import numpy as np
import torch

TENSOR_IDS = {"q": 0, "k": 1, "v": 2, "alpha": 3, "beta": 4, "state": 5, "z": 6, "x": 7, "w": 8, "bias": 9,
              "carry": 10}


def seed_for(workload_id: int, tensor: str, step: int = 0) -> int:
    ss = np.random.SeedSequence([int(workload_id), TENSOR_IDS[tensor], int(step)])
    return int(ss.generate_state(1, dtype=np.uint64)[0] & ((1 << 63) - 1))


def _normal(shape, seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32)


def gdn_inputs(B, H, n_frames, frame_len, d, dtype=torch.bfloat16, workload_id=0, step=0,
               device="cpu", gates="config", state_std=None, dv=None, keys="unit"):
    """Inputs of the frame-wise gated delta rule: q, k, v [B,H,T,d], alpha, beta [B,H,T],
    state_in [B,H,d_v,d_k] or None.  keys: "unit" (L2-normalised), "raw" or "short"
    (see the module docstring)."""
    dv = d if dv is None else dv
    T = n_frames * frame_len
    q = _normal((B, H, T, d), seed_for(workload_id, "q", step), device)
    k = _normal((B, H, T, d), seed_for(workload_id, "k", step), device)
    if keys == "unit":
        k = k / k.norm(dim=-1, keepdim=True).clamp_min(1e-30)
    elif keys in ("raw", "short"):
        g = torch.Generator(device=device)
        g.manual_seed(seed_for(workload_id, "z", step))
        u = torch.rand((B, H, T, 1), generator=g, device=device, dtype=torch.float32)
        k = k * (10.0 ** (4.0 * u - 2.0)) if keys == "raw" else k * (10.0 ** (u - 1.0)) / d ** 0.5
    else:
        raise ValueError(keys)
    v = _normal((B, H, T, dv), seed_for(workload_id, "v", step), device)
    xa = _normal((B, H, T), seed_for(workload_id, "alpha", step), device)
    xb = _normal((B, H, T), seed_for(workload_id, "beta", step), device)
    beta = torch.sigmoid(xb)
    if gates == "config":
        alpha = torch.exp(-torch.nn.functional.softplus(xa))
    elif gates == "near_one":
        alpha = torch.exp(-1e-3 * torch.nn.functional.softplus(xa))
    else:
        raise ValueError(gates)
    state = None
    if state_std is not None:
        state = state_std * _normal((B, H, dv, d), seed_for(workload_id, "state", step), device)
    return {
        "q": q.to(dtype).contiguous(),
        "k": k.to(dtype).contiguous(),
        "v": v.to(dtype).contiguous(),
        "alpha": alpha.contiguous(),
        "beta": beta.contiguous(),
        "state_in": state,
    }


def block_causal_inputs(B, H, n_frames, frame_len, d, dtype=torch.bfloat16, workload_id=1,
                        step=0, device="cpu", state_std=None, dv=None):
    """Inputs of block-causal ReLU linear attention: q, k, v ~ N(0,1) [B,H,T,d]; the
    feature map is applied by the computation, not here.  Optional carried state
    S_in [B,H,d_k,d_v] ~ N(0, std^2) and normaliser z_in = |N(0, std^2)| * d."""
    dv = d if dv is None else dv
    T = n_frames * frame_len
    q = _normal((B, H, T, d), seed_for(workload_id, "q", step), device)
    k = _normal((B, H, T, d), seed_for(workload_id, "k", step), device)
    v = _normal((B, H, T, dv), seed_for(workload_id, "v", step), device)
    s_in = z_in = None
    if state_std is not None:
        s_in = state_std * _normal((B, H, d, dv), seed_for(workload_id, "state", step), device)
        z_in = (state_std * d) * _normal((B, H, d), seed_for(workload_id, "z", step), device).abs()
    return {"q": q.to(dtype).contiguous(), "k": k.to(dtype).contiguous(),
            "v": v.to(dtype).contiguous(), "state_in": s_in, "z_in": z_in}


def softmax_inputs(B, H, n_frames, kv_frames, frame_len, d, dtype=torch.bfloat16, workload_id=6,
                   step=0, device="cpu", dv=None):
    """Inputs of frame-block-causal softmax attention: k, v ~ N(0,1) [B,H,kv_frames*N,d]
    (the first kv_frames - n_frames frames stand for cached earlier frames) and
    q ~ N(0,1) [B,H,n_frames*N,d]."""
    dv = d if dv is None else dv
    Tq, Tk = n_frames * frame_len, kv_frames * frame_len
    q = _normal((B, H, Tq, d), seed_for(workload_id, "q", step), device)
    k = _normal((B, H, Tk, d), seed_for(workload_id, "k", step), device)
    v = _normal((B, H, Tk, dv), seed_for(workload_id, "v", step), device)
    return {"q": q.to(dtype).contiguous(), "k": k.to(dtype).contiguous(), "v": v.to(dtype).contiguous()}


def tconv_inputs(B, n_frames, frame_len, channels, dtype=torch.bfloat16, workload_id=8, step=0, device="cpu",
                 carry=True):
    """Inputs of the causal temporal convolution: x ~ N(0,1) [B, F, P, C] and the carried
    last frame of the previous block ~ N(0,1) [B, P, C] (None without a carry), both in
    dtype; random-init parameters w ~ N(0, 1/3) [3, C] and bias ~ N(0, 0.1^2) [C], float32."""
    x = _normal((B, n_frames, frame_len, channels), seed_for(workload_id, "x", step), device)
    w = _normal((3, channels), seed_for(workload_id, "w", step), device) / 3 ** 0.5
    bias = 0.1 * _normal((channels,), seed_for(workload_id, "bias", step), device)
    c = _normal((B, frame_len, channels), seed_for(workload_id, "carry", step), device) if carry else None
    return {"x": x.to(dtype).contiguous(), "w": w.contiguous(), "bias": bias.contiguous(),
            "carry_in": None if c is None else c.to(dtype).contiguous()}
