"""ctypes wrapper around ``oracle_gdn.c`` (TEST INFRASTRUCTURE ONLY).

The C source is the oracle; this file only compiles it (gcc, OpenMP), marshals numpy
arrays and returns float64 results.  Inputs are widened to float32 before the call:
bf16 tensors convert to float32 exactly, so the oracle works on the same values the
GPU receives.

Definitions and citations are in the header of ``oracle_gdn.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

NORMALIZE_K = 1
ADDITIVE = 2
GATE_LOGITS = 4  # alpha, beta hold logits a, b: alpha = exp(-softplus(a)), beta = sigmoid(b)

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle_gdn.c")
_LIB_PATH = os.path.join(_HERE, "liboracle_gdn.so")
_lib = None
_lock = threading.Lock()


def build(force: bool = False) -> str:
    """Compile the oracle into ``oracle/liboracle_gdn.so`` (gcc -O2 -fopenmp)."""
    stale = (not os.path.exists(_LIB_PATH)) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)
    if force or stale:
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            lib = ctypes.CDLL(_LIB_PATH)
            fp = ctypes.POINTER(ctypes.c_float)
            dp = ctypes.POINTER(ctypes.c_double)
            i = ctypes.c_int
            lib.oracle_gdn_forward.argtypes = [fp, fp, fp, fp, fp, fp, dp, dp,
                                               i, i, i, i, i, i, ctypes.c_uint, i]
            lib.oracle_gdn_forward.restype = i
            lib.oracle_linear_attn_block_causal.argtypes = [fp, fp, fp, fp, fp, dp, dp, dp,
                                                            i, i, i, i, i, i, ctypes.c_double, i]
            lib.oracle_linear_attn_block_causal.restype = i
            lib.oracle_softmax_attn_block_causal.argtypes = [fp, fp, fp, dp, i, i, i, i, i, i, i,
                                                             ctypes.c_double, i]
            lib.oracle_softmax_attn_block_causal.restype = i
            lib.oracle_temporal_conv_block.argtypes = [fp, fp, fp, fp, dp, dp, i, i, i, i]
            lib.oracle_temporal_conv_block.restype = i
            lib.oracle_rope3d.argtypes = [fp, dp, i, i, i, i, i, i, i, i, i, ctypes.c_double]
            lib.oracle_rope3d.restype = i
            _lib = lib
    return _lib


def _f32(x):
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor -> numpy float32 (exact for bf16)
        import torch
        x = x.detach().to("cpu", torch.float32).numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float32))


def _ptr(a, ctype):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def gdn_forward(q, k, v, alpha, beta, n_frames, frame_len, state_in=None,
                flags=NORMALIZE_K, n_threads=0, want_state=True):
    """Frame-wise gated delta rule (see ``oracle_gdn.c``).

    q, k: [B, H, T, d_k]; v: [B, H, T, d_v]; alpha, beta: [B, H, T] (ignored when
    ``flags`` has ADDITIVE; may then be None); state_in: [B, H, d_v, d_k] or None.
    Returns (out [B, H, T, d_v] float64, state_out [B, H, d_v, d_k] float64 or None).
    """
    lib = _load()
    q, k, v = _f32(q), _f32(k), _f32(v)
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    if T != n_frames * frame_len or k.shape != q.shape or v.shape[:3] != (B, H, T):
        raise ValueError("shape mismatch")
    additive = bool(flags & ADDITIVE)
    alpha = _f32(alpha) if not additive or alpha is not None else None
    beta = _f32(beta) if not additive or beta is not None else None
    if not additive and (alpha is None or beta is None or alpha.shape != (B, H, T) or beta.shape != (B, H, T)):
        raise ValueError("alpha/beta must be [B, H, T]")
    s_in = _f32(state_in)
    if s_in is not None and s_in.shape != (B, H, dv, dk):
        raise ValueError("state_in must be [B, H, d_v, d_k]")
    out = np.zeros((B, H, T, dv), dtype=np.float64)
    s_out = np.zeros((B, H, dv, dk), dtype=np.float64) if want_state else None
    rc = lib.oracle_gdn_forward(_ptr(q, ctypes.c_float), _ptr(k, ctypes.c_float), _ptr(v, ctypes.c_float),
                                _ptr(alpha, ctypes.c_float), _ptr(beta, ctypes.c_float),
                                _ptr(s_in, ctypes.c_float), _ptr(s_out, ctypes.c_double),
                                _ptr(out, ctypes.c_double), B, H, n_frames, frame_len, dk, dv,
                                int(flags), int(n_threads))
    if rc != 0:
        raise RuntimeError("oracle_gdn_forward failed (%d)" % rc)
    return out, s_out


def linear_attn_block_causal(q, k, v, n_frames, frame_len, state_in=None, z_in=None,
                             eps=1e-6, n_threads=0):
    """Block-causal ReLU linear attention (see ``oracle_gdn.c``).

    Returns (out [B, H, T, d_v], state_out [B, H, d_k, d_v], z_out [B, H, d_k]), float64.
    """
    lib = _load()
    q, k, v = _f32(q), _f32(k), _f32(v)
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    if T != n_frames * frame_len or k.shape != q.shape or v.shape[:3] != (B, H, T):
        raise ValueError("shape mismatch")
    s_in, z = _f32(state_in), _f32(z_in)
    if s_in is not None and s_in.shape != (B, H, dk, dv):
        raise ValueError("state_in must be [B, H, d_k, d_v]")
    if z is not None and z.shape != (B, H, dk):
        raise ValueError("z_in must be [B, H, d_k]")
    out = np.zeros((B, H, T, dv), dtype=np.float64)
    s_out = np.zeros((B, H, dk, dv), dtype=np.float64)
    z_out = np.zeros((B, H, dk), dtype=np.float64)
    rc = lib.oracle_linear_attn_block_causal(_ptr(q, ctypes.c_float), _ptr(k, ctypes.c_float),
                                             _ptr(v, ctypes.c_float), _ptr(s_in, ctypes.c_float),
                                             _ptr(z, ctypes.c_float), _ptr(s_out, ctypes.c_double),
                                             _ptr(z_out, ctypes.c_double), _ptr(out, ctypes.c_double),
                                             B, H, n_frames, frame_len, dk, dv, float(eps), int(n_threads))
    if rc != 0:
        raise RuntimeError("oracle_linear_attn_block_causal failed (%d)" % rc)
    return out, s_out, z_out


def softmax_attn_block_causal(q, k, v, n_frames, kv_frames, frame_len, scale=0.0, n_threads=0):
    """Frame-block-causal softmax attention (see ``oracle_gdn.c``).

    q: [B, H, n_frames * frame_len, d_k]; k: [B, H, kv_frames * frame_len, d_k];
    v: [B, H, kv_frames * frame_len, d_v].  The queries' frames are the last n_frames of
    the kv_frames key frames.  scale <= 0 means 1 / sqrt(d_k).
    Returns out [B, H, n_frames * frame_len, d_v] float64.
    """
    lib = _load()
    q, k, v = _f32(q), _f32(k), _f32(v)
    B, H, Tq, dk = q.shape
    dv = v.shape[-1]
    if (Tq != n_frames * frame_len or k.shape != (B, H, kv_frames * frame_len, dk)
            or v.shape[:3] != (B, H, kv_frames * frame_len) or kv_frames < n_frames):
        raise ValueError("shape mismatch")
    out = np.zeros((B, H, Tq, dv), dtype=np.float64)
    rc = lib.oracle_softmax_attn_block_causal(_ptr(q, ctypes.c_float), _ptr(k, ctypes.c_float),
                                              _ptr(v, ctypes.c_float), _ptr(out, ctypes.c_double),
                                              B, H, n_frames, kv_frames, frame_len, dk, dv,
                                              float(scale), int(n_threads))
    if rc != 0:
        raise RuntimeError("oracle_softmax_attn_block_causal failed (%d)" % rc)
    return out


def temporal_conv_block(x, w, bias=None, carry_in=None):
    """Causal temporal convolution of one block with its carry (see ``oracle_gdn.c``).

    x: [B, F, P, C]; w: [3, C]; bias: [C] or None; carry_in: [B, P, C] or None.
    Returns (y [B, F, P, C], carry_out [B, P, C]) float64.
    """
    lib = _load()
    x, w = _f32(x), _f32(w)
    B, F, P, C = x.shape
    if w.shape != (3, C):
        raise ValueError("w must be [3, C]")
    bias, carry_in = _f32(bias), _f32(carry_in)
    if bias is not None and bias.shape != (C,):
        raise ValueError("bias must be [C]")
    if carry_in is not None and carry_in.shape != (B, P, C):
        raise ValueError("carry_in must be [B, P, C]")
    y = np.zeros((B, F, P, C), dtype=np.float64)
    carry = np.zeros((B, P, C), dtype=np.float64)
    rc = lib.oracle_temporal_conv_block(_ptr(x, ctypes.c_float), _ptr(carry_in, ctypes.c_float),
                                        _ptr(w, ctypes.c_float), _ptr(bias, ctypes.c_float),
                                        _ptr(y, ctypes.c_double), _ptr(carry, ctypes.c_double), B, F, P, C)
    if rc != 0:
        raise RuntimeError("oracle_temporal_conv_block failed (%d)" % rc)
    return y, carry


def rope3d(x, n_frames, grid_h, grid_w, d_t, d_h, frame_offset=0, base=10000.0):
    """3D rotary position embedding (see ``oracle_gdn.c``): x [B, H, T, d],
    T = n_frames * grid_h * grid_w.  Returns the rotated tensor, float64."""
    lib = _load()
    x = _f32(x)
    B, H, T, d = x.shape
    if T != n_frames * grid_h * grid_w:
        raise ValueError("T must be n_frames * grid_h * grid_w")
    y = np.zeros(x.shape, dtype=np.float64)
    rc = lib.oracle_rope3d(_ptr(x, ctypes.c_float), _ptr(y, ctypes.c_double), B, H, n_frames, grid_h, grid_w, d,
                           d_t, d_h, frame_offset, float(base))
    if rc != 0:
        raise RuntimeError("oracle_rope3d failed (%d)" % rc)
    return y
