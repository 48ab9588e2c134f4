"""Python binding of ``libgdn_mi355x.so`` (the C ABI of ``include/gdn.h``).

Argument marshalling only: tensors are passed as device pointers, the stream is torch's
current stream on the tensors' device, and the scratch workspace is a torch allocation.
Every step of the computation runs in the library's HIP kernels; if the library is not
built, importing works but every call raises ``GdnLibraryMissing``.
"""
from __future__ import annotations

import ctypes
import os

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libgdn_mi355x.so")

GDN_BF16, GDN_F32 = 0, 1
NORMALIZE_K, ADDITIVE, RELU_QK, OUT_F32, GATE_LOGITS, ROPE_QK = 1, 2, 4, 8, 16, 32
ENTRY_FORWARD, ENTRY_READONLY, ENTRY_BLOCK_CAUSAL, ENTRY_TOKEN = 0, 1, 2, 3
EXPORTS = ("gdn_frame_forward", "gdn_frame_forward_noalloc", "gdn_noalloc_scratch_bytes",
           "gdn_frame_forward_readonly", "gdn_token_forward", "linear_attn_block_causal",
           "softmax_attn_block_causal", "temporal_conv_block", "rope3d_apply", "gdn_workspace_bytes",
           "gdn_window_count", "gdn_status_str", "gdn_abi_version")


class GdnLibraryMissing(RuntimeError):
    pass


class GdnError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__("gdn error %d: %s" % (code, msg))
        self.code = code


ABI_VERSION = 9  # GDN_ABI_VERSION of include/gdn.h that Dims mirrors


class Dims(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("n_frames", ctypes.c_int32),
                ("frame_len", ctypes.c_int32), ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("flags", ctypes.c_uint32), ("workspace", ctypes.c_void_p),
                ("workspace_bytes", ctypes.c_size_t), ("phase_events", ctypes.c_void_p),
                ("phase_windows", ctypes.c_int32), ("window_units", ctypes.c_int32),
                ("group_frames", ctypes.c_int32), ("rope_d_t", ctypes.c_int32), ("rope_d_h", ctypes.c_int32),
                ("rope_grid_w", ctypes.c_int32), ("rope_frame_offset", ctypes.c_int32),
                ("rope_base", ctypes.c_float)]


_lib = None


def lib():
    """Load the shared library (raises GdnLibraryMissing when it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise GdnLibraryMissing("%s not found: run `python -m linear_attention_video_gated_amd.build`"
                                    % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        vp, fp = ctypes.c_void_p, ctypes.c_void_p
        dp = ctypes.POINTER(Dims)
        L.gdn_frame_forward.argtypes = [vp, vp, vp, fp, fp, fp, fp, vp, dp, vp]
        L.gdn_frame_forward.restype = ctypes.c_int
        L.gdn_frame_forward_noalloc.argtypes = [vp, vp, vp, fp, fp, fp, fp, vp, dp, vp]
        L.gdn_frame_forward_noalloc.restype = ctypes.c_int
        L.gdn_noalloc_scratch_bytes.argtypes = []
        L.gdn_noalloc_scratch_bytes.restype = ctypes.c_size_t
        L.gdn_token_forward.argtypes = [vp, vp, vp, fp, fp, fp, fp, vp, dp, vp]
        L.gdn_token_forward.restype = ctypes.c_int
        L.gdn_frame_forward_readonly.argtypes = [vp, vp, vp, fp, fp, fp, vp, dp, vp]
        L.gdn_frame_forward_readonly.restype = ctypes.c_int
        L.linear_attn_block_causal.argtypes = [vp, vp, vp, fp, fp, fp, fp, vp, dp, vp]
        L.linear_attn_block_causal.restype = ctypes.c_int
        L.softmax_attn_block_causal.argtypes = [vp, vp, vp, vp, ctypes.c_int32, dp, vp]
        L.softmax_attn_block_causal.restype = ctypes.c_int
        i32 = ctypes.c_int32
        L.temporal_conv_block.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, ctypes.c_uint32, vp, vp]
        L.temporal_conv_block.restype = ctypes.c_int
        L.rope3d_apply.argtypes = [vp, i32, i32, i32, i32, i32, i32, i32, i32, i32, ctypes.c_float, i32, vp, vp]
        L.rope3d_apply.restype = ctypes.c_int
        L.gdn_workspace_bytes.argtypes = [dp, ctypes.c_int]
        L.gdn_workspace_bytes.restype = ctypes.c_size_t
        L.gdn_window_count.argtypes = [dp, ctypes.c_int]
        L.gdn_window_count.restype = ctypes.c_int
        L.gdn_status_str.argtypes = [ctypes.c_int]
        L.gdn_status_str.restype = ctypes.c_char_p
        L.gdn_abi_version.argtypes = []
        L.gdn_abi_version.restype = ctypes.c_int
        if L.gdn_abi_version() != ABI_VERSION:  # the Dims layout above is that version's
            raise RuntimeError("%s has ABI version %d, this binding needs %d: rebuild it (build.py)"
                               % (LIB_PATH, L.gdn_abi_version(), ABI_VERSION))
        _lib = L
    return _lib


def status_str(code):
    return lib().gdn_status_str(int(code)).decode()


def _check(code):
    if code != 0:
        raise GdnError(code, status_str(code))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype_code(dt):
    if dt == torch.bfloat16:
        return GDN_BF16
    if dt == torch.float32:
        return GDN_F32
    raise TypeError("q/k/v must be bfloat16 or float32, got %s" % dt)


def make_dims(B, H, n_frames, frame_len, d, dtype_code, flags, workspace=None, nbytes=0, events=None, plan=None,
              rope=None):
    """events: None or a ctypes array of 6 * n hipEvent_t handles, recorded around the
    three launches of each of the call's first n windows (per-kernel timing).
    plan: None or a dict with "window_units" and/or "group_frames" (the dims' plan
    overrides, for tests and tuning).
    rope: None or a dict with "d_t", "d_h", "grid_w" and optionally "frame_offset" (0) and
    "base" (10000): q and k are rotated by the 3D rotary embedding on the kernels' load
    path (sets GDN_F_ROPE_QK)."""
    plan = plan or {}
    r = rope or {}
    if rope is not None:
        flags |= ROPE_QK
    return Dims(B, H, n_frames, frame_len, d, d, dtype_code, flags,
                None if workspace is None else workspace.data_ptr(), nbytes,
                None if events is None else ctypes.cast(events, ctypes.c_void_p).value,
                0 if events is None else len(events) // 6,
                int(plan.get("window_units", 0)), int(plan.get("group_frames", 0)),
                int(r.get("d_t", 0)), int(r.get("d_h", 0)), int(r.get("grid_w", 0)),
                int(r.get("frame_offset", 0)), float(r.get("base", 10000.0)))


def window_count(B, H, n_frames, frame_len, d, dtype=torch.bfloat16, flags=NORMALIZE_K, entry=ENTRY_FORWARD,
                 plan=None):
    """gdn_window_count: the number of windows (three launches each) such a call makes."""
    n = lib().gdn_window_count(ctypes.byref(make_dims(B, H, n_frames, frame_len, d, _dtype_code(dtype), flags,
                                                      plan=plan)), entry)
    _check(min(n, 0))
    return n


def workspace_bytes(B, H, n_frames, frame_len, d, dtype=torch.bfloat16, flags=NORMALIZE_K,
                    entry=ENTRY_FORWARD, plan=None):
    dims = make_dims(B, H, n_frames, frame_len, d, _dtype_code(dtype), flags, plan=plan)
    return lib().gdn_workspace_bytes(ctypes.byref(dims), entry)


# One scratch buffer per (device, stream): calls on different streams may run at the
# same time and must not share one.  Each buffer is allocated while its stream is
# current, so torch's caching allocator reuses its memory only in that stream's order
# (also when a larger call replaces it).
_ws_cache = {}


def _workspace(device, nbytes, stream):
    """A cached uint8 device buffer of at least nbytes for calls on `stream`."""
    if nbytes == 0:
        return None
    key = (torch.device(device), stream.cuda_stream)
    buf = _ws_cache.get(key)
    if buf is None or buf.numel() < nbytes:
        _ws_cache.pop(key, None)
        with torch.cuda.stream(stream):
            buf = torch.empty(nbytes, dtype=torch.uint8, device=device)
        _ws_cache[key] = buf
    return buf


def _stream_of(device, stream):
    return stream if stream is not None else torch.cuda.current_stream(device)


def _handle(stream):
    return ctypes.c_void_p(stream.cuda_stream)


def _shapes(q, k, v, n_frames, frame_len):
    if q.dim() != 4 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must all be [B, H, T, d] with equal shapes")
    B, H, T, d = q.shape
    if T != n_frames * frame_len:
        raise ValueError("T=%d != n_frames*frame_len=%d" % (T, n_frames * frame_len))
    for t in (q, k, v):
        if not t.is_cuda or not t.is_contiguous() or t.dtype != q.dtype:
            raise ValueError("q, k, v must be contiguous device tensors of one dtype")
    return B, H, T, d


def _out(q, out, out_dtype, flags):
    """Allocate / check the output; float32 output of bf16 inputs sets OUT_F32."""
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or q.dtype, device=q.device)
    if tuple(out.shape) != tuple(q.shape) or not out.is_contiguous() or out.device != q.device:
        raise ValueError("out must be a contiguous device tensor shaped like q")
    if out.dtype == torch.float32:
        flags |= OUT_F32
    elif out.dtype != q.dtype:
        raise ValueError("out must have q's dtype or float32")
    return out, flags


def _f32(t, shape, name):
    if t is None:
        return None
    if t.dtype != torch.float32 or not t.is_contiguous() or tuple(t.shape) != tuple(shape) or not t.is_cuda:
        raise ValueError("%s must be a contiguous float32 device tensor of shape %s" % (name, tuple(shape)))
    return t


def frame_forward(q, k, v, alpha, beta, n_frames, frame_len, state_in=None, state_out=None,
                  out=None, flags=NORMALIZE_K, return_state=True, stream=None, out_dtype=None,
                  events=None, plan=None, rope=None, _entry=ENTRY_FORWARD):
    """gdn_frame_forward.  Returns (out [B,H,T,d], state_out [B,H,d,d] float32 or None).
    out_dtype=torch.float32 (or a float32 ``out``) returns the unrounded float32 result.
    stream: a torch stream of q's device (default: its current stream); the outputs this
    function allocates and its scratch buffer belong to that stream.  plan: the dims' plan
    overrides; rope: the 3D rotary embedding applied to q and k on load (see make_dims)."""
    B, H, T, d = _shapes(q, k, v, n_frames, frame_len)
    alpha = _f32(alpha, (B, H, T), "alpha")
    beta = _f32(beta, (B, H, T), "beta")
    state_in = _f32(state_in, (B, H, d, d), "state_in")
    st = _stream_of(q.device, stream)
    with torch.cuda.device(q.device), torch.cuda.stream(st):
        out, flags = _out(q, out, out_dtype, flags)
        if state_out is None and return_state:
            state_out = torch.empty((B, H, d, d), dtype=torch.float32, device=q.device)
        state_out = _f32(state_out, (B, H, d, d), "state_out")
        code = _dtype_code(q.dtype)
        need = lib().gdn_workspace_bytes(ctypes.byref(make_dims(B, H, n_frames, frame_len, d, code, flags,
                                                                plan=plan, rope=rope)), _entry)
        ws = _workspace(q.device, need, st)
        dims = make_dims(B, H, n_frames, frame_len, d, code, flags, ws, 0 if ws is None else ws.numel(), events,
                         plan, rope)
        fn = lib().gdn_token_forward if _entry == ENTRY_TOKEN else lib().gdn_frame_forward
        _check(fn(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(state_in), _ptr(state_out), _ptr(out),
                  ctypes.byref(dims), _handle(st)))
    return out, state_out


def frame_forward_noalloc(q, k, v, alpha, beta, n_frames, frame_len, out, state_in=None, state_out=None,
                          flags=NORMALIZE_K, stream=None, plan=None, rope=None):
    """gdn_frame_forward_noalloc: gdn_frame_forward with the library's static device
    scratch instead of a workspace.  Allocates nothing: ``out`` (q's shape, q's dtype or
    float32) must be given, state_out is optional.  Returns (out, state_out)."""
    B, H, T, d = _shapes(q, k, v, n_frames, frame_len)
    alpha = _f32(alpha, (B, H, T), "alpha")
    beta = _f32(beta, (B, H, T), "beta")
    state_in = _f32(state_in, (B, H, d, d), "state_in")
    state_out = _f32(state_out, (B, H, d, d), "state_out")
    if out is None:
        raise ValueError("frame_forward_noalloc allocates nothing: pass out")
    out, flags = _out(q, out, None, flags)
    st = _stream_of(q.device, stream)
    dims = make_dims(B, H, n_frames, frame_len, d, _dtype_code(q.dtype), flags, plan=plan, rope=rope)
    with torch.cuda.device(q.device):
        _check(lib().gdn_frame_forward_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(state_in),
                                               _ptr(state_out), _ptr(out), ctypes.byref(dims), _handle(st)))
    return out, state_out


def token_forward(q, k, v, alpha, beta, n_frames, frame_len, state_in=None, state_out=None,
                  out=None, flags=NORMALIZE_K, return_state=True, stream=None, out_dtype=None,
                  events=None, plan=None, rope=None):
    """gdn_token_forward: every token reads the state after itself (o_t = S_t q_t).
    Same arguments and returns as frame_forward."""
    return frame_forward(q, k, v, alpha, beta, n_frames, frame_len, state_in=state_in, state_out=state_out,
                         out=out, flags=flags, return_state=return_state, stream=stream, out_dtype=out_dtype,
                         events=events, plan=plan, rope=rope, _entry=ENTRY_TOKEN)


def frame_forward_readonly(q, k, v, alpha, beta, n_frames, frame_len, state_in=None, out=None,
                           flags=NORMALIZE_K, stream=None, out_dtype=None, events=None, plan=None, rope=None):
    """gdn_frame_forward_readonly.  Returns out; state_in is never written."""
    B, H, T, d = _shapes(q, k, v, n_frames, frame_len)
    alpha = _f32(alpha, (B, H, T), "alpha")
    beta = _f32(beta, (B, H, T), "beta")
    state_in = _f32(state_in, (B, H, d, d), "state_in")
    st = _stream_of(q.device, stream)
    with torch.cuda.device(q.device), torch.cuda.stream(st):
        out, flags = _out(q, out, out_dtype, flags)
        code = _dtype_code(q.dtype)
        need = lib().gdn_workspace_bytes(ctypes.byref(make_dims(B, H, n_frames, frame_len, d, code, flags,
                                                                plan=plan, rope=rope)), ENTRY_READONLY)
        ws = _workspace(q.device, need, st)
        dims = make_dims(B, H, n_frames, frame_len, d, code, flags, ws, 0 if ws is None else ws.numel(), events,
                         plan, rope)
        _check(lib().gdn_frame_forward_readonly(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                                _ptr(state_in), _ptr(out), ctypes.byref(dims), _handle(st)))
    return out


def linear_attn_block_causal(q, k, v, n_frames, frame_len, state_in=None, z_in=None, state_out=None,
                             z_out=None, out=None, flags=RELU_QK, return_state=True, stream=None,
                             out_dtype=None, events=None, plan=None):
    """linear_attn_block_causal.  Returns (out, state_out [B,H,d,d], z_out [B,H,d])."""
    B, H, T, d = _shapes(q, k, v, n_frames, frame_len)
    state_in = _f32(state_in, (B, H, d, d), "state_in")
    z_in = _f32(z_in, (B, H, d), "z_in")
    st = _stream_of(q.device, stream)
    with torch.cuda.device(q.device), torch.cuda.stream(st):
        out, flags = _out(q, out, out_dtype, flags)
        if return_state:
            if state_out is None:
                state_out = torch.empty((B, H, d, d), dtype=torch.float32, device=q.device)
            if z_out is None:
                z_out = torch.empty((B, H, d), dtype=torch.float32, device=q.device)
        state_out = _f32(state_out, (B, H, d, d), "state_out")
        z_out = _f32(z_out, (B, H, d), "z_out")
        code = _dtype_code(q.dtype)
        need = lib().gdn_workspace_bytes(ctypes.byref(make_dims(B, H, n_frames, frame_len, d, code, flags,
                                                                plan=plan)), ENTRY_BLOCK_CAUSAL)
        ws = _workspace(q.device, need, st)
        dims = make_dims(B, H, n_frames, frame_len, d, code, flags, ws, 0 if ws is None else ws.numel(), events,
                         plan)
        _check(lib().linear_attn_block_causal(_ptr(q), _ptr(k), _ptr(v), _ptr(state_in), _ptr(z_in),
                                              _ptr(state_out), _ptr(z_out), _ptr(out), ctypes.byref(dims),
                                              _handle(st)))
    return out, state_out, z_out


def softmax_attn_block_causal(q, k, v, n_frames, kv_frames, frame_len, out=None, stream=None, out_dtype=None,
                              events=None):
    """softmax_attn_block_causal: q [B,H,n_frames*frame_len,d] against k, v
    [B,H,kv_frames*frame_len,d] (the last n_frames frames are the queries' own).
    Returns out shaped like q (float32 with out_dtype=torch.float32 or a float32 out)."""
    if q.dim() != 4 or k.dim() != 4 or k.shape != v.shape or k.shape[:2] != q.shape[:2] or k.shape[3] != q.shape[3]:
        raise ValueError("q must be [B, H, Tq, d] and k, v [B, H, Tk, d]")
    B, H, Tq, d = q.shape
    if Tq != n_frames * frame_len or k.shape[2] != kv_frames * frame_len:
        raise ValueError("Tq=%d, Tk=%d do not match n_frames=%d, kv_frames=%d, frame_len=%d"
                         % (Tq, k.shape[2], n_frames, kv_frames, frame_len))
    for t in (q, k, v):
        if not t.is_cuda or not t.is_contiguous() or t.dtype != q.dtype:
            raise ValueError("q, k, v must be contiguous device tensors of one dtype")
    st = _stream_of(q.device, stream)
    with torch.cuda.device(q.device), torch.cuda.stream(st):
        out, flags = _out(q, out, out_dtype, 0)
        dims = make_dims(B, H, n_frames, frame_len, d, _dtype_code(q.dtype), flags, events=events)
        _check(lib().softmax_attn_block_causal(_ptr(q), _ptr(k), _ptr(v), _ptr(out), int(kv_frames),
                                               ctypes.byref(dims), _handle(st)))
    return out


def temporal_conv_block(x, weight, bias=None, carry_in=None, carry_out=None, out=None, stream=None,
                        out_dtype=None, events=None, return_carry=True):
    """temporal_conv_block: x [B, F, P, C] (bf16 or float32), weight [3, C] and bias [C]
    float32, carry_in [B, P, C] in x's dtype or None.  Returns (y, carry_out)."""
    if x.dim() != 4 or not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous [B, F, P, C] device tensor")
    B, F, P, C = x.shape
    if carry_in is not None and (tuple(carry_in.shape) != (B, P, C) or carry_in.dtype != x.dtype
                                 or not carry_in.is_contiguous()):
        raise ValueError("carry_in must be a contiguous [B, P, C] tensor of x's dtype")
    weight = _f32(weight, (3, C), "weight")
    bias = _f32(bias, (C,), "bias")
    st = _stream_of(x.device, stream)
    with torch.cuda.device(x.device), torch.cuda.stream(st):
        if out is None:
            out = torch.empty(x.shape, dtype=out_dtype or x.dtype, device=x.device)
        if tuple(out.shape) != tuple(x.shape) or not out.is_contiguous():
            raise ValueError("out must be a contiguous tensor shaped like x")
        flags = OUT_F32 if out.dtype == torch.float32 and x.dtype != torch.float32 else 0
        if out.dtype not in (x.dtype, torch.float32):
            raise ValueError("out must have x's dtype or float32")
        if carry_out is None and return_carry:
            carry_out = torch.empty((B, P, C), dtype=x.dtype, device=x.device)
        ev = None if events is None else ctypes.cast(events, ctypes.c_void_p)
        _check(lib().temporal_conv_block(_ptr(x), _ptr(carry_in), _ptr(weight), _ptr(bias), _ptr(out),
                                         _ptr(carry_out), B, F, P, C, _dtype_code(x.dtype), flags, ev, _handle(st)))
    return out, carry_out


def rope3d_apply(x, n_frames, grid_h, grid_w, d_t, d_h, frame_offset=0, base=10000.0, stream=None, events=None):
    """rope3d_apply: rotates x [B, H, T, d] (bf16 or float32) in place and returns it."""
    if x.dim() != 4 or not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous [B, H, T, d] device tensor")
    B, H, T, d = x.shape
    if T != n_frames * grid_h * grid_w:
        raise ValueError("T=%d != n_frames * grid_h * grid_w" % T)
    ev = None if events is None else ctypes.cast(events, ctypes.c_void_p)
    st = _stream_of(x.device, stream)
    with torch.cuda.device(x.device):
        _check(lib().rope3d_apply(_ptr(x), B, H, n_frames, grid_h, grid_w, d, d_t, d_h, frame_offset, float(base),
                                  _dtype_code(x.dtype), ev, _handle(st)))
    return x
