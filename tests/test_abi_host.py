"""The C ABI library loads, exports exactly what include/gdn.h declares, and rejects bad
arguments on the host, before anything is enqueued (no GPU needed: every call here
returns from argument checking)."""
import ctypes
import os
import re
import subprocess

import pytest

from linear_attention_video_gated_amd import gdn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")

pytestmark = pytest.mark.skipif(not os.path.exists(gdn.LIB_PATH), reason="library not built")

FAKE = 0x7F0000000000  # a 256-byte aligned non-NULL address; never dereferenced here


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(\w+)\s*\(", text, re.M)))


def test_header_declares_the_documented_entry_points():
    assert declared_functions() == sorted(gdn.EXPORTS)


def test_library_exports_every_declared_symbol_and_nothing_else():
    out = subprocess.run(["nm", "-D", "--defined-only", gdn.LIB_PATH], capture_output=True, text=True).stdout
    exported = sorted({ln.split()[-1] for ln in out.splitlines() if " T " in ln and not ln.split()[-1].startswith("_")})
    assert exported == declared_functions()
    L = gdn.lib()
    for name in declared_functions():
        assert hasattr(L, name)


def test_abi_version_and_status_strings():
    assert gdn.lib().gdn_abi_version() == 9
    for code in range(0, -9, -1):
        s = gdn.status_str(code)
        assert s and s != "unknown status"
    assert gdn.status_str(-99) == "unknown status"


def dims(B=1, H=2, F=3, N=16, d=32, dtype=gdn.GDN_BF16, flags=gdn.NORMALIZE_K, ws=None, nbytes=0, wu=0, gf=0):
    return gdn.Dims(B, H, F, N, d, d, dtype, flags, ws, nbytes, None, 0, wu, gf, 0, 0, 0, 0, 10000.0)


def wsb(dm, entry=gdn.ENTRY_FORWARD):
    return gdn.lib().gdn_workspace_bytes(ctypes.byref(dm), entry)


def fwd(dm, q=FAKE, k=FAKE + 2 ** 28, v=FAKE + 2 ** 29, a=FAKE + 2 ** 30, b=FAKE + 2 ** 31,
        s_in=None, s_out=None, out=FAKE + 2 ** 32):
    return gdn.lib().gdn_frame_forward(q, k, v, a, b, s_in, s_out, out, ctypes.byref(dm), None)


def test_workspace_is_bounded_independently_of_frame_count():
    frames = [1, 2, 3, 7, 21, 100, 240, 409, 410, 1000, 5000, 100000, 200000]
    sizes = [wsb(dims(B=1, H=20, F=F, N=880, d=112)) for F in frames]
    assert min(sizes) > 0
    # one window of at most 8192 (b, h, frame) units: bounded by 8192 / (B H) frames'
    # worth of the one-frame workspace (which holds one frame per (b, h)), whatever F
    assert max(sizes) <= (8192 / 20) * sizes[0]
    # nor with the frame length (which only changes how frames are grouped)
    one = wsb(dims(F=1, N=16, d=112))
    assert one == wsb(dims(F=1, N=4000, d=112))
    for N in (1, 16, 390, 880, 4000):
        assert wsb(dims(F=240, N=N, d=112)) <= (8192 / 2) * one


def test_window_plan():
    """Windows hold whole groups of frames and at most 8192 (b, h, frame) units."""
    L = gdn.lib()
    assert L.gdn_window_count(ctypes.byref(dims(B=1, H=20, F=240, N=880, d=112)), gdn.ENTRY_FORWARD) == 1
    assert L.gdn_window_count(ctypes.byref(dims(B=1, H=20, F=1000, N=880, d=112)), gdn.ENTRY_FORWARD) == 3
    assert L.gdn_window_count(ctypes.byref(dims(B=1, H=2, F=1, N=16, d=32)), gdn.ENTRY_FORWARD) == 1
    assert L.gdn_window_count(ctypes.byref(dims(d=48)), gdn.ENTRY_FORWARD) == -7
    assert L.gdn_window_count(ctypes.byref(dims()), 9) == -7
    # block-causal calls are not cut beyond the workspace bound
    assert L.gdn_window_count(ctypes.byref(dims(B=1, H=20, F=21, N=390, d=112, flags=gdn.RELU_QK)),
                              gdn.ENTRY_BLOCK_CAUSAL) == 1


def test_plan_overrides():
    """dims.window_units and dims.group_frames cut the call differently (tests and tuning)."""
    L = gdn.lib()
    assert L.gdn_window_count(ctypes.byref(dims(B=1, H=2, F=7, N=90, d=112, wu=4)), gdn.ENTRY_FORWARD) == 4
    assert L.gdn_window_count(ctypes.byref(dims(B=1, H=2, F=7, N=90, d=112, wu=4, gf=1)), gdn.ENTRY_FORWARD) == 4
    # a group is never cut by a window: 3-frame groups in windows of >= 3 frames
    assert L.gdn_window_count(ctypes.byref(dims(B=1, H=2, F=7, N=90, d=112, wu=4, gf=3)), gdn.ENTRY_FORWARD) == 3
    # more frames per group -> fewer group maps in the workspace
    assert wsb(dims(B=1, H=2, F=40, N=90, d=112, gf=40)) < wsb(dims(B=1, H=2, F=40, N=90, d=112, gf=1))


def test_workspace_zero_for_invalid_or_empty():
    assert wsb(dims(d=48)) == 0            # unsupported d
    assert wsb(dims(dtype=7)) == 0
    assert wsb(dims(F=0)) == 0
    assert wsb(dims(), entry=9) == 0


@pytest.mark.parametrize("field,val,code", [
    ("dtype", 5, -3), ("B", -1, -2), ("frame_len", 0, -2), ("n_frames", -2, -2),
    ("d_k", 48, -7), ("flags", 64, -7), ("flags", gdn.RELU_QK, -7),
    ("window_units", -1, -2), ("group_frames", -3, -2),
])
def test_bad_dims_rejected(field, val, code):
    dm = dims()
    setattr(dm, field, val)
    assert fwd(dm) == code


def test_dv_must_equal_dk():
    dm = dims()
    dm.d_v = 64
    assert fwd(dm) == -7


def test_null_dims_and_pointers():
    assert gdn.lib().gdn_frame_forward(FAKE, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, None, None) == -1
    assert fwd(dims(), q=None) == -1
    assert fwd(dims(), a=None) == -1
    assert fwd(dims(flags=gdn.NORMALIZE_K | gdn.ADDITIVE), a=None, b=None) == -6  # gates optional, then workspace


def test_misaligned_pointer_rejected():
    dm = dims(ws=FAKE + 2 ** 34, nbytes=1 << 30)
    assert fwd(dm, q=FAKE + 2) == -4
    assert fwd(dm, s_in=FAKE + 2 ** 33 + 8) == -4


def test_missing_or_small_workspace_rejected():
    dm = dims()
    assert fwd(dm) == -6
    need = wsb(dm)
    dm.workspace, dm.workspace_bytes = FAKE + 2 ** 34, need - 1
    assert fwd(dm) == -6


def test_overlapping_output_rejected():
    dm = dims(ws=FAKE + 2 ** 34, nbytes=1 << 30)
    assert fwd(dm, out=FAKE) == -5                      # out == q
    assert fwd(dm, out=FAKE + 2 ** 28 + 256) == -5      # out inside k
    assert fwd(dm, out=FAKE + 2 ** 34 + 4096) == -5     # out inside the workspace
    assert fwd(dm, s_out=FAKE + 2 ** 29) == -5          # state_out inside v


def test_block_causal_flag_rules():
    dm = dims(flags=gdn.NORMALIZE_K)
    assert gdn.lib().linear_attn_block_causal(FAKE, FAKE, FAKE, None, None, None, None, FAKE,
                                              ctypes.byref(dm), None) == -7
    dm = dims(flags=gdn.RELU_QK)
    assert gdn.lib().linear_attn_block_causal(FAKE, FAKE + 2 ** 28, FAKE + 2 ** 29, None, None, None, None,
                                              FAKE + 2 ** 30, ctypes.byref(dm), None) == -6
    dm = dims(flags=gdn.RELU_QK | gdn.GATE_LOGITS)  # gate logits belong to the gated delta rule
    assert gdn.lib().linear_attn_block_causal(FAKE, FAKE, FAKE, None, None, None, None, FAKE,
                                              ctypes.byref(dm), None) == -7


def test_empty_batch_is_a_noop():
    assert fwd(dims(B=0)) == 0
    assert fwd(dims(H=0), q=None) == 0


def test_binding_fails_loudly_without_library(monkeypatch):
    monkeypatch.setattr(gdn, "_lib", None)
    monkeypatch.setattr(gdn, "LIB_PATH", "/nonexistent/libgdn_mi355x.so")
    with pytest.raises(gdn.GdnLibraryMissing):
        gdn.lib()


def sa(dm, kv_frames=None, q=FAKE, k=FAKE + 2 ** 28, v=FAKE + 2 ** 29, out=FAKE + 2 ** 32):
    kv = dm.n_frames if kv_frames is None else kv_frames
    return gdn.lib().softmax_attn_block_causal(q, k, v, out, kv, ctypes.byref(dm), None)


def test_softmax_attention_argument_checks():
    L = gdn.lib()
    assert L.softmax_attn_block_causal(FAKE, FAKE, FAKE, FAKE, 3, None, None) == -1
    assert sa(dims(flags=0), kv_frames=2) == -2           # fewer key frames than query frames
    assert sa(dims(flags=gdn.NORMALIZE_K)) == -7          # only OUT_F32 applies here
    assert sa(dims(flags=gdn.RELU_QK)) == -7
    assert sa(dims(flags=0, d=48)) == -7
    assert sa(dims(flags=0, dtype=7)) == -3
    dm = dims(flags=0)
    dm.frame_len = 0
    assert sa(dm) == -2
    assert sa(dims(flags=0), q=None) == -1
    assert sa(dims(flags=0), v=FAKE + 2 ** 29 + 8) == -4
    assert sa(dims(flags=0), out=FAKE + 64) == -5          # out inside q
    assert sa(dims(flags=gdn.OUT_F32), kv_frames=5, out=FAKE + 2 ** 29 + 4096) == -5  # inside v
    # nothing to compute: no pointer is looked at
    assert sa(dims(flags=0, B=0), q=None, k=None, v=None, out=None) == 0
    assert sa(dims(flags=0, F=0), kv_frames=4, q=None, k=None, v=None, out=None) == 0


def test_softmax_attention_size_limits():
    # key tensors past the element-count bound, and a grid past 2^31 workgroups
    dm = dims(flags=0, B=1, H=1, F=1, N=1 << 30, d=128)
    assert sa(dm, kv_frames=1 << 10) == -2
    dm = dims(flags=0, B=65535, H=65535, F=1, N=128, d=16)
    assert sa(dm) == -2


def test_temporal_conv_argument_checks():
    """Every call here is rejected (or has nothing to do) before any launch."""
    L = gdn.lib()
    tc = lambda B=1, F=3, P=4, C=16, dtype=gdn.GDN_BF16, flags=0, x=FAKE, cin=None, w=FAKE + 2 ** 30, b=None, \
        y=FAKE + 2 ** 31, cout=None: L.temporal_conv_block(x, cin, w, b, y, cout, B, F, P, C, dtype, flags, None, None)
    assert tc(dtype=5) == -3
    assert tc(F=-1) == -2
    assert tc(flags=gdn.NORMALIZE_K) == -7
    assert tc(C=12) == -7                      # bf16 channels come in groups of 8
    assert tc(C=12, dtype=gdn.GDN_F32, w=None) == -1  # float32: groups of 4 (then the NULL weight)
    assert tc(w=None) == -1
    assert tc(x=None) == -1
    assert tc(x=FAKE + 8) == -4
    assert tc(y=FAKE + 64) == -5                # y inside x
    assert tc(B=0) == 0 and tc(P=0, x=None, y=None) == 0
    # an empty block needs no x or y (it only passes the carry on): past the NULL check,
    # stopped by the misaligned carry_out
    assert tc(F=0, x=None, y=None, cout=FAKE + 2 ** 32 + 8) == -4


def test_rope3d_argument_checks():
    """Every call here is rejected (or has nothing to do) before any launch."""
    L = gdn.lib()
    rp = lambda x=FAKE, B=1, H=2, F=3, gh=2, gw=4, d=16, dt=4, dh=6, off=0, base=10000.0, dtype=gdn.GDN_BF16: \
        L.rope3d_apply(x, B, H, F, gh, gw, d, dt, dh, off, base, dtype, None, None)
    assert rp(dtype=9) == -3
    assert rp(dt=3, dh=7) == -7              # odd parts
    assert rp(d=12) == -7                    # bf16 rows are whole 16-byte groups
    assert rp(dt=10, dh=10) == -2            # d_w < 0
    assert rp(base=0.0) == -2
    assert rp(gh=0) == -2
    assert rp(off=1 << 24) == -2
    assert rp(x=None) == -1
    assert rp(x=FAKE + 8) == -4
    assert rp(B=0, x=None) == 0 and rp(F=0, x=None) == 0


def test_noalloc_entry_rejects_calls_beyond_its_scratch():
    """gdn_frame_forward_noalloc: a call whose workspace exceeds the static scratch returns
    GDN_ERR_WORKSPACE before anything is enqueued (the 60 s rollout in one window does);
    argument errors are those of gdn_frame_forward."""
    L = gdn.lib()
    cap = L.gdn_noalloc_scratch_bytes()
    assert cap == 64 << 20
    big = dims(B=1, H=20, F=240, N=880, d=112)
    assert wsb(big) > cap
    f = L.gdn_frame_forward_noalloc
    args = (FAKE, FAKE + 2 ** 28, FAKE + 2 ** 29, FAKE + 2 ** 30, FAKE + 2 ** 31, None, None, FAKE + 2 ** 32)
    assert f(*args, ctypes.byref(big), None) == -6
    assert f(*args, None, None) == -1
    bad = dims(d=48)
    assert f(*args, ctypes.byref(bad), None) == -7
    # a smaller window makes the same call fit
    small = dims(B=1, H=20, F=240, N=880, d=112, wu=400)
    assert 0 < wsb(small) <= cap


def test_rope_flag_rules():
    """GDN_F_ROPE_QK: the gated-delta-rule entries only; parts even and within d; the frame
    length a whole number of latent rows; frames below 2^24."""
    def rd(dt=4, dh=6, gw=4, off=0, base=100.0, N=16, d=32, F=3):
        dm = dims(N=N, d=d, F=F, flags=gdn.NORMALIZE_K | gdn.ROPE_QK)
        dm.rope_d_t, dm.rope_d_h, dm.rope_grid_w, dm.rope_frame_offset, dm.rope_base = dt, dh, gw, off, base
        return dm
    L = gdn.lib()
    assert wsb(rd()) > 0
    assert wsb(rd(), entry=gdn.ENTRY_READONLY) > 0
    assert wsb(rd(), entry=gdn.ENTRY_TOKEN) > 0                         # the per-token entry too
    bc = rd()
    bc.flags = 0
    assert L.gdn_window_count(ctypes.byref(bc), gdn.ENTRY_BLOCK_CAUSAL) == 1
    bc.flags = gdn.ROPE_QK                                              # not the block-causal entry
    assert L.gdn_window_count(ctypes.byref(bc), gdn.ENTRY_BLOCK_CAUSAL) == -7
    assert L.gdn_window_count(ctypes.byref(rd(dt=3, dh=7)), gdn.ENTRY_FORWARD) == -7   # odd parts
    assert L.gdn_window_count(ctypes.byref(rd(dt=30, dh=6)), gdn.ENTRY_FORWARD) == -2  # beyond d
    assert L.gdn_window_count(ctypes.byref(rd(gw=5)), gdn.ENTRY_FORWARD) == -2         # 16 % 5 != 0
    assert L.gdn_window_count(ctypes.byref(rd(gw=0)), gdn.ENTRY_FORWARD) == -2
    assert L.gdn_window_count(ctypes.byref(rd(base=0.0)), gdn.ENTRY_FORWARD) == -2
    assert L.gdn_window_count(ctypes.byref(rd(off=(1 << 24) - 2)), gdn.ENTRY_FORWARD) == -2
    assert L.gdn_window_count(ctypes.byref(rd(off=(1 << 24) - 3)), gdn.ENTRY_FORWARD) == 1
