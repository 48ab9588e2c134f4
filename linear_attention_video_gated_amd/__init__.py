"""MI355X (gfx950) frame-wise recurrent linear attention: the frame-wise gated delta rule
of Gated DeltaNet and block-causal ReLU linear attention, as hand-written HIP kernels
behind a C ABI (``include/gdn.h``).  This package holds the kernel sources (``csrc/``),
their build script, the ctypes binding and the seeded synthetic-input generator."""
from .gdn import (  # noqa: F401
    ADDITIVE,
    NORMALIZE_K,
    RELU_QK,
    GdnError,
    GdnLibraryMissing,
    frame_forward,
    frame_forward_readonly,
    linear_attn_block_causal,
    workspace_bytes,
)
