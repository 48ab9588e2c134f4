"""CPU oracle for the frame-wise gated delta rule, block-causal ReLU linear attention and
frame-block-causal softmax attention, the causal temporal convolution with its block
carry and the 3D rotary position embedding.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py``; never by the product package.  It shares no code
with the HIP path.  Every function here is "parity pinned" by the tests in
``tests/test_oracle_pins.py``.
"""
from .oracle import (  # noqa: F401
    NORMALIZE_K,
    ADDITIVE,
    GATE_LOGITS,
    build,
    gdn_forward,
    linear_attn_block_causal,
    softmax_attn_block_causal,
    temporal_conv_block,
    rope3d,
)
