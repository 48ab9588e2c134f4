"""Named synthetic workloads (shapes follow the latent grids of 480p / 720p video).

480p latent frame: 15 x 26 patches = 390 tokens; 720p: 22 x 40 = 880 tokens.
"""
from dataclasses import dataclass


@dataclass(frozen=True)
class Workload:
    name: str
    wid: int            # seed key
    kind: str           # "gdn" | "block_causal" | "stream" | "token" (per-token readout)
                        # | "softmax" (frame-block-causal softmax attention)
                        # | "tconv" (causal temporal convolution, channels H * d)
                        # | "rope" (3D rotary position embedding of q, in place)
    B: int
    H: int
    n_frames: int
    frame_len: int
    d: int
    dtype: str          # "bf16" | "f32"
    state_std: float = None
    steps: int = 1      # denoising steps for the streaming workload

    @property
    def T(self):
        return self.n_frames * self.frame_len


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_gdn_f32", 0, "gdn", 1, 2, 8, 16, 32, "f32"),
        Workload("block_causal_480p_21f", 1, "block_causal", 1, 20, 21, 390, 112, "bf16"),
        Workload("gdn_720p_5s", 2, "gdn", 1, 20, 21, 880, 112, "bf16"),
        Workload("gdn_720p_60s", 3, "gdn", 1, 20, 240, 880, 112, "bf16"),
        Workload("stream_denoise_b16", 4, "stream", 16, 20, 1, 880, 112, "bf16", state_std=0.1, steps=50),
        Workload("gdn_720p_60s_token", 5, "token", 1, 20, 240, 880, 112, "bf16"),
        Workload("softmax_720p_5s", 6, "softmax", 1, 20, 21, 880, 112, "bf16"),
        # one GPU's share of the 60 s rollout split into 8 frame ranges (30 frames each)
        Workload("gdn_720p_60s_share8", 7, "gdn", 1, 20, 30, 880, 112, "bf16"),
        # causal temporal convolution over one block: channels = H * d = 2240
        Workload("tconv_720p_5s", 8, "tconv", 1, 20, 21, 880, 112, "bf16"),
        # 3D RoPE of q on the 22 x 40 latent grid, d = 112 cut (36, 38, 38)
        Workload("rope_720p_5s", 9, "rope", 1, 20, 21, 880, 112, "bf16"),
        # the 60 s rollout with the 3D RoPE of q and k fused into the kernels' load path
        Workload("gdn_720p_60s_rope", 10, "gdn_rope", 1, 20, 240, 880, 112, "bf16"),
    ]
}
