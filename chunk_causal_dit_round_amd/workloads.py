"""Named round shapes (synthetic Wan2.1-shaped workloads).

832x480 video, 8x VAE, 2x2 patchify -> 30x52 tokens per latent frame; three
latent frames per chunk -> 4680 tokens; 399 latent frames -> 133 chunks
("Wave Forcing: Towards Speed-of-Light Streaming Video Generation", §5 and
App. C, App. B.4).  Head counts: 12 x 128 for the 1.3B shape, 40 x 128 for
the 14B-class shape.
"""

from dataclasses import dataclass, replace

from . import wf


@dataclass(frozen=True)
class Workload:
    name: str
    S: int
    W: int
    n_chunk: int
    F: int
    Hh: int
    Ww: int
    n_heads: int
    head_dim: int
    n_layers: int
    dtype: int = wf.WF_BF16
    mask: int = wf.WF_MASK_WAVE
    W_store: int = -1
    anchor: int = 1
    q_head_scale: bool = False     # per-head U(0.5, 2) scale on q
    max_frames: int = 0            # unbounded requests (n_chunk <= 0): frames reachable

    @property
    def n_tokens(self) -> int:
        return self.F * self.Hh * self.Ww

    def config(self) -> "wf.wf_config":
        return wf.make_config(self.S, self.W, self.n_chunk, self.F, self.Hh, self.Ww,
                              self.n_heads, self.head_dim, self.n_layers, W_store=self.W_store,
                              anchor=self.anchor, dtype=self.dtype, mask=self.mask,
                              max_frames=self.max_frames)

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# Tiny fp32 round: 3 x 4x6 tokens, 2 heads x 64, W = 2, one layer, 8 rounds.
TINY_FP32 = Workload("tiny_fp32_s2", S=2, W=2, n_chunk=6, F=3, Hh=4, Ww=6,
                     n_heads=2, head_dim=64, n_layers=1, dtype=wf.WF_F32)
# 1.3B shape, 4 steps (12 x 128, 30 layers).  The long rollout is this
# shape over all 133 chunks (137 rounds).
WAN13B_4STEP = Workload("wan1.3b_4step", S=4, W=4, n_chunk=133, F=3, Hh=30, Ww=52,
                        n_heads=12, head_dim=128, n_layers=30)
WAN13B_5STEP = Workload("wan1.3b_5step", S=5, W=6, n_chunk=133, F=3, Hh=30, Ww=52,
                        n_heads=12, head_dim=128, n_layers=30)
WAN13B_5STEP_ROLLING = WAN13B_5STEP.with_(name="wan1.3b_5step_rolling",
                                          mask=wf.WF_MASK_ROLLING)
WAN14B_4STEP = Workload("wan14b_4step", S=4, W=4, n_chunk=133, F=3, Hh=30, Ww=52,
                        n_heads=40, head_dim=128, n_layers=40, q_head_scale=True)

# The same 1.3B round over FP8 (E4M3) pages (App. C.6 variant).
WAN13B_4STEP_FP8 = WAN13B_4STEP.with_(name="wan1.3b_4step_fp8", dtype=wf.WF_FP8)
# ... and over 8-bit-key pages (FP8 keys, bf16 values: the 8-bit QK^T tier of
# App. B.1 / App. C.2 Tab. 4).
WAN13B_4STEP_FP8K = WAN13B_4STEP.with_(name="wan1.3b_4step_fp8k", dtype=wf.WF_FP8K)

ALL = {w.name: w for w in (TINY_FP32, WAN13B_4STEP, WAN13B_5STEP, WAN13B_5STEP_ROLLING,
                           WAN14B_4STEP, WAN13B_4STEP_FP8, WAN13B_4STEP_FP8K)}
