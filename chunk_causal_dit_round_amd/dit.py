"""Device buffers of the DiT block around the round (``include/wf_dit.h``).

Plumbing only: torch allocates the weights, modulation, residual stream and
workspace the C ABI asks for, and this class passes pointers.  Every step of
the block runs in libwf.so (its kernels, and hipBLASLt for the products).
"""

import torch

from . import synth, wf
from .session import Session


class DitSession:
    """A Session plus one request's DiT state: weights of every layer
    (dummy, seeded by ``tag``), per-layer modulation [L][S+1][6][C] and the
    residual stream x [S+1][N][C] (fp32)."""

    def __init__(self, session: Session, ffn_dim: int, tag: str, eps: float = 0.0):
        s = session
        self.s = s
        self.tag = tag
        self.C = s.H * s.D
        self.F = ffn_dim
        dev = s.device
        self.dc = wf.make_dit_config(ffn_dim, eps)
        self.layers = [synth.dit_layer_weights(tag, l, self.C, ffn_dim, dev) for l in range(s.L)]
        self.weights = wf.make_dit_weights(self.layers)
        self.mod = torch.stack([synth.dit_modulation(tag, l, s.S + 1, self.C, dev)
                                for l in range(s.L)]).contiguous()
        self.x = torch.zeros((s.S + 1, s.N, self.C), dtype=torch.float32, device=dev)
        self.work_bytes = wf.wf_dit_workspace_bytes(s.h, self.dc)
        self.work = torch.empty(self.work_bytes, dtype=torch.uint8, device=dev)

    def tune(self, stream=None) -> None:
        """Pick the fastest hipBLASLt algorithm of each full-width product
        (blocking; overwrites the work buffer)."""
        wf.wf_dit_tune(self.s.h, self.dc, self.weights, self.work, self.work_bytes, stream)

    def load_x0(self, rnd: int, stages=None) -> None:
        """x of every (or the given) stage <- the round's seeded layer-0 input."""
        for st in (range(self.s.S + 1) if stages is None else stages):
            self.x[st].copy_(synth.dit_x0(self.tag, rnd, st, self.s.N, self.C, self.s.device))

    def layer(self, plan, layer: int, stream=None) -> None:
        wf.wf_dit_layer(self.s.h, plan, layer, self.dc, self.weights, self.mod[layer], self.x,
                        self.work, self.work_bytes, stream)

    def round(self, plan, stream=None) -> None:
        wf.wf_dit_round(self.s.h, plan, self.dc, self.weights, self.mod, self.x, self.work,
                        self.work_bytes, stream)
