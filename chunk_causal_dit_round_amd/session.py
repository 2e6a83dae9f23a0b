"""Device buffers for one request, bound to a wf handle.

Plumbing only: torch allocates the caller-owned memory the C ABI asks for
(slot pool, anchor store, RoPE tables, per-round q/k/v/q_rot/out) and this
class passes pointers.  All compute happens in libwf.so.
"""

import torch

from . import wf

# q/k/v/q_rot/out and anchor_raw element type; FP8 and FP8K configs keep them bf16
TORCH_DTYPE = {wf.WF_F32: torch.float32, wf.WF_BF16: torch.bfloat16, wf.WF_FP8: torch.bfloat16,
               wf.WF_FP8K: torch.bfloat16}


class Session:
    def __init__(self, cfg: "wf.wf_config", device="cuda", io=True):
        self.cfg = cfg
        self.device = torch.device(device)
        self.dtype = TORCH_DTYPE[cfg.dtype]
        self.h = wf.wf_create(cfg)
        self.pool_bytes, self.anchor_bytes, self.table_bytes = wf.wf_pool_bytes(cfg)
        self.pool = torch.empty(self.pool_bytes, dtype=torch.uint8, device=self.device)
        self.anchor = torch.empty(self.anchor_bytes, dtype=torch.uint8, device=self.device)
        self.tables = torch.empty(self.table_bytes, dtype=torch.uint8, device=self.device)
        wf.wf_bind(self.h, self.pool, self.pool_bytes, self.anchor, self.anchor_bytes,
                   self.tables, self.table_bytes)
        S, N, H, D, L = cfg.S, cfg.F * cfg.Hh * cfg.Ww, cfg.n_heads, cfg.head_dim, cfg.n_layers
        self.S, self.N, self.H, self.D, self.L = S, N, H, D, L
        lay = wf.wf_page_layout(cfg)
        self.layout = lay
        self.n_slots = lay.n_slots
        self.page_bytes = lay.page_bytes
        self.T = lay.tiles
        self.Npad = lay.tokens_padded
        self.bufs = self.alloc_io() if io else None

    def alloc_io(self):
        shape = (self.L, self.S + 1, self.N, self.H, self.D)
        return {n: torch.zeros(shape, dtype=self.dtype, device=self.device)
                for n in ("q", "k", "v", "q_rot", "out")}

    # ---- views of the slot pool (layouts documented in include/wf.h) ----
    def slot_bytes(self, layer: int, slot: int):
        """All bytes of one slot of one layer (uint8), whatever the page format."""
        return self.pool.view(self.L, self.n_slots, self.page_bytes)[layer, slot]

    _slot_bytes = slot_bytes

    def page(self, layer: int, slot: int):
        """(K [H][N][D], Vt [H][D][N]) views of one slot of one layer."""
        p = self._slot_bytes(layer, slot)
        vo = self.layout.vt_offset
        return (p[:vo].view(self.dtype).view(self.H, self.N, self.D),
                p[vo:2 * vo].view(self.dtype).view(self.H, self.D, self.N))

    def fp8_page(self, layer: int, slot: int):
        """(K8 [H][Npad][D], Vt [H][D][Npad], codes [H][T][2]) views of one
        slot of an FP8 or FP8K pool (codes: exponent + 127 of K, V per tile).
        K8 and codes are uint8; Vt is uint8 E4M3 codes (FP8) or bf16 (FP8K)."""
        H, D, Np, T = self.H, self.D, self.Npad, self.T
        p = self._slot_bytes(layer, slot)
        vo, co = self.layout.vt_offset, self.layout.codes_offset
        vt = p[vo:co]
        vt = vt.view(torch.bfloat16) if self.cfg.dtype == wf.WF_FP8K else vt
        return p[:vo].view(H, Np, D), vt.view(H, D, Np), p[co:co + 2 * H * T].view(H, T, 2)

    def anchor_page(self, layer: int):
        hnd = self.H * self.N * self.D
        a = self.anchor.view(self.dtype).view(self.L, 2 * hnd)[layer]
        return a[:hnd].view(self.H, self.N, self.D), a[hnd:].view(self.H, self.D, self.N)

    # ---- thin wrappers ----
    def plan(self, k: int):
        return wf.wf_round_plan(self.h, k)

    def next_round(self) -> int:
        return wf.wf_next_round(self.h)

    def run_round(self, plan, bufs=None, stream=None):
        b = self.bufs if bufs is None else bufs
        wf.wf_round(self.h, plan, b["q"], b["k"], b["v"], b["q_rot"], b["out"], stream)

    def publish(self, plan, layer, bufs=None, stream=None):
        b = self.bufs if bufs is None else bufs
        wf.wf_kv_publish(self.h, plan, layer, b["q"][layer], b["k"][layer], b["v"][layer],
                         b["q_rot"][layer], stream)

    def attention(self, plan, layer, bufs=None, stream=None):
        b = self.bufs if bufs is None else bufs
        wf.wf_wave_attention(self.h, plan, layer, b["q_rot"][layer], b["out"][layer], stream)

    def commit(self, plan):
        wf.wf_round_commit(self.h, plan)

    def close(self):
        if self.h is not None:
            wf.wf_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
