"""Seeded synthetic inputs (q, k, v projections) for wavefront rounds.

Holds no arithmetic of the method: only random numbers and their seeds.
Every (round, layer, stage, tensor) slice has its own seed, so any single
slice can be regenerated on its own (tests rebuild the inputs a history
page was produced from without keeping old rounds around).

Values: N(0, 1) drawn in fp32 by torch's generator on the target device,
optionally scaled per head (q only), then cast to the round dtype.
"""

import math
import zlib

import torch

_MASK = (1 << 64) - 1
BASE_SEED = 42
NAMES = ("q", "k", "v")


def _splitmix(h: int, x: int) -> int:
    h = (h + 0x9E3779B97F4A7C15 + x) & _MASK
    z = h
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK
    return z ^ (z >> 31)


def seed_of(*parts) -> int:
    """Stable 63-bit seed from ints and strings."""
    h = 0
    for p in parts:
        x = zlib.crc32(p.encode()) if isinstance(p, str) else int(p) & _MASK
        h = _splitmix(h, x)
    return h & ((1 << 63) - 1)


def head_scales(n_heads: int, tag: str, lo: float = 0.5, hi: float = 2.0) -> torch.Tensor:
    """Per-head query scale c_h ~ U(lo, hi), seeded by (BASE_SEED, tag); CPU fp32."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed_of(BASE_SEED, tag, "head-scale"))
    return lo + (hi - lo) * torch.rand(n_heads, generator=g, dtype=torch.float32)


def slice_input(tag: str, rnd: int, layer: int, stage: int, name: str, n_tokens: int,
                n_heads: int, head_dim: int, device, dtype,
                q_scale: torch.Tensor = None) -> torch.Tensor:
    """One [N, H, D] projection slice, regenerated bit-for-bit from its seed."""
    g = torch.Generator(device=device)
    g.manual_seed(seed_of(BASE_SEED, tag, rnd, layer, stage, NAMES.index(name)))
    x = torch.randn((n_tokens, n_heads, head_dim), generator=g, device=device,
                    dtype=torch.float32)
    if name == "q" and q_scale is not None:
        x *= q_scale.to(device=x.device).view(1, -1, 1)
    return x.to(dtype)


def fill_round(bufs: dict, tag: str, rnd: int, n_layers: int, n_stages: int,
               q_scale: torch.Tensor = None, layers=None, stages=None) -> None:
    """Fill bufs['q'|'k'|'v'] ([L][S+1][N][H][D]) with round ``rnd``'s inputs."""
    q = bufs["q"]
    _, _, n, hh, d = q.shape
    for layer in (range(n_layers) if layers is None else layers):
        for s in (range(n_stages) if stages is None else stages):
            for name in NAMES:
                bufs[name][layer, s].copy_(slice_input(tag, rnd, layer, s, name, n, hh, d,
                                                       q.device, q.dtype, q_scale))


# ---- DiT block around the round: dummy (random-init) weights and inputs ----
def _gen(device, *parts):
    g = torch.Generator(device=device)
    g.manual_seed(seed_of(BASE_SEED, *parts))
    return g


def dit_layer_weights(tag: str, layer: int, C: int, F: int, device) -> dict:
    """One layer's weights: W [out][in] ~ N(0, 1/in) in bf16; biases
    ~ N(0, 0.1^2), RMSNorm gains ~ 1 + N(0, 0.1^2), fp32."""
    g = _gen(device, tag, "dit-weights", layer)

    def mat(o, i):
        return (torch.randn((o, i), generator=g, device=device) / math.sqrt(i)).to(torch.bfloat16)

    def vec(n, base=0.0):
        return base + 0.1 * torch.randn(n, generator=g, device=device)

    return dict(w_qkv=mat(3 * C, C), b_qkv=vec(3 * C), g_q=vec(C, 1.0), g_k=vec(C, 1.0),
                w_o=mat(C, C), b_o=vec(C), w_1=mat(F, C), b_1=vec(F), w_2=mat(C, F), b_2=vec(C))


def dit_modulation(tag: str, layer: int, n_stages: int, C: int, device) -> torch.Tensor:
    """[S+1][6][C] fp32 (shift1, scale1, gate1, shift2, scale2, gate2) per
    stage: N(0, 0.1^2), gates centred on 0.5."""
    g = _gen(device, tag, "dit-mod", layer)
    m = 0.1 * torch.randn((n_stages, 6, C), generator=g, device=device)
    m[:, 2] += 0.5
    m[:, 5] += 0.5
    return m


def dit_x0(tag: str, rnd: int, stage: int, n_tokens: int, C: int, device) -> torch.Tensor:
    """Layer-0 input [N][C] of the cell at ``stage`` in round ``rnd``: N(0, 1), fp32."""
    g = _gen(device, tag, "dit-x0", rnd, stage)
    return torch.randn((n_tokens, C), generator=g, device=device)
