"""Wan-shaped DiT block around the wavefront round, fp64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

WF ("Wave Forcing: Towards Speed-of-Light Streaming Video Generation")
splits each layer of a cell into a producer step that makes Q/K/V and applies
RoPE and a consumer step that runs attention and the rest of the block (§4.1,
Eq. 8); its runtime hooks in right after the self-attention QKV projection
and RoPE (App. B.1).  The model is Wan2.1-T2V with random-init weights (§5.3);
the pages do not spell out the block.  Reading taken here (the public Wan2.1
block, restated; FFN width an assumption):

* the cell's state x [N, C] (C = H d) is a residual stream;
* each cell s carries its own modulation (it sits at its own noise level):
  six vectors of length C, (shift1, scale1, gate1, shift2, scale2, gate2);
* attention half:  a = LN(x) (1 + scale1) + shift1;
  [q | k | v] = a W_qkv^T + b_qkv;  q <- RMSNorm(q) g_q;  k <- RMSNorm(k) g_k
  (both norms over all C channels);  q, k, v split into H heads of d;
  the round's RoPE, paging and attention give o;
  x <- x + gate1 (o W_o^T + b_o);
* FFN half:  a2 = LN(x) (1 + scale2) + shift2;
  x <- x + gate2 (GELU(a2 W_1^T + b_1) W_2^T + b_2), GELU in its tanh form;
* LN has no affine parameters; LN and RMSNorm use the same epsilon (1e-6);
* Wan's text cross-attention is left out (it needs a text encoder and is
  not part of the round).

Weights follow the nn.Linear convention: W [out, in], y = x W^T + b.

Parity status: pinned by ``tests/test_oracle_dit.py`` (torch's
``layer_norm``, ``rms_norm`` and tanh-``gelu`` in fp64; the block against a
composition of torch modules; closed-form special cases of the block).
"""

from dataclasses import dataclass
from typing import Callable, Dict, Optional

import numpy as np

from . import wf_plan as P
from . import wf_round as R

EPS = 1e-6


def layer_norm(x: np.ndarray, eps: float = EPS) -> np.ndarray:
    """(x - mean) / sqrt(var + eps) over the last axis, population variance."""
    x = np.asarray(x, dtype=np.float64)
    mu = x.mean(axis=-1, keepdims=True)
    d = x - mu
    var = (d * d).mean(axis=-1, keepdims=True)
    return d / np.sqrt(var + eps)


def rms_norm(x: np.ndarray, g: np.ndarray, eps: float = EPS) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * g over the last axis."""
    x = np.asarray(x, dtype=np.float64)
    ms = (x * x).mean(axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(g, dtype=np.float64)


def gelu_tanh(x: np.ndarray) -> np.ndarray:
    """GELU, tanh form: x/2 (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3)))."""
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * x * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (x + 0.044715 * x ** 3)))


def modulate(a: np.ndarray, shift: np.ndarray, scale: np.ndarray) -> np.ndarray:
    return a * (1.0 + scale) + shift


@dataclass
class Weights:
    """One layer's weights, fp64 (bf16 / fp32 values widened)."""
    w_qkv: np.ndarray   # [3C, C]
    b_qkv: np.ndarray   # [3C]
    g_q: np.ndarray     # [C]
    g_k: np.ndarray     # [C]
    w_o: np.ndarray     # [C, C]
    b_o: np.ndarray     # [C]
    w_1: np.ndarray     # [F, C]
    b_1: np.ndarray     # [F]
    w_2: np.ndarray     # [C, F]
    b_2: np.ndarray     # [C]


def project_qkv(w: Weights, x: np.ndarray, mod: np.ndarray, n_heads: int,
                eps: float = EPS):
    """Producer step before RoPE: x [N, C], mod [6, C] -> q, k, v [N, H, d]."""
    x = np.asarray(x, dtype=np.float64)
    n, c = x.shape
    a = modulate(layer_norm(x, eps), mod[0], mod[1])
    y = a @ w.w_qkv.T + w.b_qkv
    q = rms_norm(y[:, :c], w.g_q, eps)
    k = rms_norm(y[:, c:2 * c], w.g_k, eps)
    v = y[:, 2 * c:]
    d = c // n_heads
    return q.reshape(n, n_heads, d), k.reshape(n, n_heads, d), v.reshape(n, n_heads, d)


def finish_block(w: Weights, x: np.ndarray, mod: np.ndarray, o: np.ndarray,
                 eps: float = EPS) -> np.ndarray:
    """Consumer step after attention: rows of x [n, C] and their attention
    output o [n, H, d] -> the rows of the block output.  Row-wise only."""
    x = np.asarray(x, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64).reshape(x.shape[0], -1)
    x1 = x + mod[2] * (o @ w.w_o.T + w.b_o)
    a2 = modulate(layer_norm(x1, eps), mod[3], mod[4])
    f = gelu_tanh(a2 @ w.w_1.T + w.b_1)
    return x1 + mod[5] * (f @ w.w_2.T + w.b_2)


class DitRounds:
    """Block outputs of the cells of any round, by logical identity.

    ``x0(rnd, stage)`` gives the layer-0 input [N, C] of the cell at
    ``stage`` in round ``rnd``; ``weights(layer)`` and ``mod(layer)``
    ([S+1, 6, C], by stage) are fixed for the request.  Layer l of a cell
    reads the output of layer l-1 of the same cell in the same round; the
    attention of a layer reads the K/V that the producer steps of the same
    layer made for the chunks of its key list (``wf_round``), in whatever
    round they were made.  Everything is memoised.  ``fp8`` selects the page
    reading of the attention (``wf_round.group_output``: FP8 pages, or "k"
    for the 8-bit QK^T tier's FP8 keys with exact values).
    """

    def __init__(self, cfg: P.Config, x0: Callable, weights: Callable, mod: Callable,
                 eps: float = EPS, fp8=False):
        self.cfg, self.x0, self.weights, self.mod, self.eps = cfg, x0, weights, mod, eps
        self.fp8 = fp8          # the page reading of the attention (``wf_round``)
        self._x: Dict = {}
        self._qkv: Dict = {}

    def x_in(self, rnd: int, layer: int, stage: int) -> np.ndarray:
        """Input of ``layer`` for the cell at ``stage`` of round ``rnd``."""
        key = (rnd, layer, stage)
        if key not in self._x:
            if layer == 0:
                self._x[key] = np.asarray(self.x0(rnd, stage), dtype=np.float64)
            else:
                self._x[key] = self.layer_output(rnd, layer - 1, stage)
        return self._x[key]

    def qkv(self, rnd: int, layer: int, stage: int):
        key = (rnd, layer, stage)
        if key not in self._qkv:
            self._qkv[key] = project_qkv(self.weights(layer), self.x_in(rnd, layer, stage),
                                         np.asarray(self.mod(layer))[stage], self.cfg.n_heads,
                                         self.eps)
        return self._qkv[key]

    def raw(self, rnd: int, layer: int, stage: int, name: str) -> np.ndarray:
        """The callback ``wf_round`` asks for: a cell's q, k or v."""
        return self.qkv(rnd, layer, stage)["qkv".index(name)]

    def attention(self, rnd: int, layer: int, stage: int, rows=None) -> np.ndarray:
        return R.group_output(self.cfg, rnd, stage, layer, self.raw, rows=rows, fp8=self.fp8)

    def layer_output(self, rnd: int, layer: int, stage: int,
                     rows: Optional[np.ndarray] = None) -> np.ndarray:
        """Output of ``layer`` for the cell at ``stage`` of round ``rnd``
        (the selected token rows, all by default)."""
        x = self.x_in(rnd, layer, stage)
        o = self.attention(rnd, layer, stage, rows)
        if rows is not None:
            x = x[np.asarray(rows)]
        return finish_block(self.weights(layer), x, np.asarray(self.mod(layer))[stage], o,
                            self.eps)
