"""Oracle round: rotated queries and attention outputs by logical identity.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The oracle never looks at slots.  Each key entry of a plan names a chunk and
a kind; where that chunk's K/V came from follows from WF ("Wave Forcing:
Towards Speed-of-Light Streaming Video Generation"):

* a denoising entry (chunk c at stage j = k - c) was produced by cell j of
  the current round k (§3.1, Eq. 3 and 5);
* the live store entry (chunk k - S) was produced by the store cell of
  round k, and a history entry c by the store cell of round c + S, whose
  page was promoted after that round (App. B.3);
* the anchor is chunk 0's raw key and value, captured when chunk 0 was
  stored (round S), re-rotated for round k at the anchor position
  (App. B.3), value unchanged.

Inputs are supplied by a callback ``raw(round, layer, cell, name)`` that
returns the raw projection ``name`` in {"q", "k", "v"} of ``cell`` (stage)
in ``round`` for ``layer`` as an array [N_C, H, d].  For bf16 workloads the
callback returns the bf16 values widened to fp64, so a comparison measures
kernel error, not input quantisation.
"""

import math

import numpy as np

from . import wf_fp8 as F8
from . import wf_plan as P
from .wf_attention import attend
from .wf_rope import rope3d


def entry_source(cfg: P.Config, k: int, kind: int, chunk: int):
    """(round, cell, frame0) of the raw K/V behind a key entry of round k."""
    S = cfg.S
    if kind == P.DENOISE:
        return k, k - chunk, cfg.F * chunk
    if kind == P.STORE:
        return k, S, cfg.F * chunk
    if kind == P.HISTORY:
        return chunk + S, S, cfg.F * chunk
    if kind == P.ANCHOR:
        return S, S, P.anchor_frame0(cfg, k)
    raise ValueError(kind)


def scale_of(cfg: P.Config) -> float:
    return 1.0 / math.sqrt(cfg.head_dim)


def _fp8_page(x: np.ndarray) -> np.ndarray:
    """One page [N, H', d] as FP8 pages hold it: each head quantised per
    64-token tile (App. C.6 reading in ``wf_fp8``), dequantised."""
    out = np.empty_like(x)
    for h in range(x.shape[1]):
        out[:, h, :] = F8.fp8_tiles(x[:, h, :])
    return out


def group_keys(cfg: P.Config, k: int, stage: int, layer: int, raw, heads=None, fp8=False,
               pages=None):
    """Concatenated rotated keys and values of query stage ``stage``:
    ([N_k, H', d], [N_k, H', d]) in plan order (WF §3.1, Eq. 5).  With
    ``fp8`` each page is the FP8 page of the App. C.6 reading; with
    ``fp8="k"`` only the keys are (8-bit QK^T tier, values exact).

    ``pages``: an optional dict that keeps each page once it is made, for
    callers that ask for several stages of the same round, layer, heads and
    page reading (the stages share most of their pages)."""
    ks, vs = [], []
    for kind, chunk, _slot in P.key_entries(cfg, k, stage):
        key = (kind, chunk)
        if pages is not None and key in pages:
            kr, vr = pages[key]
        else:
            rnd, cell, frame0 = entry_source(cfg, k, kind, chunk)
            kr = np.asarray(raw(rnd, layer, cell, "k"), dtype=np.float64)
            vr = np.asarray(raw(rnd, layer, cell, "v"), dtype=np.float64)
            if heads is not None:
                kr, vr = kr[:, heads, :], vr[:, heads, :]
            kr = rope3d(kr, frame0, cfg.F, cfg.Hh, cfg.Ww, cfg.rope_theta)
            if fp8:
                kr = _fp8_page(kr)
                if fp8 != "k":
                    vr = _fp8_page(vr)
            if pages is not None:
                pages[key] = (kr, vr)
        ks.append(kr)
        vs.append(vr)
    return np.concatenate(ks, axis=0), np.concatenate(vs, axis=0)


def q_rot(cfg: P.Config, k: int, stage: int, layer: int, raw) -> np.ndarray:
    """Rotated queries of the active cell (k - stage, stage): [N_C, H, d]."""
    q = np.asarray(raw(k, layer, stage, "q"), dtype=np.float64)
    return rope3d(q, cfg.F * (k - stage), cfg.F, cfg.Hh, cfg.Ww, cfg.rope_theta)


def group_output(cfg: P.Config, k: int, stage: int, layer: int, raw,
                 rows=None, heads=None, fp8=False, pages=None) -> np.ndarray:
    """Attention output of query stage ``stage``: [len(rows), len(heads), d].

    ``rows`` / ``heads`` select query tokens and heads (all by default);
    every selected row still attends to its full key list.  With ``fp8`` the
    pages are FP8 pages (``fp8="k"``: FP8 keys, exact values) and each
    rotated query row, stored in bf16, is quantised per row (the query
    reading of ``wf_fp8.fp8_query``).  ``pages`` as in ``group_keys``.
    """
    heads = list(range(cfg.n_heads)) if heads is None else list(heads)
    qr = q_rot(cfg, k, stage, layer, raw)
    if rows is not None:
        qr = qr[np.asarray(rows)]
    kk, vv = group_keys(cfg, k, stage, layer, raw, heads, fp8=fp8, pages=pages)
    out = np.empty((qr.shape[0], len(heads), cfg.head_dim), dtype=np.float64)
    sc = scale_of(cfg)
    for hi, h in enumerate(heads):
        qh = qr[:, h, :]
        if fp8:
            qh = F8.fp8_query(F8.bf16_round(qh))
        out[:, hi, :] = attend(qh, kk[:, hi, :], vv[:, hi, :], sc)
    return out


def round_outputs(cfg: P.Config, k: int, layer: int, raw) -> dict:
    """All active groups of round k for one layer: {stage: (q_rot, out)}."""
    res = {}
    for s in range(cfg.S + 1):
        if not P.chunk_active(cfg, k - s):
            continue
        res[s] = (q_rot(cfg, k, s, layer, raw),
                  group_output(cfg, k, s, layer, raw))
    return res
