"""The derived per-element bounds of the GPU parity tests, checked on the CPU
against an emulation of the rounding steps each attention kernel documents
(include/wf.h numerics notes), so that a bound that is too tight or vacuous
shows here and not only on the GPU.

The emulation is written from the documented arithmetic, in fp64 apart from
the roundings themselves (torch's bfloat16 and float8_e4m3fn conversions,
round to nearest even):
* bf16 pages: q rounded to bf16 (q_rot in HBM), multiplied by
  c = fp32(scale log2 e) and rounded to bf16 again; K rounded to bf16; the
  weights 2^(S - m - 7) rounded to bf16 and used for both P V and the row
  sum; the output rounded to bf16.
* FP8 pages: Q, K, V already dequantised E4M3 (the oracle's operands); the
  weights 2^(S - m + 7) rounded to E4M3 and used for both sums; the output
  rounded to bf16.
* 8-bit-key pages: as FP8 with the weights rounded to bf16 and exact values.
Each emulated output is compared with the exact fp64 attention of the same
operands (the oracle's) under ``wfcheck``'s bound for that kernel.
"""

import math

import numpy as np
import pytest
import torch

from oracle import wf_fp8 as F8
from oracle.wf_attention import attend
from wfcheck import bf16_attention_tolerance, fp8_attention_tolerance

LOG2E = 1.4426950408889634


def _bf16(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).to(torch.float64).numpy()


def _e4m3(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float64)).to(torch.float8_e4m3fn).to(torch.float64).numpy()


def _weighted(w, v):
    return (w @ v) / w.sum(axis=1, keepdims=True)


def _inputs(kind, n_keys, d=128, nq=64, seed=0):
    """Unit-Gaussian rows ("broad"), keys scaled up ("peaky"), or keys whose
    gain grows along the context as in the lazy-rescale test ("wide")."""
    rng = np.random.default_rng([seed, n_keys, len(kind)])
    q = rng.standard_normal((nq, d))
    k = rng.standard_normal((n_keys, d))
    v = rng.standard_normal((n_keys, d))
    if kind == "peaky":
        k *= 3.0
    elif kind == "wide":
        k *= (1.0 + 0.8 * (np.arange(n_keys) // max(1, n_keys // 6)))[:, None]   # six 'chunks'
    return q, k, v


CASES = [("broad", 64), ("broad", 360), ("broad", 4096), ("peaky", 512), ("wide", 720)]


@pytest.mark.parametrize("kind,n_keys", CASES)
def test_bf16_bound_covers_the_kernel_roundings(kind, n_keys):
    q, k, v = _inputs(kind, n_keys)
    v = _bf16(v)                                   # bf16 inputs: the values are exact
    d = q.shape[1]
    scale = 1.0 / math.sqrt(d)
    c = float(np.float32(scale * LOG2E))
    q2 = _bf16(_bf16(q) * c)                       # twice rounded, base-2 units
    s = q2 @ _bf16(k).T
    w = _bf16(np.exp2(s - s.max(axis=1, keepdims=True) - 7.0))
    got = _bf16(_weighted(w, v))
    want = attend(q, k, v, scale)
    tol = bf16_attention_tolerance(q, k, v, scale)
    ratio = np.abs(got - want) / tol
    assert ratio.max() <= 1.0, ratio.max()
    assert ratio.max() >= 0.05, ratio.max()        # the bound is not vacuous


@pytest.mark.parametrize("kind,n_keys", CASES)
@pytest.mark.parametrize("pages", ["fp8", "fp8k"])
def test_8bit_bound_covers_the_kernel_weight_rounding(kind, n_keys, pages):
    q, k, v = _inputs(kind, n_keys, seed=1)
    d = q.shape[1]
    scale = 1.0 / math.sqrt(d)
    q8 = F8.fp8_query(F8.bf16_round(q))
    k8 = F8.fp8_tiles(k)
    v8 = F8.fp8_tiles(v) if pages == "fp8" else _bf16(v)
    s = scale * LOG2E * (q8 @ k8.T)
    if pages == "fp8":
        w = _e4m3(np.exp2(s - s.max(axis=1, keepdims=True) + 7.0))
        eps = 2.0 ** -4
    else:
        w = _bf16(np.exp2(s - s.max(axis=1, keepdims=True) - 7.0))
        eps = 2.0 ** -8
    got = _bf16(_weighted(w, v8))
    want = attend(q8, k8, v8, scale)
    tol = fp8_attention_tolerance(q8, k8, v8, scale, weight_eps=eps, out_rel=2.0 ** -8)
    ratio = np.abs(got - want) / tol
    assert ratio.max() <= 1.0, ratio.max()
    assert ratio.max() >= 0.05, ratio.max()
