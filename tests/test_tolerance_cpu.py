"""CPU checks of the tolerance helpers in ``wfcheck`` (test infrastructure):
the rounding-midpoint distance against a brute-force search of the grids,
and the fp32 rotation error bound against an fp32 rotation."""

import math

import numpy as np
import pytest
import torch

from oracle import wf_fp8 as F8
from wfcheck import _midpoint_distance, _query_term, _rotation_error, query_shift


def _brute_margin(x, grid):
    mids = (grid[1:] + grid[:-1]) / 2
    a = np.abs(x)
    i = np.searchsorted(mids, a)
    lo = np.where(i > 0, mids[np.maximum(i - 1, 0)], -np.inf)
    hi = np.where(i < len(mids), mids[np.minimum(i, len(mids) - 1)], np.inf)
    return np.minimum(a - lo, hi - a)


def test_e4m3_midpoint_distance_matches_brute_force():
    rng = np.random.default_rng(3)
    x = rng.standard_normal(100000) * np.exp2(rng.integers(-12, 9, 100000))
    x = x[np.abs(x) < 440]
    grid = np.unique(np.abs(F8.e4m3_values(np.arange(256, dtype=np.uint8))))
    grid = grid[np.isfinite(grid)]
    # exact midpoints and values next to them are included
    mids = (grid[1:] + grid[:-1]) / 2
    x = np.concatenate([x, mids, np.nextafter(mids, 0), np.nextafter(mids, 1e9), -mids[:50]])
    dist, step = _midpoint_distance(x, 3, -6)
    np.testing.assert_allclose(dist, _brute_margin(x, grid), rtol=0, atol=1e-15)
    assert (dist[len(x) - 50 - 3 * len(mids):len(x) - 50 - 2 * len(mids)] == 0).all()
    # crossing the nearest midpoint moves the code by the spacing of the two
    # grid values around that midpoint: never more than the step returned
    a = np.abs(x)
    j = np.argmin(np.abs(mids[None, :] - a[:2000, None]), axis=1)
    assert (grid[j + 1] - grid[j] <= step[:2000]).all()


def test_bf16_midpoint_distance_matches_brute_force():
    rng = np.random.default_rng(4)
    x = rng.standard_normal(20000) * 3
    g = F8.bf16_round(x)
    dist, _ = _midpoint_distance(x, 7, -126)
    # neighbours of g in bf16: step the fp32 bit pattern's upper half
    bits = torch.from_numpy(np.abs(g).astype(np.float32)).view(torch.int32).numpy() >> 16
    nb = lambda b: torch.from_numpy((b.astype(np.int32) << 16)).view(torch.float32).double().numpy()  # noqa: E731
    up, dn = nb(bits + 1), nb(bits - 1)
    brute = np.minimum(np.abs(x) - (np.abs(g) + dn) / 2, (np.abs(g) + up) / 2 - np.abs(x))
    np.testing.assert_allclose(dist, brute, rtol=0, atol=1e-15)


def test_rotation_error_bounds_an_fp32_rotation():
    rng = np.random.default_rng(5)
    n = 50000
    a = F8.bf16_round(rng.standard_normal(n) * 4)
    b = F8.bf16_round(rng.standard_normal(n) * 4)
    th = rng.uniform(0, 2 * math.pi, n)
    exact = np.stack([a * np.cos(th) - b * np.sin(th), a * np.sin(th) + b * np.cos(th)], 1)
    c32, s32 = np.cos(th).astype(np.float32), np.sin(th).astype(np.float32)
    a32, b32 = a.astype(np.float32), b.astype(np.float32)
    got = np.stack([a32 * c32 - b32 * s32, a32 * s32 + b32 * c32], 1).astype(np.float64)
    assert (np.abs(got - exact) <= _rotation_error(exact)).all()


def _kernel_query(x, scale):
    """The quantised query of the FP8 / 8-bit-key attention kernels as the
    tolerance models it: y = fp32(x) * fp32(scale log2 e) in fp32, one
    power-of-two exponent per row (the block rule on y), E4M3 by torch's
    float8_e4m3fn, divided by c again (a model of the kernel's rounding,
    used here only to check the bound that covers it)."""
    c = np.float32(scale * math.log2(math.e))
    y = (x.astype(np.float32) * c).astype(np.float64)
    out = np.empty_like(y)
    for r in range(y.shape[0]):
        e = F8.pow2_exponent(np.max(np.abs(y[r])))
        z = torch.tensor(np.ldexp(y[r], -e), dtype=torch.float32).to(torch.float8_e4m3fn)
        out[r] = np.ldexp(z.to(torch.float64).numpy(), e) / float(c)
    return out


@pytest.mark.parametrize("n_keys,key_gain,q_gain", [(64, 1.0, 1.0), (360, 1.0, 1.0), (4096, 1.0, 1.0),
                                                     (512, 3.0, 1.0), (256, 1.0, 4.0)])
def test_query_term_bounds_the_grid_change(n_keys, key_gain, q_gain):
    """The query term of ``fp8_attention_tolerance`` covers the change of
    the exact attention output when the oracle's per-row quantised query
    is replaced by the kernel's (quantised on the grid of q * scale log2 e):
    same keys and values, exact fp64 softmax on both sides.  Peaky rows
    (large key or query gain) and broad ones (4096 keys) are covered."""
    from oracle.wf_attention import attend

    rng = np.random.default_rng([7, n_keys])
    d, nq, scale = 128, 48, 1 / math.sqrt(128)
    q = rng.standard_normal((nq, d)) * q_gain
    k = F8.fp8_tiles(rng.standard_normal((n_keys, d)) * key_gain)
    v = rng.standard_normal((n_keys, d))
    x = F8.bf16_round(q)
    q8o = F8.fp8_query(x)
    q8k = _kernel_query(x, scale)
    assert not np.array_equal(q8o, q8k)          # the grids really differ
    shift = np.abs(attend(q8k, k, v, scale) - attend(q8o, k, v, scale))
    s = scale * (q8o @ k.T)
    p = np.exp(s - s.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    term = _query_term(p, k, v, p @ v, scale, query_shift(q, scale))
    ratio = (shift / term).max()
    assert ratio <= 1.0, ratio
    # and the term is not vacuous: it stays within a small factor of the
    # largest shift it has to cover
    assert term.max() < 40 * shift.max()
