"""Pins of the DiT-block reading in ``oracle/wf_dit.py`` (CPU only).

Pinned against something other than the oracle itself:
* LayerNorm, RMSNorm and tanh-GELU against torch's fp64 functional routines;
* one block on a single chunk against a composition of torch modules
  (``nn.LayerNorm``, ``nn.Linear``, ``scaled_dot_product_attention``), which
  fixes the weight layout, the q/k/v split and the head split;
* closed forms of the whole round assembly: zero gates give the identity;
  scale1 = -1 makes every value row equal, so attention must return that
  row whatever the keys and positions are;
* the causal invariant through two layers: a noisier cell's input never
  reaches a cleaner cell's output.
The last two also over FP8 pages and the 8-bit QK^T tier's pages (the
attention's page reading is pinned in ``test_oracle_fp8.py``).
"""

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as TF

from oracle import wf_dit as D
from oracle import wf_plan as P
from oracle.wf_attention import attend_heads


def _rng(seed):
    return np.random.default_rng(seed)


def test_layer_norm_matches_torch():
    x = _rng(1).standard_normal((7, 96)) * 3 + 1.5
    ref = TF.layer_norm(torch.tensor(x), (96,), eps=1e-6).numpy()
    assert np.allclose(D.layer_norm(x, 1e-6), ref, rtol=0, atol=1e-12)
    y = D.layer_norm(x, 0.0)
    assert np.allclose(y.mean(axis=1), 0, atol=1e-12)
    assert np.allclose((y * y).mean(axis=1), 1, atol=1e-12)
    # invariant under x -> a x + b (a > 0) when eps = 0
    assert np.allclose(D.layer_norm(2.5 * x - 7.0, 0.0), y, atol=1e-12)


def test_rms_norm_matches_torch():
    r = _rng(2)
    x = r.standard_normal((5, 64)) * 4
    g = 1 + 0.1 * r.standard_normal(64)
    ref = TF.rms_norm(torch.tensor(x), (64,), weight=torch.tensor(g), eps=1e-6).numpy()
    assert np.allclose(D.rms_norm(x, g, 1e-6), ref, rtol=0, atol=1e-12)
    assert np.allclose(D.rms_norm(3 * x, g, 0.0), D.rms_norm(x, g, 0.0), atol=1e-12)
    assert np.allclose(D.rms_norm(np.ones((2, 64)), g, 0.0), np.broadcast_to(g, (2, 64)))


def test_gelu_tanh_matches_torch():
    x = np.linspace(-8, 8, 2001)
    ref = TF.gelu(torch.tensor(x), approximate="tanh").numpy()
    assert np.allclose(D.gelu_tanh(x), ref, rtol=0, atol=1e-14)
    assert D.gelu_tanh(np.array([0.0]))[0] == 0.0
    assert np.allclose(D.gelu_tanh(x) - D.gelu_tanh(-x), x, atol=1e-12)
    # differs from the erf form by a few 1e-4 at most: the form is pinned
    erf = TF.gelu(torch.tensor(x)).numpy()
    assert 1e-4 < np.max(np.abs(D.gelu_tanh(x) - erf)) < 1e-3


def _weights(r, C, F):
    s = 1 / math.sqrt(C)
    return D.Weights(
        w_qkv=r.standard_normal((3 * C, C)) * s, b_qkv=0.1 * r.standard_normal(3 * C),
        g_q=1 + 0.1 * r.standard_normal(C), g_k=1 + 0.1 * r.standard_normal(C),
        w_o=r.standard_normal((C, C)) * s, b_o=0.1 * r.standard_normal(C),
        w_1=r.standard_normal((F, C)) * s, b_1=0.1 * r.standard_normal(F),
        w_2=r.standard_normal((C, F)) / math.sqrt(F), b_2=0.1 * r.standard_normal(C))


def _mod(r, C):
    m = 0.3 * r.standard_normal((6, C))
    m[2] += 1.0
    m[5] += 1.0
    return m


def test_block_matches_torch_modules_on_one_chunk():
    """Single chunk, attention over itself (no RoPE): oracle vs torch modules."""
    r = _rng(3)
    N, H, d, F = 40, 4, 16, 96
    C = H * d
    w = _weights(r, C, F)
    mod = _mod(r, C)
    x = r.standard_normal((N, C))
    q, k, v = D.project_qkv(w, x, mod, H)
    o = attend_heads(q, k, v, 1 / math.sqrt(d))
    got = D.finish_block(w, x, mod, o)

    t = lambda a: torch.tensor(a, dtype=torch.float64)  # noqa: E731
    ln = torch.nn.LayerNorm(C, eps=1e-6, elementwise_affine=False).double()

    def linear(wt, b):
        lin = torch.nn.Linear(wt.shape[1], wt.shape[0]).double()
        with torch.no_grad():
            lin.weight.copy_(t(wt))
            lin.bias.copy_(t(b))
        return lin

    m = t(mod)
    with torch.no_grad():
        xt = t(x)
        a = ln(xt) * (1 + m[1]) + m[0]
        qkv = linear(w.w_qkv, w.b_qkv)(a)
        qt, kt, vt = qkv.split(C, dim=1)
        qt = TF.rms_norm(qt, (C,), weight=t(w.g_q), eps=1e-6)
        kt = TF.rms_norm(kt, (C,), weight=t(w.g_k), eps=1e-6)
        heads = lambda z: z.view(N, H, d).transpose(0, 1)  # noqa: E731
        ot = TF.scaled_dot_product_attention(heads(qt), heads(kt), heads(vt))
        ot = ot.transpose(0, 1).reshape(N, C)
        x1 = xt + m[2] * linear(w.w_o, w.b_o)(ot)
        a2 = ln(x1) * (1 + m[4]) + m[3]
        ff = linear(w.w_2, w.b_2)(TF.gelu(linear(w.w_1, w.b_1)(a2), approximate="tanh"))
        ref = (x1 + m[5] * ff).numpy()
    assert np.allclose(got, ref, rtol=0, atol=1e-10)


def _tiny_cfg(n_layers=1):
    return P.Config(S=2, W=2, W_store=4, anchor=1, n_chunk=6, F=3, Hh=4, Ww=6,
                    n_heads=2, head_dim=16, n_layers=n_layers, mask=0)


def _rounds(cfg, seed, mod_fn=None, x_fn=None, fp8=False):
    r = _rng(seed)
    C, F = cfg.n_heads * cfg.head_dim, 64
    ws = [_weights(r, C, F) for _ in range(cfg.n_layers)]
    mods = [np.stack([_mod(r, C) for _ in range(cfg.S + 1)]) for _ in range(cfg.n_layers)]
    if mod_fn is not None:
        mods = [mod_fn(m) for m in mods]
    cache = {}

    def x0(rnd, stage):
        if (rnd, stage) not in cache:
            cache[(rnd, stage)] = np.random.default_rng((seed, rnd, stage)).standard_normal((cfg.n_c, C))
            if x_fn is not None:
                cache[(rnd, stage)] = x_fn(rnd, stage, cache[(rnd, stage)])
        return cache[(rnd, stage)]

    return D.DitRounds(cfg, x0, lambda l: ws[l], lambda l: mods[l], fp8=fp8), ws, mods


def test_zero_gates_give_identity():
    cfg = _tiny_cfg()

    def zero_gates(m):
        m = m.copy()
        m[:, 2] = 0
        m[:, 5] = 0
        return m

    dr, _, _ = _rounds(cfg, 4, zero_gates)
    for s in range(cfg.S + 1):
        assert np.array_equal(dr.layer_output(5, 0, s), dr.x_in(5, 0, s))


@pytest.mark.parametrize("fp8", [False, "k", True], ids=["exact", "fp8_keys", "fp8_pages"])
def test_constant_values_pass_through_attention(fp8):
    """scale1 = -1 and one shift1 for every stage: a = shift1 for every token
    of every cell, so every value row is shift1 W_v^T + b_v and attention
    returns it whatever RoPE, paging, the key quantisation and the softmax
    do.  Over FP8 pages the values are quantised too: each head's row then
    comes back as its E4M3 quantisation with the row's own power-of-two
    scale (every 64-token tile holds the same rows)."""
    from oracle import wf_fp8 as F8
    cfg = _tiny_cfg()
    r = _rng(5)
    shift = r.standard_normal(cfg.n_heads * cfg.head_dim)

    def fix(m):
        m = m.copy()
        m[:, 1] = -1.0
        m[:, 0] = shift
        return m

    dr, ws, mods = _rounds(cfg, 6, fix, fp8=fp8)
    C = cfg.n_heads * cfg.head_dim
    w = ws[0]
    vrow = shift @ w.w_qkv[2 * C:].T + w.b_qkv[2 * C:]
    if fp8 is True:
        d = cfg.head_dim
        vrow = np.concatenate([np.ldexp(F8.e4m3_values(c), e) for c, e in
                               (F8.quantize_block(vrow[h * d:(h + 1) * d]) for h in range(cfg.n_heads))])
    k = 5                                     # full width, history and anchor present
    for s in range(cfg.S + 1):
        o = dr.attention(k, 0, s)
        assert np.allclose(o.reshape(cfg.n_c, C), np.broadcast_to(vrow, (cfg.n_c, C)), atol=1e-12)
        x = dr.x_in(k, 0, s)
        expect = D.finish_block(w, x, mods[0][s], np.broadcast_to(vrow, (cfg.n_c, C)))
        assert np.allclose(dr.layer_output(k, 0, s), expect, atol=1e-12)


@pytest.mark.parametrize("fp8", [False, "k"], ids=["exact", "fp8_keys"])
def test_causal_invariant_through_two_layers(fp8):
    """Perturbing the input of a noisier cell (stage j < s) changes nothing
    at stage s, in either layer (WF §3.1, Eq. 4 mask 1[j >= s])."""
    cfg = _tiny_cfg(n_layers=2)
    k = 4
    base, _, _ = _rounds(cfg, 7, fp8=fp8)
    bump = lambda rnd, stage, x: x + (5.0 if (rnd == k and stage == 0) else 0.0)  # noqa: E731
    pert, _, _ = _rounds(cfg, 7, x_fn=bump, fp8=fp8)
    for s in range(1, cfg.S + 1):
        assert np.array_equal(base.layer_output(k, 1, s), pert.layer_output(k, 1, s))
    assert not np.allclose(base.layer_output(k, 1, 0), pert.layer_output(k, 1, 0))


def test_second_layer_reads_first_layer_output_and_rows_select():
    cfg = _tiny_cfg(n_layers=2)
    dr, _, _ = _rounds(cfg, 8)
    k, s = 3, 1
    assert np.array_equal(dr.x_in(k, 1, s), dr.layer_output(k, 0, s))
    rows = np.array([0, 5, 71])
    full = dr.layer_output(k, 1, s)
    assert np.allclose(dr.layer_output(k, 1, s, rows=rows), full[rows], rtol=0, atol=1e-12)


def test_block_shapes_follow_the_heads():
    r = _rng(9)
    w = _weights(r, 32, 48)
    q, k, v = D.project_qkv(w, r.standard_normal((10, 32)), _mod(r, 32), n_heads=2)
    assert q.shape == k.shape == v.shape == (10, 2, 16)
    # each q row is the RMS-normalised first third of the projection
    with pytest.raises(ValueError):
        D.project_qkv(w, r.standard_normal((10, 31)), _mod(r, 32), n_heads=2)
