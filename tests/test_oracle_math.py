"""Pins for the oracle RoPE, attention and round assembly.

RoPE is checked against complex multiplication and against closed-form
properties (norm, identity at position 0, relative-position dependence,
per-axis frequencies).  Attention is checked against torch's CPU
``scaled_dot_product_attention`` (a library routine, not the oracle's own
formula), against the causal special case of the chunk mask, and against
textbook special cases.
"""

import math

import numpy as np
import pytest
import torch

from oracle import wf_plan as P
from oracle import wf_rope as R
from oracle.wf_attention import attend
from oracle import wf_round as WR


def rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- RoPE ----

def test_axis_split():
    assert R.axis_split(128) == (22, 21, 21)
    assert R.axis_split(64) == (12, 10, 10)
    for d in range(6, 258, 2):
        nt, nh, nw = R.axis_split(d)
        assert nt + nh + nw == d // 2 and nt >= nh == nw


def test_rope_norm_and_identity():
    x = rng(1).standard_normal((72, 2, 64))
    y = R.rope3d(x, 9, 3, 4, 6)
    # every rotation pair keeps its length
    np.testing.assert_allclose(np.hypot(y[..., 0::2], y[..., 1::2]),
                               np.hypot(x[..., 0::2], x[..., 1::2]), rtol=1e-13)
    # token 0 of a chunk at frame 0 sits at the origin of all three axes
    z = R.rope3d(x, 0, 3, 4, 6)
    np.testing.assert_array_equal(z[0], x[0])


def test_rope_matches_complex_multiplication():
    """Each pair rotated as the complex number x0 + i x1 times e^{i a}, with
    the per-axis angle spelled out for d = 64: pairs 0..11 use the frame at
    10000^(-m/12), pairs 12..21 the row at 10000^(-m/10), 22..31 the column."""
    F, Hh, Ww, frame0 = 2, 3, 5, 7
    x = rng(2).standard_normal((F * Hh * Ww, 64))
    y = R.rope3d(x, frame0, F, Hh, Ww)
    for n in range(F * Hh * Ww):
        f, yy, xx = n // (Hh * Ww), (n // Ww) % Hh, n % Ww
        for p in range(32):
            if p < 12:
                a = (frame0 + f) * 10000.0 ** (-p / 12)
            elif p < 22:
                a = yy * 10000.0 ** (-(p - 12) / 10)
            else:
                a = xx * 10000.0 ** (-(p - 22) / 10)
            zc = complex(x[n, 2 * p], x[n, 2 * p + 1]) * complex(math.cos(a), math.sin(a))
            assert abs(y[n, 2 * p] - zc.real) < 1e-12
            assert abs(y[n, 2 * p + 1] - zc.imag) < 1e-12


def test_rope_relative_position():
    """q(m).k(n) depends only on m - n: shifting both frames keeps scores."""
    q = rng(3).standard_normal((24, 128))
    k = rng(4).standard_normal((24, 128))
    s1 = R.rope3d(q, 9, 1, 4, 6) @ R.rope3d(k, 3, 1, 4, 6).T
    s2 = R.rope3d(q, 409, 1, 4, 6) @ R.rope3d(k, 403, 1, 4, 6).T
    np.testing.assert_allclose(s1, s2, atol=1e-10)
    # and a different offset changes them
    s3 = R.rope3d(q, 9, 1, 4, 6) @ R.rope3d(k, 4, 1, 4, 6).T
    assert np.abs(s1 - s3).max() > 1e-3


# ----------------------------------------------------------- attention ----

@pytest.mark.parametrize("nq,nk,d", [(1, 1, 8), (7, 33, 64), (40, 300, 128)])
def test_attend_matches_torch_sdpa(nq, nk, d):
    r = rng(nq * 1000 + nk)
    q, k, v = (r.standard_normal((n, d)) * 2.0 for n in (nq, nk, nk))
    want = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None],
        torch.from_numpy(v)[None]).numpy()[0]
    got = attend(q, k, v, 1.0 / math.sqrt(d), block=5)
    np.testing.assert_allclose(got, want, atol=1e-12, rtol=0)


def test_attend_special_cases():
    r = rng(5)
    v = r.standard_normal((9, 16))
    k = r.standard_normal((9, 16))
    # equal scores -> mean of V
    out = attend(np.zeros((3, 16)), k, v, 0.25)
    np.testing.assert_allclose(out, np.broadcast_to(v.mean(0), (3, 16)), atol=1e-14)
    # one key -> that V row
    out = attend(r.standard_normal((4, 16)), k[:1], v[:1], 0.25)
    np.testing.assert_allclose(out, np.broadcast_to(v[0], (4, 16)), atol=1e-15)
    # outputs lie in the per-dimension hull of V
    q = r.standard_normal((50, 16)) * 3
    out = attend(q, k, v, 0.25)
    assert (out <= v.max(0) + 1e-12).all() and (out >= v.min(0) - 1e-12).all()


# ------------------------------------------------------ round assembly ----

class Raw:
    """Seeded raw projections per (round, layer, cell, name), fp64."""

    def __init__(self, cfg, seed=0, scale=1.0):
        self.cfg, self.seed, self.scale, self.cache = cfg, seed, scale, {}
        self.override = {}

    def __call__(self, rnd, layer, cell, name):
        key = (rnd, layer, cell, name)
        if key in self.override:
            return self.override[key]
        if key not in self.cache:
            c = self.cfg
            s = [self.seed, rnd, layer, cell, "qkv".index(name)]
            self.cache[key] = rng(s).standard_normal((c.n_c, c.n_heads, c.head_dim)) * self.scale
        return self.cache[key]


def test_round_reduces_to_causal_sdpa():
    """W = 0, no anchor, one token per chunk: in chunk order Eq. 4 is the
    lower-triangular mask, so a full round equals causal SDPA over the S+1
    chunks (store = oldest first)."""
    S = 4
    c = P.Config(S=S, W=0, W_store=0, anchor=0, n_chunk=12, F=1, Hh=1, Ww=1,
                 n_heads=3, head_dim=16, n_layers=1)
    raw = Raw(c, seed=11, scale=2.0)
    k = 7
    res = WR.round_outputs(c, k, 0, raw)
    # chunk order: store chunk k-S first, then k-S+1 ... k (stage S .. 0);
    # queries and keys of chunk k-s both at that chunk's own frame (R10)
    stages = list(range(S, -1, -1))
    q = np.concatenate([R.rope3d(raw(k, 0, s, "q"), k - s, 1, 1, 1) for s in stages])
    np.testing.assert_array_equal(np.concatenate([res[s][0] for s in stages]), q)
    kk = np.concatenate([R.rope3d(raw(k, 0, s, "k"), k - s, 1, 1, 1) for s in stages])
    vv = np.concatenate([raw(k, 0, s, "v") for s in stages])
    t = lambda a: torch.from_numpy(a.transpose(1, 0, 2).copy())
    want = torch.nn.functional.scaled_dot_product_attention(
        t(q), t(kk), t(vv), is_causal=True).numpy().transpose(1, 0, 2)
    got = np.concatenate([res[s][1] for s in stages])
    np.testing.assert_allclose(got, want, atol=1e-12)


def test_rolling_mask_reduces_to_dense_sdpa():
    """Rolling-Forcing comparison mask: each denoiser attends, unmasked, to
    anchor + history + store + every active denoising chunk."""
    c = P.Config(S=3, W=2, W_store=-1, anchor=1, n_chunk=12, F=1, Hh=2, Ww=3,
                 n_heads=2, head_dim=32, n_layers=1, mask=P.MASK_ROLLING)
    raw = Raw(c, seed=12)
    k = 9
    for s in range(c.S):
        got = WR.group_output(c, k, s, 0, raw)
        # the denoiser's queries at its chunk's own frames (R10)
        q = R.rope3d(raw(k, 0, s, "q"), c.F * (k - s), c.F, c.Hh, c.Ww)
        kk, vv = WR.group_keys(c, k, s, 0, raw)
        assert kk.shape[0] == c.n_c * (1 + 2 + 1 + 3)
        t = lambda a: torch.from_numpy(a.transpose(1, 0, 2).copy())
        want = torch.nn.functional.scaled_dot_product_attention(
            t(q), t(kk), t(vv)).numpy().transpose(1, 0, 2)
        np.testing.assert_allclose(got, want, atol=1e-12)


def test_causal_invariant_oracle():
    """Perturbing the K/V of any noisier active chunk (stage j < s) leaves the
    stage-s output bit-identical (WF §3.1, Eq. 4)."""
    c = P.Config(S=4, W=2, W_store=-1, anchor=1, n_chunk=20, F=3, Hh=2, Ww=2,
                 n_heads=2, head_dim=16, n_layers=1)
    raw = Raw(c, seed=13)
    k = 10
    base = {s: WR.group_output(c, k, s, 0, raw) for s in range(c.S + 1)}
    for j in range(c.S):
        raw.override = {(k, 0, j, "k"): raw(k, 0, j, "k") + 5.0,
                        (k, 0, j, "v"): raw(k, 0, j, "v") - 3.0}
        for s in range(j + 1, c.S + 1):
            np.testing.assert_array_equal(WR.group_output(c, k, s, 0, raw), base[s])
        # and the chunk itself does change
        assert np.abs(WR.group_output(c, k, j, 0, raw) - base[j]).max() > 1e-3
    raw.override = {}


def test_anchor_entry_source():
    c = P.Config(S=2, W=1, W_store=-1, anchor=1, n_chunk=30, F=3, Hh=1, Ww=2,
                 n_heads=1, head_dim=8, n_layers=1)
    # anchor raw K/V always come from the store cell of round S (chunk 0)
    assert WR.entry_source(c, 20, P.ANCHOR, 0) == (2, 2, 3 * (20 - 2 - 3 - 1))
    assert WR.entry_source(c, 20, P.HISTORY, 15) == (17, 2, 45)
    assert WR.entry_source(c, 20, P.STORE, 18) == (20, 2, 54)
    assert WR.entry_source(c, 20, P.DENOISE, 19) == (20, 1, 57)
