"""GPU parity of the DiT block around the round (``include/wf_dit.h``)
against the fp64 oracle (``oracle/wf_dit.py``), through the C ABI, over
bf16 pages and (with derived wider bounds) over FP8 and 8-bit-key pages.

Small shapes: every round of a request, every active cell, every element of
the residual stream after the last layer (two layers, so layer 1 reads
layer 0's output and its own K/V pages).  Full 1.3B shape (one layer,
FFN 8960): rounds 0..S+1 on the GPU, sampled token rows of every active cell
of the last round checked against the oracle.

Tolerance (derived from the arithmetic): each of the ten bf16 roundings on
the way from x to the block's update d = x_out - x_in (a, qkv, q/k/v after
the norms, q_rot and the K page, the query fragments scaled by
scale * log2(e) inside attention, the softmax weights, o, a2, the FFN hidden
activation) reaches the update with gain about one (norms are scale-free,
the weights keep RMS, GELU' <= 1.13, softmax weights lie in [0, 1]).  Round
to nearest even to 8 significant bits leaves an absolute error uniform in
+-2^-8 * 2^E for a value m * 2^E (1 <= m < 2), a relative error u * 2^-8 / m
(u uniform in [-1, 1]); with the mantissa m log-uniformly distributed,
E[1/m^2] = 3 / (8 ln 2), so the relative error has standard deviation
sigma_1 = 2^-8 * sqrt(1 / (8 ln 2)) = 0.4247 * 2^-8.  Treated as independent,
the ten give sigma = sigma_1 * sqrt(10) * rms(d) per element of a row; the bar
is 6 sigma = 3.15e-2 * rms_row(d), plus 1e-5 for values of d near zero.
"""

import gc
import math

import numpy as np
import pytest
import torch

from chunk_causal_dit_round_amd import synth, wf
from chunk_causal_dit_round_amd.dit import DitSession
from chunk_causal_dit_round_amd.session import Session
from chunk_causal_dit_round_amd.workloads import WAN13B_4STEP, Workload
from oracle import wf_dit as D
from wfcheck import oracle_cfg

pytestmark = pytest.mark.gpu

N_ROUNDINGS = 10
SIGMA_BF16 = 2.0 ** -8 * (1.0 / (8.0 * math.log(2.0))) ** 0.5   # one RNE rounding, relative
REL_TOL = 6 * SIGMA_BF16 * N_ROUNDINGS ** 0.5                  # 3.15e-2

# Over FP8 pages the oracle quantises the exact q, k (and v) while the GPU
# quantises its own, already rounded ones.  A perturbation delta of a value
# flips its E4M3 code by one step u with probability 2 |delta| / u (the
# value's distance to the nearer midpoint is uniform in [0, u/2]), so the
# code's error has variance E[2 |delta| u] = 2 sqrt(2/pi) sigma_delta E[u]
# for Gaussian delta; relative to the value, u = 2^-3 / m and, m
# log-uniform, E[u] = 2^-3 / (2 ln 2).  The perturbations come from the
# roundings upstream: k after a, qkv and its norm (3), q after those and
# q_rot (4), v after a and qkv (2).  Each flipped operand then reaches the
# update with gain about one, like the roundings above.  On FP8 pages the
# softmax weights are rounded to E4M3 instead of bf16: standard deviation
# 2^-4 sqrt(1 / (8 ln 2)) in place of one of the ten bf16 roundings.
_EU = 2.0 ** -3 / (2.0 * math.log(2.0))


def _flip_var(n_upstream):
    return 2.0 * math.sqrt(2.0 / math.pi) * math.sqrt(n_upstream) * SIGMA_BF16 * _EU


REL_TOL_FP8K = 6 * math.sqrt(N_ROUNDINGS * SIGMA_BF16 ** 2 + _flip_var(3) + _flip_var(4))
REL_TOL_FP8 = 6 * math.sqrt((N_ROUNDINGS - 1) * SIGMA_BF16 ** 2 + (16 * SIGMA_BF16) ** 2
                            + _flip_var(3) + _flip_var(4) + _flip_var(2))
ABS_FLOOR = 1e-5


@pytest.fixture(autouse=True)
def _free_memory():
    yield
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _log(msg):
    print(msg, flush=True)


def _oracle_rounds(ds: DitSession, w: Workload):
    cfg = oracle_cfg(w)
    fp8 = {wf.WF_FP8: True, wf.WF_FP8K: "k"}.get(w.dtype, False)
    weights = [D.Weights(**{n: t.detach().double().cpu().numpy() for n, t in lw.items()})
               for lw in ds.layers]
    mods = [m.double().cpu().numpy() for m in ds.mod]
    x0 = lambda rnd, st: synth.dit_x0(ds.tag, rnd, st, w.n_tokens, ds.C, ds.s.device).double().cpu().numpy()  # noqa: E731
    return D.DitRounds(cfg, x0, lambda l: weights[l], lambda l: mods[l], fp8=fp8)


def _compare(got, want, x_in, what, rel_tol=REL_TOL):
    """Max error / bound over the rows; asserts the bound."""
    d = want - x_in
    rms = np.sqrt((d * d).mean(axis=1, keepdims=True))
    bound = rel_tol * rms + ABS_FLOOR
    err = np.abs(got - want)
    ratio = float((err / bound).max())
    assert ratio <= 1.0, f"{what}: max err/bound {ratio:.3f}, max err {err.max():.3g}"
    return ratio


SMALL = [
    # 72 tokens: one partial 256-row query tile, 64-key tiles straddle pages
    (Workload("dit_s2_n72", S=2, W=2, n_chunk=6, F=3, Hh=4, Ww=6, n_heads=2, head_dim=64,
              n_layers=2), 192),
    # several query tiles + ragged tail, head_dim 128, anchor re-rotation
    (Workload("dit_s4_n360", S=4, W=2, n_chunk=8, F=3, Hh=10, Ww=12, n_heads=2, head_dim=128,
              n_layers=2), 512),
]


@pytest.mark.parametrize("tune", [False, True], ids=["heuristic", "tuned"])
@pytest.mark.parametrize("w,ffn", SMALL, ids=[w.name for w, _ in SMALL])
def test_small_dit_every_round(w, ffn, tune):
    """Every round against the oracle; with ``tuned`` the products run the
    algorithms wf_dit_tune timed fastest (the same bar: only the rounding
    order of the products changes)."""
    s = Session(w.config(), io=False)
    ds = DitSession(s, ffn, tag=w.name)
    if tune:
        ds.tune()
    orc = _oracle_rounds(ds, w)
    worst = 0.0
    try:
        for k in range(w.n_chunk + w.S):
            plan = s.plan(k)
            ds.load_x0(k)
            ds.round(plan)
            torch.cuda.synchronize()
            got = ds.x.double().cpu().numpy()
            for st in range(w.S + 1):
                if not plan.cells[st].active:
                    continue
                want = orc.layer_output(k, w.n_layers - 1, st)
                x_in = orc.x_in(k, 0, st)
                worst = max(worst, _compare(got[st], want, x_in, f"{w.name} k={k} stage={st}"))
        _log(f"{w.name}: worst err/bound {worst:.3f}")
    finally:
        s.close()


def test_inactive_rows_untouched_and_layer_calls_equal_round():
    """Rows of inactive stages keep their contents; wf_dit_layer per layer +
    commit gives the same bits as wf_dit_round."""
    w, ffn = SMALL[0]
    outs = []
    for mode in ("round", "layers"):
        s = Session(w.config(), io=False)
        ds = DitSession(s, ffn, tag=w.name)
        try:
            marker = torch.full_like(ds.x, 7.25)
            for k in range(3):
                plan = s.plan(k)
                ds.x.copy_(marker)
                ds.load_x0(k, [st for st in range(w.S + 1) if plan.cells[st].active])
                if mode == "round":
                    ds.round(plan)
                else:
                    for layer in range(w.n_layers):
                        ds.layer(plan, layer)
                    s.commit(plan)
                torch.cuda.synchronize()
                for st in range(w.S + 1):
                    if not plan.cells[st].active:
                        assert torch.equal(ds.x[st], marker[st])
            outs.append(ds.x.clone())
        finally:
            s.close()
    assert torch.equal(outs[0], outs[1])


def test_full_size_wan13b_one_layer_sampled():
    """1.3B shape (12 x 128 heads, C 1536, FFN 8960), one layer, rounds
    0..S+1 (the last with the anchor present); 48 sampled rows per active
    cell of the last round against the oracle."""
    w = WAN13B_4STEP.with_(name="dit_wan1.3b_l1", n_layers=1)
    s = Session(w.config(), io=False)
    ds = DitSession(s, 8960, tag=w.name)
    orc = _oracle_rounds(ds, w)
    last = w.S + 1
    try:
        for k in range(last + 1):
            plan = s.plan(k)
            ds.load_x0(k)
            ds.round(plan)
        torch.cuda.synchronize()
        got = ds.x.double().cpu().numpy()
        rng = np.random.default_rng(13)
        worst = 0.0
        for st in range(w.S + 1):
            rows = np.sort(rng.choice(w.n_tokens, 48, replace=False))
            rows[-1] = w.n_tokens - 1
            want = orc.layer_output(last, 0, st, rows=rows)
            x_in = orc.x_in(last, 0, st)[rows]
            worst = max(worst, _compare(got[st][rows], want, x_in, f"stage {st}"))
        _log(f"{w.name}: worst err/bound {worst:.3f}")
    finally:
        s.close()


FP8_SMALL = [
    (SMALL[1][0].with_(name="dit_fp8k_s4_n360", dtype=wf.WF_FP8K), 512, REL_TOL_FP8K),
    (SMALL[1][0].with_(name="dit_fp8_s4_n360", dtype=wf.WF_FP8), 512, REL_TOL_FP8),
]


@pytest.mark.parametrize("w,ffn,rel_tol", FP8_SMALL, ids=[w.name for w, _, _ in FP8_SMALL])
def test_small_dit_over_fp8_pages_every_round(w, ffn, rel_tol):
    """The block over 8-bit-key pages (the paper's Sage tier keeps the linear
    layers in bf16) and over FP8 pages: every round, every element of x
    after two layers, against the oracle's block over the same page reading.
    Bound: the derivation above (3.15e-2 for bf16 pages becomes
    REL_TOL_FP8K / REL_TOL_FP8 times rms_row(d))."""
    s = Session(w.config(), io=False)
    ds = DitSession(s, ffn, tag=w.name)
    orc = _oracle_rounds(ds, w)
    worst = 0.0
    try:
        for k in range(w.n_chunk + w.S):
            plan = s.plan(k)
            ds.load_x0(k)
            ds.round(plan)
            torch.cuda.synchronize()
            got = ds.x.double().cpu().numpy()
            for st in range(w.S + 1):
                if not plan.cells[st].active:
                    continue
                want = orc.layer_output(k, w.n_layers - 1, st)
                x_in = orc.x_in(k, 0, st)
                worst = max(worst, _compare(got[st], want, x_in, f"{w.name} k={k} stage={st}", rel_tol))
        _log(f"{w.name}: worst err/bound {worst:.3f} (bound {rel_tol:.3g} rms_row(d))")
    finally:
        s.close()


@pytest.mark.parametrize("dtype,rel_tol", [(wf.WF_FP8K, REL_TOL_FP8K), (wf.WF_FP8, REL_TOL_FP8)],
                         ids=["fp8k", "fp8"])
def test_full_size_wan13b_one_layer_8bit_pages_sampled(dtype, rel_tol):
    """1.3B shape, one layer, over 8-bit-key pages (FP8K) and 8-bit K/V
    pages (FP8): rounds 0..S+1, 48 sampled rows per active cell of the last
    round against the oracle."""
    tag = "fp8k" if dtype == wf.WF_FP8K else "fp8"
    w = WAN13B_4STEP.with_(name=f"dit_wan1.3b_l1_{tag}", n_layers=1, dtype=dtype)
    s = Session(w.config(), io=False)
    ds = DitSession(s, 8960, tag=w.name)
    orc = _oracle_rounds(ds, w)
    last = w.S + 1
    try:
        for k in range(last + 1):
            plan = s.plan(k)
            ds.load_x0(k)
            ds.round(plan)
        torch.cuda.synchronize()
        got = ds.x.double().cpu().numpy()
        rng = np.random.default_rng(14)
        worst = 0.0
        for st in range(w.S + 1):
            rows = np.sort(rng.choice(w.n_tokens, 48, replace=False))
            rows[-1] = w.n_tokens - 1
            want = orc.layer_output(last, 0, st, rows=rows)
            x_in = orc.x_in(last, 0, st)[rows]
            worst = max(worst, _compare(got[st][rows], want, x_in, f"stage {st}", rel_tol))
        _log(f"{w.name}: worst err/bound {worst:.3f}")
    finally:
        s.close()


def test_fp32_rounds_have_no_block():
    """An fp32 handle (bound on the GPU) rejects the block before any
    device work: WF_EUNSUPPORTED, with the reason in wf_last_error."""
    from chunk_causal_dit_round_amd.workloads import TINY_FP32
    s = Session(TINY_FP32.config(), io=False)
    try:
        fake = 1 << 20                      # never dereferenced: rejected first
        dc = wf.make_dit_config(64)
        names = [n for n, _ in wf.wf_dit_weights._fields_]
        W = wf.make_dit_weights([{n: fake for n in names}])
        st = wf.status_of(wf.wf_dit_layer, s.h, s.plan(0), 0, dc, W[0], fake, fake, fake, 1 << 30)
        assert st == wf.WF_EUNSUPPORTED
        assert "fp32" in wf.wf_last_error()
    finally:
        s.close()


def test_dit_layers_replay_in_a_hip_graph():
    """Every layer of a round through the block (norm kernels, hipBLASLt
    products, publish, attention) captured into a HIP graph: each replay
    from the same residual stream gives the eager bits."""
    w, ffn = SMALL[1]
    s = Session(w.config(), io=False)
    ds = DitSession(s, ffn, tag=w.name + "_graph")
    try:
        k_cap = 6
        for k in range(k_cap):
            plan = s.plan(k)
            ds.load_x0(k)
            ds.round(plan)
        plan = s.plan(k_cap)
        ds.load_x0(k_cap)
        x_in = ds.x.clone()

        def layers():
            for layer in range(w.n_layers):
                ds.layer(plan, layer)

        layers()                                    # eager (also makes the product plans)
        torch.cuda.synchronize()
        eager = ds.x.clone()
        ds.x.copy_(x_in)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            layers()
        torch.cuda.synchronize()
        for rep in range(3):
            ds.x.copy_(x_in)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(ds.x, eager), rep
        s.commit(plan)
    finally:
        s.close()
