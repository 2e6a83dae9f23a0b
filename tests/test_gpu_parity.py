"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Small shapes are compared element by element over every round of a request
(several query and key tiles, ragged tails, fill, steady state, drain,
anchor re-rotation, ring wrap).  Full Wan2.1 shapes are compared on sampled
query rows (each against its full key list) and on whole pages.

Tolerances: attention max-abs error 2e-2 for bf16 inputs, 1e-4 for fp32
inputs; over FP8 and 8-bit-key pages the per-element bound derived in
``wfcheck.fp8_attention_tolerance`` from the rounding of the softmax
weights; RoPE'd q/k within one bf16 unit in the last place (fp32: 2e-6
relative); values, codes, exponents and every plan field bit-exact.
"""

import gc

import pytest
import torch

from chunk_causal_dit_round_amd import wf
from chunk_causal_dit_round_amd.workloads import (TINY_FP32, WAN13B_4STEP, WAN13B_4STEP_FP8,
                                                  WAN13B_4STEP_FP8K, WAN13B_5STEP, WAN13B_5STEP_ROLLING,
                                                  WAN14B_4STEP, Workload)
import numpy as np

from oracle import wf_plan as P
from oracle import wf_round as WR
from wfcheck import Rollout, check_attention, check_publish, oracle_cfg

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _free_memory():
    yield
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _log(msg):
    print(msg, flush=True)


def full_rollout(w, check_rows=None, check_rounds=None, layers=None, mode="round"):
    ro = Rollout(w)
    try:
        for k in range(w.n_chunk + w.S):
            ro.run(k, mode=mode)
            if check_rounds is None or k in check_rounds:
                for layer in (range(w.n_layers) if layers is None else layers):
                    check_publish(ro, k, layer)
                    check_attention(ro, k, layer, rows=check_rows)
    finally:
        ro.close()


def test_tiny_fp32_every_round():
    _log("tiny fp32: 8 rounds")
    full_rollout(TINY_FP32)


def test_tiny_fp32_long_rollout_ring_wrap_and_anchor_shift():
    w = TINY_FP32.with_(name="tiny_fp32_long", n_chunk=16)
    _log("tiny fp32 long: 18 rounds")
    full_rollout(w)


SMALL_BF16 = [
    # several query tiles + ragged tail (360 = 2*128 + 104), keys straddle pages
    Workload("bf16_s4_n360", S=4, W=4, n_chunk=12, F=3, Hh=10, Ww=12, n_heads=3,
             head_dim=128, n_layers=2),
    # one partial query tile; 72-key pages straddle every 64-key tile
    Workload("bf16_s2_n72", S=2, W=2, n_chunk=10, F=3, Hh=4, Ww=6, n_heads=2,
             head_dim=128, n_layers=1),
    # head_dim 64, no anchor, explicit store window
    Workload("bf16_d64_noanchor", S=3, W=1, W_store=2, anchor=0, n_chunk=9, F=2, Hh=10,
             Ww=10, n_heads=2, head_dim=64, n_layers=1),
    # Rolling-Forcing comparison mask
    Workload("bf16_rolling", S=3, W=2, n_chunk=8, F=2, Hh=8, Ww=15, n_heads=2,
             head_dim=128, n_layers=1, mask=wf.WF_MASK_ROLLING),
    # per-head query scale U(0.5, 2)
    Workload("bf16_headscale", S=2, W=3, n_chunk=9, F=1, Hh=16, Ww=16, n_heads=4,
             head_dim=128, n_layers=1, q_head_scale=True),
    # degenerate: one step, no history, no anchor
    Workload("bf16_s1_w0", S=1, W=0, anchor=0, n_chunk=5, F=1, Hh=8, Ww=8, n_heads=1,
             head_dim=128, n_layers=1),
    # degenerate: a single chunk never fills the pipeline
    Workload("bf16_single_chunk", S=3, W=2, n_chunk=1, F=1, Hh=8, Ww=16, n_heads=2,
             head_dim=128, n_layers=1),
]


@pytest.mark.parametrize("w", SMALL_BF16, ids=lambda w: w.name)
def test_small_bf16_every_round(w):
    _log(f"{w.name}: {w.n_chunk + w.S} rounds")
    full_rollout(w)


SMALL_FP8 = [
    # FP8 pages: 360 tokens -> 6 tiles per page, the last with 40 keys;
    # several query tiles with a ragged tail
    Workload("fp8_s4_n360", S=4, W=4, n_chunk=12, F=3, Hh=10, Ww=12, n_heads=3,
             head_dim=128, n_layers=2, dtype=wf.WF_FP8),
    # N a multiple of 64: no padding tokens
    Workload("fp8_s2_n128", S=2, W=2, n_chunk=8, F=2, Hh=8, Ww=8, n_heads=2,
             head_dim=128, n_layers=1, dtype=wf.WF_FP8),
    # 72 tokens: two tiles per page, the second with 8 keys
    Workload("fp8_s2_n72", S=2, W=2, n_chunk=8, F=3, Hh=4, Ww=6, n_heads=2,
             head_dim=128, n_layers=1, dtype=wf.WF_FP8),
    # a single 64-token tile per page; Rolling-Forcing comparison mask
    Workload("fp8_rolling_n64", S=3, W=2, n_chunk=7, F=1, Hh=8, Ww=8, n_heads=2,
             head_dim=128, n_layers=1, mask=wf.WF_MASK_ROLLING, dtype=wf.WF_FP8),
    # per-head query scale U(0.5, 2), no anchor
    Workload("fp8_headscale", S=2, W=3, anchor=0, n_chunk=7, F=1, Hh=16, Ww=16, n_heads=4,
             head_dim=128, n_layers=1, q_head_scale=True, dtype=wf.WF_FP8),
]


@pytest.mark.parametrize("w", SMALL_FP8, ids=lambda w: w.name)
def test_small_fp8_every_round(w):
    _log(f"{w.name}: {w.n_chunk + w.S} rounds")
    ro = Rollout(w)
    worst = 0.0
    try:
        for k in range(w.n_chunk + w.S):
            ro.run(k)
            for layer in range(w.n_layers):
                check_publish(ro, k, layer)
                worst = max(worst, check_attention(ro, k, layer))
    finally:
        ro.close()
    _log(f"  max abs err {worst:.3e}, {ro.fp8_bound_ratio:.2f} x the FP8 bound at worst")


@pytest.mark.timeout(600)
def test_full_size_wan13b_4step_fp8_sampled():
    """The 1.3B 4-step round over FP8 pages: steady state with the anchor
    re-rotated (k=14), first and last layer, 64 sampled rows per (group,
    head) plus the last row; whole pages."""
    w = WAN13B_4STEP_FP8
    ro = Rollout(w)
    try:
        for k in range(15):
            _log(f"{w.name} round {k}")
            ro.run(k)
            if k in (4, 14):
                for layer in (0, w.n_layers - 1):
                    check_publish(ro, k, layer)
                    err = check_attention(ro, k, layer, rows=64)
                    _log(f"  k={k} layer={layer} max abs err {err:.3e}, "
                         f"{ro.fp8_bound_ratio:.2f} x the FP8 bound at worst")
    finally:
        ro.close()


@pytest.mark.timeout(600)
def test_full_size_wan13b_4step_sampled():
    """1.3B shape, 4 steps, 30 layers: fill (k=4) and steady state with the
    anchor re-rotated (k=14); first and last layer; 64 sampled rows per
    (group, head) plus the last row; whole pages."""
    w = WAN13B_4STEP
    ro = Rollout(w)
    try:
        for k in range(15):
            _log(f"{w.name} round {k}")
            ro.run(k)
            if k in (4, 14):
                for layer in (0, w.n_layers - 1):
                    check_publish(ro, k, layer)
                    err = check_attention(ro, k, layer, rows=64)
                    _log(f"  k={k} layer={layer} max abs err {err:.3e}")
    finally:
        ro.close()


@pytest.mark.timeout(900)
@pytest.mark.parametrize("w", [WAN13B_5STEP, WAN13B_5STEP_ROLLING], ids=lambda w: w.name)
def test_full_size_wan13b_5step_sampled(w):
    """1.3B shape, 5 steps (and the Rolling-Forcing mask): two steady rounds
    (17: the first with the anchor re-rotated; 18), first and last layer,
    64 sampled rows per (group, head) plus the last row; whole pages and
    q_rot of both layers in round 17."""
    ro = Rollout(w)
    try:
        for k in range(19):
            _log(f"{w.name} round {k}")
            ro.run(k)
            if k in (17, 18):
                for layer in (0, w.n_layers - 1):
                    if k == 17:
                        check_publish(ro, k, layer)
                    err = check_attention(ro, k, layer, rows=64)
                    _log(f"  k={k} layer={layer} max abs err {err:.3e}")
    finally:
        ro.close()


@pytest.mark.timeout(1200)
def test_full_size_wan14b_4step_sampled():
    """14B-class shape (40 heads, per-head query scale U(0.5, 2)): two
    steady rounds (14: the anchor's first shift; 15), first and last layer,
    64 sampled rows per (group, head) plus the last row, at the fixed 2e-2
    bar; whole pages of the first layer."""
    w = WAN14B_4STEP
    ro = Rollout(w)
    try:
        for k in range(16):
            _log(f"{w.name} round {k}")
            ro.run(k)
            if k in (14, 15):
                for layer in (0, w.n_layers - 1):
                    if layer == 0:
                        check_publish(ro, k, layer)
                    err = check_attention(ro, k, layer, rows=64)
                    _log(f"  k={k} layer={layer} max abs err {err:.3e}")
    finally:
        ro.close()


@pytest.mark.timeout(1200)
def test_full_size_wan13b_long_rollout_two_layers():
    """The 133-chunk request at the 1.3B shape (137 rounds, automatic split)
    with two layers (layers are independent, so two bound the time): the
    slot ring wraps many times (k = 24, 70, 132) and the drain rounds
    133-136 run partial widths, where the split picks other groups.  Whole
    pages, q_rot and 32 sampled rows per (group, head) plus the last row,
    both layers."""
    w = WAN13B_4STEP.with_(name="wan1.3b_4step_2layer_rollout", n_layers=2)
    checked = (24, 70, 132, 133, 134, 135, 136)
    ro = Rollout(w)
    try:
        for k in range(w.n_chunk + w.S):
            ro.run(k)
            if k in checked:
                _log(f"{w.name} round {k}")
                for layer in range(w.n_layers):
                    check_publish(ro, k, layer)
                    err = check_attention(ro, k, layer, rows=32)
                    _log(f"  k={k} layer={layer} max abs err {err:.3e}")
    finally:
        ro.close()


SMALL_FP8K = [
    # 8-bit-key pages (FP8 keys, bf16 values): the FP8 shapes' edge cases
    Workload("fp8k_s4_n360", S=4, W=4, n_chunk=12, F=3, Hh=10, Ww=12, n_heads=3,
             head_dim=128, n_layers=2, dtype=wf.WF_FP8K),
    Workload("fp8k_s2_n128", S=2, W=2, n_chunk=8, F=2, Hh=8, Ww=8, n_heads=2,
             head_dim=128, n_layers=1, dtype=wf.WF_FP8K),
    Workload("fp8k_s2_n72", S=2, W=2, n_chunk=8, F=3, Hh=4, Ww=6, n_heads=2,
             head_dim=128, n_layers=1, dtype=wf.WF_FP8K),
    Workload("fp8k_rolling_n64", S=3, W=2, n_chunk=7, F=1, Hh=8, Ww=8, n_heads=2,
             head_dim=128, n_layers=1, mask=wf.WF_MASK_ROLLING, dtype=wf.WF_FP8K),
    Workload("fp8k_headscale", S=2, W=3, anchor=0, n_chunk=7, F=1, Hh=16, Ww=16, n_heads=4,
             head_dim=128, n_layers=1, q_head_scale=True, dtype=wf.WF_FP8K),
]


@pytest.mark.parametrize("w", SMALL_FP8K, ids=lambda w: w.name)
def test_small_fp8k_every_round(w):
    _log(f"{w.name}: {w.n_chunk + w.S} rounds")
    ro = Rollout(w)
    worst = 0.0
    try:
        for k in range(w.n_chunk + w.S):
            ro.run(k)
            for layer in range(w.n_layers):
                check_publish(ro, k, layer)
                worst = max(worst, check_attention(ro, k, layer))
    finally:
        ro.close()
    _log(f"  max abs err {worst:.3e}, {ro.fp8_bound_ratio:.2f} x the bound at worst")


@pytest.mark.timeout(600)
def test_full_size_wan13b_4step_fp8k_sampled():
    """The 1.3B 4-step round over 8-bit-key pages: steady state with the
    anchor re-rotated (k=14), first and last layer, 64 sampled rows per
    (group, head) plus the last row; whole pages."""
    w = WAN13B_4STEP_FP8K
    ro = Rollout(w)
    try:
        for k in range(15):
            _log(f"{w.name} round {k}")
            ro.run(k)
            if k in (4, 14):
                for layer in (0, w.n_layers - 1):
                    check_publish(ro, k, layer)
                    err = check_attention(ro, k, layer, rows=64)
                    _log(f"  k={k} layer={layer} max abs err {err:.3e}, "
                         f"{ro.fp8_bound_ratio:.2f} x the bound at worst")
    finally:
        ro.close()


@pytest.mark.parametrize("dtype", [wf.WF_BF16, wf.WF_FP8], ids=["bf16", "fp8"])
def test_unbounded_stream_finished_and_drained(dtype):
    """A stream (n_chunk = 0, WF §1): rounds 0..13 run with no last chunk
    known, then wf_finish_stream(14) ends it and rounds 14..16 drain.  Every
    round is checked against the oracle of the 14-chunk request (pages,
    q_rot, every attention output; the plans of the first 14 rounds are the
    same), and the outputs equal, bit for bit, those of the same inputs run
    as a bounded request from the start."""
    wb = Workload(f"stream_{dtype}", S=3, W=2, n_chunk=14, F=2, Hh=8, Ww=12, n_heads=2,
                  head_dim=128, n_layers=2, dtype=dtype)
    wu = wb.with_(n_chunk=0, max_frames=wb.F * 64)
    rounds = wb.n_chunk + wb.S
    ref = []
    rb = Rollout(wb, tag=wb.name)
    try:
        for k in range(rounds):
            rb.run(k)
            torch.cuda.synchronize()
            ref.append(rb.sess.bufs["out"].clone())
    finally:
        rb.close()
    ru = Rollout(wu, tag=wb.name)
    ru.w = wb                       # the oracle's view: the request as it ends
    worst = 0.0
    try:
        for k in range(rounds):
            if k == wb.n_chunk:
                wf.wf_finish_stream(ru.sess.h, wb.n_chunk)
            ru.run(k)
            for layer in range(wb.n_layers):
                check_publish(ru, k, layer)
                worst = max(worst, check_attention(ru, k, layer))
            assert torch.equal(ru.sess.bufs["out"], ref[k]), f"round {k}: stream != bounded"
    finally:
        ru.close()
    _log(f"  {rounds} rounds, max abs err {worst:.3e}")


SPLIT_CASES = [SMALL_BF16[0], SMALL_BF16[1], SMALL_BF16[2], SMALL_BF16[3], SMALL_FP8[0], SMALL_FP8[2],
               SMALL_FP8K[0], SMALL_FP8K[2], SMALL_FP8K[3]]


@pytest.mark.parametrize("w", SPLIT_CASES, ids=lambda w: w.name)
def test_small_split_every_round(w):
    """Every round with the two longest groups split into halves over their
    pages (partial results merged by the combine kernel), against the oracle
    at the same bars as the unsplit runs."""
    _log(f"{w.name} split: {w.n_chunk + w.S} rounds")
    ro = Rollout(w, split=wf.WF_SPLIT_FORCE)
    worst = 0.0
    try:
        for k in range(w.n_chunk + w.S):
            ro.run(k, mode="layers")
            for layer in range(w.n_layers):
                worst = max(worst, check_attention(ro, k, layer))
    finally:
        ro.close()
    _log(f"  max abs err {worst:.3e}")


def test_split_modes_agree_full_size_layer():
    """1.3B steady round, one layer: the automatic split, no split and the
    forced split give the same outputs up to fp32 merge rounding and the
    bf16 rounding of the output (two bf16 units at most)."""
    w = WAN13B_4STEP.with_(n_layers=1)
    outs = {}
    for mode in (wf.WF_SPLIT_OFF, wf.WF_SPLIT_AUTO, wf.WF_SPLIT_FORCE):
        ro = Rollout(w, split=mode)
        try:
            for k in range(14):
                ro.run(k)
            outs[mode] = ro.sess.bufs["out"][0].float().clone()
        finally:
            ro.close()
    ref = outs[wf.WF_SPLIT_OFF]
    for mode in (wf.WF_SPLIT_AUTO, wf.WF_SPLIT_FORCE):
        diff = (outs[mode] - ref).abs()
        bound = 2 * 2.0 ** -8 * ref.abs() + 1e-3
        _log(f"  mode {mode}: max |diff| {diff.max().item():.3e}")
        assert bool((diff <= bound).all()), (mode, diff.max().item())


class GrowingKeys(Rollout):
    """Keys of chunk i scaled by 1 + 0.8 i: along the context (anchor first,
    then history oldest first) a query row's running max keeps growing by
    several units of log2, so the kernels' lazy rescale fires after the
    first tile, not only on it."""

    def input_slice(self, rnd, layer, stage, name):
        x = super().input_slice(rnd, layer, stage, name)
        if name == "k":
            x = (x.float() * (1.0 + 0.8 * (rnd - stage))).to(x.dtype)
        return x


def _rescale_events(ro, k, layer, fp8):
    """(row, head, tile) triples of round k where the exact running row max
    (base-2 units, tiles in the kernel's order) grows by at least 9 after
    the first tile: the kernels must move m there (their trigger is 8)."""
    w, oc = ro.w, oracle_cfg(ro.w)
    c = WR.scale_of(oc) / np.log(2.0)
    n = 0
    for st in range(w.S + 1):
        if not P.chunk_active(oc, k - st):
            continue
        kk, _ = WR.group_keys(oc, k, st, layer, ro.raw, fp8=fp8)
        q = WR.q_rot(oc, k, st, layer, ro.raw)
        n_keys = kk.shape[0]
        if fp8:
            # page-aligned 64-key tiles, the last of each page partial
            bounds = [p * w.n_tokens + min(64 * t, w.n_tokens)
                      for p in range(n_keys // w.n_tokens) for t in range((w.n_tokens + 63) // 64)]
        else:
            bounds = list(range(0, n_keys, 64))
        bounds.append(n_keys)
        for h in range(w.n_heads):
            sc = c * (q[:, h, :] @ kk[:, h, :].T)
            tile_max = np.stack([sc[:, a:b].max(axis=1) for a, b in zip(bounds[:-1], bounds[1:])], 1)
            run = np.maximum.accumulate(tile_max, axis=1)
            n += int((run[:, 1:] - run[:, :-1] >= 9.0).sum())
    return n


@pytest.mark.parametrize("dtype", [wf.WF_BF16, wf.WF_FP8K, wf.WF_FP8], ids=["bf16", "fp8k", "fp8"])
def test_lazy_rescale_after_first_tile(dtype):
    """Queries whose running max grows along the context: every round and
    layer against the oracle, and the rounds checked are ones where the
    oracle's scores require the rescale to fire after the first tile.  The
    scores reach about 40 log2 units, so bf16 is held to its derived
    per-element bound (``wfcheck.bf16_attention_tolerance``), not the fixed
    2e-2 bar."""
    w = Workload(f"growing_keys_{dtype}", S=2, W=3, n_chunk=7, F=2, Hh=6, Ww=12, n_heads=2,
                 head_dim=128, n_layers=1, dtype=dtype)
    ro = GrowingKeys(w)
    fp8 = {wf.WF_FP8K: "k", wf.WF_FP8: True}.get(dtype, False)
    events = 0
    try:
        for k in range(w.n_chunk + w.S):
            ro.run(k)
            check_attention(ro, k, 0, derived=True)
            events += _rescale_events(ro, k, 0, fp8)
    finally:
        ro.close()
    ratio = getattr(ro, "bound_ratio", 0.0) or getattr(ro, "fp8_bound_ratio", 0.0)
    _log(f"  {events} (row, head, tile) rescale events after the first tile; "
         f"{ratio:.2f} x the bound at worst")
    assert events > 100
