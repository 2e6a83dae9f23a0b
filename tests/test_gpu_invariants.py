"""GPU invariants that need no oracle values: bit-identical outputs.

* Chunk-wise causal mask (WF §3.1 Eq. 4): perturbing the K/V of a noisier
  active chunk (stage j < s) leaves every stage-s output bit-identical.
* Same-graph scheduling (WF App. B.6, Proposition 1): the order and the
  streams the per-layer work is issued on do not change a single bit, as
  long as every attention runs after its layer's publish and the attention
  calls of a handle run one after another (they share the handle's split
  scratch; include/wf.h states the rule).
* Stale slots: slots a round neither reads nor writes may hold anything
  (NaN bytes here) without touching the outputs.
* HIP graphs: a round's layers captured into a graph replay to the eager bits.
"""

import gc

import pytest
import torch

from chunk_causal_dit_round_amd import wf
from chunk_causal_dit_round_amd.workloads import Workload
from oracle import wf_plan as P
from wfcheck import Rollout, oracle_cfg

pytestmark = pytest.mark.gpu

W_INV = Workload("bf16_invariants", S=4, W=2, n_chunk=10, F=2, Hh=8, Ww=12, n_heads=2,
                 head_dim=128, n_layers=2)


@pytest.fixture(autouse=True)
def _free_memory():
    yield
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def outputs(ro):
    torch.cuda.synchronize()
    return ro.sess.bufs["out"].clone()


DTYPES = [wf.WF_BF16, wf.WF_FP8, wf.WF_FP8K]
DTYPE_IDS = ["bf16", "fp8", "fp8k"]


@pytest.mark.parametrize("dtype", DTYPES, ids=DTYPE_IDS)
def test_causal_invariant_bit_identical(dtype):
    """Over FP8 pages too: a chunk's page (and its per-tile scales) is its
    own, so a noisier chunk's K/V cannot reach a cleaner stage."""
    w = W_INV.with_(name=f"causal_{dtype}", dtype=dtype)
    k = 9  # full width, anchor present
    for j in range(w.S):
        pert = {(k, layer, j, n): 3.0 for layer in range(w.n_layers) for n in ("k", "v")}
        base, moved = Rollout(w), Rollout(w, perturb=pert)
        try:
            for r in range(k + 1):
                base.run(r)
                moved.run(r)
            a, b = outputs(base), outputs(moved)
            for s in range(j + 1, w.S + 1):
                assert torch.equal(a[:, s], b[:, s]), (j, s)
            assert not torch.equal(a[:, j], b[:, j])
        finally:
            base.close()
            moved.close()


def test_same_graph_any_issue_order_and_streams():
    w = W_INV
    runs = {m: Rollout(w) for m in ("round", "layers", "publish_all_first", "two_streams")}
    s_pub, s_att = torch.cuda.Stream(), torch.cuda.Stream()
    try:
        for k in range(w.n_chunk + w.S):
            for m, ro in runs.items():
                if m != "two_streams":
                    ro.run(k, mode=m)
                    continue
                # publish on one stream, attention on another, ordered by events
                ro.fill(k)
                torch.cuda.synchronize()
                plan = ro.sess.plan(k)
                for layer in range(w.n_layers):
                    ro.sess.publish(plan, layer, stream=s_pub)
                    ev = torch.cuda.Event()
                    ev.record(s_pub)
                    s_att.wait_event(ev)
                    ro.sess.attention(plan, layer, stream=s_att)
                ro.sess.commit(plan)
                torch.cuda.synchronize()
            ref = outputs(runs["round"])
            for m, ro in runs.items():
                assert torch.equal(outputs(ro), ref), (k, m)
    finally:
        for ro in runs.values():
            ro.close()


@pytest.mark.parametrize("dtype", DTYPES, ids=DTYPE_IDS)
def test_stale_slots_do_not_matter(dtype):
    """Every byte of the slots a round does not use is 0xFF (NaN in bf16,
    E4M3 and as an E8M0 scale code)."""
    w = W_INV.with_(name=f"stale_{dtype}", dtype=dtype)
    oc = oracle_cfg(w)
    clean, poisoned = Rollout(w), Rollout(w)
    try:
        for k in range(w.n_chunk + w.S):
            p = P.plan(oc, k)
            live = {sl for g in p["groups"] for _, _, sl in g["entries"]}
            live |= {c["slot"] for c in p["cells"] if c["active"]}
            for layer in range(w.n_layers):
                for slot in range(oc.n_slots):
                    if slot not in live:
                        poisoned.sess.slot_bytes(layer, slot).fill_(0xFF)
            clean.run(k)
            poisoned.run(k)
            a, b = outputs(clean), outputs(poisoned)
            for s in range(w.S + 1):
                if P.chunk_active(oc, k - s):
                    assert torch.isfinite(b[:, s].float()).all(), (k, s)
                    assert torch.equal(a[:, s], b[:, s]), (k, s)
    finally:
        clean.close()
        poisoned.close()


def test_order_errors_on_device():
    """Host-side ordering contract with a bound handle: attention before
    publish, a skipped round, commit before every layer is published."""
    ro = Rollout(W_INV)
    try:
        s = ro.sess
        p0 = s.plan(0)
        assert wf.status_of(s.attention, p0, 0) == wf.WF_EORDER
        s.publish(p0, 0)
        assert wf.status_of(s.commit, p0) == wf.WF_EORDER
        s.publish(p0, 1)
        s.attention(p0, 0)
        s.attention(p0, 1)
        s.commit(p0)
        assert wf.status_of(s.publish, s.plan(2), 0) == wf.WF_EORDER
        assert s.next_round() == 1
        torch.cuda.synchronize()
    finally:
        ro.close()


@pytest.mark.parametrize("dtype", DTYPES, ids=DTYPE_IDS)
def test_round_layers_replay_in_a_hip_graph(dtype):
    """The layers of a round (publish + attention per layer) captured into
    a HIP graph: every replay, with eager work and synchronisations between
    replays, gives the bits the eager calls gave.  The library enqueues only
    kernels on the caller's stream (no allocation, no memset), so the round
    can sit inside a caller's graph."""
    w = W_INV.with_(name=f"graph_{dtype}", dtype=dtype)
    ro = Rollout(w)
    s = ro.sess
    try:
        k_cap = 7                                   # steady: anchor, history, all stages
        for k in range(k_cap):
            ro.run(k)
        ro.fill(k_cap)
        plan = s.plan(k_cap)

        def layers():
            for layer in range(w.n_layers):
                s.publish(plan, layer)
                s.attention(plan, layer)

        layers()                                    # eager
        torch.cuda.synchronize()
        eager_out = s.bufs["out"].clone()
        eager_q = s.bufs["q_rot"].clone()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            layers()
        torch.cuda.synchronize()
        for rep in range(3):
            s.bufs["out"].zero_()
            s.bufs["q_rot"].fill_(float("nan"))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(s.bufs["out"], eager_out), rep
            assert torch.equal(s.bufs["q_rot"], eager_q), rep
        s.commit(plan)
        ro.run(k_cap + 1)                           # the handle carries on normally
    finally:
        ro.close()
