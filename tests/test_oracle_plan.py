"""Pins for the oracle plan (schedule, ordered key lists, slot ring).

Each test checks the oracle against something other than itself: values the
Wave Forcing page prints (tests/golden/wf_printed_values.json), closed forms
from its equations, or a brute-force simulation of slot contents.
"""

import json
import os

import pytest

from oracle import wf_plan as P

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                   "wf_printed_values.json")))


def cfg(S=4, W=4, W_store=-1, anchor=1, n_chunk=133, mask=P.MASK_WAVE,
        F=3, Hh=4, Ww=6, heads=2, d=64, L=1):
    return P.Config(S=S, W=W, W_store=W_store, anchor=anchor, n_chunk=n_chunk,
                    F=F, Hh=Hh, Ww=Ww, n_heads=heads, head_dim=d, n_layers=L,
                    mask=mask)


SMALL = [cfg(S=S, W=W, W_store=Ws, anchor=A, n_chunk=N, mask=m)
         for S in range(1, 7) for N in (1, 2, 3, 5, 8, 13, 20)
         for (W, Ws) in ((0, -1), (2, -1), (3, 3), (4, 1)) for A in (0, 1)
         for m in (P.MASK_WAVE, P.MASK_ROLLING)]


def test_occupancy_printed_value():
    g = GOLD["occupancy"]
    c = cfg(S=g["S"], n_chunk=g["n_chunk"])
    assert c.n_rounds == g["rounds"]
    cells = sum(P.plan(c, k)["n_active"] for k in range(c.n_rounds))
    occ = cells / ((c.S + 1) * c.n_rounds)
    assert round(100 * occ, 1) == g["occupancy_percent_1dp"]


def test_workload_chunk_count():
    g = GOLD["workload"]
    assert g["latent_frames"] // g["latent_frames_per_chunk"] == g["n_chunk"]


def test_figure1c_five_chunks_in_five_rounds():
    g = GOLD["continuous_output"]
    c = cfg(S=g["S"], n_chunk=40)
    # Rounds after fill: k = S .. S+4.  A chunk completes when it is stored.
    done = [P.plan(c, k)["cells"][c.S]["chunk"]
            for k in range(c.S, c.S + g["rounds_after_fill"])]
    assert len(set(done)) == g["chunks_completed"]
    assert all(x >= 0 for x in done)


@pytest.mark.parametrize("c", SMALL, ids=lambda c: f"S{c.S}N{c.n_chunk}W{c.W}/{c.W_store}A{c.anchor}m{c.mask}")
def test_schedule_invariants(c):
    S, N = c.S, c.n_chunk
    total = 0
    visits = {}
    for k in range(c.n_rounds):
        p = P.plan(c, k)
        act = [x for x in p["cells"] if x["active"]]
        total += len(act)
        assert 1 <= len(act) <= S + 1                       # Eq. 2 width
        for x in act:                                        # Eq. 3
            assert x["chunk"] + x["stage"] == k
            visits.setdefault(x["chunk"], []).append((k, x["stage"]))
        store = p["cells"][S]
        assert store["active"] == (S <= k < N + S)           # one store
        full = len(act) == S + 1
        assert full == (S <= k < N)                          # App. B.4
    assert total == N * (S + 1)                              # App. B.4 work
    # every chunk visits stages 0..S in consecutive rounds i .. i+S
    for i in range(N):
        assert visits[i] == [(i + s, s) for s in range(S + 1)]
    if N <= S:
        assert not any(sum(x["active"] for x in P.plan(c, k)["cells"]) == S + 1
                       for k in range(c.n_rounds))


@pytest.mark.parametrize("c", SMALL[::3], ids=lambda c: f"S{c.S}N{c.n_chunk}W{c.W}/{c.W_store}A{c.anchor}m{c.mask}")
def test_mask_lower_triangular_in_chunk_order(c):
    """Eq. 4 restated in chunk order: query chunk i reads active denoising
    chunk i' iff i' <= i (WF); Rolling Forcing reads every active one."""
    for k in range(c.n_rounds):
        live = {k - j for j in P.denoise_active(c, k)}
        for s in range(c.S):
            i = k - s
            if not P.chunk_active(c, i):
                continue
            got = [ch for kd, ch, _ in P.key_entries(c, k, s) if kd == P.DENOISE]
            if c.mask == P.MASK_WAVE:
                want = sorted((x for x in live if x <= i), reverse=True)
            else:
                want = sorted(live, reverse=True)
            assert got == want
            if c.mask == P.MASK_WAVE:
                assert got[0] == i                            # self first


@pytest.mark.parametrize("c", SMALL[::2], ids=lambda c: f"S{c.S}N{c.n_chunk}W{c.W}/{c.W_store}A{c.anchor}m{c.mask}")
def test_context_order_eq5(c):
    """anchor, history (oldest first), live store, denoising by stage."""
    for k in range(c.n_rounds):
        for s in range(c.S + 1):
            e = P.key_entries(c, k, s)
            if not P.chunk_active(c, k - s):
                assert e == []
                continue
            kinds = [kd for kd, _, _ in e]
            assert kinds == sorted(kinds)
            assert kinds.count(P.ANCHOR) <= 1 and kinds.count(P.STORE) <= 1
            hist = [ch for kd, ch, _ in e if kd == P.HISTORY]
            assert hist == sorted(hist) and len(set(hist)) == len(hist)
            assert all(h < k - c.S for h in hist)            # clean only
            chunks = [ch for _, ch, _ in e]
            assert len(set(chunks)) == len(chunks)            # no duplicates
            if c.anchor:
                assert 0 not in hist
            win = c.w_store if s == c.S else c.W
            assert len(hist) <= win
            if s == c.S:
                assert kinds[-1] == P.STORE and P.DENOISE not in kinds


def test_eq10_key_counts_full_round():
    """N_s = N_prefix + (S - s) N_C with N_prefix = anchor + W + store."""
    for S, W in ((4, 4), (5, 6), (2, 2), (3, 0)):
        c = cfg(S=S, W=W, n_chunk=60)
        k = S + c.w_max + 2            # full width, full window, anchor on
        for s in range(S):
            n = len(P.key_entries(c, k, s))
            assert n == (1 + W + 1) + (S - s)
        # the store reserves one query chunk out of the same budget
        assert len(P.key_entries(c, k, S)) == 1 + W + 1 + S


def test_shared_window_reading():
    c = cfg(S=4, W=4, W_store=4, n_chunk=60)
    k = 20
    assert len(P.key_entries(c, k, c.S)) == 1 + 4 + 1
    assert [len(P.key_entries(c, k, s)) for s in range(4)] == [10, 9, 8, 7]


def test_fan_out_app_b8():
    """Denoiser j is read by j noisier ranks; S(S-1)/2 + S destinations."""
    for S in range(1, 7):
        c = cfg(S=S, W=2, n_chunk=40)
        k = S + c.w_max + 3
        readers = {}
        for s in range(S + 1):
            for kd, ch, _ in P.key_entries(c, k, s):
                if kd in (P.DENOISE, P.STORE):
                    readers.setdefault((kd, ch), set()).add(s)
        remote = 0
        for (kd, ch), rs in readers.items():
            producer = S if kd == P.STORE else k - ch
            others = rs - {producer}
            if kd == P.DENOISE:
                assert len(others) == producer                # j readers
            else:
                assert others == set(range(S))
            remote += len(others)
        assert remote == S * (S - 1) // 2 + S
        # stage-0 (noisiest) page is read by its own group only
        assert readers[(P.DENOISE, k)] == {0}


def test_round_range_and_anchor_timeline():
    c = cfg(S=4, W=4, n_chunk=20)
    with pytest.raises(ValueError):
        P.plan(c, -1)
    with pytest.raises(ValueError):
        P.plan(c, c.n_rounds)
    for k in range(c.n_rounds):
        p = P.plan(c, k)
        assert p["anchor"]["capture"] == (k == c.S)
        assert p["anchor"]["present"] == (k > c.S)
        if p["anchor"]["present"]:
            # anchor sits right before the oldest retained clean page
            oldest = max(1, k - c.S - c.w_max)
            assert p["anchor"]["frame0"] == c.F * (oldest - 1)


@pytest.mark.parametrize("c", [cfg(S=4, W=4, n_chunk=133), cfg(S=5, W=6, n_chunk=133),
                               cfg(S=2, W=2, W_store=4, n_chunk=16),
                               cfg(S=3, W=0, anchor=0, n_chunk=30),
                               cfg(S=1, W=5, W_store=2, n_chunk=25),
                               cfg(S=4, W=4, n_chunk=133, mask=P.MASK_ROLLING)],
                         ids=lambda c: f"S{c.S}W{c.W}/{c.W_store}A{c.anchor}N{c.n_chunk}m{c.mask}")
def test_slot_ring_brute_force(c):
    """Simulate slot contents by identity over the whole rollout.

    Round k writes its cells' pages and (if present) the re-rotated anchor;
    every key entry it reads must find the identity it names, written in this
    round or promoted earlier and not overwritten since.  Round k+1 must not
    write any slot that round k reads (double buffering of Eq. 13)."""
    _simulate_slots(c, c.n_rounds)


@pytest.mark.parametrize("c", [cfg(S=4, W=4, n_chunk=0), cfg(S=2, W=2, W_store=4, n_chunk=-1),
                               cfg(S=3, W=0, anchor=0, n_chunk=0),
                               cfg(S=5, W=6, n_chunk=0, mask=P.MASK_ROLLING)],
                         ids=lambda c: f"S{c.S}W{c.W}/{c.W_store}A{c.anchor}m{c.mask}")
def test_unbounded_request(c):
    """An unbounded request: every round from S on is full width with one
    store, slots stay within the same n_slots over 400 rounds (the ring keeps
    attention storage bounded, App. B.8), and round k's plan equals the plan
    of a bounded request of k + 1 + S chunks (so a stream can be ended at any
    round and drain like a bounded one)."""
    rounds = 400
    _simulate_slots(c, rounds)
    for k in range(rounds):
        p = P.plan(c, k)
        assert p["n_active"] == min(k + 1, c.S + 1)
        assert p["cells"][c.S]["active"] == (k >= c.S)
        if k % 37 == 0 or k < 3 * c.S:
            b = P.Config(**{**c.__dict__, "n_chunk": k + 1 + c.S})
            assert P.plan(b, k) == p
    with pytest.raises(ValueError):
        c.n_rounds


def _simulate_slots(c, rounds):
    plans = [P.plan(c, k) for k in range(rounds)]
    content = {}
    prev_reads = set()
    for k in range(rounds):
        p = plans[k]
        writes = {}
        for x in p["cells"]:
            if x["active"]:
                kind = "clean" if x["stage"] == c.S else "denoise"
                writes[x["slot"]] = (kind, x["chunk"], k)
        if p["anchor"]["present"]:
            writes[p["anchor"]["slot"]] = ("anchor", 0, k)
        assert len(writes) == sum(x["active"] for x in p["cells"]) + p["anchor"]["present"]
        assert not (set(writes) & prev_reads)
        assert all(0 <= s < c.n_slots for s in writes)
        content.update(writes)
        reads = set()
        for g in p["groups"]:
            for kd, ch, sl in g["entries"]:
                reads.add(sl)
                have = content[sl]
                if kd == P.ANCHOR:
                    assert have == ("anchor", 0, k)
                elif kd == P.DENOISE:
                    assert have == ("denoise", ch, k)
                else:
                    assert have[0] == "clean" and have[1] == ch
                    assert have[2] == ch + c.S
        # evicted chunk is no longer read in any later round
        ev = p["evict"]
        if ev >= 0:
            for k2 in range(k + 1, rounds):
                for g in plans[k2]["groups"]:
                    assert all(not (kd == P.HISTORY and ch == ev)
                               for kd, ch, _ in g["entries"])
        prev_reads = reads


@pytest.mark.parametrize("c", [cfg(S=4, W=4, n_chunk=40), cfg(S=2, W=2, W_store=4, n_chunk=16),
                               cfg(S=3, W=0, anchor=0, n_chunk=12), cfg(S=1, W=5, W_store=2, n_chunk=25),
                               cfg(S=3, W=3, W_store=1, n_chunk=20)],
                         ids=lambda c: f"S{c.S}W{c.W}/{c.W_store}A{c.anchor}N{c.n_chunk}")
def test_evicted_chunk_is_the_oldest_retained_page(c):
    """Brute force of the clean list (App. B.3, B.8): after each round the
    store's chunk joins the retained list (the anchor chunk 0 never does, R4)
    and, past max(W, W_store) pages, the oldest leaves; that one is the
    round's evicted chunk, and every history page a later round reads is
    still retained."""
    retained = []
    for k in range(c.n_rounds):
        p = P.plan(c, k)
        for g in p["groups"]:
            for kd, ch, _ in g["entries"]:
                if kd == P.HISTORY:
                    assert ch in retained
        dropped = -1
        if p["cells"][c.S]["active"]:
            ch = k - c.S
            if not (c.anchor == 1 and ch == 0):
                retained.append(ch)
            if len(retained) > c.w_max:
                dropped = retained.pop(0)
        assert p["evict"] == dropped, (k, p["evict"], dropped)


@pytest.mark.parametrize("c", [cfg(S=3, W=2, n_chunk=9, F=1, Hh=2, Ww=3, heads=2, d=16, L=2),
                               cfg(S=2, W=1, W_store=3, anchor=0, n_chunk=6, F=2, Hh=1, Ww=3,
                                   heads=3, d=8, L=1, mask=P.MASK_ROLLING)],
                         ids=["wave", "rolling"])
def test_plan_flops_match_torch_flop_counter(c):
    """The plan's FLOPs (what the roofline divides by) equal what torch's FLOP
    counter reports for the two products of plain attention (scores Q K^T,
    then P V) of every active group over its context, every layer, in every
    round.  (The counter does not see torch's CPU scaled_dot_product_attention
    kernel, so the products are run as matmuls.)"""
    import torch
    from torch.utils.flop_counter import FlopCounterMode

    for k in range(c.n_rounds):
        p = P.plan(c, k)
        counter = FlopCounterMode(display=False)
        with counter:
            for _ in range(c.n_layers):
                for g in p["groups"]:
                    n_k = len(g["entries"]) * c.n_c
                    if n_k == 0:
                        continue
                    q = torch.zeros(1, c.n_heads, c.n_c, c.head_dim, dtype=torch.float64)
                    kv = torch.zeros(1, c.n_heads, n_k, c.head_dim, dtype=torch.float64)
                    q @ kv.transpose(-1, -2)                         # scores
                    torch.zeros(1, c.n_heads, c.n_c, n_k, dtype=torch.float64) @ kv   # P V
        assert p["flops"] == counter.get_total_flops(), k


def test_payload_bytes_formula():
    # Per-chunk K+V page size equals the page's per-edge payload formula.
    c = cfg(S=4, W=4, n_chunk=133, F=3, Hh=30, Ww=52, heads=12, d=128)
    page = 2 * c.n_c * c.n_heads * c.head_dim * 2
    assert c.n_c == 4680
    assert page == 28_753_920
