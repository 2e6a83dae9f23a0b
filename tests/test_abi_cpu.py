"""C-ABI checks that need no GPU: exports, plan parity, error paths.

``wf_round_plan`` is host-only integer code, so the C library's plans are
compared here, field by field and bit-exactly, with the independent oracle
(``oracle/wf_plan.py``).  Error paths are forced from the host; every failing
call returns before any device work.
"""

import ctypes
import os
import re

import pytest

from chunk_causal_dit_round_amd import wf
from chunk_causal_dit_round_amd.workloads import (ALL, TINY_FP32, WAN13B_4STEP, WAN13B_4STEP_FP8,
                                                  WAN13B_4STEP_FP8K)
from oracle import wf_plan as P

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    names = set()
    for f in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if f.endswith(".h"):
            text = open(os.path.join(ROOT, "include", f)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"\b(wf_[a-z_]+)\s*\(", text))
    return sorted(names)


def test_library_exports_every_declared_function():
    names = header_functions()
    assert len(names) == 22, names
    assert {"wf_dit_workspace_bytes", "wf_dit_layer", "wf_dit_round"} <= set(names)
    lib = ctypes.CDLL(wf.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def oracle_cfg(c):
    return P.Config(S=c.S, W=c.W, W_store=c.W_store, anchor=c.anchor, n_chunk=c.n_chunk,
                    F=c.F, Hh=c.Hh, Ww=c.Ww, n_heads=c.n_heads, head_dim=c.head_dim,
                    n_layers=c.n_layers, mask=c.mask)


CONFIGS = [wf.make_config(S, W, N, 3, 4, 6, 2, 64, 3, W_store=Ws, anchor=A, mask=m, dtype=wf.WF_F32)
           for S in (1, 2, 3, 4, 5, 8) for N in (1, 2, 5, 9, 16)
           for (W, Ws) in ((0, -1), (2, -1), (4, 4), (6, 2), (3, 0)) for A in (0, 1)
           for m in (wf.WF_MASK_WAVE, wf.WF_MASK_ROLLING)]
CONFIGS += [w.config() for w in ALL.values()]


@pytest.mark.parametrize("cfg", CONFIGS, ids=lambda c: f"S{c.S}W{c.W}/{c.W_store}A{c.anchor}N{c.n_chunk}m{c.mask}H{c.n_heads}")
def test_plan_parity_with_oracle(cfg):
    h = wf.wf_create(cfg)
    oc = oracle_cfg(cfg)
    try:
        for k in range(oc.n_rounds):
            got = wf.plan_to_dict(wf.wf_round_plan(h, k))
            want = P.plan(oc, k)
            for key in ("k", "cells", "groups", "anchor", "evict", "kv_tokens", "n_active"):
                assert got[key] == want[key], (k, key)
            assert got["flops"] == want["flops"]
    finally:
        wf.wf_destroy(h)


def test_plan_numbers_1p3b_4step():
    h = wf.wf_create(WAN13B_4STEP.config())
    p = wf.wf_round_plan(h, 13)
    assert [p.groups[s].n_pages for s in range(5)] == [10, 9, 8, 7, 10]
    assert abs(p.flops - 1.7763e14) / 1.7763e14 < 1e-4
    # publish: 5 cells x (q,k,v in; q_rot,K,Vt out) + anchor (2 in, 2 out), 30 layers
    nhd2 = 4680 * 12 * 128 * 2
    assert p.publish_bytes == 30 * (30 + 4) * nhd2
    wf.wf_destroy(h)


def test_pool_bytes():
    cfg = WAN13B_4STEP.config()
    pool, anc, tab = wf.wf_pool_bytes(cfg)
    page = 2 * 4680 * 12 * 128 * 2
    assert pool == 30 * 20 * page
    assert anc == 30 * page
    # frame-axis frequencies (22 doubles), then row and column cos/sin tables
    rope = 22 * 8 + (30 * 21 + 52 * 21) * 8
    nh = 4680 * 12
    # RoPE tables rounded up to 256 bytes, then the split scratch: two split
    # groups x two halves x (O [N][H][D] + (e, l) [N][H]) in fp32
    assert tab == -(-rope // 256) * 256 + 2 * 2 * (nh * 128 + 2 * nh) * 4


@pytest.mark.parametrize("w", list(ALL.values()), ids=lambda w: w.name)
def test_page_layout_matches_the_page_formats(w):
    """wf_page_layout: the slot count is the oracle's ring (4 + max(W,
    W_store) + 2 S), the sizes agree with wf_pool_bytes, and the offsets are
    those of the page formats in wf.h (K at 0; Vt after H x Npad x D keys of
    1 byte on FP8 / FP8K pages, else H x N x D elements; codes after Vt)."""
    cfg = w.config()
    lay = wf.wf_page_layout(cfg)
    pool, anc, tab = wf.wf_pool_bytes(cfg)
    oc = oracle_cfg(cfg)
    N, H, D, L = w.n_tokens, w.n_heads, w.head_dim, w.n_layers
    T = -(-N // 64)
    assert lay.n_slots == oc.n_slots
    assert (lay.pool_bytes, lay.anchor_bytes, lay.table_bytes) == (pool, anc, tab)
    assert lay.pool_bytes == L * lay.n_slots * lay.page_bytes
    assert lay.anchor_bytes == L * lay.anchor_page_bytes == L * 2 * H * N * D * (4 if w.dtype == wf.WF_F32 else 2)
    assert (lay.tokens, lay.tiles) == (N, T)
    if w.dtype in (wf.WF_FP8, wf.WF_FP8K):
        vb = 1 if w.dtype == wf.WF_FP8 else 2
        assert lay.tokens_padded == 64 * T
        assert lay.vt_offset == H * 64 * T * D
        assert lay.codes_offset == lay.vt_offset + vb * H * 64 * T * D
        assert lay.page_bytes == -(-(lay.codes_offset + 2 * H * T) // 256) * 256
    else:
        eb = 4 if w.dtype == wf.WF_F32 else 2
        assert lay.tokens_padded == N and lay.codes_offset == -1
        assert lay.vt_offset == H * N * D * eb and lay.page_bytes == 2 * lay.vt_offset
    nh = N * H
    assert lay.split_scratch_bytes == (0 if w.dtype == wf.WF_F32 else 2 * 2 * (nh * D + 2 * nh) * 4)
    assert lay.split_scratch_offset % 256 == 0
    assert lay.split_scratch_offset + lay.split_scratch_bytes == lay.table_bytes


def test_pool_bytes_fp8():
    """FP8 pages: K8 [H][Npad][D] + Vt8 [H][D][Npad] + codes [H][T][2], rounded
    up to 256 bytes; the anchor store keeps bf16 raw K and Vt."""
    cfg = WAN13B_4STEP_FP8.config()
    pool, anc, tab = wf.wf_pool_bytes(cfg)
    T = (4680 + 63) // 64
    page = -(-(2 * 12 * 64 * T * 128 + 2 * 12 * T) // 256) * 256
    assert T == 74 and pool == 30 * 20 * page
    assert anc == 30 * 2 * 4680 * 12 * 128 * 2
    assert tab == wf.wf_pool_bytes(WAN13B_4STEP.config())[2]


def test_plan_numbers_fp8():
    h = wf.wf_create(WAN13B_4STEP_FP8.config())
    p = wf.wf_round_plan(h, 13)
    assert abs(p.flops - 1.7763e14) / 1.7763e14 < 1e-4
    # per cell: q,k,v in (bf16) + q_rot out (bf16) + K, Vt out (1 byte);
    # anchor: raw K, Vt in (bf16) + anchor slot out (1 byte)
    nhd = 4680 * 12 * 128
    assert p.publish_bytes == 30 * (5 * 10 + 6) * nhd
    wf.wf_destroy(h)


def test_pool_bytes_fp8k():
    """8-bit-key pages: K8 [H][Npad][D] (1 byte) + Vt [H][D][Npad] (bf16) +
    codes [H][T][2], rounded up to 256 bytes."""
    cfg = WAN13B_4STEP_FP8K.config()
    pool, anc, tab = wf.wf_pool_bytes(cfg)
    T = 74
    page = -(-(3 * 12 * 64 * T * 128 + 2 * 12 * T) // 256) * 256
    assert pool == 30 * 20 * page
    assert anc == 30 * 2 * 4680 * 12 * 128 * 2
    assert tab == wf.wf_pool_bytes(WAN13B_4STEP.config())[2]


def test_plan_numbers_fp8k():
    """Same FLOPs as bf16; per cell q,k,v in + q_rot out (bf16), K out (1
    byte) and Vt out (bf16); anchor: raw K, Vt in + K (1) and Vt (2) out."""
    h = wf.wf_create(WAN13B_4STEP_FP8K.config())
    p = wf.wf_round_plan(h, 13)
    assert abs(p.flops - 1.7763e14) / 1.7763e14 < 1e-4
    nhd = 4680 * 12 * 128
    assert p.publish_bytes == 30 * (5 * 11 + 7) * nhd
    wf.wf_destroy(h)


def test_fp8_unsupported_shapes():
    fake = 1 << 20
    for w in (WAN13B_4STEP_FP8.with_(head_dim=64), WAN13B_4STEP_FP8.with_(Ww=51),
              # longest context 40 pages x 104 tiles > 4096 tiles
              WAN13B_4STEP_FP8.with_(W=30, Hh=40, Ww=55),
              WAN13B_4STEP_FP8K.with_(head_dim=64), WAN13B_4STEP_FP8K.with_(Ww=51),
              WAN13B_4STEP_FP8K.with_(W=30, Hh=40, Ww=55)):
        cfg = w.config()
        h = wf.wf_create(cfg)
        pb, ab, tb = wf.wf_pool_bytes(cfg)
        assert wf.status_of(wf.wf_bind, h, fake, pb, fake, ab, fake, tb) == wf.WF_EUNSUPPORTED
        assert wf.wf_last_error() != ""
        wf.wf_destroy(h)


BAD = [dict(S=0), dict(S=9), dict(W=-1), dict(W_store=-2), dict(anchor=2), dict(n_chunk=0),
       dict(F=0), dict(n_heads=0), dict(head_dim=7), dict(head_dim=4), dict(n_layers=0),
       dict(dtype=5), dict(mask=3), dict(max_frames=5), dict(rope_theta=-1.0),
       dict(rope_theta=0.5), dict(softmax_scale=-1.0), dict(W=40, S=8),
       dict(n_chunk=0, max_frames=2), dict(n_chunk=-1, max_frames=(1 << 30) + 1),
       dict(n_chunk=1 << 29)]


@pytest.mark.parametrize("bad", BAD, ids=lambda d: ",".join(f"{k}={v}" for k, v in d.items()))
def test_invalid_config_rejected(bad):
    cfg = TINY_FP32.config()
    for k, v in bad.items():
        setattr(cfg, k, v)
    assert wf.status_of(wf.wf_create, cfg) == wf.WF_EINVAL
    assert wf.wf_last_error() != ""
    assert wf.status_of(wf.wf_pool_bytes, cfg) == wf.WF_EINVAL


def test_round_range_and_order_errors():
    cfg = TINY_FP32.config()
    h = wf.wf_create(cfg)
    h2 = wf.wf_create(WAN13B_4STEP.config())
    try:
        assert wf.status_of(wf.wf_round_plan, h, -1) == wf.WF_ERANGE
        assert wf.status_of(wf.wf_round_plan, h, 8) == wf.WF_ERANGE
        assert wf.wf_next_round(h) == 0
        p1 = wf.wf_round_plan(h, 1)
        p0 = wf.wf_round_plan(h, 0)
        other = wf.wf_round_plan(h2, 0)
        # not the next round / another config: rejected before anything else
        for fn, args in ((wf.wf_kv_publish, (0, 16, 16, 16, 16)),
                         (wf.wf_wave_attention, (0, 16, 16)),
                         (wf.wf_round, (16, 16, 16, 16, 16))):
            assert wf.status_of(fn, h, p1, *args, stream=0) == wf.WF_EORDER
            assert wf.status_of(fn, h, other, *args, stream=0) == wf.WF_EORDER
            # right round, but the handle is not bound
            assert wf.status_of(fn, h, p0, *args, stream=0) == wf.WF_EINVAL
        assert wf.status_of(wf.wf_round_commit, h, p1) == wf.WF_EORDER
        assert wf.status_of(wf.wf_round_commit, h, p0) == wf.WF_EORDER   # nothing published
        # a modified plan is refused
        bad = wf.wf_round_plan(h, 0)
        bad.groups[0].slot[0] = 99
        assert wf.status_of(wf.wf_round_commit, h, bad) == wf.WF_EINVAL
        assert wf.status_of(wf.wf_reset, h) == wf.WF_OK
    finally:
        wf.wf_destroy(h)
        wf.wf_destroy(h2)


def test_bind_errors_before_device_work():
    cfg = TINY_FP32.config()
    h = wf.wf_create(cfg)
    pb, ab, tb = wf.wf_pool_bytes(cfg)
    fake = 1 << 20    # never dereferenced: every case fails before device work
    try:
        assert wf.status_of(wf.wf_bind, h, fake, pb - 1, fake, ab, fake, tb) == wf.WF_ESMALL
        assert wf.status_of(wf.wf_bind, h, fake, pb, fake, ab - 1, fake, tb) == wf.WF_ESMALL
        assert wf.status_of(wf.wf_bind, h, fake, pb, fake, ab, fake, tb - 1) == wf.WF_ESMALL
        assert wf.status_of(wf.wf_bind, h, None, pb, fake, ab, fake, tb) == wf.WF_EINVAL
        assert wf.status_of(wf.wf_bind, h, fake + 4, pb, fake, ab, fake, tb) == wf.WF_EINVAL
    finally:
        wf.wf_destroy(h)
    for w in (WAN13B_4STEP.with_(head_dim=96), WAN13B_4STEP.with_(Ww=51),
              WAN13B_4STEP.with_(F=1, Hh=7, Ww=8),
              TINY_FP32.with_(head_dim=66), TINY_FP32.with_(head_dim=256)):
        cfg = w.config()
        h = wf.wf_create(cfg)
        pb, ab, tb = wf.wf_pool_bytes(cfg)
        assert wf.status_of(wf.wf_bind, h, fake, pb, fake, ab, fake, tb) == wf.WF_EUNSUPPORTED
        wf.wf_destroy(h)


def test_strerror():
    for s in range(0, -7, -1):
        assert wf.wf_strerror(s) and wf.wf_strerror(s) != "unknown status"
    assert wf.wf_strerror(-99) == "unknown status"


def test_dit_workspace_bytes_and_errors_before_device_work():
    cfg = WAN13B_4STEP.config()
    h = wf.wf_create(cfg)
    fake = 1 << 20    # never dereferenced
    try:
        dc = wf.make_dit_config(8960)
        got = wf.wf_dit_workspace_bytes(h, dc)
        rows, C = 5 * 4680, 1536
        up = lambda x: -(-x // 256) * 256  # noqa: E731
        # a, qkv, q, k, v, q_rot, o (bf16), y (fp32), FFN hidden (bf16), GEMM workspace
        want = (up(rows * C * 2) + up(rows * 3 * C * 2) + 5 * up(rows * C * 2) + up(rows * C * 4)
                + up(rows * 8960 * 2) + (64 << 20))
        assert got == want
        for bad in (wf.make_dit_config(0), wf.make_dit_config(7), wf.make_dit_config(64, eps=-1.0)):
            assert wf.status_of(wf.wf_dit_workspace_bytes, h, bad) == wf.WF_EINVAL
        names = [n for n, _ in wf.wf_dit_weights._fields_]
        W = wf.make_dit_weights([{n: fake for n in names} for _ in range(30)])
        p0, p1 = wf.wf_round_plan(h, 0), wf.wf_round_plan(h, 1)
        args = (fake, fake, fake, got)
        assert wf.status_of(wf.wf_dit_layer, h, p1, 0, dc, W, *args, stream=0) == wf.WF_EORDER
        assert wf.status_of(wf.wf_dit_round, h, p1, dc, W, *args, stream=0) == wf.WF_EORDER
        assert wf.status_of(wf.wf_dit_layer, h, p0, 30, dc, W[0], *args, stream=0) == wf.WF_EINVAL
        assert wf.status_of(wf.wf_dit_layer, h, p0, 0, dc, W, *args, stream=0) == wf.WF_EINVAL
        assert "not bound" in wf.wf_last_error()
        assert wf.status_of(wf.wf_dit_round, h, p0, dc, W, *args, stream=0) == wf.WF_EINVAL
    finally:
        wf.wf_destroy(h)
    # C beyond the row kernels' limit
    w = WAN13B_4STEP.with_(n_heads=72)
    h = wf.wf_create(w.config())
    try:
        assert wf.status_of(wf.wf_dit_workspace_bytes, h, wf.make_dit_config(64)) == wf.WF_EUNSUPPORTED
    finally:
        wf.wf_destroy(h)


def test_split_mode_checked_on_the_host():
    h = wf.wf_create(WAN13B_4STEP.config())
    try:
        for mode in (wf.WF_SPLIT_OFF, wf.WF_SPLIT_FORCE, wf.WF_SPLIT_AUTO):
            wf.wf_set_attention_split(h, mode)
        assert wf.status_of(wf.wf_set_attention_split, h, 3) == wf.WF_EINVAL
        assert wf.status_of(wf.wf_set_attention_split, h, -1) == wf.WF_EINVAL
    finally:
        wf.wf_destroy(h)
    assert wf.status_of(wf.wf_set_attention_split, None, 0) == wf.WF_EINVAL


def test_fp32_rounds_have_no_split_scratch():
    from chunk_causal_dit_round_amd.workloads import TINY_FP32
    _, _, tab = wf.wf_pool_bytes(TINY_FP32.config())
    # 12 frame-axis frequencies (fp64, padded to 16 bytes); cos/sin of the
    # 4 rows and 6 columns, 10 pairs each (64 dims: 12, 10, 10 pairs)
    rope = 12 * 8 + (4 * 10 + 6 * 10) * 8
    assert tab == -(-rope // 256) * 256


def _plan_bytes(p):
    return bytes(memoryview(p))


@pytest.mark.parametrize("w", [TINY_FP32, WAN13B_4STEP, WAN13B_4STEP_FP8K], ids=lambda w: w.name)
def test_unbounded_request_plans(w):
    """n_chunk <= 0: the plan of every round equals the oracle's unbounded
    plan, every field of it (hash aside) equals the plan of the bounded
    request of k + 1 + S chunks, rounds stop where F (k + 1) would exceed
    max_frames, and no buffer size depends on the request's length."""
    rounds = 200
    ub = w.with_(n_chunk=0)
    cfg = ub.config()
    cfg.max_frames = w.F * rounds
    h = wf.wf_create(cfg)
    oc = oracle_cfg(cfg)
    assert oc.unbounded
    try:
        for k in range(rounds):
            got = wf.plan_to_dict(wf.wf_round_plan(h, k))
            want = P.plan(oc, k)
            for key in ("k", "cells", "groups", "anchor", "evict", "kv_tokens", "n_active"):
                assert got[key] == want[key], (k, key)
            assert got["flops"] == want["flops"]
            if k % 23 == 0:
                hb = wf.wf_create(w.with_(n_chunk=k + 1 + w.S).config())
                assert wf.plan_to_dict(wf.wf_round_plan(hb, k)) == got
                wf.wf_destroy(hb)
        assert wf.status_of(wf.wf_round_plan, h, rounds) == wf.WF_ERANGE
        assert "max_frames" in wf.wf_last_error()
    finally:
        wf.wf_destroy(h)
    assert wf.wf_pool_bytes(cfg) == wf.wf_pool_bytes(w.config())
    a, b = wf.wf_page_layout(cfg), wf.wf_page_layout(w.config())
    assert all(getattr(a, f) == getattr(b, f) for f, _ in wf.wf_layout._fields_)


def test_finish_stream_turns_into_the_bounded_request():
    """wf_finish_stream(n): the handle's following plans are byte for byte
    those of a handle created for the bounded request of n chunks (config
    hash included), fill and drain alike; plans made before are rejected;
    bounded handles and n out of range are refused."""
    w = TINY_FP32
    cfg = w.with_(n_chunk=0).config()
    cfg.max_frames = 1 << 20
    h = wf.wf_create(cfg)
    old = wf.wf_round_plan(h, 0)
    assert wf.status_of(wf.wf_finish_stream, h, 0) == wf.WF_EINVAL
    wf.wf_finish_stream(h, 7)
    hb = wf.wf_create(w.with_(n_chunk=7).config())
    try:
        for k in range(7 + w.S):
            assert _plan_bytes(wf.wf_round_plan(h, k)) == _plan_bytes(wf.wf_round_plan(hb, k))
        assert wf.status_of(wf.wf_round_plan, h, 7 + w.S) == wf.WF_ERANGE
        assert old.config_hash != wf.wf_round_plan(h, 0).config_hash
        assert wf.status_of(wf.wf_finish_stream, h, 9) == wf.WF_EINVAL      # now bounded
        assert wf.status_of(wf.wf_finish_stream, hb, 9) == wf.WF_EINVAL
        assert "bounded" in wf.wf_last_error()
    finally:
        wf.wf_destroy(h)
        wf.wf_destroy(hb)


def test_device_failure_is_reported_as_wf_edevice():
    """WF_EDEVICE, forced from the host: with no GPU visible, the table
    upload of a valid, supported and correctly sized wf_bind fails inside
    the HIP runtime; the call returns WF_EDEVICE and wf_last_error names the
    HIP error (the buffer addresses are never dereferenced: no device)."""
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is visible: the upload would run")
    cfg = TINY_FP32.config()
    h = wf.wf_create(cfg)
    try:
        pb, ab, tb = wf.wf_pool_bytes(cfg)
        fake = 1 << 20
        assert wf.status_of(wf.wf_bind, h, fake, pb, fake, ab, fake, tb) == wf.WF_EDEVICE
        err = wf.wf_last_error()
        assert err.startswith("table upload: ") and len(err) > len("table upload: "), err
        plan = wf.wf_round_plan(h, 0)
        # the handle stays unbound: later calls fail before any device work
        assert wf.status_of(wf.wf_kv_publish, h, plan, 0, fake, fake, fake, fake, 0) == wf.WF_EINVAL
    finally:
        wf.wf_destroy(h)


# ---- the attention launch's split choice (host only) ----

def _model_split(w, pages_by_stage, n_cu=256):
    """The split model wf_set_attention_split documents, written out: every
    work-group (group or half, head, 256 query rows) taken longest first by
    n_cu compute units, one at a time each; a work-group costs its key
    tiles + 2; plus the merge per split group.  Returns the strictly
    cheapest split found scanning none, the halves of every single group,
    then of every pair."""
    import heapq
    import math

    N, H, D = w.Hh * w.Ww * w.F, w.n_heads, w.head_dim
    bm = 256
    per_group = H * ((N + bm - 1) // bm)
    T = (N + 63) // 64

    def end(pages):
        free_at = [0.0] * n_cu
        e = 0.0
        for p in sorted(pages, reverse=True):
            tiles = (math.ceil(p * N / 64.0) if w.dtype == wf.WF_BF16 else float(p * T)) + 2.0
            for _ in range(per_group):
                t = heapq.heappop(free_at) + tiles
                heapq.heappush(free_at, t)
                e = max(e, t)
        return e

    tile_s = bm * 64.0 * D * 4.0 / (1.1e15 / n_cu)
    merge = 2.0 + 10.0 * N * H * D / 5e12 / tile_s
    active = [s for s in sorted(pages_by_stage) if pages_by_stage[s] > 0]

    def cost(sp):
        pages = []
        for s in active:
            n = pages_by_stage[s]
            pages += [n // 2, n - n // 2] if s in sp else [n]
        return end(pages) + merge * len(sp)

    cand = sorted([s for s in active if pages_by_stage[s] >= 2], key=lambda s: -pages_by_stage[s])
    best, best_cost = [], cost([])
    for s in cand:
        c = cost([s])
        if c < best_cost:
            best, best_cost = [s], c
    for i in range(len(cand)):
        for j in range(i + 1, len(cand)):
            c = cost([cand[i], cand[j]])
            if c < best_cost:
                best, best_cost = [cand[i], cand[j]], c
    return [(s, pages_by_stage[s] // 2) for s in best]


def _group_pages(p):
    return {s: p.groups[s].n_pages for s in range(p.S + 1)}


@pytest.mark.parametrize("w", [WAN13B_4STEP, WAN13B_4STEP_FP8, WAN13B_4STEP_FP8K],
                         ids=lambda w: w.name)
def test_split_choice_follows_the_launch_model(w):
    """AUTO's choice equals the documented model's on every distinct list of
    group lengths of the whole 1.3B request (fill, steady, drain); every
    split is of an active group, in halves; repeated queries agree."""
    h = wf.wf_create(w.config())
    try:
        seen = {}
        for k in range(w.n_chunk + w.S):
            p = wf.wf_round_plan(h, k)
            pages = _group_pages(p)
            key = tuple(pages[s] for s in sorted(pages))
            got = wf.wf_attention_split_choice(h, p)
            assert got == wf.wf_attention_split_choice(h, p)
            assert len(got) <= wf.WF_MAX_SPLIT and len({s for s, _ in got}) == len(got)
            for s, at in got:
                assert pages[s] >= 2 and at == pages[s] // 2
            if key not in seen:
                seen[key] = _model_split(w, pages)
            assert got == seen[key], (k, pages)
        steady = wf.wf_round_plan(h, 16)
        assert [steady.groups[s].n_pages for s in range(5)] == [10, 9, 8, 7, 10]
        # the steady round's choice: the 7-page group, as 3 + 4 pages
        assert wf.wf_attention_split_choice(h, steady) == [(3, 3)]
    finally:
        wf.wf_destroy(h)


def test_split_choice_off_force_and_fp32():
    h = wf.wf_create(WAN13B_4STEP.config())
    try:
        p = wf.wf_round_plan(h, 16)
        wf.wf_set_attention_split(h, wf.WF_SPLIT_OFF)
        assert wf.wf_attention_split_choice(h, p) == []
        wf.wf_set_attention_split(h, wf.WF_SPLIT_FORCE)
        # the two longest groups (10 pages: stage 0 and the store), halves
        assert wf.wf_attention_split_choice(h, p) == [(0, 5), (4, 5)]
        wf.wf_set_attention_split(h, wf.WF_SPLIT_AUTO)
        assert wf.wf_attention_split_choice(h, p) == [(3, 3)]
    finally:
        wf.wf_destroy(h)
    h = wf.wf_create(TINY_FP32.config())
    try:
        wf.wf_set_attention_split(h, wf.WF_SPLIT_FORCE)
        for k in range(TINY_FP32.n_chunk + TINY_FP32.S):
            assert wf.wf_attention_split_choice(h, wf.wf_round_plan(h, k)) == []
    finally:
        wf.wf_destroy(h)


def test_split_choice_errors():
    h = wf.wf_create(WAN13B_4STEP.config())
    other = wf.wf_create(TINY_FP32.config())
    try:
        p = wf.wf_round_plan(h, 16)
        assert wf.status_of(wf.wf_attention_split_choice, None, p) == wf.WF_EINVAL
        assert wf.status_of(wf.wf_attention_split_choice, other, p) == wf.WF_EORDER
        bad = wf.wf_round_plan(h, 16)
        bad.groups[1].n_pages += 1
        assert wf.status_of(wf.wf_attention_split_choice, h, bad) == wf.WF_EINVAL
        assert "modified" in wf.wf_last_error()
    finally:
        wf.wf_destroy(h)
        wf.wf_destroy(other)
