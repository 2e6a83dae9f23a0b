"""Pins of the FP8 (E4M3) reading in ``oracle/wf_fp8.py`` (CPU only).

Pinned against something other than the oracle itself:
* every one of the 256 codes against torch's ``float8_e4m3fn`` dtype (a
  library implementation of the OCP E4M3 format);
* round-to-nearest-even of values between codes against torch's conversion;
* closed-form exponents of the power-of-two scale rule;
* properties any correct block quantiser has: exact on representable
  values, error within half a unit in the last place, invariance of the
  codes under scaling the block by a power of two.
"""

import math

import numpy as np
import pytest
import torch

from oracle import wf_fp8 as F

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def torch_decode(codes):
    t = torch.tensor(np.asarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def torch_encode(x):
    t = torch.tensor(np.asarray(x, dtype=np.float64)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def test_every_code_matches_torch_float8_e4m3fn():
    codes = np.arange(256)
    ours = np.array([F.e4m3_decode(c) for c in codes])
    ref = torch_decode(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert np.array_equal(ours[~nan], ref[~nan])


def test_format_landmarks():
    assert F.e4m3_decode(0x7E) == 448.0                 # largest finite
    assert F.e4m3_decode(0x08) == 2.0 ** -6             # smallest normal
    assert F.e4m3_decode(0x01) == 2.0 ** -9             # smallest subnormal
    assert F.e4m3_decode(0x38) == 1.0                   # exponent bias 7
    pos = np.array([F.e4m3_decode(c) for c in range(127)])
    assert np.all(np.diff(pos) > 0)                     # codes order like values


def test_encode_matches_torch_rounding_including_ties():
    pos = np.array([F.e4m3_decode(c) for c in range(127)])
    mids = (pos[:-1] + pos[1:]) / 2                      # exact ties
    quarter = pos[:-1] + (pos[1:] - pos[:-1]) / 4
    three_q = pos[:-1] + 3 * (pos[1:] - pos[:-1]) / 4
    rng = np.random.default_rng(5)
    rand = rng.uniform(-448, 448, 4000) * 2.0 ** rng.integers(-12, 1, 4000)
    x = np.concatenate([pos, -pos, mids, -mids, quarter, three_q, rand])
    tiny = np.array([-1e-6, -0.0, 0.0, 1e-6, -2.0 ** -10, -0.00098, 2.0 ** -10])
    x = np.concatenate([x, tiny])
    ours = F.e4m3_encode(x)
    ref = torch_encode(x)
    assert np.array_equal(ours, ref)                     # codes, signed zeros included


def test_ties_go_to_even_code():
    # between 1.0 (code 0x38) and 1.125 (0x39): tie -> 0x38 (even)
    assert F.e4m3_encode(1.0625) == 0x38
    # between 1.125 (0x39) and 1.25 (0x3A): tie -> 0x3A
    assert F.e4m3_encode(1.1875) == 0x3A


def test_out_of_range_is_refused():
    with pytest.raises(ValueError):
        F.e4m3_encode(449.0)
    with pytest.raises(ValueError):
        F.e4m3_encode(np.nan)


@pytest.mark.parametrize("amax,e", [(448.0, 0), (448.0000001, 1), (224.0, -1), (224.1, 0),
                                    (1.0, -8), (0.875, -9), (3.5, -7), (3.51, -6),
                                    (1e6, 12), (0.0, 0)])
def test_scale_exponent_closed_form(amax, e):
    assert F.pow2_exponent(amax) == e
    if amax > 0:
        assert amax <= 448.0 * 2.0 ** e < 2 * amax


def test_block_quantiser_properties():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((64, 128))
    codes, e = F.quantize_block(x)
    back = np.ldexp(F.e4m3_values(codes), e)
    amax = np.max(np.abs(x))
    assert amax <= 448 * 2.0 ** e < 2 * amax
    # within half an ulp: relative 2^-4 for normals, absolute 2^-10 * 2^e below
    err = np.abs(back - x)
    bound = np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * 2.0 ** e)
    assert np.all(err <= bound * (1 + 1e-12))
    # scaling the block by a power of two shifts only the exponent
    codes2, e2 = F.quantize_block(x * 2.0 ** 5)
    assert e2 == e + 5 and np.array_equal(codes2, codes)
    # representable values come back exactly
    exact = np.ldexp(F.e4m3_values(codes), e)
    c3, e3 = F.quantize_block(exact)
    assert np.array_equal(np.ldexp(F.e4m3_values(c3), e3), exact)


def test_tiles_pad_and_scale_per_tile():
    rng = np.random.default_rng(3)
    n = 150                                              # 3 tiles, last one ragged
    x = rng.standard_normal((n, 16))
    x[64:128] *= 1000.0                                  # tile 1 much larger
    codes, exps = F.quantize_tiles(x)
    assert codes.shape == (192, 16) and exps.shape == (3,)
    assert np.all(codes[n:] == 0)                        # zero padding
    for t in range(3):
        blk = x[64 * t:min(n, 64 * (t + 1))]
        assert exps[t] == F.pow2_exponent(np.max(np.abs(blk)))
    back = F.dequantize_tiles(codes, exps, n)
    assert back.shape == x.shape
    assert np.all(np.abs(back - x) <= np.abs(x) * 2.0 ** -4 + 2.0 ** (exps.repeat(64)[:n, None] - 10))


def test_rows_quantise_each_row_separately():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((5, 128)) * np.array([1e-3, 1, 10, 100, 1e4])[:, None]
    q = F.fp8_rows(x)
    for r in range(5):
        assert np.allclose(q[r], F.fp8_tiles(x[r:r + 1], 1)[0])
        assert np.max(np.abs(q[r] - x[r])) <= np.max(np.abs(x[r])) * 2.0 ** -4


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(8)
    x = rng.standard_normal(10000) * 2.0 ** rng.integers(-20, 20, 10000)
    ref = torch.tensor(x, dtype=torch.float64).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(F.bf16_round(x), ref)


def test_fp8_round_reduces_to_dense_attention_on_dequantised_inputs():
    """group_output(fp8=True) is the plain attention of the dequantised
    pages and per-row quantised bf16 queries (a tiny config, one head)."""
    from oracle import wf_plan as P
    from oracle import wf_round as R
    from oracle.wf_attention import attend
    from oracle.wf_rope import rope3d

    cfg = P.Config(S=2, W=2, W_store=4, anchor=1, n_chunk=6, F=3, Hh=4, Ww=6,
                   n_heads=2, head_dim=64, n_layers=1, mask=0)
    rng = np.random.default_rng(21)
    cache = {}

    def raw(rnd, layer, cell, name):
        key = (rnd, layer, cell, name)
        if key not in cache:
            cache[key] = rng.standard_normal((72, 2, 64))
        return cache[key]

    k, stage = 5, 1
    got = R.group_output(cfg, k, stage, 0, raw, heads=[1], fp8=True)
    # rebuild by hand: each page quantised per 64-token tile, per head
    ks, vs = [], []
    for kind, chunk, _slot in P.key_entries(cfg, k, stage):
        rnd, cell, frame0 = R.entry_source(cfg, k, kind, chunk)
        kr = rope3d(raw(rnd, 0, cell, "k"), frame0, 3, 4, 6, cfg.rope_theta)[:, 1, :]
        ks.append(F.fp8_tiles(kr))
        vs.append(F.fp8_tiles(raw(rnd, 0, cell, "v")[:, 1, :]))
    q = rope3d(raw(k, 0, stage, "q"), 3 * (k - stage), 3, 4, 6, cfg.rope_theta)[:, 1, :]
    q = F.fp8_query(F.bf16_round(q))
    ref = attend(q, np.concatenate(ks), np.concatenate(vs), 1 / math.sqrt(64))
    assert np.allclose(got[:, 0, :], ref, rtol=0, atol=1e-12)
    # and the FP8 result stays close to the exact one (quantisation only)
    exact = R.group_output(cfg, k, stage, 0, raw, heads=[1])
    assert np.max(np.abs(got - exact)) < 0.1


def _smallest_exponent_brute(amax):
    """Smallest integer e with amax <= 448 * 2^e, by scanning (0 for 0)."""
    if amax == 0:
        return 0
    e = -200
    while amax > 448.0 * 2.0 ** e:
        e += 1
    return e


def test_query_reading_is_torch_per_row_e4m3():
    """fp8_query quantises every bf16 row on its own: divided by 2^e (e the
    smallest integer with max |row| <= 448 * 2^e, found by scanning), cast
    to torch's float8_e4m3fn (round to nearest even), cast back and
    multiplied by 2^e.  Rows span magnitudes from 1e-6 to 1e5, so some
    elements land in the subnormal range of their row's scale."""
    rng = np.random.default_rng(31)
    mags = np.exp2(rng.integers(-20, 17, 40)).astype(np.float64)
    q = F.bf16_round(rng.standard_normal((40, 128)) * mags[:, None])
    q[3, :] = 0.0                                     # an all-zero row
    q[4, 5:] = q[4, 5:] * 2.0 ** -14                  # one large, many tiny
    got = F.fp8_query(q)
    for r in range(q.shape[0]):
        e = _smallest_exponent_brute(float(np.max(np.abs(q[r]))))
        x = torch.tensor(np.ldexp(q[r], -e), dtype=torch.float32)
        ref = x.to(torch.float8_e4m3fn).to(torch.float64).numpy()
        np.testing.assert_array_equal(got[r], np.ldexp(ref, e), err_msg=f"row {r}")
    # the reading does not depend on the softmax scale: a row and the same
    # row times a power of two quantise to the same codes
    np.testing.assert_array_equal(F.fp8_query(q * 8.0), got * 8.0)


def test_fp8_keys_only_round_is_dense_attention_with_exact_values():
    """The 8-bit QK^T tier: keys quantised per 64-token tile, values exact,
    queries by the FP8 query reading (a tiny config, one head)."""
    from oracle import wf_plan as P
    from oracle import wf_round as R
    from oracle.wf_attention import attend
    from oracle.wf_rope import rope3d

    cfg = P.Config(S=2, W=2, W_store=4, anchor=1, n_chunk=6, F=3, Hh=4, Ww=6,
                   n_heads=2, head_dim=64, n_layers=1, mask=0)
    rng = np.random.default_rng(22)
    cache = {}

    def raw(rnd, layer, cell, name):
        key = (rnd, layer, cell, name)
        if key not in cache:
            cache[key] = rng.standard_normal((72, 2, 64))
        return cache[key]

    k, stage = 5, 0
    got = R.group_output(cfg, k, stage, 0, raw, heads=[0], fp8="k")
    ks, vs = [], []
    for kind, chunk, _slot in P.key_entries(cfg, k, stage):
        rnd, cell, frame0 = R.entry_source(cfg, k, kind, chunk)
        kr = rope3d(raw(rnd, 0, cell, "k"), frame0, 3, 4, 6, cfg.rope_theta)[:, 0, :]
        ks.append(F.fp8_tiles(kr))
        vs.append(raw(rnd, 0, cell, "v")[:, 0, :])
    q = rope3d(raw(k, 0, stage, "q"), 3 * (k - stage), 3, 4, 6, cfg.rope_theta)[:, 0, :]
    q = F.fp8_query(F.bf16_round(q))
    ref = attend(q, np.concatenate(ks), np.concatenate(vs), 1 / math.sqrt(64))
    assert np.allclose(got[:, 0, :], ref, rtol=0, atol=1e-12)
    # values untouched: the keys-only page differs from the full FP8 page
    _, vv_k = R.group_keys(cfg, k, stage, 0, raw, [0], fp8="k")
    _, vv = R.group_keys(cfg, k, stage, 0, raw, [0])
    assert np.array_equal(vv_k, vv)
    _, vv_kv = R.group_keys(cfg, k, stage, 0, raw, [0], fp8=True)
    assert not np.array_equal(vv_kv, vv)


@pytest.mark.parametrize("fp8", [False, "k", True])
def test_page_memo_changes_nothing(fp8):
    """group_output with a shared page dict over every stage of a round gives
    the same bits as building each stage's pages afresh."""
    from oracle import wf_plan as P
    from oracle import wf_round as R

    cfg = P.Config(S=2, W=2, W_store=4, anchor=1, n_chunk=6, F=3, Hh=4, Ww=6,
                   n_heads=2, head_dim=64, n_layers=1, mask=0)
    rng = np.random.default_rng(23)
    cache = {}

    def raw(rnd, layer, cell, name):
        key = (rnd, layer, cell, name)
        if key not in cache:
            cache[key] = rng.standard_normal((72, 2, 64))
        return cache[key]

    k, pages = 5, {}
    for stage in range(cfg.S + 1):
        a = R.group_output(cfg, k, stage, 0, raw, fp8=fp8, pages=pages)
        b = R.group_output(cfg, k, stage, 0, raw, fp8=fp8)
        assert np.array_equal(a, b)
    assert len(pages) > 0
