"""Shared helpers of the GPU parity tests: run rounds through the C ABI and
compare what they produced with the oracle (fp64, CPU).

Inputs come from ``chunk_causal_dit_round_amd.synth`` (seeded, one seed per
(round, layer, stage, tensor) slice).  The oracle never sees anything the HIP
path produced: its ``raw`` callback regenerates input slices from their seeds.
"""

import math

import numpy as np
import torch

from chunk_causal_dit_round_amd import synth, wf
from chunk_causal_dit_round_amd.session import Session
from oracle import wf_fp8 as F8
from oracle import wf_plan as P
from oracle import wf_round as WR
from oracle.wf_rope import rope3d

# bf16 RNE keeps 8 significant bits: one unit in the last place is at most
# 2^-7 of the value.  A page value may differ from RNE(exact) by one ulp when
# the fp32 rotation lands next to a rounding tie.
BF16_RTOL = 2.0 ** -7
ATT_TOL = {wf.WF_BF16: 2e-2, wf.WF_F32: 1e-4}


# The kernels rotate q and k in fp32 (fp32 tables); the oracle rotates in fp64.
# Their difference is below ROT_ERR times the largest element of the row (q)
# or of the page head (k); the page checks assert the same bound.
ROT_ERR = 2.0 ** -21


def _rotation_error(x):
    """Per-element bound on |fp32 rotation - exact| for rotated rows x [.., d]
    (pairs (2p, 2p+1) rotate together).  out = a cos - b sin with a, b exact
    in fp32 and cos, sin rounded to fp32: each product and the difference
    round once, so |err| <= 2^-23 (|a| + |b|) + 2^-24 |out| + O(2^-46), and
    |a| + |b| <= sqrt(2) times the pair's norm, which the rotation keeps.
    Doubled for margin."""
    pair = np.hypot(x[..., 0::2], x[..., 1::2])
    err = np.repeat(pair * (2.0 ** -22 * math.sqrt(2.0)), 2, axis=-1)
    err += 2.0 ** -23 * np.abs(x)
    return err


def _midpoint_distance(y, mant_bits, min_exp):
    """Distance from |y| to the nearest rounding midpoint of a floating-point
    grid with ``mant_bits`` stored mantissa bits and smallest normal
    exponent ``min_exp`` (0 exactly on a tie), and the grid spacing there
    (the larger one next to |y|).  In the binade [2^E, 2^(E+1)) the grid
    steps by u = 2^(E - mant_bits) and the midpoints sit at odd multiples of
    u / 2; just above 2^E the nearest midpoint can be the one below 2^E, half
    the lower binade's step away from 2^E.  Below 2^min_exp the step is that
    of the lowest binade."""
    a = np.abs(y)
    _, ex = np.frexp(np.maximum(a, 2.0 ** min_exp))     # a in [2^(ex-1), 2^ex)
    u = np.ldexp(1.0, ex - 1 - mant_bits)
    f = a / u
    f -= np.floor(f)
    f -= 0.5
    dist = np.abs(f)
    dist *= u
    below = a - np.ldexp(1.0, ex - 1)
    below += u / 4                                       # midpoint under 2^E
    np.minimum(dist, np.where(ex - 1 > min_exp, below, np.inf), out=dist)
    return dist, u


def key_flips(ke):
    """Possible |k8 - k8_oracle| of one page head (``ke`` [N, d], the exact
    rotated keys): one E4M3 step where the kernel's fp32 rotation may round
    to the other side of a midpoint, 0 elsewhere.

    A code is decided from the kernel's fp32 rotation; it can differ from the
    oracle's (fp64 rotation) only where the exact value, scaled by its
    64-token tile's power of two, lies within the rotation error of a
    rounding midpoint (exactly on one only for pairs at angle 0, which both
    sides rotate exactly)."""
    n, d = ke.shape
    n_t = -(-n // 64)
    kp = np.zeros((n_t * 64, d))
    kp[:n] = ke
    amax = np.abs(kp.reshape(n_t, 64 * d)).max(axis=1)
    # smallest e with amax <= 448 * 2^e (0 for an all-zero tile)
    e = np.ceil(np.log2(np.maximum(amax, 1e-300) / 448.0))
    e = np.where(amax > 448.0 * np.exp2(e), e + 1, e)
    e = np.where(amax <= 448.0 * np.exp2(e - 1), e - 1, e)
    e = np.where(amax == 0, 0.0, e)
    sc = np.repeat(np.exp2(e), 64)[:, None]
    dist, step = _midpoint_distance(kp / sc, 3, -6)
    near = (dist > 0) & (dist * sc < _rotation_error(kp))
    return np.where(near, step * sc, 0.0)[:n]


def query_shift(q, scale):
    """How the kernel's quantised query row can differ from the oracle's
    (``q`` [Nq, d]: the exact rotated query rows of one head).

    The oracle quantises x = bf16(q) per row on the E4M3 grid of x itself
    (``wf_fp8.fp8_query``).  The kernel quantises the fp32 product y = x c,
    c = fp32(scale log2 e), per row on the E4M3 grid of y (the row exponent
    eq = the smallest with max |y| <= 448 2^eq), so that Q K^T comes out in
    the softmax's base-2 units; its query is Q(y) / c.  The two grids differ
    by the factor c, which is no power of two, so the two rounding errors are
    unrelated.  Per element, q8_gpu - q8_oracle = a + b + r with
      * a = x - fp8_query(x), known exactly;
      * b = one bf16 step where the kernel's fp32 rotation may round q to the
        other bf16 neighbour (q within the rotation error of a bf16
        midpoint), else 0;
      * r = Q(y) / c - x, the kernel's own rounding: |r| <= h with h half the
        E4M3 step of y's binade (2^(E - 4) for |y| in [2^E, 2^(E+1)); the
        subnormal half step 2^(eq - 10) below 2^(eq - 6)), divided by c, plus
        the fp32 roundings of y and of c (2^-23 |x|).
    eq is taken for max |y| (1 + 2^-7), which covers a flipped row maximum.
    Returns (a, b, h), each [Nq, d]."""
    x = F8.bf16_round(q)
    a = x - F8.fp8_query(x)
    qdist, qstep = _midpoint_distance(q, 7, -126)
    b = np.where((qdist > 0) & (qdist < _rotation_error(q)), qstep, 0.0)
    c = float(np.float32(scale * math.log2(math.e)))
    y = np.abs(x) * c
    eq = np.array([F8.pow2_exponent(r) for r in y.max(axis=1) * (1.0 + 2.0 ** -7)], dtype=np.float64)
    _, ex = np.frexp(np.maximum(y, 2.0 ** -300))          # |y| in [2^(ex-1), 2^ex)
    half = np.maximum(np.ldexp(1.0, ex - 5), np.exp2(eq - 10)[:, None])
    h = half / c + 2.0 ** -23 * np.abs(x)
    return a, b, h


def _query_term(pn, k8, v8, o, scale, query, block=8):
    """Output shift from the query differences of ``query_shift``: a score
    s_j = scale q . k_j moves by scale sum_d dq_d k_jd for every key j of
    the row, so to first order O moves by scale sum_d dq_d Cov_P(k_d, V),
    Cov_P the covariance of key dim d and the values under the weights P.
    The known part a enters with its sign, the possible bf16 flips b at
    worst, and the kernel's rounding r as independent uniform errors (six
    standard deviations, variance h^2 / 3 each); the sum is taken 1.25
    times for the second order.  The covariance is formed per row from
    keys centred on their weighted mean, in fp32 (it only sizes a bound)."""
    a, b, h = (torch.from_numpy(np.ascontiguousarray(x)) for x in query)
    nq, d = a.shape
    out = torch.zeros((nq, v8.shape[1]), dtype=torch.float64)
    kt = torch.from_numpy(np.ascontiguousarray(k8.T, dtype=np.float32))     # [d, Nk]
    v32 = torch.from_numpy(np.ascontiguousarray(v8, dtype=np.float32))
    pt = torch.from_numpy(np.ascontiguousarray(pn, dtype=np.float32))
    for i0 in range(0, nq, block):
        p = pt[i0:i0 + block]                                    # [B, Nk]
        m = p @ kt.T                                             # E_P[k]: [B, d]
        pk = (kt[None] - m[:, :, None]) * p[:, None, :]          # [B, d, Nk]
        cov = torch.matmul(pk, v32).double()                     # [B, d, e]
        sl = slice(i0, i0 + block)
        mean = torch.einsum("bd,bde->be", a[sl], cov).abs()
        flip = torch.einsum("bd,bde->be", b[sl], cov.abs())
        var = torch.einsum("bd,bde->be", h[sl] ** 2 / 3.0, cov * cov)
        out[sl] = 1.25 * scale * (mean + flip + 6.0 * var.sqrt())
    return out.numpy()


def fp8_attention_tolerance(q8, k8, v8, scale, weight_eps=2.0 ** -4, out_rel=0.0, dk=None,
                            query=None, err=None):
    """Per-element bound on |O_gpu - O_oracle| over FP8 pages ([Nq, d] each).

    The oracle attends exactly over the dequantised Q, K and V.  The kernel
    in addition rounds every softmax weight P_k (to E4M3 on FP8 pages:
    relative error |eps_k| <= weight_eps = 2^-4; to bf16 on 8-bit-key pages:
    2^-8) and uses the rounded weights in both the PV product and the row
    sum, so O_gpu - O = sum_k eps_k P_k (V_k - O) / sum_k P_k (1 + eps_k).
    With the eps_k treated as independent and uniform (standard deviation
    weight_eps / sqrt 3), six standard deviations of that sum (its
    denominator bounded below by (1 - weight_eps) sum_k P_k), plus out_rel
    |O| for the rounding of the output (bf16: 2^-8), plus 1e-3 for fp32
    accumulation.
      * ``dk`` (``key_flips`` of each page, in context order): key codes
        the kernel's fp32 rotation may decide one step away from the
        oracle's.  A key element off by dk_kd moves score k of row i by at
        most f_ik = scale sum_d |q8_id| dk_kd, so weight k moves by at most
        a factor exp(f_ik) and O by at most sum_k w_k |V_k - O| / (1 - sum_k
        w_k) with w_k = P_k (exp(f_ik) - 1) (|V_k - O| <= |V_k| + |O|).
      * ``query`` = ``query_shift(...)``: the kernel quantises the query on
        another grid than the oracle (``_query_term``).  Given ``err`` (the
        observed |O_gpu - O_oracle|), the term is formed only for the rows
        where some element exceeds half the other terms: the others pass
        either way, and their err / bound, at most 0.5 without the term,
        never understates; above 0.5 the returned bound is the full one.
    """
    s = scale * (q8 @ k8.T)
    s -= s.max(axis=1, keepdims=True)
    p = np.exp(s)
    ps = p.sum(axis=1, keepdims=True)
    o = (p @ v8) / ps
    # sum_k P_k^2 (V_kd - O_d)^2 = P^2 V^2 - 2 O (P^2 V) + O^2 sum P^2
    p2 = p * p
    var = p2 @ (v8 * v8) - 2.0 * o * (p2 @ v8) + o * o * p2.sum(axis=1, keepdims=True)
    spread = np.sqrt(np.maximum(var, 0.0)) / (ps * (1.0 - weight_eps))
    tol = 6.0 * weight_eps / math.sqrt(3.0) * spread + out_rel * np.abs(o) + 1e-3
    pn = p / ps
    if dk is not None:
        w = pn * np.expm1(scale * (np.abs(q8) @ dk.T))
        ws = w.sum(axis=1, keepdims=True)
        tol = tol + (w @ np.abs(v8) + ws * np.abs(o)) / np.maximum(1.0 - ws, 0.5)
    if query is not None:
        rows = np.arange(q8.shape[0]) if err is None else np.nonzero((err > 0.5 * tol).any(axis=1))[0]
        if len(rows):
            sub = tuple(x[rows] for x in query)
            tol[rows] += _query_term(pn[rows], k8, v8, o[rows], scale, sub)
    return tol


def bf16_attention_tolerance(q, k, v, scale):
    """Per-element bound on |O_gpu - O_oracle| for bf16 rounds ([Nq, d] each;
    q and k the oracle's exact rotated rows, v the exact bf16 values).

    The oracle is exact; the kernel works from rounded operands.  Each bf16
    rounding (round to nearest even) is modelled as a relative error uniform
    in +-2^-8 (standard deviation 2^-8 / sqrt 3; the true one is smaller):
      * every element of a query row is rounded twice (q_rot in HBM, then
        the row times scale * log2(e) inside attention): the errors eta_d are
        shared by all keys of the row, so to first order
        dO = sum_d eta_d scale q_d Cov_P(k_d, V), with Cov_P the covariance
        of key dim d and the values under the softmax weights P;
      * every element of a key page is rounded once, independently per
        (key, dim): dS_j = scale sum_d q_d k_jd xi_jd, and
        dO = sum_j P_j dS_j (V_j - O);
      * every softmax weight is rounded once (as in
        ``fp8_attention_tolerance`` with weight_eps = 2^-8);
      * the output is rounded once: 2^-8 |O|.
    The three first-order terms are independent: six standard deviations of
    their sum, plus the output rounding, plus 1e-3 for fp32 accumulation.
    Unlike the fixed 2e-2 bar this grows with the scores' magnitude, which
    the two roundings of q multiply.
    """
    s = scale * (q @ k.T)
    s -= s.max(axis=1, keepdims=True)
    p = np.exp(s)
    p /= p.sum(axis=1, keepdims=True)
    o = p @ v
    u2 = 2.0 ** -16 / 3.0                       # variance of one rounding (relative)
    var_q = np.empty_like(o)
    for i in range(q.shape[0]):
        pk = k * p[i][:, None]
        cov = pk.T @ v - np.outer(pk.sum(axis=0), o[i])          # [d, d]: Cov_P(k_d, V_e)
        var_q[i] = 2.0 * u2 * scale ** 2 * ((q[i][:, None] * cov) ** 2).sum(axis=0)
    p2 = p * p
    w_k = p2 * (u2 * scale ** 2 * ((q * q) @ (k * k).T))         # P_j^2 var(dS_j)
    var_k = w_k @ (v * v) - 2.0 * o * (w_k @ v) + o * o * w_k.sum(axis=1, keepdims=True)
    var_p = u2 * (p2 @ (v * v) - 2.0 * o * (p2 @ v) + o * o * p2.sum(axis=1, keepdims=True)) \
        / (1.0 - 2.0 ** -8) ** 2
    sd = np.sqrt(np.maximum(var_q, 0.0) + np.maximum(var_k, 0.0) + np.maximum(var_p, 0.0))
    return 6.0 * sd + 2.0 ** -8 * np.abs(o) + 1e-3


def oracle_cfg(w):
    return P.Config(S=w.S, W=w.W, W_store=w.W_store, anchor=w.anchor, n_chunk=w.n_chunk,
                    F=w.F, Hh=w.Hh, Ww=w.Ww, n_heads=w.n_heads, head_dim=w.head_dim,
                    n_layers=w.n_layers, mask=w.mask)


class Rollout:
    """One request of workload ``w`` on the GPU, round by round."""

    def __init__(self, w, device="cuda", gen_device=None, tag=None, perturb=None, split=None):
        self.w = w
        self.tag = tag or w.name
        self.sess = Session(w.config(), device=device)
        if split is not None:
            wf.wf_set_attention_split(self.sess.h, split)
        self.gen_device = gen_device or ("cpu" if w.n_tokens * w.n_heads * w.head_dim < 1 << 20
                                         else device)
        self.q_scale = synth.head_scales(w.n_heads, self.tag) if w.q_head_scale else None
        self.perturb = perturb or {}      # (round, layer, stage, name) -> additive offset
        self._raw_cache = {}

    # ---- inputs ----
    def input_slice(self, rnd, layer, stage, name):
        s = self.sess
        x = synth.slice_input(self.tag, rnd, layer, stage, name, s.N, s.H, s.D,
                              self.gen_device, s.dtype, self.q_scale)
        off = self.perturb.get((rnd, layer, stage, name))
        if off is not None:
            x = (x.float() + off).to(s.dtype)
        return x

    def fill(self, k):
        b = self.sess.bufs
        for layer in range(self.w.n_layers):
            for s in range(self.w.S + 1):
                for name in synth.NAMES:
                    b[name][layer, s].copy_(self.input_slice(k, layer, s, name))

    def raw(self, rnd, layer, stage, name):
        """Oracle input callback: fp64 copy of a regenerated slice."""
        key = (rnd, layer, stage, name)
        if key not in self._raw_cache:
            if len(self._raw_cache) > 64:
                self._raw_cache.clear()
            self._raw_cache[key] = self.input_slice(rnd, layer, stage, name).to(
                torch.float64).cpu().numpy()
        return self._raw_cache[key]

    # ---- rounds ----
    def run(self, k, mode="round", stream=None):
        s = self.sess
        assert s.next_round() == k
        self.fill(k)
        plan = s.plan(k)
        if mode == "round":
            s.run_round(plan, stream=stream)
        elif mode == "layers":
            for layer in range(self.w.n_layers):
                s.publish(plan, layer, stream=stream)
                s.attention(plan, layer, stream=stream)
            s.commit(plan)
        elif mode == "publish_all_first":
            for layer in range(self.w.n_layers):
                s.publish(plan, layer, stream=stream)
            for layer in reversed(range(self.w.n_layers)):
                s.attention(plan, layer, stream=stream)
            s.commit(plan)
        else:
            raise ValueError(mode)
        return plan

    def close(self):
        self.sess.close()


def to64(t):
    return t.detach().to(torch.float64).cpu().numpy()


def _check_fp8_page(s, layer, slot, kr, v, what):
    """One FP8 (or FP8K) page vs the oracle's quantisation of the exact
    rotated key ``kr`` and the value ``v`` ([N, H, D] fp64).  V codes and
    every scale exponent must match bit for bit (V is exact bf16 input); on
    FP8K pages the bf16 values must equal the input and their exponent code
    is 2^0.  K codes are made from the fp32 rotation: each dequantised value
    lies within half a unit in the last place of the exact rotated key, plus
    the fp32 rotation error (a few 2^-24 of the page's largest key)."""
    K8, Vt8, codes = (to64(t) if t.dtype == torch.bfloat16 else t.cpu().numpy()
                      for t in s.fp8_page(layer, slot))
    N = s.N
    bf16_values = s.cfg.dtype == wf.WF_FP8K
    for h in range(s.H):
        if bf16_values:
            np.testing.assert_array_equal(Vt8[h][:, :N].T, v[:, h, :], err_msg=f"{what} h={h}: V")
            assert (codes[h, :, 1] == 127).all(), f"{what} h={h}: V exponent codes"
        else:
            vc, ve = F8.quantize_tiles(v[:, h, :])
            diff = np.argwhere(Vt8[h].T != vc)
            if len(diff):
                n0, d0 = diff[0]
                raise AssertionError(f"{what} h={h}: {len(diff)} V codes differ, first at token "
                                     f"{n0} dim {d0}: gpu 0x{Vt8[h][d0, n0]:02x} oracle "
                                     f"0x{vc[n0, d0]:02x} v={v[n0, h, d0]!r} e={ve[n0 // 64]}")
            assert np.array_equal(codes[h, :, 1].astype(np.int64) - 127, ve), \
                f"{what} h={h}: V exponents"
        _kc, ke = F8.quantize_tiles(kr[:, h, :])
        ge = codes[h, :, 0].astype(np.int64) - 127
        assert np.array_equal(ge, ke), f"{what} h={h}: K exponents"
        e_tok = np.repeat(ge, 64)[:N, None].astype(np.float64)
        deq = F8.e4m3_values(K8[h][:N]) * np.exp2(e_tok)
        want = kr[:, h, :]
        rot_err = 2.0 ** -21 * np.abs(want).max()
        bound = 2.0 ** -4 * (np.abs(want) + rot_err) + np.exp2(e_tok - 10) + rot_err
        bad = np.abs(deq - want) > bound
        assert not bad.any(), f"{what} h={h}: {bad.sum()} K codes off"
        assert not K8[h][N:].any() and not Vt8[h][:, N:].any(), f"{what} h={h}: padding not zero"


def check_publish_fp8(ro, k, layer):
    w, s = ro.w, ro.sess
    oc = oracle_cfg(w)
    torch.cuda.synchronize()
    for st in range(w.S + 1):
        i = k - st
        if not P.chunk_active(oc, i):
            continue
        qr = rope3d(ro.raw(k, layer, st, "q"), w.F * i, w.F, w.Hh, w.Ww)
        _close_rope(to64(s.bufs["q_rot"][layer, st]), qr, False, f"q_rot k={k} l={layer} s={st}")
        kr = rope3d(ro.raw(k, layer, st, "k"), w.F * i, w.F, w.Hh, w.Ww)
        _check_fp8_page(s, layer, P.cell_slot(oc, k, st), kr, ro.raw(k, layer, st, "v"),
                        f"page k={k} l={layer} s={st}")
    if P.anchor_present(oc, k):
        kr = rope3d(ro.raw(w.S, layer, w.S, "k"), P.anchor_frame0(oc, k), w.F, w.Hh, w.Ww)
        _check_fp8_page(s, layer, P.anchor_slot(oc, k), kr, ro.raw(w.S, layer, w.S, "v"),
                        f"anchor k={k} l={layer}")
    if P.anchor_present(oc, k) or k == w.S:
        K, Vt = s.anchor_page(layer)
        if k >= w.S and w.anchor:
            np.testing.assert_array_equal(to64(K).transpose(1, 0, 2), ro.raw(w.S, layer, w.S, "k"))
            np.testing.assert_array_equal(to64(Vt).transpose(2, 0, 1), ro.raw(w.S, layer, w.S, "v"))


def check_publish(ro, k, layer, rows=None):
    """q_rot and every page the round wrote vs oracle RoPE of the inputs."""
    w, s = ro.w, ro.sess
    if w.dtype in (wf.WF_FP8, wf.WF_FP8K):
        return check_publish_fp8(ro, k, layer)
    oc = oracle_cfg(w)
    torch.cuda.synchronize()
    exact = s.dtype == torch.float32
    sel = slice(None) if rows is None else torch.as_tensor(rows)
    for st in range(w.S + 1):
        i = k - st
        if not P.chunk_active(oc, i):
            continue
        qr = rope3d(ro.raw(k, layer, st, "q"), w.F * i, w.F, w.Hh, w.Ww)
        got = to64(s.bufs["q_rot"][layer, st])
        _close_rope(got[sel], qr[sel], exact, f"q_rot k={k} l={layer} s={st}")
        slot = P.cell_slot(oc, k, st)
        K, Vt = s.page(layer, slot)
        kr = rope3d(ro.raw(k, layer, st, "k"), w.F * i, w.F, w.Hh, w.Ww)
        _close_rope(to64(K).transpose(1, 0, 2)[sel], kr[sel], exact, f"K k={k} l={layer} s={st}")
        np.testing.assert_array_equal(to64(Vt).transpose(2, 0, 1), ro.raw(k, layer, st, "v"))
    if P.anchor_present(oc, k):
        K, Vt = s.page(layer, P.anchor_slot(oc, k))
        kr = rope3d(ro.raw(w.S, layer, w.S, "k"), P.anchor_frame0(oc, k), w.F, w.Hh, w.Ww)
        _close_rope(to64(K).transpose(1, 0, 2), kr, exact, f"anchor K k={k} l={layer}")
        np.testing.assert_array_equal(to64(Vt).transpose(2, 0, 1), ro.raw(w.S, layer, w.S, "v"))


def _close_rope(got, want, exact, what):
    err = np.abs(got - want)
    if exact:
        lim = 2e-6 * (1 + np.abs(want))
    else:
        lim = BF16_RTOL * np.abs(want) + 1e-6
    bad = err > lim
    assert not bad.any(), f"{what}: {bad.sum()} elements off, max err {err.max():.3e}"


def check_attention(ro, k, layer, rows=None, heads=None, stages=None, seed=0, derived=False):
    """Attention output vs the oracle; all rows, or ``rows`` random rows per
    group.  FP8 and FP8K rounds use their derived per-element bounds; bf16
    rounds the fixed 2e-2 bar, or with ``derived`` the per-element bound of
    ``bf16_attention_tolerance`` (inputs whose scores reach tens of log2
    units, where the rounding of q alone exceeds the fixed bar)."""
    w, s = ro.w, ro.sess
    oc = oracle_cfg(w)
    torch.cuda.synchronize()
    tol = ATT_TOL.get(w.dtype)
    worst = 0.0
    rng = np.random.default_rng([seed, k, layer])
    flips_of = {}
    pages_of = {}          # (page reading) -> the oracle's pages of this round and layer

    def page_flips(kind, chunk, hs):
        """key_flips of one context page (all selected heads), once per call."""
        if (kind, chunk) not in flips_of:
            rnd, cell, frame0 = WR.entry_source(oc, k, kind, chunk)
            kr = rope3d(np.asarray(ro.raw(rnd, layer, cell, "k"), dtype=np.float64)[:, hs, :],
                        frame0, w.F, w.Hh, w.Ww, oc.rope_theta)
            flips_of[(kind, chunk)] = np.stack([key_flips(kr[:, i, :]) for i in range(len(hs))], 1)
        return flips_of[(kind, chunk)]

    for st in (range(w.S + 1) if stages is None else stages):
        if not P.chunk_active(oc, k - st):
            continue
        r = None
        if rows is not None:
            r = np.sort(rng.choice(s.N, size=min(rows, s.N), replace=False))
            r[-1] = s.N - 1           # always include the ragged tail row
        fp8 = {wf.WF_FP8: True, wf.WF_FP8K: "k"}.get(w.dtype, False)
        pages = pages_of.setdefault(fp8, {})
        want = WR.group_output(oc, k, st, layer, ro.raw, rows=r, heads=heads, fp8=fp8, pages=pages)
        got = to64(s.bufs["out"][layer, st])
        if r is not None:
            got = got[r]
        if heads is not None:
            got = got[:, list(heads), :]
        assert np.isfinite(got).all()
        err = np.abs(got - want)
        if derived and w.dtype == wf.WF_BF16:
            hs = list(range(w.n_heads)) if heads is None else list(heads)
            qr = WR.q_rot(oc, k, st, layer, ro.raw)
            if r is not None:
                qr = qr[r]
            kk, vv = WR.group_keys(oc, k, st, layer, ro.raw, hs, pages=pages)
            tol = np.empty_like(err)
            for hi, h in enumerate(hs):
                tol[:, hi, :] = bf16_attention_tolerance(qr[:, h, :], kk[:, hi, :], vv[:, hi, :],
                                                         WR.scale_of(oc))
            ratio = (err / tol).max()
            worst = max(worst, err.max())
            ro.bound_ratio = max(getattr(ro, "bound_ratio", 0.0), ratio)
            assert ratio <= 1.0, (f"attention k={k} l={layer} s={st}: max abs err "
                                  f"{err.max():.3e}, {ratio:.2f} x the bound")
            continue
        if fp8:
            hs = list(range(w.n_heads)) if heads is None else list(heads)
            qr = WR.q_rot(oc, k, st, layer, ro.raw)
            if r is not None:
                qr = qr[r]
            kk, vv = WR.group_keys(oc, k, st, layer, ro.raw, hs, fp8=fp8, pages=pages)
            dk = np.concatenate([page_flips(kind, chunk, hs)
                                 for kind, chunk, _slot in P.key_entries(oc, k, st)], axis=0)
            # weights rounded to E4M3 (FP8) or bf16 (FP8K); the output is
            # bf16 on both (peaky rows have |O| near 1, where its rounding
            # exceeds the 1e-3 floor)
            eps, out_rel = (2.0 ** -4 if fp8 is True else 2.0 ** -8), 2.0 ** -8
            tol = np.empty_like(err)
            sc = WR.scale_of(oc)
            for hi, h in enumerate(hs):
                q8 = F8.fp8_query(F8.bf16_round(qr[:, h, :]))
                tol[:, hi, :] = fp8_attention_tolerance(q8, kk[:, hi, :], vv[:, hi, :], sc, eps,
                                                        out_rel, dk=dk[:, hi, :],
                                                        query=query_shift(qr[:, h, :], sc),
                                                        err=err[:, hi, :])
            ratio = (err / tol).max()
            worst = max(worst, err.max())
            ro.fp8_bound_ratio = max(getattr(ro, "fp8_bound_ratio", 0.0), ratio)
            assert ratio <= 1.0, (f"attention k={k} l={layer} s={st}: max abs err "
                                  f"{err.max():.3e}, {ratio:.2f} x the bound")
            continue
        worst = max(worst, err.max())
        assert err.max() <= tol, f"attention k={k} l={layer} s={st}: max abs err {err.max():.3e} > {tol}"
    return worst
