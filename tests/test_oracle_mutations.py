"""The oracle's pins catch plausible mistakes (CPU only).

Each case plants one mistake in a temporary copy of ``oracle/`` -- a wrong
sign, index, axis, window bound or rounding rule, a dropped term -- and runs
the pin tests that should catch it (``test_oracle_*.py``, which check the
oracle against torch, closed forms, printed values and brute force, never
against itself) against that copy.  Every case must make them fail: a
mistake the pins let through would leave the GPU path checked against a
wrong reference.  The repository's own ``oracle/`` is never modified.
"""

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TESTS = os.path.join(ROOT, "tests")
PINS = {
    "math": "test_oracle_math.py",
    "plan": "test_oracle_plan.py",
    "fp8": "test_oracle_fp8.py",
    "dit": "test_oracle_dit.py",
}

# (id, oracle file, exact text, replacement, pin files expected to fail)
MUTATIONS = [
    # 3D RoPE (R9, R10)
    ("rope_sin_sign", "wf_rope.py", "out[..., 0::2] = x0 * c - x1 * s", "out[..., 0::2] = x0 * c + x1 * s",
     ["math"]),
    ("rope_freq_2m", "wf_rope.py", "freq = theta ** (-np.arange(na, dtype=np.float64) / na)",
     "freq = theta ** (-2.0 * np.arange(na, dtype=np.float64) / na)", ["math"]),
    ("rope_row_col_swapped", "wf_rope.py", "y = (n // Ww) % Hh", "y = (n // Hh) % Ww", ["math"]),
    ("rope_axis_split", "wf_rope.py", "nt = head_dim // 2 - 2 * nh", "nt = head_dim // 2 - nh", ["math"]),
    ("rope_cos_sign", "wf_rope.py", "out[..., 1::2] = x0 * s + x1 * c", "out[..., 1::2] = x0 * s - x1 * c",
     ["math"]),
    ("rope_frame_axis_drops_chunk", "wf_rope.py", "return frame0 + f, y, x", "return f, y, x", ["math"]),
    # attention (Eq. 4-5; scale 1/sqrt(d))
    ("attend_no_scale", "wf_attention.py", "s = scale * (q[r0:r0 + block] @ k.T)",
     "s = q[r0:r0 + block] @ k.T", ["math"]),
    ("attend_norm_axis", "wf_attention.py", "p /= p.sum(axis=1, keepdims=True)",
     "p /= p.sum(axis=0, keepdims=True)", ["math"]),
    ("round_scale_1_over_d", "wf_round.py", "return 1.0 / math.sqrt(cfg.head_dim)",
     "return 1.0 / cfg.head_dim", ["math"]),
    # where a key entry's K/V comes from (App. B.3)
    ("history_from_wrong_round", "wf_round.py", "return chunk + S, S, cfg.F * chunk",
     "return chunk + S - 1, S, cfg.F * chunk", ["math"]),
    ("anchor_not_rerotated", "wf_round.py", "return S, S, P.anchor_frame0(cfg, k)", "return S, S, 0",
     ["math"]),
    ("values_rotated_too", "wf_round.py", "kr = rope3d(kr, frame0, cfg.F, cfg.Hh, cfg.Ww, cfg.rope_theta)",
     "kr = rope3d(kr, frame0, cfg.F, cfg.Hh, cfg.Ww, cfg.rope_theta); "
     "vr = rope3d(vr, frame0, cfg.F, cfg.Hh, cfg.Ww, cfg.rope_theta)", ["math"]),
    ("query_position_of_round", "wf_round.py", "rope3d(q, cfg.F * (k - stage), cfg.F",
     "rope3d(q, cfg.F * k, cfg.F", ["math"]),
    # the plan (Eq. 3-5, Eq. 10, App. B.2-B.3)
    ("mask_excludes_self", "wf_plan.py", "(j >= s if cfg.mask == MASK_WAVE else True)",
     "(j > s if cfg.mask == MASK_WAVE else True)", ["plan"]),
    ("mask_reads_noisier", "wf_plan.py", "(j >= s if cfg.mask == MASK_WAVE else True)",
     "(j <= s if cfg.mask == MASK_WAVE else True)", ["plan"]),
    ("history_window_short_by_one", "wf_plan.py", "lo = max(cfg.anchor, k - cfg.S - window)",
     "lo = max(cfg.anchor, k - cfg.S - window + 1)", ["plan"]),
    ("store_uses_denoiser_window", "wf_plan.py", "window = cfg.w_store if s == S else cfg.W",
     "window = cfg.W", ["plan"]),
    ("denoisers_reversed", "wf_plan.py", "for j in sorted(readable):",
     "for j in sorted(readable, reverse=True):", ["plan"]),
    ("ring_too_short", "wf_plan.py", "return 2 + (c % cfg.ring)", "return 2 + (c % (cfg.ring - 1))",
     ["plan"]),
    ("no_double_buffer", "wf_plan.py", "return 2 + cfg.ring + (k % 2) * cfg.S + j",
     "return 2 + cfg.ring + j", ["plan"]),
    ("anchor_frame_off_by_one", "wf_plan.py", "return cfg.F * max(0, k - cfg.S - cfg.w_max - 1)",
     "return cfg.F * max(0, k - cfg.S - cfg.w_max)", ["plan", "math"]),
    ("anchor_one_round_early", "wf_plan.py", "return cfg.anchor == 1 and k >= cfg.S + 1",
     "return cfg.anchor == 1 and k >= cfg.S", ["plan"]),
    ("store_ends_one_round_early", "wf_plan.py", "return chunk_active(cfg, k - cfg.S)",
     "return chunk_active(cfg, k - cfg.S) and k - cfg.S + 1 < cfg.n_chunk", ["plan"]),
    ("store_counted_as_denoiser", "wf_plan.py", "return [s for s in range(cfg.S) if chunk_active(cfg, k - s)]",
     "return [s for s in range(cfg.S + 1) if chunk_active(cfg, k - s)]", ["plan"]),
    ("history_reads_live_store", "wf_plan.py", "hi = k - cfg.S - 1", "hi = k - cfg.S", ["plan"]),
    ("slot_count_short", "wf_plan.py", "return 4 + self.w_max + 2 * self.S", "return 3 + self.w_max + 2 * self.S",
     ["plan"]),
    ("store_budget_reading", "wf_plan.py", "return self.W + self.S if self.W_store < 0 else self.W_store",
     "return self.W + self.S - 1 if self.W_store < 0 else self.W_store", ["plan"]),
    ("evict_one_late", "wf_plan.py", "c = k - cfg.S - cfg.w_max\n", "c = k - cfg.S - cfg.w_max - 1\n",
     ["plan"]),
    ("unbounded_has_no_chunks", "wf_plan.py", "return i >= 0 and (cfg.unbounded or i < cfg.n_chunk)",
     "return i >= 0 and i < cfg.n_chunk", ["plan"]),
    ("anchor_captured_late", "wf_plan.py", "return cfg.anchor == 1 and k == cfg.S\n",
     "return cfg.anchor == 1 and k == cfg.S + 1\n", ["plan"]),
    ("flops_one_product", "wf_plan.py", "flops = float(cfg.n_layers) * 4.0 * n_c",
     "flops = float(cfg.n_layers) * 2.0 * n_c", ["plan"]),
    ("denoise_page_position", "wf_round.py", "return k, k - chunk, cfg.F * chunk",
     "return k, k - chunk, cfg.F * (chunk + 1)", ["math"]),
    # E4M3 pages (R15-R17)
    ("e4m3_ties_up", "wf_fp8.py", "pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))",
     "pick_hi = (d_hi <= d_lo)", ["fp8"]),
    ("e4m3_subnormal_exponent", "wf_fp8.py", "return sign * math.ldexp(man / 8.0, -6)",
     "return sign * math.ldexp(man / 8.0, -7)", ["fp8"]),
    ("e4m3_bias_8", "wf_fp8.py", "return sign * math.ldexp(1.0 + man / 8.0, exp - 7)",
     "return sign * math.ldexp(1.0 + man / 8.0, exp - 8)", ["fp8"]),
    ("fp8_scale_sign", "wf_fp8.py", "return e4m3_encode(np.ldexp(x, -e)), e",
     "return e4m3_encode(np.clip(np.ldexp(x, e), -448.0, 448.0)), e", ["fp8"]),
    ("e4m3_fnuz_max", "wf_fp8.py", "E4M3_MAX = 448.0", "E4M3_MAX = 240.0", ["fp8"]),
    ("fp8_tile_size", "wf_fp8.py", "TILE = 64", "TILE = 32", ["fp8"]),
    ("bf16_seven_bits", "wf_fp8.py", "scaled = np.ldexp(m, 8)", "scaled = np.ldexp(m, 7)", ["fp8"]),
    ("fp8_query_skips_bf16", "wf_round.py", "qh = F8.fp8_query(F8.bf16_round(qh))",
     "qh = F8.fp8_query(qh)", ["fp8"]),
    ("fp8k_values_quantised", "wf_round.py", "if fp8 != \"k\":", "if True:", ["fp8"]),
    ("fp8_rows_scale_sign", "wf_fp8.py", "out[r] = np.ldexp(e4m3_values(c), e)",
     "out[r] = np.ldexp(e4m3_values(c), -e)", ["fp8"]),
    # the DiT block around the round (R19-R21)
    ("gelu_constant", "wf_dit.py", "(x + 0.044715 * x ** 3)", "(x + 0.04715 * x ** 3)", ["dit"]),
    ("layer_norm_eps_outside", "wf_dit.py", "return d / np.sqrt(var + eps)",
     "return d / (np.sqrt(var) + eps)", ["dit"]),
    ("modulation_without_one", "wf_dit.py", "return a * (1.0 + scale) + shift", "return a * scale + shift",
     ["dit"]),
    ("ffn_gate_of_attention", "wf_dit.py", "return x1 + mod[5] * (f @ w.w_2.T + w.b_2)",
     "return x1 + mod[2] * (f @ w.w_2.T + w.b_2)", ["dit"]),
    ("attention_residual_dropped", "wf_dit.py", "x1 = x + mod[2] * (o @ w.w_o.T + w.b_o)",
     "x1 = mod[2] * (o @ w.w_o.T + w.b_o)", ["dit"]),
    ("q_from_k_columns", "wf_dit.py", "q = rms_norm(y[:, :c], w.g_q, eps)",
     "q = rms_norm(y[:, c:2 * c], w.g_q, eps)", ["dit"]),
    ("rms_norm_axis", "wf_dit.py", "ms = (x * x).mean(axis=-1, keepdims=True)",
     "ms = (x * x).mean(axis=0, keepdims=True)", ["dit"]),
    ("shift_scale_swapped", "wf_dit.py", "a = modulate(layer_norm(x, eps), mod[0], mod[1])",
     "a = modulate(layer_norm(x, eps), mod[1], mod[0])", ["dit"]),
    ("k_norm_gain_of_q", "wf_dit.py", "k = rms_norm(y[:, c:2 * c], w.g_k, eps)",
     "k = rms_norm(y[:, c:2 * c], w.g_q, eps)", ["dit"]),
]


def _plant(tmp, mutation):
    _, fname, old, new, pins = mutation
    shutil.copytree(os.path.join(ROOT, "oracle"), os.path.join(tmp, "oracle"),
                    ignore=shutil.ignore_patterns("__pycache__"))
    tdir = os.path.join(tmp, "tests")
    os.makedirs(tdir)
    shutil.copy(os.path.join(TESTS, "conftest.py"), tdir)
    shutil.copytree(os.path.join(TESTS, "golden"), os.path.join(tdir, "golden"))
    for p in pins:
        shutil.copy(os.path.join(TESTS, PINS[p]), tdir)
    path = os.path.join(tmp, "oracle", fname)
    text = open(path).read()
    assert text.count(old) == 1, f"{mutation[0]}: the text to mutate must occur exactly once in {fname}"
    open(path, "w").write(text.replace(old, new))
    return [os.path.join(tdir, PINS[p]) for p in pins]


def _run(mutation):
    tmp = tempfile.mkdtemp(prefix="oracle_mut_")
    try:
        files = _plant(tmp, mutation)
        env = dict(os.environ, PYTHONDONTWRITEBYTECODE="1")
        r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                            "-p", "no:xdist", "-W", "ignore", *files],
                           cwd=tmp, env=env, capture_output=True, text=True, timeout=600)
        return mutation[0], r.returncode, r.stdout[-600:]
    finally:
        shutil.rmtree(tmp, ignore_errors=True)


def test_mutations_are_distinct_and_present():
    ids = [m[0] for m in MUTATIONS]
    assert len(ids) == len(set(ids))
    for m in MUTATIONS:
        text = open(os.path.join(ROOT, "oracle", m[1])).read()
        assert text.count(m[2]) == 1, m[0]


@pytest.mark.timeout(900)
def test_every_planted_mistake_fails_a_pin():
    # the unmutated oracle passes the same pin files (the baseline)
    base = _run(("unmutated", "wf_plan.py", "MASK_WAVE, MASK_ROLLING = 0, 1",
                 "MASK_WAVE, MASK_ROLLING = 0, 1", list(PINS)))
    assert base[1] == 0, base[2]
    workers = max(1, min(6, (os.cpu_count() or 2) - 1))
    with ThreadPoolExecutor(workers) as ex:
        results = list(ex.map(_run, MUTATIONS))
    survived = [(name, out) for name, rc, out in results if rc != 1]
    assert not survived, "mistakes the pins did not catch (pytest exit code != 1):\n" + "\n".join(
        f"{n}: {o}" for n, o in survived)
