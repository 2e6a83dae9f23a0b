"""Throughput of steady wavefront rounds on one MI355X.

A step is one whole round (for every layer: K/V publish, then the batched
wavefront attention; then commit) of the Wan2.1-1.3B-shaped 4-step request:
S = 4, W = 4 (store window 8), 4680 tokens per chunk, 12 heads x 128, 30
layers, bf16.  Rounds 0..12 fill the pipeline and the history window
(untimed); warmup rounds follow; then exactly `--steps` steady rounds are
timed between two device synchronisations.  Inputs (two seeded sets,
alternating by round) are resident in HBM before timing starts.

Output: one JSON line.  `value` = rounds per second (one chunk completes per
round).  `roofline` is the attention kernel's: algorithmic FLOPs per launch
(readable key tokens only) / its mean duration from HIP events recorded on
the launch stream around every attention launch in the timed region.
`cpu_baseline` is the fp64 oracle on a bounded sample, timed on this host.

Other modes (one JSON line each):
  --workload tiny_fp32_s2
                     a request shorter than the steady window (the tiny fp32
                     round: 6 chunks, 8 rounds): a step is the whole request
                     from round 0 (fill, full width, drain); the fp32 path is
                     bound by the vector ALUs (157.3 TFLOP/s fp32).
  --rollout          the whole long request (133 chunks, 137 rounds) with fresh
                     per-round inputs (generated between rounds, untimed): steady,
                     full-width and whole-request rounds/s.
  --copy-calibration a plain device copy of known size, for scaling the HBM
                     FETCH_SIZE / WRITE_SIZE counters to bytes.
  --workload wan1.3b_4step_fp8
                     the same round over FP8 (E4M3) pages; roofline against the
                     dense fp8 MFMA peak.
  --workload wan1.3b_4step_fp8k
                     the same round over 8-bit-key pages (FP8 keys, bf16 values);
                     roofline against the blend of the fp8 and bf16 peaks.
  --dit              the whole DiT forward of a steady round: every layer of the
                     Wan-shaped block (norms, QKV / output / FFN products, qk norm,
                     publish, attention) for all S+1 cells, dummy weights, FFN
                     width --ffn (8960 for the 1.3B shape); whole-round TFLOP/s
                     against the bf16 MFMA peak (with --workload
                     wan1.3b_4step_fp8k or _fp8: attention over those pages, the
                     peak blended by FLOPs).  With --rollout: the whole
                     133-chunk request through the DiT.
"""

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA
# 8-bit-key pages: half the attention FLOPs (Q K^T) on the fp8 matrix cores,
# half (P V) on the bf16 ones; at both peaks a launch takes F/2/5.0 + F/2/2.5,
# so its peak is the harmonic blend, 3.33 PFLOP/s.
PEAK_FP8K_TFLOPS = 1.0 / (0.5 / PEAK_FP8_TFLOPS + 0.5 / PEAK_BF16_TFLOPS)
PEAK_HBM_GBPS = 8000.0
PEAK_FP32_TFLOPS = 157.3    # MI355X fp32 vector (plain FMA on the SIMDs)
CSRC = os.path.join(ROOT, "chunk_causal_dit_round_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")

# Attention instance per page type: peak, dtype label, kernel and its source.
PAGE_KINDS = {
    "bf16": dict(peak=PEAK_BF16_TFLOPS, dtype="bf16", kernel="wf_attention_bf16_kernel<128>",
                 src="wf_attention.hip", what="bf16 MFMA peak"),
    "fp8": dict(peak=PEAK_FP8_TFLOPS, dtype="fp8", kernel="wf_attention_fp8_kernel",
                src="wf_attention_fp8.hip", what="fp8 MFMA peak (FP8 E4M3 pages)"),
    "fp8k": dict(peak=PEAK_FP8K_TFLOPS, dtype="fp8 QK^T + bf16 PV", kernel="wf_attention_fp8k_kernel",
                 src="wf_attention_fp8k.hip",
                 what="blended fp8 / bf16 MFMA peak (8-bit-key pages: FP8 K, bf16 V)"),
}

# The committed counter summary (profiles/) that each workload's attention
# traffic comes from: FETCH_SIZE + WRITE_SIZE per launch, scaled by a device
# copy of known size.
TRAFFIC_FILES = {
    "wan1.3b_4step": "attention_bf16_wan1.3b_4step_kernel_trace_and_traffic.txt",
    "wan1.3b_4step_fp8": "attention_fp8_wan1.3b_4step_kernel_trace_and_traffic.txt",
    "wan1.3b_4step_fp8k": "attention_fp8k_wan1.3b_4step_kernel_trace_and_traffic.txt",
    "wan1.3b_5step": "attention_bf16_wan1.3b_5step_kernel_trace_and_traffic.txt",
    "wan1.3b_5step_rolling": "attention_bf16_wan1.3b_5step_rolling_kernel_trace_and_traffic.txt",
    "wan14b_4step": "attention_bf16_wan14b_4step_kernel_trace_and_traffic.txt",
}


def measured_traffic(kind, workload):
    """HBM bytes per attention launch from the workload's committed counter
    summary, or None if there is none or the kernel source changed since
    the counters were taken."""
    name = TRAFFIC_FILES.get(workload)
    if name is None:
        return None
    try:
        fields = dict(line.split(":", 1) for line in open(os.path.join(PROFILES, name)) if ":" in line)
        src = hashlib.sha256(open(os.path.join(CSRC, kind["src"]), "rb").read()).hexdigest()
        if fields.get("kernel_source_sha256", "").strip() != src:
            return None
        return float(fields["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="wan1.3b_4step")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=0,
                    help="heads of one layer the oracle baseline times (0: all, one whole layer)")
    ap.add_argument("--rollout", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--dit", action="store_true")
    ap.add_argument("--ffn", type=int, default=0, help="DiT FFN width (0: 8960, or 13824 at 40 heads)")
    ap.add_argument("--split", choices=("auto", "off", "force"), default="auto",
                    help="attention split mode of the steady-round bench (wf_set_attention_split)")
    return ap.parse_args()


def copy_calibration():
    """A plain device copy of 2 GiB, five times (read 2 GiB + write 2 GiB each)."""
    import torch
    n = 2 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / 5
    print(json.dumps({"mode": "copy_calibration", "bytes_read": n, "bytes_written": n,
                      "ms_per_copy": dt * 1e3, "gbps": 2 * n / dt / 1e9}), flush=True)


def rollout(w):
    """Every round of one request, fresh inputs per round (untimed)."""
    import torch

    from chunk_causal_dit_round_amd import synth
    from chunk_causal_dit_round_amd.session import Session

    sess = Session(w.config(), device="cuda")
    n_rounds = w.n_chunk + w.S
    w_store = w.W + w.S if w.W_store < 0 else w.W_store
    k_steady = w.S + max(w.W, w_store) + 1
    stream = torch.cuda.current_stream()
    times = []
    for k in range(n_rounds):
        synth.fill_round(sess.bufs, "rollout", k, w.n_layers, w.S + 1)
        plan = sess.plan(k)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        sess.run_round(plan, stream=stream)
        e1.record(stream)
        e1.synchronize()
        times.append(e0.elapsed_time(e1) / 1e3)
        if k % 20 == 0:
            print(f"# rollout round {k}: {times[-1] * 1e3:.1f} ms", file=sys.stderr, flush=True)
    steady = times[k_steady:w.n_chunk]
    full = times[w.S:w.n_chunk]
    res = {"mode": "rollout", "metric": "wavefront rounds/sec (=chunks/sec)",
           "workload": f"{w.name} long rollout, {w.n_chunk} chunks, {n_rounds} rounds",
           "steady_rounds_per_s": 1.0 / statistics.median(steady),
           "steady_rounds": [k_steady, w.n_chunk - 1],
           "full_width_rounds_per_s": 1.0 / statistics.median(full),
           "request_chunks_per_s": w.n_chunk / sum(times),
           "request_seconds": sum(times),
           "slowest_round_ms": max(times) * 1e3, "fastest_round_ms": min(times) * 1e3}
    print(json.dumps(res), flush=True)


def oracle_baseline(w, k, layer, heads, raw, fp8=False):
    """Time the oracle on `heads` of one layer of round k (every group)."""
    import numpy as np  # noqa: F401
    from oracle import wf_plan as P
    from oracle import wf_round as WR

    oc = P.Config(S=w.S, W=w.W, W_store=w.W_store, anchor=w.anchor, n_chunk=w.n_chunk, F=w.F,
                  Hh=w.Hh, Ww=w.Ww, n_heads=w.n_heads, head_dim=w.head_dim,
                  n_layers=w.n_layers, mask=w.mask)
    threads = None
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 0) for i in threadpool_info()), default=None)
    except Exception:
        pass
    t0 = time.perf_counter()
    for s in range(w.S + 1):
        if P.chunk_active(oc, k - s):
            WR.group_output(oc, k, s, layer, raw, heads=heads, fp8=fp8)
    dt = time.perf_counter() - t0
    frac = len(heads) / (w.n_heads * w.n_layers)   # share of one round
    t_round = dt / frac
    cores = len(os.sched_getaffinity(0))
    which = ("all heads (one whole layer)" if len(heads) == w.n_heads
             else f"heads {list(heads)} of {w.n_heads}")
    return {"value": 1.0 / t_round, "unit": "rounds/s", "cores": threads or cores,
            "kind": "oracle",
            "sample": f"fp64 oracle, round k={k}, layer {layer}, {which}, every query group "
                      f"over its full context: {dt:.1f} s, scaled by {1 / frac:.0f} to one round "
                      f"({w.n_layers} layers x {w.n_heads} heads); host has {cores} cores"}


def request_bench(args, w):
    """A request shorter than the steady window (the tiny fp32 round): a
    step is the whole request, every round (fill, full width, drain) from
    round 0, with each round's seeded inputs resident in HBM.  value =
    rounds/s over the timed requests."""
    import torch

    from chunk_causal_dit_round_amd import synth, wf
    from chunk_causal_dit_round_amd.session import Session

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    sess = Session(w.config(), device=dev)
    wf.wf_set_attention_split(sess.h, {"auto": wf.WF_SPLIT_AUTO, "off": wf.WF_SPLIT_OFF,
                                       "force": wf.WF_SPLIT_FORCE}[args.split])
    S, L = w.S, w.n_layers
    n_rounds = w.n_chunk + w.S
    sets = []
    for k in range(n_rounds):
        b = sess.alloc_io() if k else sess.bufs
        synth.fill_round(b, "bench", k, L, S + 1)
        if k:
            b["q_rot"], b["out"] = sess.bufs["q_rot"], sess.bufs["out"]
        sets.append(b)
    plans = [sess.plan(k) for k in range(n_rounds)]
    stream = torch.cuda.current_stream()

    def request(ev=None):
        wf.wf_reset(sess.h)
        for k in range(n_rounds):
            for layer in range(L):
                sess.publish(plans[k], layer, sets[k], stream)
                if ev is not None:
                    ev[k][layer][0].record(stream)
                sess.attention(plans[k], layer, sets[k], stream)
                if ev is not None:
                    ev[k][layer][1].record(stream)
            sess.commit(plans[k])

    for _ in range(args.warmup):
        request()
    torch.cuda.synchronize()
    events = [[[[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(L)]
               for _ in range(n_rounds)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        request(events[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    att_s = sum(e[k][l][0].elapsed_time(e[k][l][1]) for e in events for k in range(n_rounds)
                for l in range(L)) / 1e3
    flops = sum(p.flops for p in plans) * args.steps
    achieved = flops / att_s / 1e12
    fp32 = w.dtype == wf.WF_F32
    # fp32 rounds run plain fp32 FMA on the vector ALUs, whose published peak
    # is 157.3 TFLOP/s (256 CUs x 2.4 GHz x 256 FLOP per CU per clock)
    peak = PEAK_FP32_TFLOPS if fp32 else PEAK_BF16_TFLOPS
    res = {
        "metric": "wavefront rounds/sec (=chunks/sec) and attention TFLOP/s",
        "value": args.steps * n_rounds / elapsed, "unit": "rounds/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": 1e3 * elapsed / args.steps, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp32" if fp32 else "bf16", "data": "synthetic",
        "config": {"workload": f"{w.name} whole request ({w.n_chunk} chunks, {n_rounds} rounds: "
                               f"fill, full width, drain), a step = the whole request",
                   "S": w.S, "W": w.W, "tokens_per_chunk": w.n_tokens, "heads": w.n_heads,
                   "head_dim": w.head_dim, "layers": L, "n_rounds": n_rounds},
        "roofline": {"bound": "alu" if fp32 else "mfma", "achieved": achieved, "peak": peak,
                     "unit": "TFLOP/s", "frac": achieved / peak, "traffic": None,
                     "kernel": "wf_attention_f32_kernel" if fp32 else "wf_attention_bf16_kernel",
                     "flops_per_request": flops / args.steps,
                     "attention_ms_per_request": 1e3 * att_s / args.steps},
    }
    if not args.no_cpu_baseline:
        from oracle import wf_plan as P
        from oracle import wf_round as WR

        def raw(rnd, layer, stage, name):
            x = synth.slice_input("bench", rnd, layer, stage, name, sess.N, sess.H, sess.D, dev,
                                  sess.dtype)
            return x.to(torch.float64).cpu().numpy()
        oc = P.Config(S=w.S, W=w.W, W_store=w.W_store, anchor=w.anchor, n_chunk=w.n_chunk,
                      F=w.F, Hh=w.Hh, Ww=w.Ww, n_heads=w.n_heads, head_dim=w.head_dim,
                      n_layers=w.n_layers, mask=w.mask)
        for k in range(n_rounds):               # inputs regenerated before timing
            for layer in range(L):
                for st in range(S + 1):
                    for name in ("q", "k", "v"):
                        raw(k, layer, st, name)
        t0 = time.perf_counter()
        for k in range(n_rounds):
            for layer in range(L):
                WR.round_outputs(oc, k, layer, raw)
        dt = time.perf_counter() - t0
        res["cpu_baseline"] = {"value": n_rounds / dt, "unit": "rounds/s",
                               "cores": len(os.sched_getaffinity(0)), "kind": "oracle",
                               "sample": f"fp64 oracle, the whole request ({n_rounds} rounds, "
                                         f"every layer, group and head, input generation "
                                         f"untimed): {dt:.2f} s"}
    print(json.dumps(res), flush=True)


def dit_oracle_baseline(ds, w, k):
    """Oracle time of one steady DiT round, assembled from timed pieces of
    layer 0 (fp64): one cell's norm + QKV projection (full rows), the
    attention of 256 sampled query rows of each stage over its full context,
    and the output projection + FFN of those rows; scaled to N rows, S+1
    cells and L layers."""
    import numpy as np
    import torch

    from chunk_causal_dit_round_amd import synth
    from oracle import wf_dit as D
    from oracle import wf_plan as P
    from oracle import wf_round as WR

    oc = P.Config(S=w.S, W=w.W, W_store=w.W_store, anchor=w.anchor, n_chunk=w.n_chunk, F=w.F,
                  Hh=w.Hh, Ww=w.Ww, n_heads=w.n_heads, head_dim=w.head_dim,
                  n_layers=w.n_layers, mask=w.mask)
    wt = D.Weights(**{n: t.double().cpu().numpy() for n, t in ds.layers[0].items()})
    mod = ds.mod[0].double().cpu().numpy()
    # round r starts from input set r % 2 on the GPU side
    x0 = lambda rnd, st: synth.dit_x0(ds.tag, rnd % 2, st, w.n_tokens, ds.C, ds.s.device).double().cpu().numpy()  # noqa: E731
    fp8 = {2: True, 3: "k"}.get(w.dtype, False)          # FP8 / FP8K page readings
    dr = D.DitRounds(oc, x0, lambda l: wt, lambda l: mod, fp8=fp8)
    rows = np.arange(0, w.n_tokens, w.n_tokens // 256)[:256]
    # projections of every page a steady round reads (one per cell and history page)
    t0 = time.perf_counter()
    dr.qkv(k, 0, 0)
    t_proj = time.perf_counter() - t0
    for st in range(w.S + 1):                      # the rest, untimed: shared inputs
        for kind, chunk, _ in P.key_entries(oc, k, st):
            rnd, cell, _f = WR.entry_source(oc, k, kind, chunk)
            dr.qkv(rnd, 0, cell)
    t_attn = t_fin = 0.0
    for st in range(w.S + 1):
        t0 = time.perf_counter()
        o = dr.attention(k, 0, st, rows=rows)
        t_attn += time.perf_counter() - t0
        t0 = time.perf_counter()
        D.finish_block(wt, dr.x_in(k, 0, st)[rows], mod[st], o)
        t_fin += time.perf_counter() - t0
    scale = w.n_tokens / len(rows)
    t_layer = (w.S + 1) * t_proj + (t_attn + t_fin) * scale
    t_round = t_layer * w.n_layers
    cores = len(os.sched_getaffinity(0))
    torch.cuda.synchronize()
    return {"value": 1.0 / t_round, "unit": "rounds/s", "cores": cores, "kind": "oracle",
            "sample": f"fp64 oracle, layer 0 of round {k}: one cell's norm + QKV projection "
                      f"{t_proj:.1f} s (x {w.S + 1} cells), attention + output projection + FFN "
                      f"of {len(rows)} query rows per cell {t_attn + t_fin:.1f} s (x {scale:.1f}); "
                      f"one layer {t_layer:.0f} s, x {w.n_layers} layers"}


def dit_rollout(args, w):
    """Every round of one request through the whole DiT (fresh seeded layer-0
    inputs per round, generated between rounds and untimed)."""
    import torch

    from chunk_causal_dit_round_amd.dit import DitSession
    from chunk_causal_dit_round_amd.session import Session

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    ffn = args.ffn or (13824 if w.n_heads == 40 else 8960)
    sess = Session(w.config(), device=dev, io=False)
    ds = DitSession(sess, ffn, tag="rollout-dit")
    ds.tune()                        # fastest hipBLASLt algorithm per product (blocking, untimed)
    n_rounds = w.n_chunk + w.S
    w_store = w.W + w.S if w.W_store < 0 else w.W_store
    k_steady = w.S + max(w.W, w_store) + 1
    stream = torch.cuda.current_stream()
    times = []
    for k in range(n_rounds):
        ds.load_x0(k)
        plan = sess.plan(k)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        ds.round(plan, stream)
        e1.record(stream)
        e1.synchronize()
        times.append(e0.elapsed_time(e1) / 1e3)
        if k % 20 == 0:
            print(f"# DiT rollout round {k}: {times[-1] * 1e3:.1f} ms", file=sys.stderr, flush=True)
    steady = times[k_steady:w.n_chunk]
    res = {"mode": "dit_rollout", "metric": "DiT rounds/sec (=chunks/sec), whole request",
           "workload": f"{w.name} long rollout through the whole DiT (dummy weights, FFN {ffn}), "
                       f"{w.n_chunk} chunks, {n_rounds} rounds",
           "steady_rounds_per_s": 1.0 / statistics.median(steady),
           "request_chunks_per_s": w.n_chunk / sum(times),
           "request_seconds": sum(times),
           "latent_frames_per_s": w.n_chunk * w.F / sum(times),
           "slowest_round_ms": max(times) * 1e3, "fastest_round_ms": min(times) * 1e3}
    print(json.dumps(res), flush=True)


def dit_bench(args, w):
    """Steady whole-DiT rounds: wf_dit_round over all layers."""
    import torch

    from chunk_causal_dit_round_amd import synth, wf
    from chunk_causal_dit_round_amd.dit import DitSession
    from chunk_causal_dit_round_amd.session import Session

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    ffn = args.ffn or (13824 if w.n_heads == 40 else 8960)
    sess = Session(w.config(), device=dev, io=False)
    ds = DitSession(sess, ffn, tag="bench-dit")
    S, L, N, C = w.S, w.n_layers, w.n_tokens, ds.C
    w_store = w.W + w.S if w.W_store < 0 else w.W_store
    k_steady = w.S + max(w.W, w_store) + 1
    if k_steady + args.warmup + args.steps > w.n_chunk:
        print("steps + warmup exceed the steady rounds of one request", file=sys.stderr)
        sys.exit(2)
    # two resident layer-0 input sets; round r starts from set r % 2
    x_sets = []
    for i in range(2):
        ds.load_x0(i)
        x_sets.append(ds.x.clone())
    stream = torch.cuda.current_stream()
    ds.tune(stream)                  # fastest hipBLASLt algorithm per product (blocking, untimed)

    def run(k):
        ds.x.copy_(x_sets[k % 2])
        plan = sess.plan(k)
        ds.round(plan, stream)
        return plan

    for k in range(k_steady + args.warmup):
        run(k)
    torch.cuda.synchronize()
    k0 = k_steady + args.warmup
    t0 = time.perf_counter()
    plans = [run(k0 + i) for i in range(args.steps)]
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    M = (S + 1) * N
    gemm_flops = 2.0 * M * C * (3 * C + C + 2 * ffn) * L
    attn_flops = plans[0].flops
    total = (gemm_flops + attn_flops) * args.steps
    achieved = total / elapsed / 1e12
    # products at the bf16 peak, attention at its page type's peak: a round
    # at both peaks takes gemm / 2.5 + attention / P_attn
    kind = PAGE_KINDS[{wf.WF_FP8: "fp8", wf.WF_FP8K: "fp8k"}.get(w.dtype, "bf16")]
    peak = (gemm_flops + attn_flops) / (gemm_flops / PEAK_BF16_TFLOPS + attn_flops / kind["peak"])
    res = {
        "mode": "dit",
        "metric": "DiT rounds/sec (=chunks/sec): whole Wan-shaped DiT forward of a wavefront round",
        "value": args.steps / elapsed, "unit": "rounds/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": 1e3 * elapsed / args.steps, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if kind["dtype"] == "bf16" else "bf16 products, attention " + kind["dtype"],
        "data": "synthetic",
        "config": {"workload": f"{w.name} steady round, whole DiT forward (dummy weights)",
                   "S": S, "W": w.W, "W_store": w_store, "tokens_per_chunk": N, "heads": w.n_heads,
                   "head_dim": w.head_dim, "dim": C, "ffn_dim": ffn, "layers": L,
                   "rounds_timed": [k0, k0 + args.steps - 1]},
        "flops_per_round": {"products": gemm_flops, "attention": attn_flops},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": peak,
                     "unit": "TFLOP/s", "frac": achieved / peak, "traffic": None,
                     "kernel": "whole round (products + attention)"},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = dit_oracle_baseline(ds, w, k0)
    print(json.dumps(res), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              f"(the round's multi-GPU sharding is described, not built)", file=sys.stderr)
        sys.exit(2)
    import torch

    from chunk_causal_dit_round_amd import synth, wf
    from chunk_causal_dit_round_amd.session import Session
    from chunk_causal_dit_round_amd.workloads import ALL

    w = ALL[args.workload]
    if args.copy_calibration:
        copy_calibration()
        return
    if args.rollout and not args.dit:
        rollout(w)
        return
    if args.dit:
        if args.rollout:
            dit_rollout(args, w)
        else:
            dit_bench(args, w)
        return
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    sess = Session(w.config(), device=dev)
    wf.wf_set_attention_split(sess.h, {"auto": wf.WF_SPLIT_AUTO, "off": wf.WF_SPLIT_OFF,
                                       "force": wf.WF_SPLIT_FORCE}[args.split])
    S, L = w.S, w.n_layers
    w_store = w.W + w.S if w.W_store < 0 else w.W_store
    k_steady = w.S + max(w.W, w_store) + 1         # full width and full window
    n_rounds = w.n_chunk + w.S
    if w.n_chunk + w.S <= 64:
        request_bench(args, w)
        return
    if k_steady + args.warmup + args.steps > w.n_chunk:
        print("steps + warmup exceed the steady rounds of one request", file=sys.stderr)
        sys.exit(2)

    # Two resident input sets; round r uses set r % 2.
    sets = [sess.bufs, sess.alloc_io()]
    for i, b in enumerate(sets):
        synth.fill_round(b, "bench", i, L, S + 1)
        if i == 1:
            b["q_rot"], b["out"] = sets[0]["q_rot"], sets[0]["out"]
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    def run_round(k, ev=None):
        b = sets[k % 2]
        plan = sess.plan(k)
        if ev is None:
            sess.run_round(plan, b, stream)
            return plan
        for layer in range(L):
            ev[0][layer].record(stream)
            sess.publish(plan, layer, b, stream)
            ev[1][layer].record(stream)
            sess.attention(plan, layer, b, stream)
            ev[2][layer].record(stream)
        sess.commit(plan)
        return plan

    for k in range(k_steady + args.warmup):
        run_round(k)
    torch.cuda.synchronize()

    events = [[[torch.cuda.Event(enable_timing=True) for _ in range(L)] for _ in range(3)]
              for _ in range(args.steps)]
    k0 = k_steady + args.warmup
    plans = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        plans.append(run_round(k0 + i, events[i]))
    torch.cuda.synchronize()
    t1 = time.perf_counter()

    elapsed = t1 - t0
    ms_step = 1e3 * elapsed / args.steps
    att_ms = [e[1][l].elapsed_time(e[2][l]) for e in events for l in range(L)]
    round_ms = [e[0][0].elapsed_time(e[2][L - 1]) for e in events]     # device time per round
    pub_ms = [e[0][l].elapsed_time(e[1][l]) for e in events for l in range(L)]
    att_avg = sum(att_ms) / len(att_ms)
    pub_avg = sum(pub_ms) / len(pub_ms)
    flops_launch = plans[0].flops / L            # every timed round is steady: same work
    pub_bytes_launch = plans[0].publish_bytes / L
    achieved = flops_launch / (att_avg * 1e-3) / 1e12
    total_flops = sum(p.flops for p in plans)
    kind = PAGE_KINDS[{wf.WF_FP8: "fp8", wf.WF_FP8K: "fp8k"}.get(w.dtype, "bf16")]
    fp8 = {wf.WF_FP8: True, wf.WF_FP8K: "k"}.get(w.dtype, False)
    peak = kind["peak"]

    res = {
        "metric": "wavefront rounds/sec (=chunks/sec) and attention TFLOP/s vs " + kind["what"],
        "value": args.steps / elapsed,
        "unit": "rounds/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": kind["dtype"],
        "data": "synthetic",
        "config": {"workload": f"{w.name} steady wavefront round", "S": w.S, "W": w.W,
                   "W_store": w_store, "anchor": w.anchor, "n_chunk": w.n_chunk,
                   "tokens_per_chunk": w.n_tokens, "heads": w.n_heads,
                   "head_dim": w.head_dim, "layers": L,
                   "rounds_timed": [k0, k0 + args.steps - 1], "n_rounds": n_rounds,
                   "attention_split": args.split},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": peak,
                     "unit": "TFLOP/s", "frac": achieved / peak,
                     "traffic": measured_traffic(kind, w.name),
                     "kernel": kind["kernel"],
                     "flops_per_launch": flops_launch, "avg_launch_ms": att_avg},
        "attention_tflops_round": total_flops / elapsed / 1e12,
        # one exp per readable (query, key, head): N_q N_k H = FLOPs / (4 d)
        "softmax_exps_per_round": plans[0].flops / (4.0 * w.head_dim),
        "median_round_ms": statistics.median(round_ms) if round_ms else None,
        "publish": {"avg_launch_ms": pub_avg, "bytes_per_launch": pub_bytes_launch,
                    "gbps": pub_bytes_launch / (pub_avg * 1e-3) / 1e9,
                    "hbm_frac": pub_bytes_launch / (pub_avg * 1e-3) / 1e9 / PEAK_HBM_GBPS},
    }

    if not args.no_cpu_baseline:
        def raw(rnd, layer, stage, name):
            x = synth.slice_input("bench", rnd % 2, layer, stage, name, sess.N, sess.H, sess.D,
                                  dev, sess.dtype)
            return x.to(torch.float64).cpu().numpy()
        heads = list(range(args.cpu_heads or w.n_heads))
        res["cpu_baseline"] = oracle_baseline(w, k0, 0, heads, raw, fp8=fp8)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
