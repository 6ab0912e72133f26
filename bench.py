#!/usr/bin/env python3
"""Handoff throughput of the cross-model KV handoff on one MI355X.

One step = one whole handoff of the 16K-token 8B-to-32B-shaped workload: map the source KV
to the latent, score and select the top-30% positions, reconstruct the translated cache of
the complement, then for each of the 64 target layers project Q/K/V of the selected
positions, rotate and scatter K/V into the mixed cache (one kernel) and run the sparse causal
attention.
All inputs are synthetic (seeded) and resident in HBM before timing.  Each timed step is
bracketed by HIP events on its launch stream, with a 512 MiB device write before it (outside
its events) so that it starts with cold caches; the value is T / the median step time.

Prints one JSON line: handoff tokens/s (positions handed off per second), the roofline of
the dominant kernel (the sparse attention, timed with HIP events on its launch stream
over the timed steps), per-stage times, the score GEMM and the top-k apart, the same step
captured in a HIP graph and replayed (time per step and a bit-for-bit check against the eager
outputs), the HBM rate of the standalone RoPE + scatter entry point on the same rows (outside
the timed steps), the rates this GPU reaches on a large library GEMM and a device copy, the
fp64 CPU oracle timed on a bounded sample of the same workload (extrapolated to one handoff),
and the same measurement, with fewer steps, of the 0.6B-to-14B-shaped 4K, the 8B-to-70B-shaped
8K and the batched paged workloads (other_workloads).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

METRIC = "handoff tokens/s (map+select+recompute-attn) at 16K; % of MFMA/HBM roofline"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 matrix peak
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attention_traffic_8B-to-32B-T16384.json")
ATTN_SOURCE = os.path.join(ROOT, "cross_model_kv_amd", "csrc", "attn_bf16.hip")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def f64(t):
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def stage_work(wl, T, k, pos_sum, layers_per_launch=1.0):
    """Algorithmic flops / bytes of every stage of one handoff (per launch for the per-layer
    stages, which process layers_per_launch layers per launch)."""
    d_t, n_qkv = wl.d_t, wl.n_qkv
    w = {
        "map_latent": dict(flops=2.0 * T * wl.d_src * wl.r, bytes=2.0 * (T * wl.d_src + wl.d_src * wl.r + T * wl.r)),
        "score_select": dict(flops=2.0 * T * wl.r * wl.r, bytes=2.0 * T * wl.r + 4.0 * wl.r * wl.r + 4.0 * T),
        "reconstruct": dict(flops=2.0 * (T - k) * wl.r * d_t * wl.L_t,
                            bytes=2.0 * ((T - k) * d_t * wl.L_t + wl.L_t * wl.r * d_t + T * wl.r)),
        # one kernel: gathered rows and W_qkv in, q rows and the rotated k / v cache rows out
        "qkv_rope_scatter": dict(flops=2.0 * k * wl.D * n_qkv,
                                 bytes=2.0 * (k * wl.D + wl.D * n_qkv + k * wl.H_q * wl.d_h + 2.0 * k * d_t)),
        "sparse_attention": dict(flops=4.0 * wl.H_q * wl.d_h * pos_sum,
                                 bytes=2.0 * (T * d_t + 2.0 * k * wl.H_q * wl.d_h)),
    }
    for n in ("qkv_rope_scatter", "sparse_attention"):
        w[n] = {key: v * layers_per_launch for key, v in w[n].items()}
    return w


def cpu_baseline(inp, wl, S, T, k, pos_sum):
    """The fp64 oracle as it is, timed on a bounded sample of the workload and scaled to one
    handoff: 512 source rows of the map, 256 rows of reconstruct + score (all layers), the
    full-length select, one layer's Q/K/V projection of 512 selected rows, one layer's scatter,
    and one layer's attention of 24 selected queries spread over the positions."""
    from oracle import kvx_oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([int(i.get("num_threads", 1)) for i in threadpool_info()] or [1])
    except Exception:
        cores = os.cpu_count() or 1
    rng = np.random.default_rng(0)
    parts = {}

    rows = np.sort(rng.choice(T, 512, replace=False))
    x = f64(inp.x_src[rows])
    w_s = f64(inp.w_s)
    t0 = time.perf_counter()
    z = O.map_latent(x, w_s)
    parts["map_latent"] = (time.perf_counter() - t0) * T / len(rows)
    del w_s, x

    w_l, u = f64(inp.w_l), f64(inp.u)
    zr = z[:256]
    t0 = time.perf_counter()
    _, _, Y = O.reconstruct(zr, w_l, wl.H_kv, wl.d_h)
    parts["reconstruct"] = (time.perf_counter() - t0) * T / len(zr)
    t0 = time.perf_counter()
    s = O.rank_disagreement(Y, u)
    parts["score"] = (time.perf_counter() - t0) * T / len(zr)
    del Y, w_l, u
    s_full = np.tile(s, T // len(s) + 1)[:T] * (1.0 + 1e-9 * np.arange(T))
    t0 = time.perf_counter()
    O.select(s_full, k)
    parts["select"] = time.perf_counter() - t0

    sel_rows = np.sort(rng.choice(S, min(512, len(S)), replace=False))
    xq = f64(inp.x_l[0][torch.as_tensor(sel_rows, device=inp.x_l.device)])
    wq = f64(inp.w_qkv[0])
    t0 = time.perf_counter()
    q, kk, vv = O.recompute_qkv(xq, wq, sel_rows, wl.H_q, wl.H_kv, wl.d_h, wl.rope_base)
    parts["qkv_project"] = (time.perf_counter() - t0) * k / len(sel_rows) * wl.L_t
    del xq, wq
    Kc = rng.standard_normal((T, wl.H_kv, wl.d_h))
    Vc = rng.standard_normal((T, wl.H_kv, wl.d_h))
    t0 = time.perf_counter()
    O.scatter(Kc, Vc, sel_rows, kk, vv)
    parts["rope_scatter"] = (time.perf_counter() - t0) * k / len(sel_rows) * wl.L_t
    qi = np.linspace(0, len(sel_rows) - 1, 24).astype(int)
    t0 = time.perf_counter()
    O.sparse_causal_attention(q[qi], Kc, Vc, sel_rows[qi])
    dt = time.perf_counter() - t0
    parts["sparse_attention"] = dt * pos_sum / float(np.sum(sel_rows[qi] + 1)) * wl.L_t
    total = sum(parts.values())
    cpu_model = None
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), None)
    except OSError:
        pass
    host = {"cpu_model": cpu_model, "nproc": os.cpu_count(),
            "blas_threads_env": {v: os.environ.get(v) for v in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS")
                                 if os.environ.get(v) is not None}}
    return {"value": T / total, "unit": "tokens/s", "cores": int(cores), "kind": "oracle", "host": host,
            "extrapolated": True,
            "sample": (f"extrapolated: fp64 numpy oracle on a sample of the {wl.name} workload (map 512 rows, "
                       f"reconstruct+score 256 rows x {wl.L_t} layers, full select, 1 layer of qkv (512 rows), "
                       "scatter, attention of 24 queries of 1 layer), each part scaled linearly to one handoff "
                       "(rows, layers, sum of causal lengths); the attention part dominates the total"),
            "seconds_per_handoff": total, "parts_s": {k2: round(v2, 4) for k2, v2 in parts.items()}}


def copy_calibration():
    """A plain device copy of 1 GiB, for scaling HBM byte counters (FETCH_SIZE / WRITE_SIZE)."""
    n = 1 << 29
    x = torch.ones(n, dtype=torch.bfloat16, device="cuda")
    y = torch.empty_like(x)
    for _ in range(5):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_each_way": 2 * n, "launches": 5}))


def measured_peaks(stream):
    """What this GPU reaches on a large square bf16 product through the vendor library
    (torch.matmul, 8192^3) and on a 1 GiB device copy: context for the datasheet fractions."""
    n = 8192
    a = torch.randn(n, n, device="cuda").to(torch.bfloat16)
    b = torch.randn(n, n, device="cuda").to(torch.bfloat16)
    for _ in range(3):
        c = a @ b
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(10):
        c = a @ b
    e1.record(stream)
    torch.cuda.synchronize()
    gemm_tflops = 2.0 * n ** 3 / (e0.elapsed_time(e1) / 10 * 1e-3) / 1e12
    del a, b, c
    m = 1 << 29
    x = torch.ones(m, dtype=torch.bfloat16, device="cuda")
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    e0.record(stream)
    for _ in range(10):
        y.copy_(x)
    e1.record(stream)
    torch.cuda.synchronize()
    copy_gbs = 2.0 * 2 * m / (e0.elapsed_time(e1) / 10 * 1e-3) / 1e9
    return {"bf16_gemm_tflops": round(gemm_tflops, 1), "gemm": "torch.matmul 8192x8192x8192 bf16",
            "copy_gbs": round(copy_gbs, 1), "copy": "1 GiB device copy (read + write)"}


def chain_layer_work(wl, k, pos_sum):
    """Algorithmic flops / bytes of one chained target layer (bf16 storage)."""
    HD, D, F, n_qkv, d_t = wl.H_q * wl.d_h, wl.D, wl.F, wl.n_qkv, wl.d_t
    parts = {
        "rmsnorm x2": (0.0, 2.0 * 2 * 2.0 * k * D),
        "qkv_rope_scatter": (2.0 * k * D * n_qkv, 2.0 * (k * D + D * n_qkv + k * HD + k * d_t)),
        "sparse_attention": (4.0 * wl.H_q * wl.d_h * pos_sum, 2.0 * (k * d_t + 2.0 * k * HD)),
        "o_proj+residual": (2.0 * k * HD * D, 2.0 * (k * HD + D * HD + 2.0 * k * D)),
        "swiglu": (2.0 * k * D * 2 * F, 2.0 * (k * D + 2.0 * F * D + k * F)),
        "down+residual": (2.0 * k * F * D, 2.0 * (k * F + D * F + 2.0 * k * D)),
    }
    return parts


def chain_cpu_baseline(inp, cw, wl, S, T, k, pos_sum):
    """The fp64 oracle's chained layer on a bounded sample, scaled to one chained handoff: the
    handoff's own stages as in cpu_baseline, plus one layer's norms, projections and MLP on
    128 selected rows (the attention part is already in the handoff's sample)."""
    from oracle import kvx_oracle as O
    base = cpu_baseline(inp, wl, S, T, k, pos_sum)
    rng = np.random.default_rng(1)
    rows = np.sort(rng.choice(S, min(128, len(S)), replace=False))
    x = f64(inp.x_l[0][torch.as_tensor(rows, device=inp.x_l.device)])
    o = rng.standard_normal((len(rows), wl.H_q * wl.d_h))
    w_o, g1, g2 = f64(cw.w_o[0]), f64(cw.gamma_in[0]), f64(cw.gamma_post[0])
    wg, wu, wd = f64(cw.w_gate[0]), f64(cw.w_up[0]), f64(cw.w_down[0])
    t0 = time.perf_counter()
    O.rmsnorm(x, g1, wl.norm_eps)
    x1 = x + o @ w_o.T
    x2 = x1 + O.swiglu_mlp(O.rmsnorm(x1, g2, wl.norm_eps), wg, wu, wd)
    dt = (time.perf_counter() - t0) * k / len(rows) * wl.L_t
    total = base["seconds_per_handoff"] + dt
    base["parts_s"]["norms+o_proj+mlp"] = round(dt, 4)
    base.update(value=T / total, seconds_per_handoff=total,
                sample=base["sample"] + "; plus 1 layer of norms, output projection and gated MLP on 128 rows, "
                                        "scaled by selected rows and layers")
    return base


def main_chain(args, wl, flush):
    """The handoff with the selected rows chained through every target layer."""
    from cross_model_kv_amd import kvx, synth
    from cross_model_kv_amd.handoff import ChainedHandoff

    dev = torch.device("cuda:0")
    t_gen = time.perf_counter()
    inp = synth.generate(wl, args.seed, dev)
    cw = synth.chain_weights(wl, args.seed, dev)
    h = ChainedHandoff(inp, cw, dev)
    torch.cuda.synchronize()
    log(f"[bench] {wl.name} chained: inputs and one-time preparation {time.perf_counter() - t_gen:.1f}s")
    T, k = h.batch.n_tokens, h.batch.total_sel
    stream = torch.cuda.current_stream(dev)
    names = ["map_latent", "score_select", "reconstruct", "gather_rows", "target_layer"]

    def step(ev=None):
        def mark(key):
            if ev is not None:
                e = torch.cuda.Event(enable_timing=True)
                e.record(stream)
                ev.setdefault(key, []).append(e)
        mark("t0")
        h.map()
        mark("map_latent")
        h.select()
        mark("score_select")
        h.reconstruct()
        mark("reconstruct")
        h.start_rows()
        mark("gather_rows")
        for l in range(wl.L_t):
            h.chain_layer(l)
            mark("target_layer")

    times, marks, wall = timed_steps(step, stream, args.steps, args.warmup, flush)
    order = ["map_latent", "score_select", "reconstruct", "gather_rows"] + ["target_layer"] * wl.L_t
    step_stage_ms, avg_launch_ms = stage_times(marks, order, names, args.steps)
    med = float(np.median(times))

    # the dominant kernel of a chained layer, the gated MLP's gate/up GEMM, timed live on its
    # launch stream with the layer-0 weights and the chain's own rows
    xn = torch.empty_like(h.x)
    hmid = torch.empty((max(k, 1), wl.F), dtype=torch.bfloat16, device=dev)
    kvx.rmsnorm(h.x, cw.gamma_post[0], wl.norm_eps, y=xn)
    ws = torch.empty(max(kvx.target_layer_workspace(kvx.BF16, h.batch, wl.D, wl.F, wl.H_q, wl.H_kv, wl.d_h), 16),
                     dtype=torch.uint8, device=dev)
    for _ in range(2):
        kvx.swiglu(xn[:k], cw.w_gate[0], cw.w_up[0], hmid[:k], ws)
    n_rep = 20
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(n_rep):
        kvx.swiglu(xn[:k], cw.w_gate[0], cw.w_up[0], hmid[:k], ws)
    e1.record(stream)
    torch.cuda.synchronize()
    swiglu_ms = e0.elapsed_time(e1) / n_rep

    S = h.S.cpu().numpy()
    pos_sum = float(np.sum(S.astype(np.float64) + 1.0))
    parts = chain_layer_work(wl, k, pos_sum)
    layer_flops = sum(f for f, _ in parts.values())
    layer_ms = avg_launch_ms["target_layer"]
    hand = stage_work(wl, T, k, pos_sum)
    stages = {n: {"ms_per_step": round(step_stage_ms[n], 4),
                  "ms_per_launch": round(avg_launch_ms[n], 5)} for n in names}
    for n in ("map_latent", "score_select", "reconstruct"):
        stages[n]["tflops"] = round(hand[n]["flops"] / (stages[n]["ms_per_launch"] * 1e-3) / 1e12, 2)
    stages["target_layer"]["tflops"] = round(layer_flops / (layer_ms * 1e-3) / 1e12, 2)
    stages["target_layer"]["algorithmic_flops_per_launch"] = layer_flops
    sw_flops = parts["swiglu"][0]
    achieved = sw_flops / (swiglu_ms * 1e-3) / 1e12
    line = {
        "metric": "chained handoff tokens/s (map+select+recompute through every target layer) at 16K",
        "value": T / (med * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": med, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name + "-chained", "T": T, "requests": h.batch.n_req, "target_layers": wl.L_t,
                   "H_q": wl.H_q, "H_kv": wl.H_kv, "d_h": wl.d_h, "D": wl.D, "F": wl.F, "selected": k,
                   "cache": "paged" if wl.paged else "contiguous", "parallelism": "none"},
        "roofline": {"kernel": "swiglu (gate/up GEMM)", "bound": "mfma", "achieved": round(achieved, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": None, "algorithmic_flops_per_launch": sw_flops, "avg_launch_ms": round(swiglu_ms, 5)},
        "stages": stages,
    }
    if wl.vocab > 0:
        line["ttft"] = time_to_first_token(args, wl, inp, cw, h, med)
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a sample")
        line["cpu_baseline"] = chain_cpu_baseline(inp, cw, wl, S, T, k, pos_sum)
    print(json.dumps(line), flush=True)


def time_to_first_token(args, wl, inp, cw, h, handoff_ms):
    """Time to first token: the chained handoff plus the first-token step (the last prompt
    position through every layer over the mixed cache, final norm, vocabulary projection,
    argmax), against a full re-prefill with the same kernels (every position recomputed,
    then the LM head of the last row)."""
    import dataclasses
    from cross_model_kv_amd import kvx
    from cross_model_kv_amd.handoff import ChainedHandoff

    stream = torch.cuda.current_stream(h.device)
    h.prepare_first_token()
    for _ in range(2):
        h.first_token()
    n_rep = 5
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(n_rep):
        h.first_token()
    e1.record(stream)
    torch.cuda.synchronize()
    ft_ms = e0.elapsed_time(e1) / n_rep
    # full re-prefill: the same inputs with a 100% budget (mapper stages run with nothing to do)
    log("[bench] full re-prefill for the TTFT comparison")
    full = ChainedHandoff(dataclasses.replace(inp, pcts=[100] * len(inp.lengths)), cw, h.device,
                          keep_all_outputs=False)
    last_rows = torch.tensor([c - 1 for c in full.batch.cu_tokens[1:]], dtype=torch.long, device=h.device)
    xn = torch.empty((len(inp.lengths), wl.D), dtype=torch.bfloat16, device=h.device)
    logits = torch.empty((len(inp.lengths), wl.vocab), dtype=torch.bfloat16, device=h.device)
    ws = torch.empty(max(kvx.linear_workspace(kvx.BF16, len(inp.lengths), wl.vocab, wl.D), 16), dtype=torch.uint8,
                     device=h.device)

    def prefill():
        full.run()
        kvx.rmsnorm(full.x[last_rows], cw.gamma_final, wl.norm_eps, y=xn)
        kvx.linear(xn, cw.w_lm, logits, ws)
        kvx.argmax(logits)

    prefill()
    torch.cuda.synchronize()
    n_full = 2
    e0.record(stream)
    for _ in range(n_full):
        prefill()
    e1.record(stream)
    torch.cuda.synchronize()
    full_ms = e0.elapsed_time(e1) / n_full
    ttft = handoff_ms + ft_ms
    del full
    torch.cuda.empty_cache()
    return {"handoff_ms": round(handoff_ms, 3), "first_token_ms": round(ft_ms, 3), "ttft_ms": round(ttft, 3),
            "full_prefill_ttft_ms": round(full_ms, 3), "speedup_vs_full_prefill": round(full_ms / ttft, 3),
            "ttft_saved": round(1.0 - ttft / full_ms, 4),
            "note": "full prefill = every position through every chained layer with the same kernels, then the "
                    "LM head of the last row; both on this GPU, inputs resident"}


FLUSH_BYTES = 512 << 20        # written between timed steps: more than the 256 MB last-level cache


def timed_steps(step, stream, steps, warmup, flush):
    """W untimed warmups, then K steps each bracketed by its own HIP events on the launch stream,
    with a 512 MiB device write before every timed step (outside its events) so that no step
    starts with the previous step's operands in the last-level cache or the L2s.  Returns the
    per-step times (ms), the per-stage event marks and the wall time of the timed loop (s)."""
    for _ in range(warmup):
        step(None)
    torch.cuda.synchronize()
    marks = {}
    ends = []
    t0 = time.perf_counter()
    for s in range(steps):
        flush.fill_(s & 0x7F)
        step(marks)
        e = torch.cuda.Event(enable_timing=True)
        e.record(stream)
        ends.append(e)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    times = [marks["t0"][s].elapsed_time(ends[s]) for s in range(steps)]
    return times, marks, wall


def stage_times(marks, order, names, steps):
    """Per-stage ms per step and per launch from the marks (each stage ends where the next begins)."""
    idx = {n: 0 for n in names}
    stage_ms = {n: 0.0 for n in names}
    launches = {n: 0 for n in names}
    for s in range(steps):
        prev = marks["t0"][s]
        for n in order:
            e = marks[n][idx[n]]
            idx[n] += 1
            stage_ms[n] += prev.elapsed_time(e)
            launches[n] += 1
            prev = e
    return ({n: stage_ms[n] / steps for n in names}, {n: stage_ms[n] / launches[n] for n in names})


def measure_handoff(wl, args, steps, warmup, flush, dev):
    """Inputs of workload wl generated and resident, then K timed handoffs.  Returns the Handoff,
    its inputs and the measurements (median step time, per-stage times and rates)."""
    from cross_model_kv_amd import kvx, synth
    from cross_model_kv_amd.handoff import Handoff

    t_gen = time.perf_counter()
    inp = synth.generate(wl, args.seed, dev)
    h = Handoff(inp, dev)
    torch.cuda.synchronize()
    log(f"[bench] {wl.name}: inputs and one-time preparation {time.perf_counter() - t_gen:.1f}s")
    T = h.batch.n_tokens           # all positions of the batch (one request: T)
    k = h.batch.total_sel
    # the target layers run in chunks (Handoff.chunks): one projection launch and one attention
    # launch per chunk, every layer of a chunk at once
    chunks = h.chunks
    lc = max(n for _, n in chunks)
    qkv_l = torch.empty((lc, max(k, 1), wl.n_qkv), dtype=torch.bfloat16, device=dev)
    qkv = qkv_l[0]
    ws_qkv = h.ws_attn
    stream = torch.cuda.current_stream(dev)
    names = ["map_latent", "score_select", "reconstruct", "qkv_rope_scatter", "sparse_attention"]

    def step(ev=None):
        def mark(key):
            if ev is not None:
                e = torch.cuda.Event(enable_timing=True)
                e.record(stream)
                ev.setdefault(key, []).append(e)
        mark("t0")
        h.map()
        mark("map_latent")
        h.select()
        mark("score_select")
        h.reconstruct()
        mark("reconstruct")
        for l0, n in chunks:
            if n == 1:                 # a layer alone: the single-layer calls with their workspaces
                kvx.qkv_rope_scatter(l0, inp.x_l[l0], inp.w_qkv[l0], wl.H_q, wl.H_kv, wl.d_h, h.rope, h.batch,
                                     h.S, h.cache, qkv, ws_qkv)
                mark("qkv_rope_scatter")
                kvx.sparse_attention(l0, qkv, wl.H_q, wl.H_kv, wl.d_h, h.rope, h.batch, h.S, h.cache, h.out[l0],
                                     h.lse[l0], ws_qkv)
                mark("sparse_attention")
                continue
            kvx.qkv_rope_scatter_layers(l0, inp.x_l[l0:l0 + n], inp.w_qkv[l0:l0 + n], wl.H_q, wl.H_kv, wl.d_h,
                                        h.rope, h.batch, h.S, h.cache, qkv_l[:n])
            mark("qkv_rope_scatter")
            kvx.sparse_attention_layers(l0, qkv_l[:n], wl.H_q, wl.H_kv, wl.d_h, h.rope, h.batch, h.S, h.cache,
                                        h.out[l0:l0 + n], h.lse[l0:l0 + n])
            mark("sparse_attention")

    times, marks, wall = timed_steps(step, stream, steps, warmup, flush)
    order = ["map_latent", "score_select", "reconstruct"] + ["qkv_rope_scatter", "sparse_attention"] * len(chunks)
    step_stage_ms, avg_launch_ms = stage_times(marks, order, names, steps)
    med = float(np.median(times))
    S = h.S.cpu().numpy()
    pos_sum = float(np.sum(S.astype(np.float64) + 1.0))
    # per launch: the per-layer stages cover L_t / len(chunks) layers on average
    work = stage_work(wl, T, k, pos_sum, wl.L_t / len(chunks))
    stages = {}
    for n in names:
        t = avg_launch_ms[n] * 1e-3
        w = work[n]
        stages[n] = {"ms_per_step": round(step_stage_ms[n], 4), "ms_per_launch": round(avg_launch_ms[n], 5),
                     "tflops": round(w["flops"] / t / 1e12, 2) if w["flops"] else None,
                     "gbs": round(w["bytes"] / t / 1e9, 1)}
    att_ms = avg_launch_ms["sparse_attention"]
    achieved = work["sparse_attention"]["flops"] / (att_ms * 1e-3) / 1e12
    # the handoff at 100% of every stage's roofline (bf16 peak for the matrix-core stages)
    roof_ms = sum(w["flops"] / (PEAK_BF16_TFLOPS * 1e12) * 1e3 * (len(chunks) if n in ("qkv_rope_scatter",
                                                                                      "sparse_attention") else 1)
                  for n, w in work.items())
    res = {
        "value": T / (med * 1e-3), "ms_per_step": med, "T": T, "k": k,
        "step_ms": {"median": round(med, 4), "mean": round(float(np.mean(times)), 4),
                    "min": round(float(np.min(times)), 4), "max": round(float(np.max(times)), 4)},
        "wall_ms_per_step_with_flush": round(wall * 1e3 / steps, 4),
        "stages": stages,
        "roofline": {"kernel": "sparse_attention", "bound": "mfma", "achieved": round(achieved, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "algorithmic_flops_per_launch": work["sparse_attention"]["flops"],
                     "avg_launch_ms": round(att_ms, 5)},
        "handoff_at_roofline_ms": round(roof_ms, 3),
        "frac_of_roofline_time": round(roof_ms / med, 4),
        "layers_per_launch": [n for _, n in chunks],
    }
    ctx = dict(h=h, inp=inp, step=step, qkv=qkv, ws_qkv=ws_qkv, S=S, pos_sum=pos_sum, work=work, stream=stream)
    return res, ctx


def score_select_split(h, stream, reps=20):
    """The score GEMM and the top-k kernel apart (outside the timed steps): kvx_select_topk alone
    on the step's own scores, timed with HIP events; the score GEMM is the rest of kvx_score_select."""
    from cross_model_kv_amd import kvx
    sc = h.scores.clone()
    out = (torch.empty_like(h.sel), torch.empty_like(h.rest))
    e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
    for _ in range(2):
        h.select()
        kvx.select_topk(sc, h.batch, out)
    e0.record(stream)
    for _ in range(reps):
        h.select()
    e1.record(stream)
    for _ in range(reps):
        kvx.select_topk(sc, h.batch, out)
    e2.record(stream)
    torch.cuda.synchronize()
    both = e0.elapsed_time(e1) / reps
    sel = e1.elapsed_time(e2) / reps
    return both, sel


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="8B-to-32B-shape-T16384")
    ap.add_argument("--seed", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="time only the headline workload (no 4K, 70B-shaped and batched lines)")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--chain", action="store_true",
                    help="chain the selected rows through every target layer (norms, output projection, MLP)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the handoff path here is single-GPU.",
              file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return

    from cross_model_kv_amd import kvx, workloads

    wl = workloads.ALL[args.workload]
    dev = torch.device("cuda:0")
    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
    if args.chain:
        main_chain(args, wl, flush)
        return
    res, ctx = measure_handoff(wl, args, args.steps, args.warmup, flush, dev)
    h, inp, step, qkv, stream = ctx["h"], ctx["inp"], ctx["step"], ctx["qkv"], ctx["stream"]
    T, k, S, pos_sum, work = res["T"], res["k"], ctx["S"], ctx["pos_sum"], ctx["work"]

    # The same step captured once in a HIP graph (no entry point allocates, copies or synchronises)
    # and replayed: its time per step, and whether every replay reproduces the eager outputs bit
    # for bit.  Reported beside the eager line; the step above is the measured one.
    graph = None
    try:
        ref_out, ref_sel = h.out.clone(), h.S.clone()
        side = torch.cuda.Stream(dev)
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            step()
        stream.wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        torch.cuda.synchronize()
        same = True
        g.replay()
        torch.cuda.synchronize()
        same = same and torch.equal(h.out, ref_out) and torch.equal(h.S, ref_sel)
        gt = []
        for i in range(args.steps):
            flush.fill_(i & 0x7F)
            ge0, ge1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            ge0.record(stream)
            g.replay()
            ge1.record(stream)
            gt.append((ge0, ge1))
        torch.cuda.synchronize()
        same = same and torch.equal(h.out, ref_out) and torch.equal(h.S, ref_sel)
        graph = {"ms_per_step": round(float(np.median([a.elapsed_time(b) for a, b in gt])), 3),
                 "replays_equal_eager": bool(same)}
        del g
    except RuntimeError as e:          # reported, not fatal: the eager line is the measurement
        graph = {"error": str(e)[:200]}

    # The step fuses RoPE + scatter into the projection's epilogue.  The standalone entry point
    # (kvx_rope_scatter, HBM-bound) is timed here on the same selected rows, after the timed
    # steps and outside them, for its bandwidth: 2 * k * H_kv * d_h bf16 values read and written.
    for l in range(2):
        kvx.rope_scatter(l, qkv, wl.H_q, wl.H_kv, wl.d_h, h.rope, h.batch, h.S, h.cache)
    reps = 4
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        for l in range(wl.L_t):
            kvx.rope_scatter(l, qkv, wl.H_q, wl.H_kv, wl.d_h, h.rope, h.batch, h.S, h.cache)
    e1.record(stream)
    torch.cuda.synchronize()
    sc_ms = e0.elapsed_time(e1) / (reps * wl.L_t)
    sc_bytes = 8.0 * k * wl.H_kv * wl.d_h
    sc_gbs = sc_bytes / (sc_ms * 1e-3) / 1e9
    scatter = {"kernel": "rope_scatter (kvx_rope_scatter on the step's selected rows; outside the timed step, "
                         "which fuses RoPE + scatter into the projection)",
               "bound": "hbm", "achieved": round(sc_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
               "frac": round(sc_gbs / PEAK_HBM_GBS, 4), "bytes_per_launch": sc_bytes,
               "avg_launch_ms": round(sc_ms, 5)}

    # The reconstruction for a mapper whose keys carry no rotary phase (kvx_reconstruct_rope:
    # translated keys rotated at their positions in the same GEMM's epilogue), timed on the
    # step's complement rows beside the plain reconstruction, outside the timed steps.
    def time_rec(rope_t, reps=5):
        for _ in range(2):
            kvx.reconstruct(h.z, inp.w_l, wl.H_kv, wl.d_h, h.batch, h.cache, rows=h.C, rope=rope_t)
        r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        r0.record(stream)
        for _ in range(reps):
            kvx.reconstruct(h.z, inp.w_l, wl.H_kv, wl.d_h, h.batch, h.cache, rows=h.C, rope=rope_t)
        r1.record(stream)
        torch.cuda.synchronize()
        return r0.elapsed_time(r1) / reps
    rec_plain_ms, rec_rope_ms = time_rec(None), time_rec(h.rope)
    # the normalized score (outside energy over total energy: two score GEMMs, one select) on
    # the step's latent, outside the timed steps
    op_tot = kvx.score_prepare(inp.w_l, inp.u[:, :, :0])
    nbuf = (torch.empty_like(h.scores), torch.empty_like(h.sel), torch.empty_like(h.rest))
    for _ in range(2):
        kvx.score_select_normalized(h.z, h.op, op_tot, h.batch, inp.pcts, out=nbuf)
    n0, n1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n0.record(stream)
    for _ in range(10):
        kvx.score_select_normalized(h.z, h.op, op_tot, h.batch, inp.pcts, out=nbuf)
    n1.record(stream)
    torch.cuda.synchronize()
    normalized = {"kernel": "score_select_normalized (two score GEMMs and one select), outside the timed step",
                  "ms": round(n0.elapsed_time(n1) / 10, 5)}
    # the projection with QK-norm (q and k normalised per head before the rotation) on one layer
    # of the step's rows, beside the same projection without it (both whole tiles, no split)
    gq = torch.ones(wl.d_h, dtype=torch.float32, device=dev)
    def time_qkv(qk, reps=10):
        def run():
            if qk:
                kvx.qkv_rope_scatter_qknorm(0, inp.x_l[0], inp.w_qkv[0], wl.H_q, wl.H_kv, wl.d_h, gq, gq, 1e-6, h.rope,
                                            h.batch, h.S, h.cache, qkv)
            else:
                kvx.qkv_rope_scatter_layers(0, inp.x_l[0:1], inp.w_qkv[0:1], wl.H_q, wl.H_kv, wl.d_h, h.rope, h.batch,
                                            h.S, h.cache, qkv.view(1, *qkv.shape))
        for _ in range(2):
            run()
        q0, q1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        q0.record(stream)
        for _ in range(reps):
            run()
        q1.record(stream)
        torch.cuda.synchronize()
        return q0.elapsed_time(q1) / reps
    qk_plain_ms, qk_norm_ms = time_qkv(False), time_qkv(True)
    qknorm = {"kernel": "qkv_rope_scatter_qknorm on one layer (whole tiles), outside the timed step",
              "ms": round(qk_norm_ms, 5), "plain_ms": round(qk_plain_ms, 5),
              "tflops": round(2.0 * k * wl.D * wl.n_qkv / (qk_norm_ms * 1e-3) / 1e12, 2)}
    # direct scoring of the stored cache (every layer's K/V of every position, against the
    # calibration bases), summed and selected, and per layer with every layer's own top-k
    cop = kvx.score_cache_prepare(inp.u, kvx.BF16)
    cws = torch.empty(4 * wl.L_t * -(-wl.c // 256) * T + 256, dtype=torch.uint8, device=dev)
    cbuf = (torch.empty_like(h.scores), torch.empty_like(h.sel), torch.empty_like(h.rest))
    energy = torch.empty((wl.L_t, T), dtype=torch.float32, device=dev)
    lbuf = (torch.empty((wl.L_t, k), dtype=torch.int32, device=dev),
            torch.empty((wl.L_t, T - k), dtype=torch.int32, device=dev))
    def time_direct(per_layer, reps=5):
        def run():
            if per_layer:
                kvx.score_cache(h.cache, 0, wl.H_kv, wl.d_h, cop, h.batch, energy=energy, ws=cws)
                kvx.select_topk_layers(energy, h.batch, out=lbuf)
            else:
                kvx.score_cache_select(h.cache, 0, wl.H_kv, wl.d_h, cop, h.batch, inp.pcts, ws=cws, out=cbuf)
        run()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            run()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps
    dsum_ms, dlay_ms = time_direct(False), time_direct(True)
    d_t = 2 * wl.H_kv * wl.d_h
    dflops = 2.0 * T * d_t * 2 * wl.c * wl.L_t              # hi and lo halves of the basis
    direct_score = {"kernel": "score_cache_select (direct scoring of the stored cache, all layers) and score_cache + "
                              "select_topk_layers (per-layer sets), outside the timed step",
                    "ms": round(dsum_ms, 5), "per_layer_sets_ms": round(dlay_ms, 5), "bound": "mfma",
                    "tflops_executed": round(dflops / (dsum_ms * 1e-3) / 1e12, 2),
                    "cache_gbs": round(2.0 * T * d_t * wl.L_t / (dsum_ms * 1e-3) / 1e9, 1)}
    del cop, cws, cbuf, energy, lbuf
    rec_flops = work["reconstruct"]["flops"]
    rotated_keys = {"kernel": "reconstruct with rotated translated keys (kvx_reconstruct_rope), outside the timed step",
                    "ms": round(rec_rope_ms, 5), "tflops": round(rec_flops / (rec_rope_ms * 1e-3) / 1e12, 2),
                    "plain_ms": round(rec_plain_ms, 5)}

    # score GEMM and top-k apart: the score is a dense contraction (matrix cores, executed as
    # 2 T r 2r flops with the hi/lo operator), the top-k a latency-bound pass over T scores
    both_ms, sel_ms = score_select_split(h, stream)
    gemm_ms = max(both_ms - sel_ms, 1e-6)
    r = wl.r
    score_split = {
        "score_gemm": {"ms": round(gemm_ms, 5), "bound": "mfma",
                       "tflops_executed": round(2.0 * T * r * 2 * r / (gemm_ms * 1e-3) / 1e12, 2),
                       "frac_of_bf16_peak": round(2.0 * T * r * 2 * r / (gemm_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                       "gbs": round((2.0 * T * r + 2.0 * r * 2 * r + 4.0 * T * (r // 256)) / (gemm_ms * 1e-3) / 1e9, 1)},
        "select": {"ms": round(sel_ms, 5), "bound": "latency",
                   "note": "one workgroup per request; radix passes over the request's keys in LDS"},
    }

    traffic = None
    if os.path.exists(TRAFFIC_FILE) and wl.name == "8B-to-32B-shape-T16384":
        # HBM bytes counted by rocprofv3 (FETCH_SIZE, WRITE_SIZE scaled by a 1 GiB copy); valid only for
        # the kernel source they were counted on
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
        with open(ATTN_SOURCE, "rb") as f:
            if hashlib.sha256(f.read()).hexdigest() == rec.get("kernel_source_sha256"):
                traffic = rec.get("hbm_bytes_per_launch")
    roofline = dict(res["roofline"])
    roofline["traffic"] = traffic
    peaks = measured_peaks(stream)
    peaks["attention_frac_of_gemm"] = round(roofline["achieved"] / peaks["bf16_gemm_tflops"], 4)
    peaks["scatter_frac_of_copy"] = round(sc_gbs / peaks["copy_gbs"], 4)
    line = {
        "metric": METRIC,
        "value": res["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "T": T, "requests": h.batch.n_req, "source_layers": wl.L_s,
                   "d_src": wl.d_src, "latent_rank": wl.r,
                   "target_layers": wl.L_t, "H_q": wl.H_q, "H_kv": wl.H_kv, "d_h": wl.d_h, "D": wl.D,
                   "calibration_rank": wl.c, "budget_pct": list(h.inp.pcts) if wl.batched else wl.pct,
                   "selected": k, "cache": "paged" if wl.paged else "contiguous", "parallelism": "none"},
        "timing": {"per_step": "HIP events on the launch stream around each step; value = T / median step",
                   "flush_between_steps_bytes": FLUSH_BYTES, **res["step_ms"],
                   "wall_ms_per_step_with_flush": res["wall_ms_per_step_with_flush"]},
        "roofline": roofline,
        "handoff_at_roofline_ms": res["handoff_at_roofline_ms"],
        "frac_of_roofline_time": res["frac_of_roofline_time"],
        "layers_per_launch": res["layers_per_launch"],
        "stages": res["stages"],
        "score_select_split": score_split,
        "scatter_standalone": scatter,
        "reconstruct_rotated_keys": rotated_keys,
        "score_select_normalized": normalized,
        "qkv_qknorm": qknorm,
        "direct_score": direct_score,
        "graph": graph,
        "measured_peaks": peaks,
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a sample")
        line["cpu_baseline"] = cpu_baseline(inp, wl, S, T, k, pos_sum)
    del h, inp, ctx, qkv, step
    torch.cuda.empty_cache()

    # the other workloads of the pages' model pairs, each timed the same way (fewer steps)
    if not args.no_other_workloads:
        others = {}
        for name in ("0.6B-to-14B-shape-T4096", "8B-to-70B-shape-T8192", "batched-16req-paged16"):
            if name == wl.name:
                continue
            o_res, o_ctx = measure_handoff(workloads.ALL[name], args, max(3, min(args.steps, 5)),
                                           max(1, min(args.warmup, 2)), flush, dev)
            others[name] = {"tokens_per_s": round(o_res["value"], 1), "ms_per_step": round(o_res["ms_per_step"], 4),
                            "T": o_res["T"], "selected": o_res["k"], "step_ms": o_res["step_ms"],
                            "roofline": o_res["roofline"], "handoff_at_roofline_ms": o_res["handoff_at_roofline_ms"],
                            "frac_of_roofline_time": o_res["frac_of_roofline_time"],
                            "layers_per_launch": o_res["layers_per_launch"],
                            "stages": {n: {kk: v for kk, v in st.items() if kk in ("ms_per_step", "tflops")}
                                       for n, st in o_res["stages"].items()}}
            del o_ctx
            torch.cuda.empty_cache()
        line["other_workloads"] = others
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
