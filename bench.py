#!/usr/bin/env python3
"""Benchmark: committed tokens/s of masked-diffusion decoding on one MI355X.

Workload (default): the dense 8B-shaped dLLM in bf16 at batch 1 -- 32 layers,
d 4096, 32 heads x 128, SwiGLU FFN 12288, vocab 126464, a prompt of 512
random ids and 256 generated positions in blocks of 32, vicinity w 16,
tau 0.9, credit on, smoothing alpha 0.3 over the top-8, planting +8 with
probability 0.75.  Weights N(0, 0.02) drawn on the GPU; all inputs resident in
HBM before the timed region.

One bench step = one whole generation of the batch (every block: full KV
refresh, then denoise+commit steps replayed from a HIP graph until the block
is committed).  value = committed tokens / wall time over the timed steps.

Also reported:
  step_latency_ms / step_latency_p90_ms: one denoise+commit step, median and
    p90 over every graph replay of a run (replay time / graph_unroll,
    event-timed; block refreshes excluded).
  roofline: the dominant kernel (the skinny bf16 GEMM that runs the QKV and
    gate|up projections of every layer), timed with HIP events on the stream it
    is launched on, over rotating layers so every launch streams its weights
    from HBM; algorithmic bytes = weights + input activations + fp32 output.
    With more than 128 window rows (batch 16, long context) the projections
    run the fat GEMM instead, priced in TFLOP/s against bf16 MFMA peak.
  batch16: the same weights on the batch-16 request mix (prompts U{128..1024},
    ragged), one warm-up and one timed generation (dense 8B workload only).
  decode_accounting: commits through the threshold gate, the credit gate and
    the fallback, idle graph steps past a block's end, commits-per-step
    histogram.  Under the workloads' literal planting every step commits one
    token through the fallback.
  supplementary_calibrated_planting: the batch-1 and batch-16 workloads (and
    with --supplementary-long the long-context one) with the planting bias
    raised by ln(V-1), so that planted positions pass the threshold gate:
    tokens/s, step latency and the same accounting.  A separate reading of
    the planting, labelled as such; `value` is always the literal workload.
  cpu_baseline: the CPU oracle on a bounded sample -- one full refresh and
    the median of three full steps (every layer, LM head, vocab stats,
    commit) when a refresh takes under 25 s on the host, else one layer of
    each scaled to the model's layers -- scaled to the run's refresh and step
    counts.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                       [--no-batch16] [--no-cpu-baseline] [--queue Q [--budget T]]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
KERNEL = "gemm_skinny_kernel<bf16, MT=4, NT=2>"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_skinny_qkv_gateup_dense8b_traffic.json")
MODEL_NAMES = {"dense8b_b1": "dense 8B-shaped dLLM", "dense8b_b16": "dense 8B-shaped dLLM",
               "dense8b_long_b4": "dense 8B-shaped dLLM, 8K prompt",
               "moe_b1": "MoE dLLM (64 experts top-8 + shared)", "tiny_f32": "tiny dLLM"}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def source_hash() -> str:
    """Hash of the sources the skinny projection kernel is built from (its
    recorded HBM traffic is reported only while they are unchanged)."""
    h = hashlib.sha256()
    for f in ("gemm.hip", "gemm_split.h", "common.h"):
        h.update(open(os.path.join(ROOT, "diffusion_vicinity_kv_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def dominant_kernel_timing(wc, weights, iters=40):
    """Average launch time and bytes of the QKV / gate|up projections at the
    step's row count, alternating over rotating layers."""
    import torch
    from diffusion_vicinity_kv_amd import binding as B
    m = wc.model
    d = m.d_model
    F = m.shared_ffn if m.is_moe else m.ffn_dim
    gu_key = "shared_gate_up" if m.is_moe else "w_gate_up"
    rows = min(wc.max_len, wc.decode.block_len + 2 * wc.decode.vicinity_w) * wc.batch
    A = torch.randn(rows, d, device="cuda")
    lib = B.load()
    out = torch.empty(max(lib.dinfer_linear_out_elems(rows, 3 * d, d, B.BF16),
                          lib.dinfer_linear_out_elems(rows, 2 * F, d, B.BF16)), device="cuda")
    # the two projections in the packed layout the library reads
    layers = [{k: B.pack_linear(L[k]) for k in ("wqkv", gu_key)}
              for L in weights["layers"] if L is not None]
    shapes = []
    for i in range(iters):
        L = layers[i % len(layers)]
        W = L["wqkv"] if i % 2 == 0 else L[gu_key]
        shapes.append(W)
    for W in shapes[:4]:
        B.linear(A, W, out)
    torch.cuda.synchronize()
    # the launches replayed from one captured graph, back to back on one
    # stream as in the step's own graph: events around the replays time the
    # kernels, not the host's launch rate (which a profiler slows down)
    cap = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        for W in shapes:
            B.linear(A, W, out)
    st = torch.cuda.current_stream()
    g.replay()
    torch.cuda.synchronize()
    reps = 3
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(reps):
        g.replay()
    e1.record(st)
    torch.cuda.synchronize()
    avg_ms = e0.elapsed_time(e1) / (reps * len(shapes))
    nbytes = sum(W.shape[0] * d * 2 + rows * d * 4 + rows * W.shape[0] * 4 for W in shapes)
    nflops = sum(2 * rows * W.shape[0] * d for W in shapes)
    del g
    return avg_ms, nbytes / len(shapes), nflops / len(shapes), rows


def cpu_baseline(wc, gpu_refreshes_per_run, gpu_steps_per_run, committed_per_run,
                 full_budget_s=25.0):
    """Oracle timed on a bounded sample of the workload, scaled to one run.

    One layer of the full refresh is timed first.  If a whole refresh of
    every layer fits full_budget_s, the sample is one full refresh and three
    full steps (all layers, the LM head, vocab statistics and commit; the
    step time is their median), on a model whose layers all reuse layer 0's
    weights -- the oracle's cost depends on the shapes only, and one fp64
    copy of a layer keeps the host memory small.  Otherwise the one-layer
    refresh and twelve one-layer window steps are scaled to the model's
    layers."""
    import numpy as np
    import oracle
    import synth
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()
                       if i.get("user_api") == "blas"] or [os.cpu_count()])
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    m = wc.model
    nl = m.n_layers
    w = synth.make_weights(m, wc.seed, device="cpu", layers=[0])
    req = synth.make_requests(wc)
    rb = req.get("router_bias")

    def new_run(om):
        return oracle.OracleRun(om, wc.decode, req["tokens"][0].numpy(), int(req["prompt_len"][0]),
                                int(req["gen_len"][0]), req["plant_id"][0].numpy(),
                                float(req["plant_bias"][0]), None if rb is None else rb[0].numpy())

    def one_step(om, run, lo, hi):
        e = run.window_embeddings(lo, hi)
        t0 = time.perf_counter()
        h = om.forward_rows(run.cache, np.arange(lo, hi), e, run.L, run._router_bias_block())
        t_layers = time.perf_counter() - t0
        t0 = time.perf_counter()
        st = run.stats(om.logits(h[run.bs - lo: run.be - lo]))
        run.commit(st)
        return t_layers, time.perf_counter() - t0

    om = oracle.OracleModel(m, w, layers=[0])
    run = new_run(om)
    t0 = time.perf_counter()
    run.start_block(0)                           # one layer of the full refresh
    t_ref_layer = time.perf_counter() - t0
    lo, hi = run.window()
    base = {"unit": "tokens/s", "cores": int(threads), "kind": "oracle"}
    if nl * t_ref_layer <= full_budget_s:
        om.layer_ids = list(range(nl))            # every layer on layer 0's weights
        om.layers = {li: om.layers[0] for li in om.layer_ids}
        run = new_run(om)
        t0 = time.perf_counter()
        run.start_block(0)
        t_refresh = time.perf_counter() - t0
        steps = [sum(one_step(om, run, lo, hi)) for _ in range(3)]
        t_step = float(np.median(steps))
        t_run = gpu_refreshes_per_run * t_refresh + gpu_steps_per_run * t_step
        return {**base, "value": round(committed_per_run / t_run, 4),
                "sample": (f"fp64 NumPy oracle, all {nl} layers (sharing one layer's weights): one "
                           f"full refresh of {run.L} rows ({t_refresh:.2f} s) and the median of 3 "
                           f"full steps of {hi - lo} window rows with the LM head, vocab stats and "
                           f"commit ({', '.join(f'{x:.2f}' for x in steps)} s); scaled to "
                           f"{gpu_refreshes_per_run} refreshes and {gpu_steps_per_run} steps per "
                           f"run ({t_run:.1f} s; {t_ref_layer + t_refresh + sum(steps):.1f} s "
                           "measured)"),
                "step_s": round(t_step, 3), "refresh_s": round(t_refresh, 3)}
    reps = 12                                    # window steps of one layer (averaged)
    t_step_layer = t_head = 0.0
    for _ in range(reps):
        a, b = one_step(om, run, lo, hi)
        t_step_layer += a / reps
        t_head += b / reps
    t_refresh = nl * t_ref_layer
    t_step = nl * t_step_layer + t_head
    t_run = gpu_refreshes_per_run * t_refresh + gpu_steps_per_run * t_step
    sample_s = t_ref_layer + reps * (t_step_layer + t_head)
    return {**base, "value": round(committed_per_run / t_run, 4),
            "sample": (f"fp64 NumPy oracle: 1 of {nl} layers of the full refresh "
                       f"({run.L} rows, {t_ref_layer:.2f} s); {reps} window steps of 1 layer "
                       f"({hi - lo} rows, {t_step_layer:.2f} s each) with the LM head + vocab "
                       f"stats + commit ({t_head:.2f} s each); scaled to {nl} layers, "
                       f"{gpu_refreshes_per_run} refreshes and {gpu_steps_per_run} steps per run "
                       f"({t_run:.1f} s projected; {sample_s:.1f} s measured)"),
            "step_s": round(t_step, 3), "refresh_s": round(t_refresh, 3)}


def run_workload(wc, w, req, unroll, warmup, steps):
    """Timed whole generations of one request batch; also the event-timed
    latency of one denoise+commit step from graph replays of the first block."""
    import torch
    from diffusion_vicinity_kv_amd.engine import Engine
    m = wc.model
    max_len = req["tokens"].shape[1]
    eng = Engine(m, wc.decode, w, wc.batch, max_len, graph_unroll=unroll)
    tokens0 = req["tokens"].cuda().contiguous()
    tokens = tokens0.clone()
    plant_id = req["plant_id"].cuda().contiguous()
    plant_bias = req["plant_bias"].cuda().contiguous()
    P, G = req["prompt_len"].tolist(), req["gen_len"].tolist()
    rb = req.get("router_bias")
    router_bias = None if rb is None else rb.cuda().contiguous()

    def bind():
        tokens.copy_(tokens0)
        eng.set_batch(tokens, P, G, plant_id, plant_bias, router_bias)

    def one_run():
        bind()
        return eng.run_to_completion()

    def accounting():
        """The last run's decode accounting summed over the batch."""
        ds = eng.view()["decode_stats"].cpu().sum(dim=0).tolist()
        hist = {k: int(n) for k, n in enumerate(ds[4:69]) if n}
        return {"threshold_commits": int(ds[0]), "credit_commits": int(ds[1]),
                "fallback_commits": int(ds[2]), "idle_steps": int(ds[3]),
                "commits_per_step_hist": hist}

    for i in range(warmup):
        s = one_run()
        log(f"[bench] warmup {i}: {s}")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    runs = []
    for i in range(steps):
        runs.append(one_run())
        log(f"[bench] step {i}: {runs[-1]}")
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    committed = sum(r["committed"] for r in runs)
    value = committed / elapsed
    acct = accounting()

    # denoise-step latency over every step of one more run: each graph replay
    # (unroll steps) event-timed on the library's stream (torch's current
    # stream), block refreshes outside the timed replays
    st = torch.cuda.current_stream()
    bind()
    need, lat = [True] * wc.batch, []
    while True:
        if any(need):
            eng.refresh_kv(need)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        if unroll > 0:
            eng.step_graph(unroll)
        else:
            eng.denoise_step()
            eng.commit()
        e1.record(st)
        need, unfinished = eng.advance_blocks()    # waits for the stream
        lat.append(e0.elapsed_time(e1) / max(unroll, 1))
        if unfinished == 0:
            break
    lat.sort()
    step_ms = lat[len(lat) // 2]
    step_p90_ms = lat[int(0.9 * (len(lat) - 1))]

    eng.close()
    return {"value": value, "elapsed": elapsed / steps, "step_ms": step_ms,
            "step_p90_ms": step_p90_ms, "replays": len(lat), "runs": runs,
            "committed": committed, "accounting": acct}


def calibrated(wc):
    """The supplementary planting reading: bias b' = b + ln(V - 1), so that a
    planted position's confidence is about e^b / (e^b + 1) (0.9997 at b = 8)
    whatever the vocabulary size, and the threshold gate fires."""
    import math
    return wc.with_(plant_bias=wc.plant_bias + math.log(wc.model.vocab - 1))


def supplementary_leg(name, w, unroll):
    """One warm-up and one timed generation of a workload under calibrated
    planting, with its decode accounting."""
    import synth
    wc = calibrated(synth.preset(name))
    r = run_workload(wc, w, synth.make_requests(wc), unroll, 1, 1)
    return {"workload": name, "planting": f"calibrated: bias {wc.plant_bias:.3f} = "
            f"{synth.preset(name).plant_bias:g} + ln(V-1)", "batch": wc.batch,
            "hierarchical": bool(wc.decode.hierarchical), "value": round(r["value"], 3),
            "unit": "tokens/s", "ms_per_run": round(r["elapsed"] * 1e3, 1),
            "step_latency_ms": round(r["step_ms"], 3), "steps_per_run": r["runs"][0]["steps"],
            "refreshes_per_run": r["runs"][0]["refreshes"],
            "refresh_ms_per_run": round(r["runs"][0]["refresh_ms"], 1), **r["accounting"]}


def run_queue_workload(wc, w, n_requests, unroll, budget=None):
    """Continuous batching: n_requests of the workload's request mix through
    its wc.batch slots (a finished slot takes the next queued request); with a
    budget (rows per step) the deficit scheduler admits the refreshes.  All
    requests arrive at the start, so a request's latency is its finish time."""
    import torch
    import synth
    from diffusion_vicinity_kv_amd.engine import Engine
    req = synth.make_requests(wc.with_(batch=n_requests))
    max_len = req["tokens"].shape[1]
    S = wc.batch
    eng = Engine(wc.model, wc.decode, w, S, max_len, graph_unroll=unroll)
    tokens = req["tokens"][:S].cuda().contiguous()
    plant_id = req["plant_id"][:S].cuda().contiguous()
    plant_bias = req["plant_bias"][:S].cuda().contiguous()
    P, G = req["prompt_len"].tolist(), req["gen_len"].tolist()
    eng.set_batch(tokens, P[:S], G[:S], plant_id, plant_bias)
    queue = [{"tokens": req["tokens"][i].cuda(), "prompt_len": P[i], "gen_len": G[i],
              "plant_id": req["plant_id"][i].cuda(), "plant_bias": float(req["plant_bias"][i])}
             for i in range(S, n_requests)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    res = eng.run_queue(queue, token_budget=budget)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    lat = sorted(t - t0 for t in res["finish_time"].values())
    rnd = sorted(res["round_s"])
    eng.close()
    committed = sum(G)        # every response position is committed (no end-of-sequence id)
    return {"requests": n_requests, "slots": S, "value": round(committed / elapsed, 3),
            "unit": "tokens/s", "wall_s": round(elapsed, 3), "steps": res["steps"],
            "refreshes": res["refreshes"], "token_budget_per_step": budget,
            "mean_latency_s": round(sum(lat) / len(lat), 3),
            "p90_latency_s": round(lat[int(0.9 * (len(lat) - 1))], 3),
            # a round is graph_unroll steps plus the refreshes admitted before
            # them: the longest rounds are the decode stalls refreshes cause
            "rounds": len(rnd), "median_round_ms": round(1e3 * rnd[len(rnd) // 2], 2),
            "max_round_ms": round(1e3 * rnd[-1], 2)}


def gemm_shapes(shapes, reps=32):
    """Projection kernel timing at the given (M, N, K) shapes: dinfer_linear
    on random fp32 activations and enough packed bf16 weight matrices per
    shape to span 1 GiB (rotated, so weights stream from HBM rather than the
    256 MB last-level cache), `reps` launches captured in a
    graph and replayed twice between events; per shape the average launch
    time, algorithmic TFLOP/s (2 M N K) and its fraction of the bf16 peak."""
    import torch
    from diffusion_vicinity_kv_amd import binding as B
    lib = B.load()
    out = []
    for M, N, K in shapes:
        g = torch.Generator(device="cuda").manual_seed(M + N + K)
        A = torch.randn(M, K, device="cuda", generator=g)
        n_weights = min(reps, max(4, -(-(1 << 30) // (N * K * 2))))
        Ws = [B.pack_linear((torch.randn(N, K, device="cuda", generator=g) * 0.02)
                            .to(torch.bfloat16)) for _ in range(n_weights)]
        dst = torch.empty(lib.dinfer_linear_out_elems(M, N, K, B.BF16), device="cuda")
        S = B.linear(A, Ws[0], dst)
        torch.cuda.synchronize()
        cap = torch.cuda.Stream()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr, stream=cap):
            for i in range(reps):
                B.linear(A, Ws[i % n_weights], dst)
        gr.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        gr.replay()
        gr.replay()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / (2 * reps)
        tf = 2.0 * M * N * K / us / 1e6
        out.append({"M": M, "N": N, "K": K, "splits": S, "us": round(us, 2),
                    "tflops": round(tf, 1), "frac_bf16_peak": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
                    "weight_gbs": round(N * K * 2 / us / 1e3, 1)})
        del gr, Ws, A, dst
        torch.cuda.empty_cache()
    return out


def trace_summary(csv_path, top=40):
    """Per (kernel, grid size) totals of a rocprofv3 kernel-trace CSV, as a
    markdown table: the same kernel runs with different grids in a block
    refresh (all prompt rows) and in a denoise step (the window rows), and
    this is what tells them apart."""
    import csv
    import collections
    agg = collections.defaultdict(lambda: [0, 0.0])
    def dims(r, stem):
        xyz = [r.get(f"{stem}_{a}") for a in "XYZ"]
        if all(xyz):
            return "x".join(xyz)
        return r.get(stem, "")

    for r in csv.DictReader(open(csv_path)):
        name = r["Kernel_Name"].replace("(anonymous namespace)::", "")
        if name.startswith("void "):
            name = name[5:]
        us = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        key = (name.split("(")[0][:110], dims(r, "Grid_Size"), dims(r, "Workgroup_Size"))
        agg[key][0] += 1
        agg[key][1] += us
    total = sum(v[1] for v in agg.values())
    lines = ["| kernel | grid (work-items x, y, z) | workgroup | calls | total ms | avg us | % |",
             "|---|---:|---:|---:|---:|---:|---:|"]
    for (name, grid, wg), (n, us) in sorted(agg.items(), key=lambda kv: -kv[1][1])[:top]:
        lines.append(f"| `{name}` | {grid} | {wg} | {n} | {us / 1e3:.2f} | {us / n:.2f} | "
                     f"{100 * us / total:.1f} |")
    lines.append(f"\nTotal kernel time {total / 1e3:.1f} ms over {sum(v[0] for v in agg.values())} "
                 "dispatches.")
    return "\n".join(lines)


def traffic_record(k_fetch, k_write, c_fetch, c_write, commands):
    """The dominant kernel's HBM traffic per launch from two rocprofv3 --pmc
    runs of --kernel-only (FETCH_SIZE, WRITE_SIZE; KiB per dispatch), each
    scaled by what the same counter reads for the 1 GiB copy of --calib-copy,
    keyed on the hash of the kernel's sources."""
    import csv

    def mean(path, counter, match):
        vals = [float(r["Counter_Value"]) for r in csv.DictReader(open(path))
                if r["Counter_Name"] == counter and match in r["Kernel_Name"]]
        if not vals:
            raise SystemExit(f"no {counter} rows for {match} in {path}")
        return sum(vals) / len(vals), len(vals)

    kf, n = mean(k_fetch, "FETCH_SIZE", "gemm_skinny_kernel")
    kw, _ = mean(k_write, "WRITE_SIZE", "gemm_skinny_kernel")
    cf, _ = mean(c_fetch, "FETCH_SIZE", "copyBuffer")
    cw, _ = mean(c_write, "WRITE_SIZE", "copyBuffer")
    copy_bytes = 1 << 30
    ff, wf = copy_bytes / 1024 / cf, copy_bytes / 1024 / cw
    return {"kernel": f"{KERNEL} (QKV and gate|up projections, 64 rows)",
            "workload": "dense8b_b1 window: 64 rows x d 4096, N = 12288 (QKV) and 24576 (gate|up), "
                        "alternating; weights packed k-step-major",
            "source_hash": source_hash(),
            "source_files": [f"diffusion_vicinity_kv_amd/csrc/{f}"
                             for f in ("gemm.hip", "gemm_split.h", "common.h")],
            "dispatches": n, "fetch_kib_per_dispatch": round(kf, 1),
            "write_kib_per_dispatch": round(kw, 1),
            "calibration": {"copy_bytes": copy_bytes, "copy_kernel": "__amd_rocclr_copyBuffer",
                            "copy_fetch_kib": cf, "copy_write_kib": cw,
                            "fetch_factor": ff, "write_factor": wf},
            "bytes_per_launch": int(round((kf * ff + kw * wf) * 1024)),
            "commands": commands}


def step_only(wc, w, req, n_steps):
    """One block refresh and n_steps eager denoise+commit steps of the
    workload (no graph), for counter runs: the difference of two such runs
    with different n_steps is the per-step traffic of the step's kernels."""
    import torch
    from diffusion_vicinity_kv_amd.engine import Engine
    max_len = req["tokens"].shape[1]
    eng = Engine(wc.model, wc.decode, w, wc.batch, max_len, graph_unroll=0)
    tokens = req["tokens"].cuda().contiguous()
    rb = req.get("router_bias")
    eng.set_batch(tokens, req["prompt_len"].tolist(), req["gen_len"].tolist(),
                  req["plant_id"].cuda().contiguous(), req["plant_bias"].cuda().contiguous(),
                  None if rb is None else rb.cuda().contiguous())
    eng.refresh_kv()
    for _ in range(n_steps):
        eng.denoise_step()
        eng.commit()
    torch.cuda.synchronize()
    eng.close()


def counter_totals(paths):
    """Sum of each counter over every dispatch of rocprofv3 counter CSVs
    (KiB for FETCH_SIZE / WRITE_SIZE), with the dispatch count."""
    import csv
    tot, n = {}, {}
    for path in paths:
        for r in csv.DictReader(open(path)):
            c = r["Counter_Name"]
            tot[c] = tot.get(c, 0.0) + float(r["Counter_Value"])
            n[c] = n.get(c, 0) + 1
    return {c: {"sum": tot[c], "dispatches": n[c]} for c in tot}


def run_expert_sweep(wc, w, slot_list, intervals, blocks, unroll):
    """TIDE-style expert cache on the MoE workload: the first `blocks` blocks
    of its request with `slots` experts per layer in HBM and the rest read
    from a pinned host store, for each (slots, interval); beside the run with
    every expert in HBM.  Reports tokens/s, hit rates, bytes moved, and
    whether the tokens equal the all-in-HBM run's (they must: the cache is
    lossless)."""
    import torch
    import synth
    from diffusion_vicinity_kv_amd.engine import Engine
    wcs = wc.with_(gen_len=blocks * wc.decode.block_len)
    req = synth.make_requests(wcs)
    max_len = req["tokens"].shape[1]
    P, G = req["prompt_len"].tolist(), req["gen_len"].tolist()
    out = []

    def one(slots, interval):
        eng = Engine(wcs.model, wcs.decode, w, wcs.batch, max_len, graph_unroll=unroll)
        if slots is not None:
            eng.expert_offload(slots, interval)
        tokens = req["tokens"].cuda().contiguous()
        args = (P, G, req["plant_id"].cuda().contiguous(), req["plant_bias"].cuda().contiguous(),
                req["router_bias"].cuda().contiguous())
        eng.set_batch(tokens, *args)                 # warm-up (graph capture)
        eng.run_to_completion()
        if slots is not None:
            eng.expert_report(reset=True)
        tokens.copy_(req["tokens"].cuda())
        eng.set_batch(tokens, *args)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        st = eng.run_to_completion()
        torch.cuda.synchronize()
        el = time.perf_counter() - t0
        rep = eng.expert_report() if slots is not None else None
        toks = tokens.clone()
        eng.close()
        del eng
        torch.cuda.empty_cache()
        return el, st, rep, toks

    el0, st0, _, tok0 = one(None, 0)
    out.append({"slots": wc.model.n_experts, "interval": None, "store": "all experts in HBM",
                "value": round(st0["committed"] / el0, 3), "unit": "tokens/s",
                "steps": st0["steps"], "refreshes": st0["refreshes"]})
    log(f"[bench] expert sweep: all in HBM {out[-1]}")
    for slots in slot_list:
        for interval in intervals:
            el, st, rep, toks = one(slots, interval)
            rows = rep["row_hits"] + rep["row_misses"]
            ex = rep["expert_hits"] + rep["expert_misses"]
            out.append({"slots": slots, "interval": interval, "value": round(st["committed"] / el, 3),
                        "unit": "tokens/s", "steps": st["steps"], "refreshes": st["refreshes"],
                        "row_hit_rate": round(rep["row_hits"] / max(rows, 1), 4),
                        "expert_hit_rate": round(rep["expert_hits"] / max(ex, 1), 4),
                        "placements": rep["placements"], "bytes_placed": rep["bytes_placed"],
                        "bytes_host_read": rep["bytes_host_read"],
                        "tokens_equal_all_in_hbm": bool(torch.equal(toks, tok0))})
            log(f"[bench] expert sweep: {out[-1]}")
    return {"workload": wc.name, "blocks": blocks, "gen_len": wcs.gen_len, "points": out}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="dense8b_b1")
    ap.add_argument("--unroll", type=int, default=8)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-batch16", action="store_true",
                    help="skip the batch-16 companion figure of the dense 8B workload")
    ap.add_argument("--queue", type=int, default=0,
                    help="also run this many batch-16-mix requests through the 16 slots with "
                         "continuous batching (dense 8B workload only)")
    ap.add_argument("--budget", default="",
                    help="with --queue: also run the queue with the deficit token-budget "
                         "scheduler at these rows per step (comma-separated)")
    ap.add_argument("--no-supplementary", action="store_true",
                    help="skip the supplementary calibrated-planting runs of the dense 8B "
                         "workloads (batch 1 and the batch-16 mix)")
    ap.add_argument("--supplementary-long", action="store_true",
                    help="also run the long-context workload (batch 4, 8K prompt, hierarchical) "
                         "under calibrated planting (about a minute)")
    ap.add_argument("--expert-sweep", default="",
                    help="MoE workload: comma-separated expert slots per layer for the HBM "
                         "expert cache over a pinned host store (TIDE-style placement)")
    ap.add_argument("--expert-interval", default="0",
                    help="with --expert-sweep: comma-separated placement intervals in steps "
                         "(0: block starts only)")
    ap.add_argument("--expert-blocks", type=int, default=2,
                    help="with --expert-sweep: blocks of the request to run")
    ap.add_argument("--gemm-shapes", default="",
                    help="only time the projection kernels at these MxNxK shapes "
                         "(comma-separated, e.g. 1024x12288x4096,64x12288x4096)")
    ap.add_argument("--kernel-only", action="store_true",
                    help="only the dominant-kernel timing loop (for counter runs)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="one plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--trace-summary", default="",
                    help="print per-(kernel, grid) totals of this rocprofv3 kernel-trace CSV "
                         "as a markdown table (no GPU work)")
    ap.add_argument("--traffic-record", nargs=4, default=None,
                    metavar=("KERNEL_FETCH_CSV", "KERNEL_WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                    help="write the dominant kernel's HBM traffic record from the counter CSVs of "
                         "--kernel-only and --calib-copy runs (no GPU work)")
    ap.add_argument("--traffic-out", default=TRAFFIC_FILE)
    ap.add_argument("--step-only", type=int, default=0,
                    help="one block refresh and this many eager denoise+commit steps of the "
                         "workload, nothing else (counter runs)")
    ap.add_argument("--counter-totals", nargs="+", default=None,
                    help="print each counter's sum over every dispatch of these rocprofv3 counter "
                         "CSVs (no GPU work)")
    args = ap.parse_args()
    if args.counter_totals:
        print(json.dumps(counter_totals(args.counter_totals)))
        return
    if args.trace_summary:
        print(trace_summary(args.trace_summary))
        return
    if args.traffic_record:
        cmds = [f"rocprofv3 --pmc {c} --output-format csv -d <dir> -o run -- python3 -u bench.py {m}"
                for m in ("--kernel-only", "--calib-copy") for c in ("FETCH_SIZE", "WRITE_SIZE")]
        rec = traffic_record(*args.traffic_record, cmds)
        with open(args.traffic_out, "w") as f:
            json.dump(rec, f, indent=1)
        print(json.dumps({k: rec[k] for k in ("bytes_per_launch", "dispatches", "source_hash")}))
        return
    if args.gpus != 1:
        print(f"bench.py: this library runs on one GPU; --gpus {args.gpus} is not supported "
              "(the multi-GPU layout is described in the design notes, not built)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    if args.gemm_shapes:
        shapes = [tuple(int(x) for x in t.split("x")) for t in args.gemm_shapes.split(",")]
        for r in gemm_shapes(shapes):
            print(json.dumps(r), flush=True)
        return
    wc = synth.preset(args.workload)
    m = wc.model

    if args.calib_copy:
        n = 1 << 28                                   # 1 GiB of fp32
        src = torch.ones(n, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"calib copy: {n * 4} bytes read, {n * 4} bytes written")
        return

    log(f"[bench] drawing {m.n_layers}-layer weights on the GPU ({args.workload})")
    w = synth.make_weights(m, wc.seed, device="cuda")
    req = synth.make_requests(wc)
    torch.cuda.synchronize()

    if args.step_only:
        log(f"[bench] step-only: refresh + {args.step_only} eager steps")
        step_only(wc, w, req, args.step_only)
        log("[bench] step-only done")
        return

    if args.kernel_only:
        avg_ms, avg_bytes, _, rows = dominant_kernel_timing(wc, w, iters=64)
        log(f"[bench] kernel-only: {avg_ms * 1e3:.1f} us/launch, {avg_bytes / avg_ms / 1e6:.0f} GB/s")
        return

    if args.expert_sweep:
        if not m.is_moe:
            print("bench.py: --expert-sweep needs an MoE workload", file=sys.stderr)
            sys.exit(2)
        sweep = run_expert_sweep(wc, w, [int(x) for x in args.expert_sweep.split(",")],
                                 [int(x) for x in args.expert_interval.split(",")],
                                 args.expert_blocks, args.unroll)
        print(json.dumps({"expert_cache_sweep": sweep}), flush=True)
        return

    res = run_workload(wc, w, req, args.unroll, args.warmup, args.steps)
    value, elapsed, step_ms = res["value"], res["elapsed"], res["step_ms"]
    runs = res["runs"]
    committed = res["committed"]
    b16 = None
    if args.workload == "dense8b_b1" and not args.no_batch16:
        # the same weights, batch 16 (step-level batching of ragged requests)
        wc16 = synth.preset("dense8b_b16")
        log("[bench] batch 16 companion run (dense8b_b16 requests, same weights)")
        r16 = run_workload(wc16, w, synth.make_requests(wc16), args.unroll, 1, 1)
        b16 = {"workload": "dense8b_b16", "value": round(r16["value"], 3), "unit": "tokens/s",
               "batch": wc16.batch, "ms_per_run": round(r16["elapsed"] * 1e3, 1),
               "step_latency_ms": round(r16["step_ms"], 3),
               "step_latency_p90_ms": round(r16["step_p90_ms"], 3),
               "steps_per_run": r16["runs"][0]["steps"],
               "refresh_ms_per_run": round(r16["runs"][0]["refresh_ms"], 1),
               **r16["accounting"]}
        torch.cuda.empty_cache()
    supp = None
    if args.workload == "dense8b_b1" and not args.no_supplementary:
        supp = []
        names = ["dense8b_b1", "dense8b_b16"] + (["dense8b_long_b4"] if args.supplementary_long else [])
        for name in names:
            log(f"[bench] supplementary: {name} under calibrated planting")
            supp.append(supplementary_leg(name, w, args.unroll))
            log(f"[bench]   {supp[-1]}")
            torch.cuda.empty_cache()
    cb = None
    if args.workload == "dense8b_b1" and args.queue > 0:
        wc16 = synth.preset("dense8b_b16")
        log(f"[bench] continuous batching: {args.queue} requests through {wc16.batch} slots")
        cb = run_queue_workload(wc16, w, args.queue, args.unroll)
        torch.cuda.empty_cache()
        budgets = [int(b) for b in args.budget.split(",") if b.strip()]
        if budgets:
            cb = {"fifo": cb, "deficit": []}
            for b in budgets:
                log(f"[bench] continuous batching, deficit budget {b} rows/step")
                cb["deficit"].append(run_queue_workload(wc16, w, args.queue, args.unroll, b))
                torch.cuda.empty_cache()

    avg_ms, avg_bytes, avg_flops, rows = dominant_kernel_timing(wc, w)
    if rows <= 128:
        # skinny path: a weight stream
        achieved = avg_bytes / (avg_ms * 1e-3) / 1e9
        traffic = None
        if args.workload == "dense8b_b1" and os.path.exists(TRAFFIC_FILE):
            t = json.load(open(TRAFFIC_FILE))
            if t.get("source_hash") == source_hash():
                traffic = t.get("bytes_per_launch")
        roofline = {"bound": "hbm", "kernel": KERNEL, "achieved": round(achieved, 1),
                    "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                    "traffic": traffic, "avg_launch_us": round(avg_ms * 1e3, 2),
                    "bytes_per_launch": int(avg_bytes)}
    else:
        # fat path (many window rows): a dense contraction, priced against bf16 MFMA
        tflops = avg_flops / (avg_ms * 1e-3) / 1e12
        roofline = {"bound": "mfma", "kernel": "gemm_fat_kernel<bf16>", "achieved": round(tflops, 1),
                    "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
                    "avg_launch_us": round(avg_ms * 1e3, 2), "flops_per_launch": int(avg_flops)}

    steps_per_run = sum(r["steps"] for r in runs) / len(runs)
    refreshes_per_run = sum(r["refreshes"] for r in runs) / len(runs)
    committed_per_run = committed / len(runs)
    # weights once + KV read once per layer + window KV write, per step.  MoE:
    # every expert counts (a 64+-row window routes rows to nearly all of them)
    d, V, nl = m.d_model, m.vocab, m.n_layers
    if m.is_moe:
        ffn_w = m.n_experts * (3 * d * m.expert_ffn + d) + 3 * d * m.shared_ffn
    else:
        ffn_w = 3 * d * m.ffn_dim
    weight_bytes = (nl * (3 * d * d + d * d + ffn_w) + V * d) * 2
    kv_bytes = nl * wc.batch * 2 * (wc.max_len * d * 2 + rows // wc.batch * d * 2)
    step_bytes = weight_bytes + kv_bytes

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (bounded oracle sample)")
        cpu = cpu_baseline(wc, int(round(refreshes_per_run)), int(round(steps_per_run)),
                           committed_per_run)

    out = {
        "metric": f"committed tokens/s (batch {wc.batch}, {MODEL_NAMES.get(args.workload, args.workload)}, bf16)",
        "value": round(value, 3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed * 1e3, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": f"synthetic: N(0,0.02) random-init weights of the "
                f"{MODEL_NAMES.get(args.workload, args.workload)} shape, random prompt ids, "
                "seeded planting" + (", seeded per-block router preference bias" if m.is_moe else ""),
        "config": {"workload": args.workload, "batch": wc.batch, "prompt_len": wc.prompt_len[0],
                   "gen_len": wc.gen_len, "block_len": wc.decode.block_len,
                   "vicinity_w": wc.decode.vicinity_w, "layers": nl, "d_model": d,
                   "vocab": V, "graph_unroll": args.unroll},
        "step_latency_ms": round(step_ms, 4),
        "step_latency_p90_ms": round(res["step_p90_ms"], 4), "latency_replays": res["replays"],
        "steps_per_run": steps_per_run,
        "refreshes_per_run": refreshes_per_run,
        "refresh_ms_per_run": round(sum(r["refresh_ms"] for r in runs) / len(runs), 3),
        "step_roofline": {"bound": "hbm", "bytes": step_bytes,
                          "achieved": round(step_bytes / (step_ms * 1e-3) / 1e9, 1),
                          "peak": HBM_PEAK_GBS, "unit": "GB/s",
                          "frac": round(step_bytes / (step_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
        "decode_accounting": res["accounting"],
        "roofline": roofline,
        "batch16": b16,
        "supplementary_calibrated_planting": supp,
        "continuous_batching": cb,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
