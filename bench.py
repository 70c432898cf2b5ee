"""Benchmark of one compensated block-sparse decode step on one MI355X.

Workload: a Llama-3.1-8B-shaped attention layer decoding with a 128K-token
context and a 512-token budget (B=1, Hq=32, Hkv=8, d=128, 16-token blocks,
r=4, bf16), synthetic seeded inputs.  A step is one ckv_decode_step call
(score every block, select the top-k, attend exactly to the selected blocks
with Mean compensation of the rest).  Steps rotate over `--layers` copies of
the layer (distinct buffers), so each step reads its summaries from HBM, not
from the last-level cache, as a model's layer loop would.

Prints one JSON line.  `value` is microseconds per layer decode step (lower
is better); the effective HBM rate over the algorithmic bytes is reported
beside it, with the roofline of the step's kernels, full dense decode on the
same GPU, and the CPU oracle timed on the host.
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "µs per layer decode step & effective HBM GB/s (% peak) at 128K ctx, 512 budget"
HBM_PEAK_GBPS = 8000.0
KERNEL_SOURCES = ("kernels.hip", "fused.hip", "step_common.hpp", "device.hpp", "internal.hpp")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "compensated_kv_selection_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(M: int, Hkv: int, d: int, r: int, k: int, bs: int, kv_bytes: int) -> dict:
    """Bytes a decode step must move: every block's summary (mean key, mean
    value, r grouped variances per KV head, one count per block) plus the
    selected blocks' keys and values."""
    summary = M * Hkv * (2 * d * kv_bytes + 4 * r) + 4 * M
    selected = Hkv * k * bs * d * 2 * kv_bytes
    return {"summary": summary, "selected_kv": selected, "total": summary + selected}


def read_traffic(kernel_tag: str, src_hash: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"{kernel_tag}_traffic.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"kernel_source_hash:\s*([0-9a-f]+)", text)
    m_bytes = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_hash or not m_bytes or m_hash.group(1) != src_hash:
        return None
    return float(m_bytes.group(1))


def rocprof_summary(directory: str) -> str:
    """Per-kernel table of the rocprofv3 CSV output (-f csv) under a directory:
    dispatch counts and durations from *kernel_stats.csv, and the mean per
    dispatch of each counter in *counter_collection.csv."""
    import csv
    import glob
    from collections import defaultdict
    lines = []
    for path in sorted(glob.glob(os.path.join(directory, "**", "*kernel_stats.csv"), recursive=True)):
        lines.append("| kernel | calls | average (us) | min (us) | max (us) | share of GPU time |")
        lines.append("|---|---|---|---|---|---|")
        with open(path) as f:
            for row in csv.DictReader(f):
                lines.append(f"| {row['Name'][:90]} | {row['Calls']} | {float(row['AverageNs']) / 1e3:.3f} | "
                             f"{float(row['MinNs']) / 1e3:.3f} | {float(row['MaxNs']) / 1e3:.3f} | "
                             f"{float(row['Percentage']):.2f}% |")
    for path in sorted(glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True)):
        acc = defaultdict(lambda: [0.0, 0])
        with open(path) as f:
            for row in csv.DictReader(f):
                key = (row["Kernel_Name"][:90], row["Counter_Name"])
                acc[key][0] += float(row["Counter_Value"])
                acc[key][1] += 1
        lines.append("| kernel | counter | dispatches | mean per dispatch |")
        lines.append("|---|---|---|---|")
        for (name, counter), (tot, cnt) in sorted(acc.items()):
            lines.append(f"| {name} | {counter} | {cnt} | {tot / cnt:.1f} |")
    return "\n".join(lines) if lines else f"no rocprofv3 CSV files under {directory}"


def graph_time_us(torch, fn, n: int) -> float:
    """Mean time of fn(i), i = 0..n-1, captured in one HIP graph and replayed
    (events on the current stream around the timed replay)."""
    for i in range(3):
        fn(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n):
            fn(i)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / n


# ---- CPU baseline: the oracle on the host's cores ---------------------------

_ORACLE_JOB = {}


def _oracle_one_kv_head(g: int) -> float:
    """One decode step of KV head g (and its query heads) in the oracle; the
    heads are independent, so the KV heads of a step can run side by side."""
    from oracle import compkv_oracle as O
    j = _ORACLE_JOB
    G = j["G"]
    sub = O.Summaries(j["summ"].mean_k[:, g:g + 1], j["summ"].mean_v[:, g:g + 1], j["summ"].gvar[:, g:g + 1],
                      j["summ"].count)
    res = O.decode_step(j["q"][g * G:(g + 1) * G], j["k"][:, g:g + 1], j["v"][:, g:g + 1], sub,
                        budget_tokens=j["budget"], block_size=j["bs"], r=j["r"])
    return float(res.out.sum())


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_oracle_baseline(w, runs: int = 5) -> dict:
    """The CPU oracle's decode step on the same layer, summaries prebuilt:
    the median of `runs` steps on one core (one process, one BLAS thread),
    and the median of `runs` steps on the host's cores (one process per KV
    head, up to the cores this process may use, each with one BLAS thread).
    Runs before anything touches the GPU (the worker processes are forked)."""
    import multiprocessing as mp
    import statistics
    import numpy as np
    from threadpoolctl import threadpool_limits
    from oracle import compkv_oracle as O
    q, k, v = O.sequence_arrays(w.q[0], w.k_tokens[0], w.v_tokens[0], w.dtype)
    t0 = time.perf_counter()
    summ = O.build_summaries(k, v, w.block_size, w.r_groups, w.dtype)
    build_s = time.perf_counter() - t0
    _ORACLE_JOB.update(q=q, k=k, v=v, summ=summ, G=w.num_q_heads // w.num_kv_heads, budget=w.budget_tokens,
                       bs=w.block_size, r=w.r_groups)
    H = w.num_kv_heads
    one = []
    with threadpool_limits(limits=1):
        for _ in range(runs):
            t0 = time.perf_counter()
            O.decode_step(q, k, v, summ, budget_tokens=w.budget_tokens, block_size=w.block_size, r=w.r_groups)
            one.append(time.perf_counter() - t0)
    avail = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    workers = max(1, min(H, avail, 16))
    many = []
    with threadpool_limits(limits=1):
        with mp.get_context("fork").Pool(workers) as pool:
            pool.map(_oracle_one_kv_head, range(H))  # warm the workers
            for _ in range(runs):
                t0 = time.perf_counter()
                pool.map(_oracle_one_kv_head, range(H))
                many.append(time.perf_counter() - t0)
    _ORACLE_JOB.clear()
    med_one, med_many = statistics.median(one), statistics.median(many)
    return {"value": round(med_many * 1e6, 1), "unit": "us/step", "cores": workers, "kind": "oracle",
            "sample": (f"median of {runs} float64 numpy oracle decode steps of the same {int(w.seq_lens[0])}-token "
                       f"layer, summaries prebuilt ({build_s:.1f} s), {workers} processes of one BLAS thread "
                       f"each taking a KV head; host CPU"),
            "one_core_us": round(med_one * 1e6, 1), "one_core_runs_us": [round(x * 1e6) for x in one],
            "all_cores_runs_us": [round(x * 1e6) for x in many], "nproc": os.cpu_count(),
            "usable_cpus": avail, "cpu_model": cpu_model()}


# ---- GPU timing --------------------------------------------------------------


GRAPH_MIN_STEPS = 20  # steps per captured graph, so that its launch gap is spread thin


def replays_for(steps: int, want: int = 10, min_per: int = GRAPH_MIN_STEPS) -> int:
    """The largest replay count <= want that divides `steps` and leaves at
    least min(min_per, steps) steps per replay."""
    for r in range(min(want, steps), 0, -1):
        if steps % r == 0 and steps // r >= min(min_per, steps):
            return r
    return 1


def timed_replays(torch, fn, steps: int, replays: int, extra: int = 0):
    """Capture steps // replays consecutive steps fn(0), fn(1), ... into one
    HIP graph, replay it `replays` times back to back with an event between
    replays (on the capturing stream), and return (us per step over all
    `steps`, per-replay us per step).  With `extra`, the per-replay figures
    come from that many further replays of the same graph after the timed
    ones instead (for a distribution when the timed steps fill few replays);
    they do not enter the first figure."""
    per = steps // replays
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(per):
            fn(i)
    g.replay()  # untimed: the first replay uploads the graph
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(replays + 1)]
    ev[0].record()
    for r in range(replays):
        g.replay()
        ev[r + 1].record()
    torch.cuda.synchronize()
    samples = [ev[r].elapsed_time(ev[r + 1]) * 1e3 / per for r in range(replays)]
    total = ev[0].elapsed_time(ev[replays]) * 1e3 / (per * replays)
    if extra > 0:
        ex = [torch.cuda.Event(enable_timing=True) for _ in range(extra + 1)]
        ex[0].record()
        for r in range(extra):
            g.replay()
            ex[r + 1].record()
        torch.cuda.synchronize()
        samples = [ex[r].elapsed_time(ex[r + 1]) * 1e3 / per for r in range(extra)]
    return total, samples


def distribution(samples) -> dict:
    import numpy as np
    a = np.asarray(samples, dtype=np.float64)
    return {"median": round(float(np.median(a)), 3), "p10": round(float(np.percentile(a, 10)), 3),
            "p90": round(float(np.percentile(a, 90)), 3), "samples": len(a)}


def sweep(args, dev0) -> int:
    """Step latency over context lengths and budgets: 32K, 64K, 128K tokens x
    512, 1024, 2048-token budgets (the CompKV review's length/budget grid is
    not printed; this is its plainest reading), Llama-3.1-8B layer shape,
    synthetic inputs.  Steps rotate over enough layer copies that their
    summaries exceed the last-level cache."""
    import torch
    from compensated_kv_selection_amd import compkv as C
    from compensated_kv_selection_amd import workloads as W
    from compensated_kv_selection_amd.tensors import to_device
    for L in (32768, 65536, 131072):
        w = W.make_decode_inputs(name=f"sweep_{L}", seq_lens=[L], num_q_heads=32, num_kv_heads=8, head_dim=128,
                                 block_size=16, r_groups=4, budget_tokens=512, dtype="bf16", n_needles=16,
                                 n_outliers=4, seed=args.seed)
        base = to_device(w, dev0)
        dims = base.dims
        M = -(-L // 16)
        summary_bytes = M * 8 * (2 * 128 * 2 + 4 * 4) + 4 * M
        n_layers = max(2, -(-(512 << 20) // summary_bytes))
        layers = []
        for li in range(n_layers):
            kc = base.k_cache if li == 0 else base.k_cache.clone()
            vc = base.v_cache if li == 0 else base.v_cache.clone()
            summ = C.allocate_summaries(dims, dev0)
            C.build_summaries(dims, kc, vc, base.block_table, base.seq_lens, summ)
            layers.append((kc, vc, summ))
        torch.cuda.synchronize()
        out = torch.empty((1, 32, 128), dtype=torch.float32, device=dev0)
        lse = torch.empty((1, 32), dtype=torch.float32, device=dev0)
        dws = C.allocate_workspace(C.dense_workspace_bytes(dims), dev0)

        def dstep(i):
            kc, vc, _ = layers[i % n_layers]
            C.dense_decode_attention(dims, base.q, kc, vc, base.block_table, base.seq_lens, dws, out=out, lse=lse)

        dense_us = graph_time_us(torch, dstep, 32)
        for budget in (512, 1024, 2048):
            ws = C.allocate_workspace(C.workspace_bytes(dims, budget), dev0)
            kk = min(M, budget // 16)
            sel = torch.empty((1, 8, max(1, kk)), dtype=torch.int32, device=dev0)
            nsel = torch.empty((1, 8), dtype=torch.int32, device=dev0)

            def step(i):
                kc, vc, summ = layers[i % n_layers]
                C.decode_step(dims, base.q, kc, vc, summ, base.block_table, base.seq_lens, budget, ws,
                              selected=sel, num_selected=nsel, out=out, lse=lse)

            us = graph_time_us(torch, step, 100)
            ab = algorithmic_bytes(M, 8, 128, 4, kk, 16, 2)
            gbps = ab["total"] / (us * 1e-6) / 1e9
            print(json.dumps({"sweep": "decode step latency", "seq_len": L, "budget_tokens": budget,
                              "us_per_step": round(us, 2), "launches": C.decode_step_launches(dims, budget),
                              "algorithmic_bytes": ab["total"], "effective_GBps": round(gbps, 1),
                              "pct_hbm_peak": round(100 * gbps / HBM_PEAK_GBPS, 2),
                              "dense_us": round(dense_us, 2), "speedup_vs_dense": round(dense_us / us, 2),
                              "layer_copies": n_layers, "data": "synthetic"}), flush=True)
        del layers
        torch.cuda.empty_cache()
    return 0


def sweep_r(args, dev0) -> int:
    """Step latency over the number of variance groups r (1, 2, 4, 8, 16,
    128 = d) at 128K context and a 512-token budget, for the CompKV score and
    for estimated-mass selection with compensation (the decoupled baseline).
    Steps rotate over layer copies whose summaries exceed the last-level
    cache; graph replay."""
    import torch
    from compensated_kv_selection_amd import compkv as C
    from compensated_kv_selection_amd import workloads as W
    from compensated_kv_selection_amd.tensors import to_device

    w = W.make_preset("llama_128k", seed=args.seed)
    base = to_device(w, dev0)
    M = -(-131072 // 16)
    out = torch.empty((1, 32, 128), dtype=torch.float32, device=dev0)
    lse = torch.empty((1, 32), dtype=torch.float32, device=dev0)
    sel = torch.empty((1, 8, 32), dtype=torch.int32, device=dev0)
    nsel = torch.empty((1, 8), dtype=torch.int32, device=dev0)
    for r in (1, 2, 4, 8, 16, 128):
        dims = dataclasses.replace(base.dims, r_groups=r)
        n_layers = 16
        layers = []
        for li in range(n_layers):
            kc = base.k_cache if li == 0 else base.k_cache.clone()
            vc = base.v_cache if li == 0 else base.v_cache.clone()
            summ = C.allocate_summaries(dims, dev0)
            C.build_summaries(dims, kc, vc, base.block_table, base.seq_lens, summ)
            layers.append((kc, vc, summ))
        torch.cuda.synchronize()
        ws = C.allocate_workspace(C.workspace_bytes(dims, 512), dev0)
        res = {}
        for name, mode in (("compkv", C.SCORE_COMPKV), ("mass_hat_compensated", C.SCORE_MASS)):
            def step(i, mode=mode):
                kc, vc, summ = layers[i % n_layers]
                C.decode_step(dims, base.q, kc, vc, summ, base.block_table, base.seq_lens, 512, ws, mode,
                              selected=sel, num_selected=nsel, out=out, lse=lse)
            res[name] = round(graph_time_us(torch, step, 100), 2)
        summary_bytes = M * 8 * (2 * 128 * 2 + 4 * r) + 4 * M
        print(json.dumps({"sweep": "decode step latency over r", "seq_len": 131072, "budget_tokens": 512,
                          "r_groups": r, "us_per_step": res, "algorithmic_bytes": summary_bytes + 8 * 32 * 8192,
                          "layer_copies": n_layers, "data": "synthetic"}), flush=True)
        del layers
        torch.cuda.empty_cache()
    return 0


def decode_loop_result(args, dev0, n_layers: int) -> dict:
    """Prefill plus a generation loop at 128K context (Llama-3.1-8B layer
    shape): the bulk summary build over 131072 tokens, then 64 decode steps,
    each appending one token (written into its page and the tail block's
    summary refreshed) and running the step with a 2048-token budget, in one
    ckv_decode_step_append call (with --loop-two-launch: ckv_append_tokens,
    then ckv_decode_step).  The steps of all layer copies are captured into
    one HIP graph and replayed; a step visits every layer copy in turn, as a
    model's layer loop would, so summaries come from HBM."""
    import numpy as np
    import torch
    from compensated_kv_selection_amd import compkv as C
    from compensated_kv_selection_amd import workloads as W
    from compensated_kv_selection_amd.decode_loop import DecodeLoop
    from compensated_kv_selection_amd.tensors import to_device

    n_steps = 64
    w = W.make_preset("prefill_128k_loop", seed=args.seed)
    steps = W.make_append_steps(w, n_steps, seed=args.seed + 1)
    kc, vc = w.paged_cache()
    base = to_device(w, dev0, k_cache=kc, v_cache=vc)
    del kc, vc
    dims = base.dims
    n_layers = max(1, n_layers)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    loops, build_ms = [], []
    for li in range(n_layers):
        dev = base if li == 0 else dataclasses.replace(
            base, k_cache=base.k_cache.clone(), v_cache=base.v_cache.clone(), q=base.q.clone(),
            seq_lens=base.seq_lens.clone())
        summ = C.allocate_summaries(dims, dev0)
        torch.cuda.synchronize()
        ev[0].record()
        C.build_summaries(dims, dev.k_cache, dev.v_cache, dev.block_table, dev.seq_lens, summ)
        ev[1].record()
        torch.cuda.synchronize()
        build_ms.append(ev[0].elapsed_time(ev[1]))
        loops.append(DecodeLoop(dev, summ, w.block_table, w.seq_lens, steps, w.dtype,
                                fused=not args.loop_two_launch))

    def run_all():
        for t in range(n_steps):
            for lp in loops:
                lp.step(t)

    run_all()  # eager pass
    torch.cuda.synchronize()
    for lp in loops:
        C.workspace_status(lp.ws)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run_all()
    g.replay()  # untimed: first replay uploads the graph
    torch.cuda.synchronize()
    ev[0].record()
    g.replay()
    ev[1].record()
    torch.cuda.synchronize()
    for lp in loops:
        C.workspace_status(lp.ws)
    us = ev[0].elapsed_time(ev[1]) * 1e3 / (n_steps * n_layers)
    M = -(-(int(w.seq_lens[0]) + n_steps) // 16)
    ab = algorithmic_bytes(M, 8, 128, 4, min(M, w.budget_tokens // 16), 16, 2)
    res = {"decode_loop": "prefill + 64 appending decode steps, graph replay",
           "seq_len_start": int(w.seq_lens[0]), "steps": n_steps,
           "budget_tokens": w.budget_tokens, "layer_copies": n_layers,
           "prefill_build_us": round(float(np.median(build_ms)) * 1e3, 1),
           "us_per_layer_step": round(us, 2),
           "step_algorithmic_bytes": ab["total"],
           "step_effective_GBps": round(ab["total"] / (us * 1e-6) / 1e9, 1),
           "per_layer_step": ("ckv_append_tokens (new key and value into their page, "
                              "tail-block summary), then ckv_decode_step" if args.loop_two_launch
                              else "ckv_decode_step_append (append and step)"),
           "launches_per_layer_step": (1 + C.decode_step_launches(dims, w.budget_tokens)
                                       if args.loop_two_launch
                                       else C.decode_step_append_launches(dims, w.budget_tokens)),
           "data": "synthetic"}
    del loops, base
    torch.cuda.empty_cache()
    return res


def decode_loop(args, dev0) -> int:
    print(json.dumps(decode_loop_result(args, dev0, args.loop_layers)), flush=True)
    return 0


def batched_result(args, dev0, n_layers: int, w=None) -> dict:
    """The batched ragged decode step: 16 sequences of 16K to 64K tokens
    (Hq 32, Hkv 8, d 128, bf16, paged), 1024-token budget, steps rotating
    over layer copies, graph replay."""
    import torch
    from compensated_kv_selection_amd import compkv as C
    from compensated_kv_selection_amd import workloads as W
    from compensated_kv_selection_amd.tensors import to_device
    w = w if w is not None else W.make_preset("batched_ragged", seed=args.seed)
    base = to_device(w, dev0)
    dims = base.dims
    layers = []
    for li in range(n_layers):
        kc = base.k_cache if li == 0 else base.k_cache.clone()
        vc = base.v_cache if li == 0 else base.v_cache.clone()
        summ = C.allocate_summaries(dims, dev0)
        C.build_summaries(dims, kc, vc, base.block_table, base.seq_lens, summ)
        layers.append((kc, vc, summ))
    budget = w.budget_tokens
    ws = C.allocate_workspace(C.workspace_bytes(dims, budget), dev0)
    kmax = max(1, dims.kmax(budget))
    sel = torch.empty((dims.batch, dims.num_kv_heads, kmax), dtype=torch.int32, device=dev0)
    nsel = torch.empty((dims.batch, dims.num_kv_heads), dtype=torch.int32, device=dev0)
    out = torch.empty((dims.batch, dims.num_q_heads, dims.head_dim), dtype=torch.float32, device=dev0)
    lse = torch.empty((dims.batch, dims.num_q_heads), dtype=torch.float32, device=dev0)

    def step(i):
        kc, vc, summ = layers[i % n_layers]
        C.decode_step(dims, base.q, kc, vc, summ, base.block_table, base.seq_lens, budget, ws,
                      selected=sel, num_selected=nsel, out=out, lse=lse)

    for i in range(4):
        step(i)
    torch.cuda.synchronize()
    us, samples = timed_replays(torch, step, 40, 2, extra=10)
    C.workspace_status(ws)
    ab = {"total": 0}
    for Lb in w.seq_lens:
        Mb = -(-int(Lb) // 16)
        ab["total"] += algorithmic_bytes(Mb, w.num_kv_heads, w.head_dim, w.r_groups,
                                         min(Mb, budget // 16), 16, 2)["total"]
    res = {"workload": (f"batched_ragged: {w.batch} sequences of {int(w.seq_lens.min())} to "
                        f"{int(w.seq_lens.max())} tokens ({int(w.seq_lens.sum())} in all), Hq {w.num_q_heads}, "
                        f"Hkv {w.num_kv_heads}, d {w.head_dim}, budget {budget} tokens, {n_layers} rotating "
                        f"layer buffers"),
           "us_per_step": round(us, 2), "distribution_us": distribution(samples),
           "algorithmic_bytes": ab["total"], "effective_GBps": round(ab["total"] / (us * 1e-6) / 1e9, 1),
           "pct_hbm_peak": round(100 * ab["total"] / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 2),
           "launches": C.decode_step_launches(dims, budget), "data": "synthetic"}
    del layers, base
    torch.cuda.empty_cache()
    return res


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--layers", type=int, default=16, help="distinct layer buffers the steps rotate over")
    ap.add_argument("--workload", default="llama_128k")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-runs", type=int, default=5, help="oracle steps per CPU-baseline median")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="leave out the batched ragged step and the 128K decode loop")
    ap.add_argument("--copy-mb", type=int, default=0,
                    help="only run a plain elementwise copy of this many MiB (counter calibration)")
    ap.add_argument("--rocprof-summary", default="",
                    help="only print a per-kernel summary of the rocprofv3 CSV files under this directory")
    ap.add_argument("--sweep", action="store_true",
                    help="only time the step over context lengths 32K, 64K, 128K x budgets 512, 1024, 2048 "
                         "tokens (Llama-3.1-8B layer shape), with dense decode per length; one JSON line each")
    ap.add_argument("--sweep-r", action="store_true",
                    help="only time the step at 128K / 512 for r = 1, 2, 4, 8, 16, 128 variance groups, "
                         "CompKV and estimated-mass selection; one JSON line per r")
    ap.add_argument("--decode-loop", action="store_true",
                    help="only time the prefill summary build and a 64-step appending decode loop at 128K "
                         "context, 2048-token budget, captured into one HIP graph; one JSON line")
    ap.add_argument("--loop-layers", type=int, default=8, help="layer copies the decode loop visits per step")
    ap.add_argument("--loop-two-launch", action="store_true",
                    help="decode loop: append and step as two calls instead of ckv_decode_step_append")
    args = ap.parse_args()

    if args.rocprof_summary:
        print(rocprof_summary(args.rocprof_summary))
        return 0

    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU; --gpus {args.gpus} is not supported "
              "(across GPUs the decode step would shard by sequence or by KV head, one share per process)",
              file=sys.stderr, flush=True)
        return 2

    import numpy as np
    import torch

    from compensated_kv_selection_amd import compkv as C
    from compensated_kv_selection_amd import workloads as W
    from compensated_kv_selection_amd.tensors import to_device

    w = None
    cpu = None
    headline = not (args.sweep or args.decode_loop or args.sweep_r or args.copy_mb)
    if headline:
        t_gen = time.time()
        w = W.make_preset(args.workload, seed=args.seed)
        print(f"[bench] generated {args.workload} in {time.time() - t_gen:.1f}s", file=sys.stderr, flush=True)
        if not args.no_cpu and w.batch == 1:
            # before anything touches the GPU: the oracle's worker processes are forked
            t0 = time.time()
            cpu = cpu_oracle_baseline(w, args.cpu_runs)
            print(f"[bench] CPU oracle baseline in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    dev0 = "cuda:0"
    torch.cuda.set_device(0)

    if args.copy_mb:
        # torch.neg over fp32: one elementwise kernel that reads n and writes n bytes
        n = args.copy_mb * (1 << 20)
        x = torch.ones(n // 4, dtype=torch.float32, device=dev0)
        y = torch.empty_like(x)
        for _ in range(5):
            torch.neg(x, out=y)
        torch.cuda.synchronize()
        print(json.dumps({"copy_kernel": "torch.neg fp32", "read_bytes": n, "write_bytes": n,
                          "launches": 5}), flush=True)
        return 0

    C.load_library()
    if args.sweep:
        return sweep(args, dev0)
    if args.decode_loop:
        return decode_loop(args, dev0)
    if args.sweep_r:
        return sweep_r(args, dev0)
    base = to_device(w, dev0)
    dims = base.dims
    budget = w.budget_tokens
    L = int(w.seq_lens.max())
    M = -(-L // w.block_size)
    kv_bytes = 2 if w.dtype == "bf16" else 4
    kk = min(M, budget // w.block_size)

    # Layer copies (distinct buffers); summaries built per layer.
    layers = []
    for li in range(args.layers):
        kc = base.k_cache if li == 0 else base.k_cache.clone()
        vc = base.v_cache if li == 0 else base.v_cache.clone()
        summ = C.allocate_summaries(dims, dev0)
        layers.append((kc, vc, summ))
    torch.cuda.synchronize()

    # Prefill summary build over the whole context (timed, reported beside the
    # step): one untimed build, then the layer copies' builds back to back
    # between two events, so that launch gaps do not count.
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    C.build_summaries(dims, layers[0][0], layers[0][1], base.block_table, base.seq_lens, layers[0][2])
    torch.cuda.synchronize()
    ev[0].record()
    for kc, vc, summ in layers:
        C.build_summaries(dims, kc, vc, base.block_table, base.seq_lens, summ)
    ev[1].record()
    torch.cuda.synchronize()
    build_us = ev[0].elapsed_time(ev[1]) * 1e3 / len(layers)

    ws = C.allocate_workspace(C.workspace_bytes(dims, budget), dev0)
    sel = torch.empty((dims.batch, dims.num_kv_heads, max(1, dims.kmax(budget))), dtype=torch.int32, device=dev0)
    nsel = torch.empty((dims.batch, dims.num_kv_heads), dtype=torch.int32, device=dev0)
    out = torch.empty((dims.batch, dims.num_q_heads, dims.head_dim), dtype=torch.float32, device=dev0)
    lse = torch.empty((dims.batch, dims.num_q_heads), dtype=torch.float32, device=dev0)

    def step(i):
        kc, vc, summ = layers[i % len(layers)]
        C.decode_step(dims, base.q, kc, vc, summ, base.block_table, base.seq_lens, budget, ws,
                      selected=sel, num_selected=nsel, out=out, lse=lse)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    C.workspace_status(ws)
    # The timed region: `steps` steps, as `replays` replays of one HIP graph of
    # steps / replays consecutive steps, back to back on the launch stream,
    # with an event between replays; synchronized before and after.
    replays = replays_for(args.steps)
    extra_replays = 10 if replays < 5 else 0  # the distribution from further replays of the same graph
    t0 = time.perf_counter()
    us_per_step, samples = timed_replays(torch, step, args.steps, replays, extra=extra_replays)
    wall_s = time.perf_counter() - t0
    # every bounded wait of the timed steps ended in time (else this raises
    # and the run fails: the outputs of those steps would be unspecified)
    C.workspace_status(ws)
    print(f"[bench] {args.steps} steps ({replays} graph replays): {us_per_step:.2f} us/step (events), "
          f"wall {wall_s:.2f} s", file=sys.stderr, flush=True)

    launches = C.decode_step_launches(dims, budget)
    ab = {"summary": 0, "selected_kv": 0, "total": 0}
    for Lb in w.seq_lens:
        Mb = -(-int(Lb) // w.block_size)
        abb = algorithmic_bytes(Mb, w.num_kv_heads, w.head_dim, w.r_groups, min(Mb, budget // w.block_size),
                                w.block_size, kv_bytes)
        for key in ab:
            ab[key] += abb[key]
    kv_all = sum(-(-int(Lb) // w.block_size) for Lb in w.seq_lens) * w.num_kv_heads * w.block_size * w.head_dim \
        * 2 * kv_bytes  # every page's keys and values
    tokens_desc = (f"{L} tokens" if w.batch == 1 else
                   f"{int(w.seq_lens.min())} to {L} tokens per sequence ({int(w.seq_lens.sum())} in all)")
    # one launch per step: the per-launch time is the per-step time
    avg_launch_us = us_per_step / launches
    achieved = ab["total"] / (us_per_step * 1e-6) / 1e9
    eff_gbps = achieved

    dense = None
    if not args.no_dense:
        dws = C.allocate_workspace(C.dense_workspace_bytes(dims), dev0)
        dout = torch.empty_like(out)
        dlse = torch.empty_like(lse)

        def dstep(i):
            kc, vc, _ = layers[i % len(layers)]
            C.dense_decode_attention(dims, base.q, kc, vc, base.block_table, base.seq_lens, dws,
                                     out=dout, lse=dlse)

        for i in range(3):
            dstep(i)
        torch.cuda.synchronize()
        dense_us, dsamples = timed_replays(torch, dstep, 48, 2, extra=6)
        C.workspace_status(dws)
        dense = {"us_per_step": round(dense_us, 2), "distribution_us": distribution(dsamples),
                 "bytes": kv_all, "GBps": round(kv_all / (dense_us * 1e-6) / 1e9, 1),
                 "pct_hbm_peak": round(100 * kv_all / (dense_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 2),
                 "speedup_of_compkv": round(dense_us / us_per_step, 2)}

    src_hash = kernel_source_hash()
    traffic = read_traffic("decode_step_" + args.workload, src_hash)
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
            "kernel": ("ckv::fused_step_kernel (one launch per decode step)" if launches == 1 else
                       "ckv::step_kernel x3 (score, select, attend; timed together)"),
            "algorithmic_bytes_per_launch": ab["total"], "avg_launch_us": round(avg_launch_us, 3),
            "launch_timing": f"HIP events on the launch stream around {replays} back-to-back replays of a "
                             f"graph of {args.steps // replays} steps, {launches} launch(es) per step"
                             + (f"; distribution_us from {extra_replays} further replays of the same graph"
                                if extra_replays else "")}
    extra = {}
    if not args.no_extra and args.workload == "llama_128k":
        del layers
        torch.cuda.empty_cache()
        t0 = time.time()
        extra["batched_ragged"] = batched_result(args, dev0, n_layers=2)
        print(f"[bench] batched ragged step in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
        t0 = time.time()
        extra["prefill_128k_loop"] = decode_loop_result(args, dev0, n_layers=args.loop_layers)
        print(f"[bench] 128K decode loop in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    line = {
        "metric": METRIC, "value": round(us_per_step, 3), "unit": "us/step", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(us_per_step / 1e3, 6),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: decode step, batch {w.batch}, {tokens_desc}, Hq "
                               f"{w.num_q_heads}, Hkv {w.num_kv_heads}, d {w.head_dim}, block "
                               f"{w.block_size}, r {w.r_groups}, budget {budget} tokens ({kk} blocks), "
                               f"{args.layers} rotating layer buffers",
                   "global_batch": w.batch, "seq_len": L, "budget_tokens": budget},
        "distribution_us": distribution(samples),
        "effective_GBps": round(eff_gbps, 1), "pct_hbm_peak": round(100 * eff_gbps / HBM_PEAK_GBPS, 2),
        "algorithmic_bytes": ab, "roofline": roof, "dense": dense,
        "summary_build": {"us": round(build_us, 1),
                          "bytes": kv_all + ab["summary"],
                          "GBps": round((kv_all + ab["summary"]) / (build_us * 1e-6) / 1e9, 1)},
        "cpu_baseline": cpu, "workspace_error_word": 0, "kernel_source_hash": src_hash,
    }
    line.update(extra)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
