"""Phase timestamps of the single-launch decode step.

    python -m compensated_kv_selection_amd.build --phase-trace
    python -m compensated_kv_selection_amd.phase_trace [--workload llama_128k] [--budget N]

Runs the step as bench.py does (a HIP graph of consecutive steps over 16
rotating layer buffers) with libcompkv_trace.so, the library built with
CKV_PHASE_TRACE.  In that build, thread 0 of every workgroup of the single
launch stores the 100 MHz constant-rate clock (s_memrealtime) at fixed points
of its work into the workspace's per-block score region, which the single
launch leaves unused.  This reads the marks left
by the last step and prints, per phase, the median and the maximum over the
workgroups, in microseconds from the first workgroup's entry.  The trace
build stores a handful of words per workgroup, so its step takes about as
long as the product's (compare its us/step line with bench.py's).
"""
from __future__ import annotations

import argparse
import os
import sys

import numpy as np
import torch

from . import compkv as C
from . import build
from . import workloads as W
from .tensors import to_device

MARKS_PER_SLOT = 32
CONTROL = {0: "entry", 1: "q staged", 2: "mean keys scored", 3: "header and weights published",
           4: "headers read", 5: "candidates published", 6: "candidates read",
           12: "radix select: start", 13: "radix select: T known", 14: "selected blocks counted",
           7: "selection known",
           8: "exact attention done", 10: "partial: reductions done", 15: "partial: value sums read",
           9: "partial published", 16: "merge: every partial read", 11: "merged (output written)"}
VALUE = {0: "entry", 1: "weights read", 2: "mean values summed", 3: "partial published"}


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="llama_128k")
    ap.add_argument("--budget", type=int, default=0, help="token budget (default: the workload's)")
    ap.add_argument("--steps", type=int, default=64, help="steps in the graph; the marks are the last step's")
    args = ap.parse_args(argv)
    if not os.path.exists(build.TRACE_LIB_PATH):
        raise RuntimeError(f"{build.TRACE_LIB_PATH} is not built; run "
                           "`python -m compensated_kv_selection_amd.build --phase-trace`")
    C.load_library(build.TRACE_LIB_PATH)
    dev = "cuda:0"
    w = W.make_preset(args.workload, seed=0)
    base = to_device(w, dev)
    dims = base.dims
    budget = args.budget or w.budget_tokens
    if C.decode_step_launches(dims, budget) != 1:
        raise RuntimeError("this workload and budget do not run as a single launch")
    layers = []
    for li in range(16):
        kc = base.k_cache if li == 0 else base.k_cache.clone()
        vc = base.v_cache if li == 0 else base.v_cache.clone()
        summ = C.allocate_summaries(dims, dev)
        C.build_summaries(dims, kc, vc, base.block_table, base.seq_lens, summ)
        layers.append((kc, vc, summ))
    ws = C.allocate_workspace(C.workspace_bytes(dims, budget), dev)

    def step(i):
        kc, vc, summ = layers[i % len(layers)]
        C.decode_step(dims, base.q, kc, vc, summ, base.block_table, base.seq_lens, budget, ws)

    for i in range(20):
        step(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(args.steps):
            step(i)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    C.workspace_status(ws)
    print(f"{args.workload}, budget {budget}: {e0.elapsed_time(e1) * 1e3 / args.steps:.2f} us/step (trace build)")

    # the marks: after the control words, [pair][2 n_chunks][32] 64-bit words
    # (control slots 0..n_chunks-1, value slots n_chunks + chunk)
    pairs = dims.batch * dims.num_kv_heads
    nch = -(-dims.max_blocks_per_seq // 256)
    ctrl_bytes = -(-(C.CTRL_WORDS_HEADER + C.CTRL_WORDS_PER_PAIR * pairs) * 4 // 256) * 256
    n = pairs * 2 * nch * MARKS_PER_SLOT
    words = ws[ctrl_bytes: ctrl_bytes + 8 * n].view(torch.int64).cpu().numpy().reshape(pairs, 2 * nch,
                                                                                      MARKS_PER_SLOT)
    times = words[:, :, :24]  # marks; counts and notes from 24
    t0 = times[:, :nch, 0][times[:, :nch, 0] > 0].min()
    us = (times.astype(np.float64) - t0) * 1e-2  # 100 MHz ticks

    def table(part_us, part_ticks, names):
        for i, name in names.items():
            v = part_us[:, :, i][part_ticks[:, :, i] > 0]
            if v.size:
                print(f"  {name:38s} {np.median(v):7.2f} {v.max():7.2f}")

    print("control workgroups, us from the first entry: median, max")
    table(us[:, :nch], times[:, :nch], CONTROL)
    print("value workgroups")
    table(us[:, nch:], times[:, nch:], VALUE)
    # shader clock over entry .. partial published (s_memtime notes 25, 26)
    span = (times[:, :nch, 9] - times[:, :nch, 0]).astype(np.float64)
    cyc = (words[:, :nch, 26] - words[:, :nch, 25]).astype(np.float64)
    ok = (span > 0) & (cyc > 0)
    if ok.any():
        print(f"shader clock over entry .. partial published: {np.median(cyc[ok] / span[ok] * 100.0):.0f} MHz")
    return 0


if __name__ == "__main__":
    sys.exit(main())
