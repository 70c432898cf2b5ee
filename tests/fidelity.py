"""Selection fidelity of CompKV against attention-mass selection on synthetic
inputs: analogs of the review's App. B.1 (KL divergence and relative L2 error
of the output against exact attention, residual ranking vs mass ranking) and
App. B.2 (Spearman correlation of the practical score with the exact
residual, and the share of the best attainable residual the selection keeps),
over the number of variance groups r.

Every figure is computed in the CPU oracle.  With ``gpu=True`` the selections
and the scores are the GPU's (through the C ABI); otherwise the oracle's.

    python tests/fidelity.py [--gpu] [--len 32768] [--seed 0] [--json PATH]
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import os
import sys
from typing import List, Optional, Sequence

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
for p in (HERE, os.path.dirname(HERE)):
    if p not in sys.path:
        sys.path.insert(0, p)

from compensated_kv_selection_amd import workloads as W  # noqa: E402
from oracle import compkv_oracle as O  # noqa: E402

R_VALUES = (1, 2, 4, 8, 128)

# (label, oracle score mode, compensate, selection available on the GPU)
SELECTIONS = (
    ("residual (exact)", "residual_exact", True, False),
    ("mass (exact)", "mass_exact", True, False),
    ("mass (exact), no comp.", "mass_exact", False, False),
    ("CompKV", "compkv", True, True),
    ("mass_hat + Mean comp.", "mass_hat", True, True),
    ("mass_hat, no comp.", "mass_hat", False, True),
)


@dataclasses.dataclass
class Row:
    selection: str
    r: Optional[int]          # None for the exact-score rankings (no summaries involved)
    compensate: bool
    kl: float                 # mean over query heads of KL(p_hat || p)
    rel_l2: float             # mean over query heads of ||out - dense|| / ||dense||
    capture: float            # mean over KV heads of the residual capture
    spearman: Optional[float]  # mean over KV heads, ranked score vs exact group residual
    source: str               # "oracle" or "gpu": where selection and scores come from


def workload(length: int = 32768, seed: int = 0, r: int = 4, budget: int = 512) -> W.DecodeInputs:
    """One Llama-3.1-8B-shaped sequence (32 query heads, 8 KV heads, d = 128)."""
    return W.make_preset("llama_32k", seed=seed, seq_lens=[length], r_groups=r, budget_tokens=budget)


def _gpu_selection(w: W.DecodeInputs, score_mode: str, compensate: bool):
    from compensated_kv_selection_amd import compkv as C
    from parity_util import run_gpu
    mode = {"compkv": C.SCORE_COMPKV, "mass_hat": C.SCORE_MASS}[score_mode]
    g = run_gpu(w, score_mode=mode, compensate=compensate)
    n = int(g.num_selected[0, 0])
    sel = np.sort(g.selected[0, :, :n].astype(np.int64), axis=1)
    M = -(-int(w.seq_lens[0]) // w.block_size)
    return sel, g.group_scores[0, :, :M].astype(np.float64), g


def fidelity_rows(w: W.DecodeInputs, r_values: Sequence[int] = R_VALUES, gpu: bool = False,
                  gpu_outputs: Optional[List] = None) -> List[Row]:
    """Rows of the fidelity table for sequence 0 of ``w``.  When ``gpu`` is
    set and ``gpu_outputs`` is a list, each GPU run's (label, r, GPU output,
    oracle output for the GPU's selection, dense output) is appended to it."""
    bs, budget = w.block_size, w.budget_tokens
    q, k, v = O.sequence_arrays(w.q[0], w.k_tokens[0], w.v_tokens[0], w.dtype)
    Hkv = k.shape[1]
    dense = O.dense_attention(q, k, v)
    rows: List[Row] = []
    resid_g = None
    for r in r_values:
        summ = O.build_summaries(k, v, bs, r, w.dtype)
        if resid_g is None:
            # The exact residual uses the stored mean key only, not r.
            _, resid, _ = O.exact_block_stats(q, k, summ, bs)
            resid_g = O.group_sum(resid, Hkv)
        for label, mode, comp, on_gpu in SELECTIONS:
            exact = not on_gpu
            if exact and r != r_values[0]:
                continue
            if gpu and on_gpu:
                sel, score, g = _gpu_selection(dataclasses.replace(w, r_groups=r), mode, comp)
                src = "gpu"
            else:
                st = O.decode_step(q, k, v, summ, budget_tokens=budget, block_size=bs, r=r,
                                   score_mode=mode, compensate=comp)
                sel, score, g, src = st.selected, st.rank_score, None, "oracle"
            f = O.selection_fidelity(q, k, v, summ, sel, bs, comp, dense)
            if g is not None and gpu_outputs is not None:
                ora_out, _ = O.compensated_attention(q, k, v, summ, sel, bs, comp)
                gpu_outputs.append((label, r, g.out[0].astype(np.float64), ora_out, dense[0]))
            rho = None if exact else float(np.mean([O.spearman(score[h], resid_g[h])
                                                    for h in range(Hkv)]))
            rows.append(Row(label, None if exact else r, comp, float(f.kl.mean()),
                            float(f.rel_l2.mean()), float(O.residual_capture(resid_g, sel).mean()),
                            rho, src))
    return rows


def markdown(rows: List[Row]) -> str:
    out = ["| selection | r | Mean comp. | KL(p̂‖p) | rel. L2 | residual capture | Spearman | from |",
           "|---|---|---|---|---|---|---|---|"]
    for x in rows:
        out.append(f"| {x.selection} | {'-' if x.r is None else x.r} | {'yes' if x.compensate else 'no'} "
                   f"| {x.kl:.4f} | {x.rel_l2:.4f} | {x.capture:.4f} | "
                   f"{'-' if x.spearman is None else f'{x.spearman:.4f}'} | {x.source} |")
    return "\n".join(out)


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpu", action="store_true", help="selections and scores from the GPU")
    ap.add_argument("--len", type=int, default=32768)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--budget", type=int, default=512)
    ap.add_argument("--json", default=None, help="also write the rows here")
    a = ap.parse_args(argv)
    w = workload(a.len, a.seed, budget=a.budget)
    print(f"[fidelity] len={a.len} seed={a.seed} budget={a.budget} gpu={a.gpu}", flush=True)
    rows = fidelity_rows(w, gpu=a.gpu)
    print(markdown(rows), flush=True)
    if a.json:
        with open(a.json, "w") as fh:
            json.dump({"len": a.len, "seed": a.seed, "budget": a.budget,
                       "rows": [dataclasses.asdict(x) for x in rows]}, fh, indent=1)
    return 0


if __name__ == "__main__":
    sys.exit(main())
