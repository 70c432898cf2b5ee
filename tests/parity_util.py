"""Run one decode step on the GPU (through the C ABI) and in the CPU oracle on
the same generated inputs, and compare them.

Tolerances:
  summaries  mean key / mean value: the oracle's mean (1/n) sum_t k_t is exact
             to float64 rounding (sums of <= 16 bf16 or f32 values are exact
             in float64).  The GPU forms k0 + (sum_t (k_t - k0)) / n in fp32,
             so per channel its value before storage is within
             (n + 2) 2^-24 (max_t |k_t - k0| + |mean|) of the exact mean; the
             test allows twice that, plus (bf16 storage) one unit in the last
             place of the stored value, since the two roundings to bf16 can
             land on neighbouring values.  Near a mean close to zero the
             first term dominates.
             grouped variance: 1e-5 relative (fp32 two-pass sums of <= 16
             terms, then a mean over <= 128 channels).
  selection  block ids bit-exact.  (a) against a CPU top-k of the GPU's own
             fp32 scores (the decision in the kernel's precision); (b)
             against the oracle's fp64 selection wherever the oracle's k-th
             and (k+1)-th scores differ by more than NEAR_TIE relative;
             closer boundaries are reported and the GPU set is checked to be
             a valid top-k within NEAR_TIE.
  output     2e-3 max-abs (bf16 inputs, fp32 accumulation); lse 1e-4 abs.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np
import torch

from compensated_kv_selection_amd import compkv as C
from compensated_kv_selection_amd.tensors import to_device, torch_to_storage
from compensated_kv_selection_amd import workloads as W
from compensated_kv_selection_amd.workloads import DecodeInputs
from oracle import compkv_oracle as O
from ws_layout import PUBLISHED_REGIONS, published_row_words, workspace_regions

NEAR_TIE = 1e-5
OUT_ATOL = 2e-3
LSE_ATOL = 1e-4


@dataclasses.dataclass
class GpuResult:
    mean_k: np.ndarray   # storage dtype, [B, Hkv, max_blocks, d]
    mean_v: np.ndarray
    gvar: np.ndarray     # [B, Hkv, max_blocks, r]
    count: np.ndarray    # [B, max_blocks]
    selected: np.ndarray     # [B, Hkv, kmax]
    num_selected: np.ndarray  # [B, Hkv]
    group_scores: Optional[np.ndarray]  # [B, Hkv, max_blocks] float32
    out: np.ndarray          # [B, Hq, d]
    lse: np.ndarray          # [B, Hq]


def check_workspace_clean(ws, dims, budget):
    """Every call leaves the control words (but each pair's step counter) and
    the fused step's published headers and candidates zero, ready for the
    next call."""
    ctrl = C.workspace_control(ws, dims.batch, dims.num_kv_heads)
    assert int(ctrl[2]) == 0, (f"error word {int(ctrl[2])} (1: a bounded wait ran out, 2: a workgroup ran on "
                               f"an XCD it was not placed on); header words {ctrl[:8].tolist()}")
    ctrl = ctrl.clone()
    ctrl[C.CTRL_WORDS_HEADER + C.CTRL_EPOCH::C.CTRL_WORDS_PER_PAIR] = 0
    assert int(ctrl.abs().sum()) == 0, f"control words not reset: {ctrl.nonzero().flatten().tolist()}"
    regions = workspace_regions(dims.batch, dims.num_q_heads, dims.num_kv_heads, dims.head_dim,
                                dims.max_blocks_per_seq, budget)
    assert sum(regions) == ws.numel(), (sum(regions), ws.numel())
    epochs = C.workspace_control(ws, dims.batch, dims.num_kv_heads)[
        C.CTRL_WORDS_HEADER + C.CTRL_EPOCH::C.CTRL_WORDS_PER_PAIR].tolist()
    rows = published_row_words(dims.num_q_heads, dims.num_kv_heads, dims.max_blocks_per_seq, budget)
    bgs = dims.batch * dims.num_kv_heads
    for r in PUBLISHED_REGIONS:
        lo = sum(regions[:r])
        words = ws[lo:lo + regions[r]].view(torch.int64).cpu()
        n = rows[r]
        for bg, ep in enumerate(epochs):
            half = (ep + 1) % 2   # the half the next call publishes into
            seg = words[(half * bgs + bg) * n:(half * bgs + bg + 1) * n]
            assert int((seg != 0).sum()) == 0, f"published words of region {r}, pair {bg} not cleared"


def run_gpu(w: DecodeInputs, budget: Optional[int] = None, score_mode: int = C.SCORE_COMPKV,
            compensate: bool = True, fused: bool = False, device="cuda:0", dev=None,
            summaries=None) -> GpuResult:
    budget = w.budget_tokens if budget is None else budget
    dev = dev or to_device(w, device)
    dims = dev.dims
    if summaries is None:
        summaries = C.allocate_summaries(dims, device)
        C.build_summaries(dims, dev.k_cache, dev.v_cache, dev.block_table, dev.seq_lens, summaries)
    ws = C.allocate_workspace(C.workspace_bytes(dims, budget), device)
    gs = None
    if fused:
        sel, nsel, out, lse = C.decode_step(dims, dev.q, dev.k_cache, dev.v_cache, summaries,
                                            dev.block_table, dev.seq_lens, budget, ws, score_mode)
    else:
        gs = torch.full((dims.batch, dims.num_kv_heads, dims.max_blocks_per_seq), float("nan"),
                        dtype=torch.float32, device=device)
        sel, nsel = C.score_select(dims, dev.q, summaries, dev.block_table, dev.seq_lens, budget, ws,
                                   score_mode, group_scores=gs)
        out, lse = C.compensated_decode_attention(dims, dev.q, dev.k_cache, dev.v_cache, summaries,
                                                  dev.block_table, dev.seq_lens, budget, sel, nsel, ws,
                                                  compensate=compensate)
    torch.cuda.synchronize()
    C.workspace_status(ws)   # raises if a bounded wait ran out or a workgroup left its XCD
    check_workspace_clean(ws, dims, budget)
    return GpuResult(torch_to_storage(summaries.mean_k), torch_to_storage(summaries.mean_v),
                     summaries.gvar.cpu().numpy(), summaries.count.cpu().numpy(),
                     sel.cpu().numpy(), nsel.cpu().numpy(),
                     None if gs is None else gs.cpu().numpy(), out.cpu().numpy(), lse.cpu().numpy())


@dataclasses.dataclass
class OracleSeq:
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    summ: O.Summaries
    step: O.StepResult


ORACLE_MODES = {C.SCORE_COMPKV: "compkv", C.SCORE_MASS: "mass_hat"}


def run_oracle(w: DecodeInputs, budget: Optional[int] = None, score_mode: int = C.SCORE_COMPKV,
               compensate: bool = True, seqs=None) -> List[Optional[OracleSeq]]:
    budget = w.budget_tokens if budget is None else budget
    res = []
    for b in range(w.batch):
        if seqs is not None and b not in seqs:
            res.append(None)
            continue
        q, k, v = O.sequence_arrays(w.q[b], w.k_tokens[b], w.v_tokens[b], w.dtype)
        summ = O.build_summaries(k, v, w.block_size, w.r_groups, w.dtype)
        step = O.decode_step(q, k, v, summ, budget_tokens=budget, block_size=w.block_size,
                             r=w.r_groups, score_mode=ORACLE_MODES[score_mode], compensate=compensate)
        res.append(OracleSeq(q, k, v, summ, step))
    return res


def check_summaries(w: DecodeInputs, g: GpuResult, ora: List[Optional[OracleSeq]]) -> None:
    for b, o in enumerate(ora):
        if o is None:
            continue
        M = w.num_blocks(b)
        gk = g.mean_k[b, :, :M].transpose(1, 0, 2)   # -> [M, Hkv, d], the oracle's order
        gv_ = g.mean_v[b, :, :M].transpose(1, 0, 2)
        gg = g.gvar[b, :, :M].transpose(1, 0, 2)
        gc = g.count[b, :M]
        np.testing.assert_array_equal(gc, o.summ.count, err_msg=f"count seq {b}")
        for name, gpu, tok in (("mean_k", gk, o.k), ("mean_v", gv_, o.v)):
            ref = o.summ.mean_k if name == "mean_k" else o.summ.mean_v
            gval = gpu.astype(np.float64) if w.dtype == "f32" else \
                (gpu.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
            for i in range(M):
                blk = tok[i * w.block_size:(i + 1) * w.block_size]
                n = blk.shape[0]
                spread = np.abs(blk - blk[0][None]).max(axis=0)
                # fp32 accumulation error of k0 + sum(k - k0) / n, doubled ...
                bound = 2 * (n + 2) * 2.0 ** -24 * (spread + np.abs(ref[i]))
                if w.dtype == "bf16":
                    # ... plus one unit in the last place of the stored bf16 value
                    mag = np.maximum(np.abs(ref[i]), 2.0 ** -126)
                    bound = bound + 2.0 ** (np.floor(np.log2(mag)) - 7)
                err = np.abs(gval[i] - ref[i])
                assert np.all(err <= bound), f"{name} seq {b} block {i}: {err.max()} > bound"
        np.testing.assert_allclose(gg, o.summ.gvar, rtol=1e-5, atol=1e-7, err_msg=f"gvar seq {b}")


def cpu_topk(scores: np.ndarray, k: int) -> np.ndarray:
    order = np.lexsort((np.arange(scores.size), -scores))
    return np.sort(order[:k])


def check_selection_isolated(w: DecodeInputs, g: GpuResult, budget: int) -> None:
    """GPU selection == CPU top-k over the GPU's own fp32 scores, bit-exact."""
    kmax = min(w.max_blocks, budget // w.block_size)
    for b in range(w.batch):
        M = w.num_blocks(b)
        kk = min(M, kmax)
        for h in range(w.num_kv_heads):
            assert g.num_selected[b, h] == kk
            s = g.group_scores[b, h, :M]
            assert np.all(np.isfinite(s)) and np.all(s >= 0)
            np.testing.assert_array_equal(g.selected[b, h, :kk], cpu_topk(s, kk), err_msg=f"seq {b} head {h}")
            if kmax > kk:
                assert np.all(g.selected[b, h, kk:kmax] == -1)


def check_selection_valid(rank: np.ndarray, kk: int, gsel: np.ndarray, gap: float, osel: np.ndarray,
                          where: str) -> bool:
    """Check one (sequence, KV head) selection against the oracle's ranked
    scores.  A decisive boundary (relative gap >= NEAR_TIE) or an exact tie
    (gap 0: equal fp64 scores, which the kernels reproduce exactly, e.g.
    duplicated or constant-key blocks) must give the oracle's set: ties go to
    the lowest block index.  A near tie (0 < gap < NEAR_TIE) must give a valid
    top-k within NEAR_TIE: every block clearly above the k-th score taken, no
    block clearly below it.  Returns True for a near tie."""
    assert gsel.shape == (kk,) and np.all(np.diff(gsel) > 0), f"{where}: not ascending and distinct"
    if gap >= NEAR_TIE or gap == 0.0:
        np.testing.assert_array_equal(gsel, osel, err_msg=where)
        return False
    kth = np.sort(rank)[::-1][kk - 1]
    must = np.nonzero(rank > kth * (1 + NEAR_TIE))[0]
    assert set(must.tolist()) <= set(gsel.tolist()), f"{where}: missed a clear winner"
    assert np.all(rank[gsel] >= kth * (1 - NEAR_TIE)), f"{where}: took a clear loser"
    return True


def check_selection_vs_oracle(w: DecodeInputs, g: GpuResult, ora: List[Optional[OracleSeq]],
                              report: Optional[list] = None) -> int:
    """Returns the number of (seq, KV head) boundaries that were near-ties."""
    near = 0
    for b, o in enumerate(ora):
        if o is None:
            continue
        kk = o.step.selected.shape[1]
        for h in range(w.num_kv_heads):
            gsel = g.selected[b, h, :kk]
            if check_selection_valid(o.step.rank_score[h], kk, gsel, float(o.step.gaps[h]),
                                     o.step.selected[h], f"seq {b} KV head {h}"):
                near += 1
                if report is not None:
                    report.append((b, h, float(o.step.gaps[h]), bool(np.array_equal(gsel, o.step.selected[h]))))
    return near


def check_group_scores(w: DecodeInputs, g: GpuResult, ora: List[Optional[OracleSeq]], rtol: float = 1e-4) -> int:
    """The GPU's fp32 ranked scores against the oracle's, element by element.
    Compared where the block's stored mean key is the same on both sides
    (bf16: the two roundings of the mean can land one unit apart, which
    moves that block's logit by up to tau |q| 2^-8 |mean|, far more than the
    scoring arithmetic's error; such blocks are counted and must be rare)
    and where the score is not near fp32's underflow (the kernels form
    exp(log score - log Z_hat), so scores below ~1e-30 of the pair's largest
    may flush to zero).  Returns the number of scores compared."""
    n = 0
    for b, o in enumerate(ora):
        if o is None:
            continue
        M = w.num_blocks(b)
        if w.dtype == "bf16":
            gk = (g.mean_k[b, :, :M].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        else:
            gk = g.mean_k[b, :, :M].astype(np.float64)
        same_row = np.all(gk == o.summ.mean_k.transpose(1, 0, 2), axis=2)   # [Hkv, M]
        for h in range(w.num_kv_heads):
            ref = o.step.rank_score[h]
            got = g.group_scores[b, h, :M].astype(np.float64)
            big = ref > max(1e-30, 1e-25 * ref.max())
            cmp = big & same_row[h] if w.dtype == "bf16" else big
            assert cmp.sum() >= 0.99 * big.sum(), f"seq {b} KV head {h}: too many differing mean keys"
            np.testing.assert_allclose(got[cmp], ref[cmp], rtol=rtol, atol=0,
                                       err_msg=f"group scores seq {b} KV head {h}")
            assert np.all(got[~big] <= 1e-20), f"seq {b} KV head {h}: tiny scores"
            n += int(cmp.sum())
    return n


def oracle_output_for(o: OracleSeq, selected: np.ndarray, w: DecodeInputs, compensate: bool = True):
    return O.compensated_attention(o.q, o.k, o.v, o.summ, selected, w.block_size, compensate)


def check_outputs(w: DecodeInputs, g: GpuResult, ora: List[Optional[OracleSeq]],
                  compensate: bool = True) -> float:
    """Compare with the oracle's attention on the GPU's own selection; return max abs error."""
    worst = 0.0
    for b, o in enumerate(ora):
        if o is None:
            continue
        kk = o.step.selected.shape[1]
        sel = g.selected[b, :, :kk].astype(np.int64)
        out, lse = oracle_output_for(o, sel, w, compensate)
        err = np.abs(g.out[b] - out).max()
        worst = max(worst, float(err))
        assert err <= OUT_ATOL, f"seq {b}: out max abs error {err}"
        fin = np.isfinite(lse)
        np.testing.assert_array_equal(np.isfinite(g.lse[b]), fin)
        if fin.any():
            lerr = np.abs(g.lse[b][fin] - lse[fin]).max()
            assert lerr <= LSE_ATOL, f"seq {b}: lse error {lerr}"
    return worst


def duplicated_blocks_case(seed: int = 77, seq_len: int = 140000, n_copies: int = 12) -> tuple:
    """A 2-KV-head, 4-query-heads-per-KV-head bf16 workload in which one hot
    block (keys along the group's mean query, with spread) is copied, keys
    and values, to n_copies block positions, three of them on both sides of
    chunk boundaries (blocks 255, 256, 511; chunks are 256 blocks).  Returns
    (inputs, ascending copy positions).  With a budget of 8 blocks the copies
    straddle the k-th place, so the selection is decided by the lower-index
    rule."""
    w = W.make_decode_inputs(name="dup", seq_lens=[seq_len], num_q_heads=8, num_kv_heads=2, head_dim=128,
                             r_groups=4, budget_tokens=128, dtype="bf16", n_needles=0, n_outliers=2,
                             seed=seed)
    rng = np.random.default_rng(seed + 1)
    M = w.num_blocks(0)
    rest = rng.choice(np.arange(512, M - 1), size=n_copies - 3, replace=False)
    copies = np.unique(np.concatenate([[255, 256, 511], rest]))
    k, v = w.k_tokens[0], w.v_tokens[0]
    src = int(copies[-1])
    q = W.bf16_bits_to_f32(w.q[0])
    for g in range(2):
        qm = q[g * 4:(g + 1) * 4].mean(axis=0)
        hot = 1.0 * qm[None, :] + rng.standard_normal((16, 128), dtype=np.float32)
        k[src * 16:(src + 1) * 16, g] = W.f32_to_bf16_bits(hot.astype(np.float32))
    for c in copies[:-1]:
        k[c * 16:(c + 1) * 16] = k[src * 16:(src + 1) * 16]
        v[c * 16:(c + 1) * 16] = v[src * 16:(src + 1) * 16]
    return w, copies


def concentrated_blocks_case(seed: int = 91, n_hot: int = 48, hot_chunk: int = 1, n_blocks: int = 2048,
                             budget_blocks: int = 96) -> tuple:
    """A 2-KV-head, 4-query-heads-per-KV-head bf16 workload of n_blocks
    blocks (by default 8 chunks of 256).  For KV head 0 only, n_hot blocks of
    one chunk carry keys along the group's mean query with a wide spread
    (large mass and large within-block variance), so that they top the
    ranking; KV head 1 keeps i.i.d. keys with 8 ordinary needles.  With a
    budget of 96 blocks, KV head 0's pair has a chunk holding more of its top
    k than the chunk's first candidates, and KV head 1's pair does not.
    Returns (inputs, the hot blocks)."""
    w = W.make_decode_inputs(name="concentrated", seq_lens=[n_blocks * 16], num_q_heads=8, num_kv_heads=2,
                             head_dim=128, r_groups=4, budget_tokens=budget_blocks * 16, dtype="bf16",
                             n_needles=8, n_outliers=2, seed=seed)
    rng = np.random.default_rng(seed + 1)
    hot = np.sort(rng.choice(np.arange(hot_chunk * 256, (hot_chunk + 1) * 256), size=n_hot, replace=False))
    k = w.k_tokens[0]
    q = W.bf16_bits_to_f32(w.q[0])
    qm = q[0:4].mean(axis=0)
    for i in hot:
        rows = 0.7 * qm[None, :] + 2.0 * rng.standard_normal((16, 128), dtype=np.float32)
        k[i * 16:(i + 1) * 16, 0] = W.f32_to_bf16_bits(rows.astype(np.float32))
    return w, hot
