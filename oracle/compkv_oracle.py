"""CompKV oracle: a plain, slow, float64 CPU implementation of one
compensation-aware block-sparse decode step.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import or run this module.  The GPU library never does,
and this module shares no code with it (only the seeded input generators are
common, and they hold none of the method's arithmetic).

What is computed, and where it is described (pages cited by title/section):

* [abstract] "CompKV: Compensation-Aware KV Selection for Long-Context LLM
  Inference", shd-paper.top listing, original English abstract: the context
  is cut into blocks, a chosen subset is attended exactly and the rest gets a
  coarse correction; the authors tie the error that the block-mean correction
  leaves to two quantities, the attention the block draws and the spread of
  its logits, and estimate that error from small per-block statistics to rank
  the blocks.
* [review] evolve.pub review of the same paper, "Summary": with Mean
  compensation each omitted block stands in with the logit of its mean; an
  exact KL identity holds; how much an omitted block leaves unexplained
  depends on both its attention mass and the variance of its logits (paper
  Section 3, Eqs. 4-7); scores come from the mean key, the key variance in
  r channel groups (4 by default) and the mean value, with a mass estimate
  taken to second order.
* [review FAQ] 2d + r + 1 scalars per block, updated incrementally as tokens
  enter the cache.
* [review Strengths] App. A.1 exact log-partition KL identity; A.2-A.3
  mass-times-variance residual with remainder control; A.5 removing
  compensation recovers attention-mass Top-K; B.1 oracle residual ranking.

The pages print none of the equations, so each step below is written from
their verbal statements.  Readings taken where they are silent:

  R1  softmax scale 1/sqrt(d).
  R2  r contiguous, equal channel groups C_t = [t*d/r, (t+1)*d/r).
  R3  grouped variance = mean over the group's channels of the per-channel
      population variance (divide by n) of the block's keys.
  R4  the "+1" of 2d + r + 1 is the block's token count n.
  R5  second-order mass estimate  A = n * exp(s_bar) * (1 + var_hat / 2);
      practical residual score     S = A * var_hat / 2;
      estimated log-partition      Z_hat = sum over blocks of A.
  R6  GQA: one selection per KV head, shared by its G query heads
      (query head h reads KV head h // G); group score
      S_g = sum over h in g of S_h / Z_hat_h.
  R7  k = min(M, budget // block_size) blocks, a partial tail block counts
      as one; no forced sink or recent blocks; ties go to the lower index.
  R8  summaries are stored as: mean key and mean value rounded to the KV
      dtype (bf16: nearest, ties to even), grouped variances rounded to f32;
      scoring and compensation use the stored values.
  R9  "updated incrementally" = the tail block's summary is recomputed from
      its raw tokens when a token is appended.

The pages print no value for the readings R2, R5 and R6.  Each is pinned
where the mathematics fixes it (tests/test_oracle_pins.py): the grouped
estimate (R2, R3) is exact when a block's key deviations are uncorrelated
with equal variance inside each group, and reduces to closed forms at r = 1
and r = d; the practical score (R5) and its GQA group sum (R6) converge, head
by head and summed over the group, to the exact per-head normalised residual
as the blocks' spread shrinks, and the group selection then equals the
brute-force minimiser of the summed KL over every k-subset.  Beyond second
order in the spread, the form of R5 is a reading, not a derived fact.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence

import numpy as np

# ---------------------------------------------------------------------------
# Storage formats
# ---------------------------------------------------------------------------


def widen(x: np.ndarray, dtype: str) -> np.ndarray:
    """Storage array -> float64 (exact).  bf16 arrays hold raw uint16 bits."""
    if dtype == "bf16":
        bits = np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    if dtype in ("f32", "f64"):
        return np.asarray(x, dtype=np.float64)
    raise ValueError(dtype)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value, ties to even.

    bfloat16 keeps 8 significant bits and float32's exponent range.  Normal
    values: write x = m * 2**e with 0.5 <= |m| < 1, round m * 2**8 to an
    integer (numpy's rint rounds halves to even), scale back.  Below 2**-126
    the spacing is fixed at 2**-133.  Rounding happens once, from float64.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    normal = np.ldexp(np.rint(m * 256.0), e - 8)
    tiny_step = 2.0 ** -133
    sub = np.rint(x / tiny_step) * tiny_step
    out = np.where(np.abs(x) < 2.0 ** -126, sub, normal)
    return out


def round_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """Value after storing ``x`` in ``dtype`` (reading R8)."""
    if dtype == "bf16":
        return round_bf16(x)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
    if dtype == "f64":
        return np.asarray(x, dtype=np.float64)
    raise ValueError(dtype)


# ---------------------------------------------------------------------------
# Block summaries: mean key, grouped key variance, mean value, count
# ([review] Summary; [review FAQ]: 2d + r + 1 scalars per block)
# ---------------------------------------------------------------------------


@dataclasses.dataclass
class Summaries:
    mean_k: np.ndarray   # [M, Hkv, d]  stored mean key
    mean_v: np.ndarray   # [M, Hkv, d]  stored mean value
    gvar: np.ndarray     # [M, Hkv, r]  stored grouped key variance
    count: np.ndarray    # [M]          tokens in the block

    @property
    def num_blocks(self) -> int:
        return int(self.count.shape[0])


def scalars_per_block(d: int, r: int) -> int:
    """Summary footprint per block and KV head: d (mean key) + d (mean value)
    + r (grouped variances) + 1 (count) ([review FAQ])."""
    return 2 * d + r + 1


def summarize_block(k_blk: np.ndarray, v_blk: np.ndarray, r: int, kv_dtype: str):
    """Summary of one block.  ``k_blk``, ``v_blk``: [n, Hkv, d] float64."""
    n, H, d = k_blk.shape
    if d % r:
        raise ValueError("r must divide head_dim")
    mu = k_blk.sum(axis=0) / n                          # mean key per channel
    nu = v_blk.sum(axis=0) / n                          # mean value per channel
    var = ((k_blk - mu[None]) ** 2).sum(axis=0) / n     # population variance per channel
    gvar = var.reshape(H, r, d // r).mean(axis=2)      # mean over each channel group (R2, R3)
    return (round_storage(mu, kv_dtype), round_storage(nu, kv_dtype),
            round_storage(gvar, "f32"), n)


def build_summaries(k: np.ndarray, v: np.ndarray, block_size: int, r: int,
                    kv_dtype: str) -> Summaries:
    """Bulk (prefill) summary build over all blocks of one sequence.

    ``k``, ``v``: [L, Hkv, d] float64 in logical token order.  Block i holds
    tokens [i*b, min((i+1)*b, L)).
    """
    L, H, d = k.shape
    M = -(-L // block_size)
    mean_k = np.zeros((M, H, d))
    mean_v = np.zeros((M, H, d))
    gvar = np.zeros((M, H, r))
    count = np.zeros(M, dtype=np.int64)
    for i in range(M):
        lo, hi = i * block_size, min(L, (i + 1) * block_size)
        mean_k[i], mean_v[i], gvar[i], count[i] = summarize_block(k[lo:hi], v[lo:hi], r, kv_dtype)
    return Summaries(mean_k, mean_v, gvar, count)


def append_summaries(summ: Optional[Summaries], k: np.ndarray, v: np.ndarray,
                     block_size: int, r: int, kv_dtype: str) -> Summaries:
    """Decode-time update after the newest token (the last row of ``k``/``v``)
    entered the cache: recompute only the block holding it (reading R9)."""
    L, H, d = k.shape
    i = (L - 1) // block_size
    lo, hi = i * block_size, L
    blk = summarize_block(k[lo:hi], v[lo:hi], r, kv_dtype)
    if summ is None:
        summ = Summaries(np.zeros((0, H, d)), np.zeros((0, H, d)), np.zeros((0, H, r)),
                         np.zeros(0, dtype=np.int64))
    M = summ.num_blocks
    if i == M:   # the token opened a new block
        summ = Summaries(np.concatenate([summ.mean_k, blk[0][None]]),
                         np.concatenate([summ.mean_v, blk[1][None]]),
                         np.concatenate([summ.gvar, blk[2][None]]),
                         np.concatenate([summ.count, [blk[3]]]))
    elif i == M - 1:
        summ.mean_k[i], summ.mean_v[i], summ.gvar[i], summ.count[i] = blk
    else:
        raise ValueError("append must extend the last block or open the next one")
    return summ


# ---------------------------------------------------------------------------
# Block scoring ([review] Summary, paper Section 3 Eqs. 4-7; [abstract])
# ---------------------------------------------------------------------------


@dataclasses.dataclass
class Scores:
    s_bar: np.ndarray        # [Hq, M] block-mean logit  tau * q . mu
    var_hat: np.ndarray      # [Hq, M] grouped estimate of the within-block logit variance
    log_mass_hat: np.ndarray  # [Hq, M] log of A = n e^{s_bar} (1 + var_hat/2)
    log_z_hat: np.ndarray    # [Hq]    log of Z_hat = sum_i A_i
    head_score: np.ndarray   # [Hq, M] S_h / Z_hat_h  (normalized practical residual score)
    group_score: np.ndarray  # [Hkv, M] sum over the group's heads of head_score


def block_scores(q: np.ndarray, summ: Summaries, r: int) -> Scores:
    """Score every block from its stored summary.

    For query head h (KV head g = h // G), block i with stored mean key mu_i,
    grouped variances gvar_i[t] and count n_i:

      s_bar   = tau * q_h . mu_i                      block-mean logit
      var_hat = tau^2 * sum_t |q_h restricted to C_t|^2 * gvar_i[t]
      A       = n_i * exp(s_bar) * (1 + var_hat / 2)   second-order mass estimate
      S       = A * var_hat / 2                        practical residual score
      Z_hat   = sum_i A_i
      group score of block i = sum over h in g of S_{h,i} / Z_hat_h

    Exponentials are taken relative to the head's largest s_bar; the shift
    cancels in S / Z_hat.
    """
    Hq, d = q.shape
    M, Hkv, _ = summ.mean_k.shape
    G = Hq // Hkv
    tau = 1.0 / math.sqrt(d)
    n = summ.count.astype(np.float64)
    s_bar = np.zeros((Hq, M))
    var_hat = np.zeros((Hq, M))
    log_mass_hat = np.zeros((Hq, M))
    log_z_hat = np.zeros(Hq)
    head_score = np.zeros((Hq, M))
    for h in range(Hq):
        g = h // G
        s_bar[h] = tau * (summ.mean_k[:, g, :] @ q[h])
        qn = (q[h].reshape(r, d // r) ** 2).sum(axis=1)          # |q_{C_t}|^2
        var_hat[h] = tau * tau * (summ.gvar[:, g, :] @ qn)
        c = s_bar[h].max()
        mass = n * np.exp(s_bar[h] - c) * (1.0 + var_hat[h] / 2.0)   # A * e^{-c}
        z = mass.sum()                                               # Z_hat * e^{-c}
        score = mass * var_hat[h] / 2.0                              # S * e^{-c}
        head_score[h] = score / z
        with np.errstate(divide="ignore"):
            log_mass_hat[h] = np.log(mass) + c
        log_z_hat[h] = math.log(z) + c
    group_score = np.zeros((Hkv, M))
    for h in range(Hq):
        group_score[h // G] += head_score[h]
    return Scores(s_bar, var_hat, log_mass_hat, log_z_hat, head_score, group_score)


def exact_block_stats(q: np.ndarray, k: np.ndarray, summ: Summaries, block_size: int):
    """Per-block exact quantities that need the raw keys (oracle-only).

    With exact logits s_j = tau q_h . k_j and Z_h = sum_j exp(s_j):

      mass[h, i]  = sum_{j in block i} exp(s_j) / Z_h           exact attention mass of the block
      resid[h, i] = (sum_{j in block i} exp(s_j) - n_i exp(s_bar_{h,i})) / Z_h
                                                              residual left by Mean compensation
      log_z[h]    = log Z_h

    s_bar comes from the stored mean key, as in the compensation itself.
    """
    Hq, d = q.shape
    L, Hkv, _ = k.shape
    G = Hq // Hkv
    tau = 1.0 / math.sqrt(d)
    M = summ.num_blocks
    mass = np.zeros((Hq, M))
    resid = np.zeros((Hq, M))
    log_z = np.zeros(Hq)
    for h in range(Hq):
        g = h // G
        s = tau * (k[:, g, :] @ q[h])
        c = s.max()
        e = np.exp(s - c)
        z = e.sum()
        s_bar = tau * (summ.mean_k[:, g, :] @ q[h])
        for i in range(M):
            lo, hi = i * block_size, min(L, (i + 1) * block_size)
            blk = e[lo:hi].sum()
            mass[h, i] = blk / z
            resid[h, i] = (blk - summ.count[i] * math.exp(s_bar[i] - c)) / z
        log_z[h] = math.log(z) + c
    return mass, resid, log_z


def group_sum(per_head: np.ndarray, Hkv: int) -> np.ndarray:
    Hq, M = per_head.shape
    G = Hq // Hkv
    out = np.zeros((Hkv, M))
    for h in range(Hq):
        out[h // G] += per_head[h]
    return out


# ---------------------------------------------------------------------------
# Top-k selection under the token budget (reading R7)
# ---------------------------------------------------------------------------


def num_selected_blocks(M: int, budget_tokens: int, block_size: int) -> int:
    return min(M, budget_tokens // block_size)


def select_topk(group_score: np.ndarray, k: int):
    """Per KV head: the k blocks with the largest score, ties to the lower
    block index, returned in ascending index order.

    Also returns, per KV head, the relative gap between the k-th and the
    (k+1)-th largest score (inf when every block is taken), so callers can
    tell a decisive boundary from a near-tie.
    """
    Hkv, M = group_score.shape
    sel = np.zeros((Hkv, k), dtype=np.int64)
    gaps = np.full(Hkv, np.inf)
    idx = np.arange(M)
    for g in range(Hkv):
        order = np.lexsort((idx, -group_score[g]))   # score descending, index ascending
        sel[g] = np.sort(order[:k])
        if 0 < k < M:
            a, b = group_score[g, order[k - 1]], group_score[g, order[k]]
            gaps[g] = (a - b) / max(abs(a), 1e-300)
        elif k == 0 and M > 0:
            gaps[g] = np.inf
    return sel, gaps


# ---------------------------------------------------------------------------
# Exact attention over selected blocks + Mean compensation of the rest
# ([abstract]; [review] Summary: omitted blocks contribute their block-mean
#  logit; the block enters with its token count and carries its mean value)
# ---------------------------------------------------------------------------


def compensated_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, summ: Summaries,
                          selected: np.ndarray, block_size: int, compensate: bool = True):
    """Attention output and log-sum-exp for each query head.

    Selected blocks contribute their tokens exactly: weight exp(s_j), value
    v_j with s_j = tau q . k_j.  Each omitted block contributes (when
    ``compensate``) one term: weight n_i exp(s_bar_i), value mean_v_i.

      out = sum(weights * values) / sum(weights),  lse = log sum(weights)

    With nothing to attend to (k = 0 and no compensation) the output is zero
    and lse is -inf.
    """
    Hq, d = q.shape
    L, Hkv, _ = k.shape
    G = Hq // Hkv
    tau = 1.0 / math.sqrt(d)
    M = summ.num_blocks
    out = np.zeros((Hq, d))
    lse = np.full(Hq, -np.inf)
    for h in range(Hq):
        g = h // G
        sel = [int(i) for i in selected[g]]
        sel_set = set(sel)
        tok = [j for i in sel for j in range(i * block_size, min(L, (i + 1) * block_size))]
        logits = tau * (k[tok, g, :] @ q[h]) if tok else np.zeros(0)
        wlog = [logits]                      # log of each term's weight
        vals = [v[tok, g, :] if tok else np.zeros((0, d))]
        if compensate:
            omitted = np.array([i for i in range(M) if i not in sel_set], dtype=np.int64)
            if omitted.size:
                s_bar = tau * (summ.mean_k[omitted, g, :] @ q[h])     # block-mean logits
                wlog.append(np.log(summ.count[omitted].astype(np.float64)) + s_bar)
                vals.append(summ.mean_v[omitted, g, :])
        wlog = np.concatenate(wlog)
        vals = np.concatenate(vals, axis=0)
        if wlog.size == 0:
            continue
        m = wlog.max()
        w = np.exp(wlog - m)
        l = w.sum()
        out[h] = (w[:, None] * vals).sum(axis=0) / l
        lse[h] = m + math.log(l)
    return out, lse


def dense_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray):
    """Textbook softmax attention of each query head over all tokens."""
    Hq, d = q.shape
    L, Hkv, _ = k.shape
    G = Hq // Hkv
    tau = 1.0 / math.sqrt(d)
    out = np.zeros((Hq, d))
    lse = np.zeros(Hq)
    for h in range(Hq):
        g = h // G
        s = tau * (k[:, g, :] @ q[h])
        m = s.max()
        w = np.exp(s - m)
        out[h] = (w @ v[:, g, :]) / w.sum()
        lse[h] = m + math.log(w.sum())
    return out, lse


# ---------------------------------------------------------------------------
# One decode step for one sequence
# ---------------------------------------------------------------------------

SCORE_MODES = ("compkv", "mass_hat", "residual_exact", "mass_exact")


@dataclasses.dataclass
class StepResult:
    selected: np.ndarray      # [Hkv, k] ascending block ids
    gaps: np.ndarray          # [Hkv] relative k-th / (k+1)-th score gap
    out: np.ndarray           # [Hq, d]
    lse: np.ndarray           # [Hq]
    scores: Scores
    rank_score: np.ndarray    # [Hkv, M] the score that was ranked


def decode_step(q: np.ndarray, k: np.ndarray, v: np.ndarray, summ: Summaries, *,
                budget_tokens: int, block_size: int, r: int, score_mode: str = "compkv",
                compensate: bool = True) -> StepResult:
    """Score, select and attend for one sequence (float64 inputs).

    score_mode:
      "compkv"         group score of the practical residual S / Z_hat (the method)
      "mass_hat"       group score of the estimated mass A / Z_hat
      "residual_exact" group score of the exact residual / Z (oracle only, needs raw keys)
      "mass_exact"     group score of the exact block mass / Z (oracle only)
    """
    Hq = q.shape[0]
    Hkv = k.shape[1]
    sc = block_scores(q, summ, r)
    if score_mode == "compkv":
        rank = sc.group_score
    elif score_mode == "mass_hat":
        rank = group_sum(np.exp(sc.log_mass_hat - sc.log_z_hat[:, None]), Hkv)
    elif score_mode in ("residual_exact", "mass_exact"):
        mass, resid, _ = exact_block_stats(q, k, summ, block_size)
        rank = group_sum(resid if score_mode == "residual_exact" else mass, Hkv)
    else:
        raise ValueError(score_mode)
    kk = num_selected_blocks(summ.num_blocks, budget_tokens, block_size)
    sel, gaps = select_topk(rank, kk)
    out, lse = compensated_attention(q, k, v, summ, sel, block_size, compensate)
    return StepResult(sel, gaps, out, lse, sc, rank)


# ---------------------------------------------------------------------------
# Batched helpers over the storage arrays of a paged workload
# ---------------------------------------------------------------------------


def sequence_arrays(q_store, k_store, v_store, dtype: str):
    """Widen one sequence's storage arrays to float64."""
    return widen(q_store, dtype), widen(k_store, dtype), widen(v_store, dtype)


def kl_divergence(p_hat: np.ndarray, p: np.ndarray) -> float:
    """KL(p_hat || p) = sum p_hat log(p_hat / p) over the support of p_hat."""
    m = p_hat > 0
    return float((p_hat[m] * (np.log(p_hat[m]) - np.log(p[m]))).sum())


# ---------------------------------------------------------------------------
# Selection fidelity ([review Strengths]: App. B.1 compares ranking blocks by
# the exact residual with ranking them by attention mass, through the KL
# divergence to exact attention and the relative L2 error of the output;
# App. B.2 measures how well the practical score tracks the exact residual,
# by rank correlation and by the share of the best attainable residual that
# its selection keeps)
# ---------------------------------------------------------------------------


def token_distribution(q: np.ndarray, k: np.ndarray, summ: Summaries, selected: np.ndarray,
                       block_size: int, h: int, compensate: bool = True) -> np.ndarray:
    """Attention distribution of query head h over all L tokens under a
    selection: a token of a selected block keeps its weight exp(s_j); every
    token of an omitted block gets its block's mean-key weight exp(s_bar)
    (Mean compensation) or weight zero (no compensation).  Normalised."""
    Hq, d = q.shape
    L, Hkv, _ = k.shape
    g = h // (Hq // Hkv)
    tau = 1.0 / math.sqrt(d)
    logit = tau * (k[:, g, :] @ q[h])
    blk = np.arange(L) // block_size
    chosen = np.zeros(summ.num_blocks, dtype=bool)
    chosen[np.asarray(selected[g], dtype=np.int64)] = True
    if compensate:
        s_bar = tau * (summ.mean_k[:, g, :] @ q[h])
        logit = np.where(chosen[blk], logit, s_bar[blk])
    else:
        logit = np.where(chosen[blk], logit, -np.inf)
    if not np.isfinite(logit).any():
        return np.zeros(L)
    w = np.exp(logit - logit.max())
    return w / w.sum()


def dense_distribution(q: np.ndarray, k: np.ndarray, h: int) -> np.ndarray:
    """Softmax of query head h's exact logits over all tokens."""
    Hq, d = q.shape
    g = h // (Hq // k.shape[1])
    s = (k[:, g, :] @ q[h]) / math.sqrt(d)
    w = np.exp(s - s.max())
    return w / w.sum()


@dataclasses.dataclass
class Fidelity:
    kl: np.ndarray       # [Hq] KL(p_hat || p) against exact attention
    rel_l2: np.ndarray   # [Hq] ||out - out_dense||_2 / ||out_dense||_2


def selection_fidelity(q: np.ndarray, k: np.ndarray, v: np.ndarray, summ: Summaries,
                       selected: np.ndarray, block_size: int, compensate: bool = True,
                       dense=None) -> Fidelity:
    """How far one selection (with or without Mean compensation) lands from
    exact attention, per query head.  ``dense`` may pass in a previous
    ``dense_attention`` result."""
    Hq = q.shape[0]
    out, _ = compensated_attention(q, k, v, summ, selected, block_size, compensate)
    d_out, _ = dense if dense is not None else dense_attention(q, k, v)
    kl = np.array([kl_divergence(token_distribution(q, k, summ, selected, block_size, h, compensate),
                                 dense_distribution(q, k, h)) for h in range(Hq)])
    rel = np.linalg.norm(out - d_out, axis=1) / np.linalg.norm(d_out, axis=1)
    return Fidelity(kl, rel)


def average_ranks(x: np.ndarray) -> np.ndarray:
    """Ranks 1..n in ascending order of x; equal values share the mean of the
    ranks they span."""
    x = np.asarray(x, dtype=np.float64)
    order = np.argsort(x, kind="stable")
    xs = x[order]
    ranks = np.empty(x.size)
    i = 0
    while i < x.size:
        j = i
        while j + 1 < x.size and xs[j + 1] == xs[i]:
            j += 1
        ranks[order[i:j + 1]] = 0.5 * (i + j) + 1.0
        i = j + 1
    return ranks


def spearman(a: np.ndarray, b: np.ndarray) -> float:
    """Spearman rank correlation: the Pearson correlation of the two
    samples' average ranks."""
    ra, rb = average_ranks(a), average_ranks(b)
    ra -= ra.mean()
    rb -= rb.mean()
    return float((ra * rb).sum() / math.sqrt((ra * ra).sum() * (rb * rb).sum()))


def residual_capture(resid: np.ndarray, selected: np.ndarray) -> np.ndarray:
    """Per KV head: the exact residual the selection keeps, as a share of the
    most any selection of the same size can keep (the top-k by the exact
    residual).  ``resid`` is [Hkv, M], e.g. the group sum of resid / Z."""
    Hkv = resid.shape[0]
    out = np.zeros(Hkv)
    for g in range(Hkv):
        sel = np.asarray(selected[g], dtype=np.int64)
        best = np.sort(resid[g])[::-1][:sel.size].sum()
        out[g] = resid[g, sel].sum() / best if best > 0 else 1.0
    return out
