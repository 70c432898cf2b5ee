"""Selection-fidelity measures (review "Strengths": App. B.1 KL and relative
L2 against exact attention for residual vs mass ranking; App. B.2 Spearman
correlation of the practical score with the exact residual, and residual
capture).

CPU tests pin the measures themselves: the rank correlation against scipy
and its closed form without ties, the token-level KL against the exact
log-partition identity (App. A.1) and, without compensation, against the
log of the kept mass (App. A.5), and the optimality of the exact-residual and
exact-mass selections that the KL must reflect.  The GPU test computes the
same table from the GPU's own selections and scores and checks it against the
oracle's.
"""
import itertools
import math

import numpy as np
import pytest
import scipy.stats

from compensated_kv_selection_amd import workloads as W
from oracle import compkv_oracle as O
import fidelity as F


def _problem(seed, L=64, Hq=4, Hkv=2, d=16, b=4, r=4, spread=1.5):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((Hq, d))
    k = rng.standard_normal((L, Hkv, d)) * rng.uniform(0.2, spread, size=(L, 1, 1))
    v = rng.standard_normal((L, Hkv, d))
    return q, k, v, O.build_summaries(k, v, b, r, "f64")


def test_average_ranks_share_ties():
    assert O.average_ranks(np.array([3.0, 1.0, 3.0, 2.0])).tolist() == [3.5, 1.0, 3.5, 2.0]
    assert O.average_ranks(np.array([5.0, 5.0, 5.0])).tolist() == [2.0, 2.0, 2.0]


@pytest.mark.parametrize("seed", range(4))
def test_spearman_matches_scipy_and_closed_form(seed):
    rng = np.random.default_rng(900 + seed)
    a = rng.integers(0, 12, size=200).astype(float)     # many ties
    b = a + rng.integers(-4, 5, size=200)
    assert O.spearman(a, b) == pytest.approx(scipy.stats.spearmanr(a, b).statistic, abs=1e-12)
    x, y = rng.standard_normal(50), rng.standard_normal(50)   # no ties
    dr = O.average_ranks(x) - O.average_ranks(y)
    n = x.size
    assert O.spearman(x, y) == pytest.approx(1 - 6 * (dr ** 2).sum() / (n * (n * n - 1)), abs=1e-12)
    assert O.spearman(x, np.exp(x)) == pytest.approx(1.0)
    assert O.spearman(x, -x) == pytest.approx(-1.0)


@pytest.mark.parametrize("seed", range(3))
def test_token_kl_is_the_log_partition_gap(seed):
    # App. A.1: with Mean compensation KL(p_hat || p) = log Z - log Z_hat.
    # App. A.5: without it, KL = -log(exact mass of the selected blocks).
    q, k, v, summ = _problem(1000 + seed)
    b, Hkv, G = 4, 2, 2
    dense_out, dense_lse = O.dense_attention(q, k, v)
    rng = np.random.default_rng(seed)
    sel = np.sort(np.stack([rng.choice(summ.num_blocks, 5, replace=False) for _ in range(Hkv)]), axis=1)
    _, lse = O.compensated_attention(q, k, v, summ, sel, b, True)
    f = O.selection_fidelity(q, k, v, summ, sel, b, True)
    assert np.allclose(f.kl, dense_lse - lse, atol=1e-12, rtol=0)
    assert np.all(f.kl > 0)
    f0 = O.selection_fidelity(q, k, v, summ, sel, b, False)
    for h in range(q.shape[0]):
        p = O.dense_distribution(q, k, h)
        kept = sum(p[i * b:(i + 1) * b].sum() for i in sel[h // G])
        assert f0.kl[h] == pytest.approx(-math.log(kept), abs=1e-12)
    out0, _ = O.compensated_attention(q, k, v, summ, sel, b, False)
    rel = np.linalg.norm(out0 - dense_out, axis=1) / np.linalg.norm(dense_out, axis=1)
    assert np.allclose(f0.rel_l2, rel, atol=1e-14, rtol=0)


def test_everything_selected_is_exact():
    q, k, v, summ = _problem(1100, L=30)
    sel = np.tile(np.arange(summ.num_blocks), (2, 1))
    for comp in (True, False):
        f = O.selection_fidelity(q, k, v, summ, sel, 4, comp)
        assert np.all(np.abs(f.kl) < 1e-13) and np.all(f.rel_l2 < 1e-13)


@pytest.mark.parametrize("seed", range(4))
def test_residual_capture_against_every_subset(seed):
    rng = np.random.default_rng(1200 + seed)
    M, kk = 9, 3
    resid = rng.exponential(size=(2, M))
    best = [max(resid[g, list(c)].sum() for c in itertools.combinations(range(M), kk))
            for g in range(2)]
    for c in itertools.combinations(range(M), kk):
        sel = np.array([c, c])
        cap = O.residual_capture(resid, sel)
        assert np.allclose(cap, [resid[g, list(c)].sum() / best[g] for g in range(2)], rtol=1e-14)
        assert np.all(cap <= 1 + 1e-15)
    top, _ = O.select_topk(resid, kk)
    assert np.allclose(O.residual_capture(resid, top), 1.0)


@pytest.mark.parametrize("seed", range(3))
def test_single_head_kl_ranks_the_selections(seed):
    # One query head: the top-k by exact residual has the least compensated
    # KL of all k-subsets (App. A.1), and without compensation the top-k by
    # exact mass has the least KL (App. A.5); every other rule does no better.
    w = W.make_decode_inputs(seq_lens=[2048 + 7 * seed], num_q_heads=1, num_kv_heads=1, head_dim=64,
                             r_groups=4, budget_tokens=128, dtype="bf16", n_needles=4,
                             n_outliers=2, seed=1300 + seed)
    q, k, v = O.sequence_arrays(w.q[0], w.k_tokens[0], w.v_tokens[0], w.dtype)
    summ = O.build_summaries(k, v, 16, 4, w.dtype)
    dense = O.dense_attention(q, k, v)

    def kl(mode, comp):
        st = O.decode_step(q, k, v, summ, budget_tokens=128, block_size=16, r=4, score_mode=mode,
                           compensate=comp)
        return float(O.selection_fidelity(q, k, v, summ, st.selected, 16, comp, dense).kl[0])

    best = kl("residual_exact", True)
    for mode in ("compkv", "mass_hat", "mass_exact"):
        assert best <= kl(mode, True) + 1e-12
    best0 = kl("mass_exact", False)
    for mode in ("compkv", "mass_hat", "residual_exact"):
        assert best0 <= kl(mode, False) + 1e-12


def test_oracle_table_small():
    # A small Llama-shaped case (4 KV heads sharing 16 query heads, d = 128).
    # On this synthetic data CompKV keeps more of the residual and lands
    # closer to exact attention than ranking by estimated mass, with or
    # without compensating the mass-ranked selection.
    w = W.make_decode_inputs(seq_lens=[8192], num_q_heads=16, num_kv_heads=4, head_dim=128,
                             r_groups=4, budget_tokens=256, dtype="bf16", n_needles=8,
                             n_outliers=4, seed=1400)
    rows = F.fidelity_rows(w, r_values=(4, 128))
    print("\n" + F.markdown(rows))
    by = {(x.selection, x.r): x for x in rows}
    assert by[("residual (exact)", None)].capture == pytest.approx(1.0)
    assert by[("residual (exact)", None)].kl <= by[("mass (exact)", None)].kl
    assert by[("mass (exact), no comp.", None)].kl <= by[("mass_hat, no comp.", 4)].kl + 1e-12
    for r in (4, 128):
        ck, mc, mn = by[("CompKV", r)], by[("mass_hat + Mean comp.", r)], by[("mass_hat, no comp.", r)]
        assert ck.kl < mc.kl < mn.kl
        assert ck.capture > mc.capture
        assert ck.spearman > mc.spearman
        assert mc.capture == mn.capture and mc.spearman == mn.spearman   # same selection


@pytest.mark.gpu
def test_gpu_fidelity_sweep():
    """The r sweep on one 32K-token Llama-shaped sequence at a 512-token
    budget, with the GPU's selections and scores, against the oracle's."""
    import torch
    from compensated_kv_selection_amd import compkv as C
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests need an MI355X")
    C.load_library()
    w = F.workload(32768)
    outs = []
    print("[case] fidelity sweep len=32768 budget=512 r=" + ",".join(map(str, F.R_VALUES)), flush=True)
    g_rows = F.fidelity_rows(w, gpu=True, gpu_outputs=outs)
    o_rows = F.fidelity_rows(w, gpu=False)
    print("\n" + F.markdown(g_rows), flush=True)
    assert len(g_rows) == len(o_rows)
    for g, o in zip(g_rows, o_rows):
        assert (g.selection, g.r, g.compensate) == (o.selection, o.r, o.compensate)
        assert g.kl == pytest.approx(o.kl, rel=1e-3)
        assert g.rel_l2 == pytest.approx(o.rel_l2, rel=1e-3)
        assert g.capture == pytest.approx(o.capture, rel=1e-3)
        if o.spearman is not None:
            assert g.spearman == pytest.approx(o.spearman, abs=1e-3)
    for label, r, gout, oout, _ in outs:
        err = float(np.abs(gout - oout).max())
        assert err <= 2e-3, (label, r, err)
    by = {(x.selection, x.r): x for x in g_rows}
    for r in F.R_VALUES:
        ck, mc, mn = by[("CompKV", r)], by[("mass_hat + Mean comp.", r)], by[("mass_hat, no comp.", r)]
        assert ck.kl < mc.kl < mn.kl
        assert ck.capture > mc.capture
