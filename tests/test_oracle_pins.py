"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: a closed
form, a textbook or library routine (torch's bf16 rounding, torch's
scaled-dot-product attention, scipy's softmax), a brute-force search, or an
identity the pages state (CompKV review, evolve.pub: "Summary", "Strengths"
App. A.1-A.5, FAQ).  They run on the CPU only.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch
from scipy.special import logsumexp, softmax

from oracle import compkv_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_problem(seed, L=37, Hq=4, Hkv=2, d=16, spread=1.0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((Hq, d))
    k = rng.standard_normal((L, Hkv, d)) * spread
    v = rng.standard_normal((L, Hkv, d))
    return q, k, v


def token_logits(q, k, h, G):
    d = q.shape[1]
    return (k[:, h // G, :] @ q[h]) / math.sqrt(d)


def compensated_token_distribution(q, k, h, G, selected_blocks, b, compensate=True):
    """Token-level construction, independent of the oracle: every token of an
    omitted block gets the mean of its block's exact logits (Mean
    compensation); without compensation omitted tokens get zero weight."""
    s = token_logits(q, k, h, G).copy()
    L = s.shape[0]
    M = -(-L // b)
    keep = np.zeros(L, dtype=bool)
    for i in range(M):
        lo, hi = i * b, min(L, (i + 1) * b)
        if i in selected_blocks:
            keep[lo:hi] = True
        else:
            s[lo:hi] = s[lo:hi].mean()
    if compensate:
        return softmax(s), logsumexp(s)
    s_sel = np.where(keep, s, -np.inf)
    return softmax(s_sel), logsumexp(s_sel)


# ---------------------------------------------------------------------------
# Storage rounding
# ---------------------------------------------------------------------------


def test_bf16_rounding_matches_torch_on_float32_values():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(200_000).astype(np.float32),
        (rng.standard_normal(50_000) * 1e-30).astype(np.float32),
        (rng.standard_normal(50_000) * 1e30).astype(np.float32),
        np.array([0.0, -0.0, 1.0, -1.0], dtype=np.float32),
    ])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = O.round_bf16(x.astype(np.float64))
    np.testing.assert_array_equal(got, ref)


def test_bf16_rounding_ties_and_single_rounding():
    # spacing of bf16 on [1, 2) is 2^-7
    assert O.round_bf16(np.array(1 + 2.0 ** -8))[()] == 1.0               # tie -> even (down)
    assert O.round_bf16(np.array(1 + 3 * 2.0 ** -8))[()] == 1 + 2.0 ** -6  # tie -> even (up)
    assert O.round_bf16(np.array(-(1 + 3 * 2.0 ** -8)))[()] == -(1 + 2.0 ** -6)
    # just above a tie: one rounding from float64 goes up; rounding through
    # float32 first would land on the tie and then go down to 1.0
    assert O.round_bf16(np.array(1 + 2.0 ** -8 + 2.0 ** -40))[()] == 1 + 2.0 ** -7


# ---------------------------------------------------------------------------
# Summaries: closed forms, footprint, bulk == appends (review Summary, FAQ)
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("n", [16, 5, 1])
def test_summary_closed_forms_arithmetic_progression(n):
    d, r, H = 8, 4, 2
    j = np.arange(n, dtype=np.float64)
    a = np.linspace(-1, 1, H * d).reshape(H, d)
    s = np.linspace(0.25, 2.0, H * d).reshape(H, d)
    k = a[None] + j[:, None, None] * s[None]          # k_j = a + j s
    v = 2.0 * a[None] - j[:, None, None] * s[None]
    summ = O.build_summaries(k, v, block_size=16, r=r, kv_dtype="f64")
    mu_expected = a + s * (n - 1) / 2.0
    var_expected = s ** 2 * (n * n - 1) / 12.0         # population variance of an AP
    gvar_expected = var_expected.reshape(H, r, d // r).mean(axis=2)
    np.testing.assert_allclose(summ.mean_k[0], mu_expected, rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(summ.mean_v[0], 2 * a - s * (n - 1) / 2.0, rtol=1e-14, atol=1e-14)
    # gvar is stored in f32
    np.testing.assert_allclose(summ.gvar[0], gvar_expected, rtol=2 ** -24, atol=1e-30)
    assert summ.count[0] == n


def test_summary_rounding_to_bf16_and_f32():
    rng = np.random.default_rng(3)
    k = np.round(rng.standard_normal((16, 1, 8)) * 64) / 64      # exact means in float32
    v = np.round(rng.standard_normal((16, 1, 8)) * 64) / 64
    sb = O.build_summaries(k, v, 16, 2, "bf16")
    mean = k.sum(0) / 16
    ref = torch.from_numpy(mean.astype(np.float32)).to(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(sb.mean_k[0], ref)
    sf = O.build_summaries(k, v, 16, 2, "f32")
    np.testing.assert_array_equal(sf.mean_k[0], mean.astype(np.float32).astype(np.float64))


def test_footprint_is_2d_plus_r_plus_1():
    for d, r in [(128, 4), (64, 4), (128, 1), (128, 128)]:
        assert O.scalars_per_block(d, r) == 2 * d + r + 1
        k = np.zeros((16, 1, d))
        s = O.build_summaries(k, k, 16, r, "f64")
        per_block = s.mean_k[0].size + s.mean_v[0].size + s.gvar[0].size + 1
        assert per_block == 2 * d + r + 1


def test_bulk_equals_chain_of_appends():
    q, k, v = rand_problem(5, L=53)
    bulk = O.build_summaries(k, v, 16, 4, "bf16")
    summ = None
    for L in range(1, 54):
        summ = O.append_summaries(summ, k[:L], v[:L], 16, 4, "bf16")
    np.testing.assert_array_equal(summ.mean_k, bulk.mean_k)
    np.testing.assert_array_equal(summ.mean_v, bulk.mean_v)
    np.testing.assert_array_equal(summ.gvar, bulk.gvar)
    np.testing.assert_array_equal(summ.count, bulk.count)


# ---------------------------------------------------------------------------
# Scores
# ---------------------------------------------------------------------------


def test_block_mean_logit_is_mean_of_token_logits():
    # Linearity: tau q . mean(k) equals the mean of the block's exact logits.
    q, k, v = rand_problem(7, L=45, Hq=4, Hkv=2, d=16)
    summ = O.build_summaries(k, v, 8, 4, "f64")
    sc = O.block_scores(q, summ, 4)
    for h in range(4):
        s = token_logits(q, k, h, 2)
        for i in range(summ.num_blocks):
            assert sc.s_bar[h, i] == pytest.approx(s[i * 8:(i + 1) * 8].mean(), abs=1e-13)


def test_grouped_variance_exact_when_r_equals_d_and_one_channel_varies():
    # With r = d and deviations confined to one channel, the key covariance
    # is diagonal, so the grouped estimate is the exact within-block logit variance.
    rng = np.random.default_rng(11)
    d, b, M = 8, 6, 5
    q = rng.standard_normal((1, d))
    k = np.zeros((M * b, 1, d))
    for i in range(M):
        base = rng.standard_normal(d)
        c = i % d
        k[i * b:(i + 1) * b, 0, :] = base
        k[i * b:(i + 1) * b, 0, c] += rng.standard_normal(b) * (i + 1)
    summ = O.build_summaries(k, k, b, d, "f64")
    sc = O.block_scores(q, summ, d)
    s = token_logits(q, k, 0, 1)
    for i in range(M):
        exact = np.var(s[i * b:(i + 1) * b])
        assert sc.var_hat[0, i] == pytest.approx(exact, rel=1e-6)   # gvar is stored in f32


def test_grouped_variance_r1_closed_form():
    q, k, v = rand_problem(13, L=32, Hq=2, Hkv=1, d=16)
    summ = O.build_summaries(k, v, 16, 1, "f64")
    sc = O.block_scores(q, summ, 1)
    for h in range(2):
        for i in range(2):
            blk = k[i * 16:(i + 1) * 16, 0, :]
            mean_var = np.var(blk, axis=0).mean()
            expected = (q[h] @ q[h]) / 16 * mean_var       # tau^2 |q|^2 mean_c var_c
            assert sc.var_hat[h, i] == pytest.approx(expected, rel=1e-6)


def test_second_order_residual_and_score_limit():
    # Review "Strengths" (App. A.2-A.3, Eqs. 5-7): the residual of an omitted
    # block is mass x within-block logit variance / 2 to leading order.
    rng = np.random.default_rng(21)
    d, b, M = 8, 16, 6
    q = rng.standard_normal((1, d))
    base = rng.standard_normal((M, d))
    eta = np.zeros((M, b, d))
    for i in range(M):
        eta[i, :, i % d] = rng.standard_normal(b)          # one channel varies: var_hat exact (r = d)
    prev_r = prev_s = None
    for eps in (1e-1, 1e-2, 1e-3):
        k = (base[:, None, :] + eps * eta).reshape(M * b, 1, d)
        summ = O.build_summaries(k, k, b, d, "f64")
        sc = O.block_scores(q, summ, d)
        mass, resid, log_z = O.exact_block_stats(q, k, summ, b)
        R = resid[0] * math.exp(log_z[0])                 # unnormalized residual
        s = token_logits(q, k, 0, 1).reshape(M, b)
        sigma2 = s.var(axis=1)
        lead = b * np.exp(s.mean(axis=1)) * sigma2 / 2
        dev_r = np.abs(R / lead - 1).max()
        S_hat = sc.head_score[0] * math.exp(sc.log_z_hat[0])
        dev_s = np.abs(S_hat / R - 1).max()
        if prev_r is not None:
            assert dev_r < prev_r / 5 and dev_s < prev_s / 5      # converges with eps
        prev_r, prev_s = dev_r, dev_s
    assert dev_r < 5e-3 and dev_s < 5e-3


def test_second_order_mass_estimate_is_more_accurate_than_first_order():
    rng = np.random.default_rng(22)
    d, b, M = 8, 16, 4
    q = rng.standard_normal((1, d))
    base = rng.standard_normal((M, d))
    eta = np.zeros((M, b, d))
    for i in range(M):
        eta[i, :, i] = rng.standard_normal(b)
    k = (base[:, None, :] + 0.05 * eta).reshape(M * b, 1, d)
    summ = O.build_summaries(k, k, b, d, "f64")
    sc = O.block_scores(q, summ, d)
    mass, resid, log_z = O.exact_block_stats(q, k, summ, b)
    true_mass = mass[0] * math.exp(log_z[0])
    A2 = np.exp(sc.log_mass_hat[0])
    A1 = summ.count * np.exp(sc.s_bar[0])
    assert np.all(np.abs(A2 / true_mass - 1) < np.abs(A1 / true_mass - 1) / 10)


def test_group_score_sums_normalized_head_scores():
    # Reading R6: the group score is the sum over the KV head's query heads of
    # S_h / Z_hat_h, each head taken on its own as a one-head problem.
    q, k, v = rand_problem(17, L=64, Hq=6, Hkv=2, d=16)
    summ = O.build_summaries(k, v, 8, 4, "bf16")
    sc = O.block_scores(q, summ, 4)
    for g in range(2):
        total = np.zeros(summ.num_blocks)
        for h in range(3 * g, 3 * g + 3):
            sub = O.Summaries(summ.mean_k[:, g:g + 1], summ.mean_v[:, g:g + 1],
                              summ.gvar[:, g:g + 1], summ.count)
            one = O.block_scores(q[h:h + 1], sub, 4)
            A = summ.count * np.exp(one.s_bar[0]) * (1 + one.var_hat[0] / 2)
            total += A * one.var_hat[0] / 2 / A.sum()
        np.testing.assert_allclose(sc.group_score[g], total, rtol=1e-12)


# ---------------------------------------------------------------------------
# Attention with Mean compensation
# ---------------------------------------------------------------------------


def torch_dense(q, k, v):
    Hq, d = q.shape
    G = Hq // k.shape[1]
    kk = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(G, dim=0)   # [Hq, L, d]
    vv = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(G, dim=0)
    qq = torch.from_numpy(q)[:, None, :]
    out = torch.nn.functional.scaled_dot_product_attention(qq[None], kk[None], vv[None])[0, :, 0]
    lse = torch.logsumexp((kk @ qq.transpose(1, 2))[..., 0] / math.sqrt(d), dim=-1)
    return out.numpy(), lse.numpy()


@pytest.mark.parametrize("mode", O.SCORE_MODES)
@pytest.mark.parametrize("compensate", [True, False])
def test_full_budget_is_dense_attention(mode, compensate):
    q, k, v = rand_problem(23, L=37, Hq=4, Hkv=2, d=16)
    summ = O.build_summaries(k, v, 4, 4, "bf16")
    res = O.decode_step(q, k, v, summ, budget_tokens=40, block_size=4, r=4,
                        score_mode=mode, compensate=compensate)
    assert res.selected.shape == (2, 10)
    ref_out, ref_lse = torch_dense(q, k, v)
    np.testing.assert_allclose(res.out, ref_out, atol=1e-12)
    np.testing.assert_allclose(res.lse, ref_lse, atol=1e-12)
    o2, l2 = O.dense_attention(q, k, v)
    np.testing.assert_allclose(o2, ref_out, atol=1e-12)
    np.testing.assert_allclose(l2, ref_lse, atol=1e-12)


@pytest.mark.parametrize("seed", range(4))
def test_compensated_output_equals_token_level_construction(seed):
    q, k, v = rand_problem(100 + seed, L=45, Hq=4, Hkv=2, d=16)
    b = 4
    summ = O.build_summaries(k, v, b, 4, "f64")
    for budget in (0, 8, 20):
        res = O.decode_step(q, k, v, summ, budget_tokens=budget, block_size=b, r=4)
        for h in range(4):
            p_hat, lse = compensated_token_distribution(q, k, h, 2, set(res.selected[h // 2]), b)
            np.testing.assert_allclose(res.out[h], p_hat @ v[:, h // 2, :], atol=1e-12)
            assert res.lse[h] == pytest.approx(lse, abs=1e-12)


@pytest.mark.parametrize("seed", range(4))
def test_uncompensated_output_is_softmax_over_selected_tokens(seed):
    q, k, v = rand_problem(200 + seed, L=45, Hq=4, Hkv=2, d=16)
    b = 4
    summ = O.build_summaries(k, v, b, 4, "f64")
    res = O.decode_step(q, k, v, summ, budget_tokens=16, block_size=b, r=4, compensate=False)
    for h in range(4):
        p_hat, lse = compensated_token_distribution(q, k, h, 2, set(res.selected[h // 2]), b,
                                                    compensate=False)
        np.testing.assert_allclose(res.out[h], p_hat @ v[:, h // 2, :], atol=1e-12)
        assert res.lse[h] == pytest.approx(lse, abs=1e-12)


def test_nothing_to_attend_gives_zero_and_minus_inf():
    q, k, v = rand_problem(9, L=20, Hq=2, Hkv=1, d=8)
    summ = O.build_summaries(k, v, 4, 4, "f64")
    res = O.decode_step(q, k, v, summ, budget_tokens=0, block_size=4, r=4, compensate=False)
    assert np.all(res.out == 0) and np.all(np.isneginf(res.lse))


@pytest.mark.parametrize("seed", range(3))
def test_exact_kl_identity(seed):
    # Review "Strengths", App. A.1: KL(p_hat || p) = log Z - log Z_hat >= 0.
    q, k, v = rand_problem(300 + seed, L=48, Hq=2, Hkv=1, d=16, spread=1.5)
    b = 4
    summ = O.build_summaries(k, v, b, 4, "f64")
    dense_out, dense_lse = torch_dense(q, k, v)
    for budget in (0, 12, 24):
        res = O.decode_step(q, k, v, summ, budget_tokens=budget, block_size=b, r=4)
        for h in range(2):
            p = softmax(token_logits(q, k, h, 2))
            p_hat, _ = compensated_token_distribution(q, k, h, 2, set(res.selected[0]), b)
            kl = O.kl_divergence(p_hat, p)
            assert kl == pytest.approx(dense_lse[h] - res.lse[h], abs=1e-12)
            assert kl >= -1e-15 and res.lse[h] <= dense_lse[h] + 1e-12


def _brute_force_best(q, k, b, M, kk, compensate):
    p = softmax(token_logits(q, k, 0, 1))
    kls = {}
    for sub in itertools.combinations(range(M), kk):
        p_hat, _ = compensated_token_distribution(q, k, 0, 1, set(sub), b, compensate)
        kls[sub] = O.kl_divergence(p_hat, p)
    ranked = sorted(kls.items(), key=lambda t: t[1])
    return ranked[0][0], ranked[0][1], ranked[1][1]


@pytest.mark.parametrize("seed", range(6))
def test_brute_force_min_kl_is_exact_residual_topk(seed):
    # Minimizing KL under Mean compensation = taking the k largest exact residuals.
    rng = np.random.default_rng(400 + seed)
    d, b, M, kk = 6, 4, 8, 3
    q = rng.standard_normal((1, d))
    k = (rng.standard_normal((M * b, 1, d)) * rng.uniform(0.2, 2.0, size=(M * b, 1, 1)))
    v = rng.standard_normal((M * b, 1, d))
    summ = O.build_summaries(k, v, b, d, "f64")
    best, kl0, kl1 = _brute_force_best(q, k, b, M, kk, True)
    assert kl1 - kl0 > 1e-9 * max(kl0, 1e-12)
    res = O.decode_step(q, k, v, summ, budget_tokens=kk * b, block_size=b, r=d,
                        score_mode="residual_exact")
    assert tuple(res.selected[0]) == best
    assert res.lse[0] == pytest.approx(torch_dense(q, k, v)[1][0] - kl0, abs=1e-12)


@pytest.mark.parametrize("seed", range(6))
def test_without_compensation_min_kl_is_mass_topk(seed):
    # Review "Key claims"/"Strengths", App. A.5: removing Mean compensation
    # recovers attention-mass Top-K.
    rng = np.random.default_rng(500 + seed)
    d, b, M, kk = 6, 4, 8, 3
    q = rng.standard_normal((1, d))
    k = (rng.standard_normal((M * b, 1, d)) * rng.uniform(0.2, 2.0, size=(M * b, 1, 1)))
    v = rng.standard_normal((M * b, 1, d))
    summ = O.build_summaries(k, v, b, d, "f64")
    best, kl0, kl1 = _brute_force_best(q, k, b, M, kk, False)
    assert kl1 - kl0 > 1e-9 * max(kl0, 1e-12)
    res = O.decode_step(q, k, v, summ, budget_tokens=kk * b, block_size=b, r=d,
                        score_mode="mass_exact", compensate=False)
    assert tuple(res.selected[0]) == best


def test_mass_and_residual_rankings_can_differ():
    # The case the pages argue from: the two optimal sets differ for some inputs.
    differ = 0
    for seed in range(20):
        rng = np.random.default_rng(600 + seed)
        d, b, M, kk = 6, 4, 8, 3
        q = rng.standard_normal((1, d))
        k = (rng.standard_normal((M * b, 1, d)) * rng.uniform(0.2, 2.0, size=(M * b, 1, 1)))
        v = rng.standard_normal((M * b, 1, d))
        summ = O.build_summaries(k, v, b, d, "f64")
        a = O.decode_step(q, k, v, summ, budget_tokens=12, block_size=b, r=d, score_mode="residual_exact")
        m = O.decode_step(q, k, v, summ, budget_tokens=12, block_size=b, r=d, score_mode="mass_exact")
        differ += int(tuple(a.selected[0]) != tuple(m.selected[0]))
    assert differ > 0


def test_constant_key_blocks_make_compensation_exact():
    rng = np.random.default_rng(31)
    d, b, M, Hq, Hkv = 8, 4, 9, 4, 2
    q = rng.standard_normal((Hq, d))
    # float32-representable keys (as the caches hold): a block's sum of equal
    # rows is exact in float64, so its mean is that row exactly
    keys = rng.standard_normal((M, Hkv, d)).astype(np.float32).astype(np.float64)
    k = np.repeat(keys, b, axis=0)[: M * b - 1]          # ragged tail block
    v = rng.standard_normal((M * b - 1, Hkv, d))
    summ = O.build_summaries(k, v, b, 4, "f64")
    ref_out, ref_lse = torch_dense(q, k, v)
    for budget in (0, 4, 12, 36):
        res = O.decode_step(q, k, v, summ, budget_tokens=budget, block_size=b, r=4)
        assert np.all(res.rank_score == 0)
        kk = budget // b
        np.testing.assert_array_equal(res.selected, np.tile(np.arange(kk), (Hkv, 1)))  # ties -> lowest ids
        np.testing.assert_allclose(res.out, ref_out, atol=1e-12)
        np.testing.assert_allclose(res.lse, ref_lse, atol=1e-12)
        _, resid, _ = O.exact_block_stats(q, k, summ, b)
        assert np.abs(resid).max() < 1e-15


def test_single_token_blocks_make_compensation_exact():
    q, k, v = rand_problem(37, L=11, Hq=2, Hkv=1, d=8)
    summ = O.build_summaries(k, v, 1, 4, "f64")
    assert np.all(summ.gvar == 0)
    ref_out, ref_lse = torch_dense(q, k, v)
    for budget in (0, 3, 11):
        res = O.decode_step(q, k, v, summ, budget_tokens=budget, block_size=1, r=4)
        np.testing.assert_allclose(res.out, ref_out, atol=1e-12)
        np.testing.assert_allclose(res.lse, ref_lse, atol=1e-12)


def test_duplicated_block_ties_to_lower_index():
    rng = np.random.default_rng(41)
    d, b, M = 8, 4, 8
    q = rng.standard_normal((1, d))
    k = rng.standard_normal((M * b, 1, d)) * 0.1
    hot = rng.standard_normal((b, 1, d)) * 3.0 + q[0] / 2
    k[5 * b:6 * b] = hot
    k[2 * b:3 * b] = hot                                  # block 2 duplicates block 5
    v = rng.standard_normal((M * b, 1, d))
    summ = O.build_summaries(k, v, b, 4, "bf16")
    res = O.decode_step(q, k, v, summ, budget_tokens=b, block_size=b, r=4)
    assert res.rank_score[0, 2] == res.rank_score[0, 5]
    assert res.rank_score[0, 2] == res.rank_score[0].max()
    assert list(res.selected[0]) == [2]
    assert res.gaps[0] == 0.0
    res2 = O.decode_step(q, k, v, summ, budget_tokens=2 * b, block_size=b, r=4)
    assert list(res2.selected[0]) == [2, 5]


def test_selection_is_ascending_and_budget_sized():
    q, k, v = rand_problem(43, L=100, Hq=4, Hkv=2, d=16)
    summ = O.build_summaries(k, v, 16, 4, "bf16")
    for budget, kk in ((0, 0), (15, 0), (16, 1), (47, 2), (112, 7), (10_000, 7)):
        res = O.decode_step(q, k, v, summ, budget_tokens=budget, block_size=16, r=4)
        assert res.selected.shape == (2, kk)
        for g in range(2):
            assert np.all(np.diff(res.selected[g]) > 0)
            order = np.lexsort((np.arange(7), -res.rank_score[g]))
            assert set(res.selected[g]) == set(order[:kk])


# ---------------------------------------------------------------------------
# Hand-worked example (tests/golden/hand_example.json)
# ---------------------------------------------------------------------------


def test_hand_worked_example():
    with open(os.path.join(GOLDEN, "hand_example.json")) as f:
        ex = json.load(f)
    q = np.array(ex["q"], dtype=np.float64)
    k = np.array(ex["k"], dtype=np.float64)
    v = np.array(ex["v"], dtype=np.float64)
    b, r, budget = ex["block_size"], ex["r"], ex["budget_tokens"]
    e = math.e
    e15 = math.exp(1.5)
    summ = O.build_summaries(k, v, b, r, "f64")
    np.testing.assert_allclose(summ.mean_k[:, 0], [[1.5, 0], [0, 0]], atol=0)
    np.testing.assert_allclose(summ.mean_v[:, 0], [[2, 0], [0, 3]], atol=0)
    np.testing.assert_allclose(summ.gvar[:, 0], [[0, 0], [1, 0]], atol=0)
    sc = O.block_scores(q, summ, r)
    np.testing.assert_allclose(sc.s_bar[0], [1.5, 0], atol=1e-15)
    np.testing.assert_allclose(sc.var_hat[0], [0, 1], atol=1e-15)
    np.testing.assert_allclose(np.exp(sc.log_mass_hat[0]), [2 * e15, 3], rtol=1e-14)
    assert math.exp(sc.log_z_hat[0]) == pytest.approx(2 * e15 + 3, rel=1e-14)
    np.testing.assert_allclose(sc.group_score[0], [0, 1.5 / (2 * e15 + 3)], rtol=1e-14)

    res = O.decode_step(q, k, v, summ, budget_tokens=budget, block_size=b, r=r)
    assert list(res.selected[0]) == [1]
    den = e + 1 / e + 2 * e15
    np.testing.assert_allclose(res.out[0], [4 * e15 / den, (2 * e + 4 / e) / den], rtol=1e-14)
    assert res.lse[0] == pytest.approx(math.log(den), abs=1e-14)

    for mode in ("mass_exact", "mass_hat"):
        rm = O.decode_step(q, k, v, summ, budget_tokens=budget, block_size=b, r=r, score_mode=mode)
        assert list(rm.selected[0]) == [0]
        den_m = 2 * e15 + 2
        np.testing.assert_allclose(rm.out[0], [4 * e15 / den_m, 6 / den_m], rtol=1e-14)
        assert rm.lse[0] == pytest.approx(math.log(den_m), abs=1e-14)
        kl = math.log((2 * e15 + e + 1 / e) / (2 * e15 + 2))
        assert res.lse[0] - rm.lse[0] == pytest.approx(kl, abs=1e-14)

    rr = O.decode_step(q, k, v, summ, budget_tokens=budget, block_size=b, r=r, score_mode="residual_exact")
    assert list(rr.selected[0]) == [1]
    mass, resid, log_z = O.exact_block_stats(q, k, summ, b)
    Z = math.exp(log_z[0])
    np.testing.assert_allclose(resid[0] * Z, [0, e + 1 / e - 2], atol=1e-14)
    np.testing.assert_allclose(mass[0] * Z, [2 * e15, e + 1 / e], rtol=1e-14)


# ---------------------------------------------------------------------------
# Widening of stored values, grouped-variance layout, and the GQA aggregation
# ---------------------------------------------------------------------------


def test_widen_bf16_matches_torch_for_every_bit_pattern():
    # Every one of the 65536 bf16 bit patterns (zeros, subnormals, infinities,
    # both signs) widens to the value torch gives it; NaNs stay NaN.
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    with np.errstate(invalid="ignore"):   # signalling NaN patterns
        got = O.widen(bits, "bf16")
    nan = np.isnan(ref)
    assert nan.sum() == 2 * 127                 # exponent all ones, nonzero fraction, two signs
    np.testing.assert_array_equal(np.isnan(got), nan)
    np.testing.assert_array_equal(got[~nan], ref[~nan])
    assert np.signbit(got[0x8000]) and got[0x8000] == 0.0
    f = np.random.default_rng(1).standard_normal(1000).astype(np.float32)
    np.testing.assert_array_equal(O.widen(f, "f32"), torch.from_numpy(f).to(torch.float64).numpy())


@pytest.mark.parametrize("r", [2, 4])
def test_grouped_variance_exact_for_uncorrelated_group_constant_deviations(r):
    # If a block's key deviations are uncorrelated across channels and have
    # one variance a_t^2 inside each channel group t, the within-block logit
    # variance tau^2 q^T C q is exactly tau^2 sum_t |q_{C_t}|^2 a_t^2, which is
    # what the grouped estimate gives with contiguous groups.  Rows of a
    # Hadamard matrix (zero mean, mutually orthogonal) make the sample
    # covariance exactly diagonal.
    from scipy.linalg import hadamard
    rng = np.random.default_rng(50 + r)
    d, b = 8, 16
    Hm = hadamard(16).astype(np.float64)
    q = rng.standard_normal((1, d))
    a = rng.uniform(0.2, 1.5, size=r)
    base = rng.standard_normal(d)
    dev = np.stack([a[c // (d // r)] * Hm[1 + c] for c in range(d)], axis=1)   # [b, d]
    k = (base[None] + dev)[:, None, :]
    summ = O.build_summaries(k, k, b, r, "f64")
    sc = O.block_scores(q, summ, r)
    exact = np.var(token_logits(q, k, 0, 1))
    assert sc.var_hat[0, 0] == pytest.approx(exact, rel=1e-6)     # gvar is stored in f32
    # teeth: interleaved groups (channel c in group c mod r) would not be exact
    gv_inter = np.array([np.mean([a[c // (d // r)] ** 2 for c in range(t, d, r)]) for t in range(r)])
    qn_inter = np.array([(q[0, t::r] ** 2).sum() for t in range(r)])
    assert abs((qn_inter @ gv_inter) / d - exact) > 1e-3 * exact


def _exact_head_residuals(q, k, h, G, b):
    """Per block, the exact residual R of Mean compensation over the head's
    partition function Z, from the token logits (independent of the oracle):
    R_i = sum_{j in i} e^{s_j} - n_i e^{mean_j s_j}."""
    s = token_logits(q, k, h, G)
    L = s.shape[0]
    M = -(-L // b)
    e = np.exp(s)
    Z = e.sum()
    R = np.array([e[i * b:(i + 1) * b].sum() - min(b, L - i * b) * math.exp(s[i * b:(i + 1) * b].mean())
                  for i in range(M)])
    return R / Z


@pytest.mark.parametrize("G", [2, 4])
def test_group_score_limit_is_the_exact_group_residual(G):
    # Each head's KL under Mean compensation is -log(1 - sum_omitted R_h/Z_h)
    # (review "Strengths", App. A.1), so to first order a block matters to
    # the KV head's query heads through sum_h R_h/Z_h, each head normalised
    # by its own partition function.  With r = d and one varying channel
    # per block the variance estimate is exact, and as the blocks' spread
    # shrinks each head's S_h/Z_hat_h and the group score must approach the
    # exact normalised residuals.  The heads' logit scales differ by 10x, so
    # normalising by a shared Z would not converge.
    rng = np.random.default_rng(700 + G)
    d, b, M, Hkv = 8, 16, 6, 2
    Hq = G * Hkv
    scales = np.geomspace(0.3, 3.0, G)
    q = rng.standard_normal((Hq, d)) * np.tile(scales, Hkv)[:, None]
    base = rng.standard_normal((M, Hkv, d))
    eta = np.zeros((M, b, Hkv, d))
    for i in range(M):
        for g in range(Hkv):
            eta[i, :, g, (i + 2 * g) % d] = rng.standard_normal(b)
    prev_h = prev_g = None
    for eps in (1e-1, 1e-2, 1e-3):
        k = (base[:, None] + eps * eta).reshape(M * b, Hkv, d)
        summ = O.build_summaries(k, k, b, d, "f64")
        sc = O.block_scores(q, summ, d)
        rho = np.zeros((Hkv, M))
        dev_h = 0.0
        for h in range(Hq):
            rh = _exact_head_residuals(q, k, h, G, b)
            dev_h = max(dev_h, float(np.abs(sc.head_score[h] / rh - 1).max()))
            rho[h // G] += rh
        dev_g = float(np.abs(sc.group_score / rho - 1).max())
        if prev_h is not None:
            assert dev_h < prev_h / 5 and dev_g < prev_g / 5      # converges with eps
        prev_h, prev_g = dev_h, dev_g
        # teeth: one Z_hat shared by the group's heads misses the exact sum
        z_hat = np.exp(sc.log_z_hat)
        raw = sc.head_score * z_hat[:, None]
        shared = np.stack([raw[g * G:(g + 1) * G].sum(0) / z_hat[g * G:(g + 1) * G].sum() for g in range(Hkv)])
        assert np.abs(shared / rho - 1).max() > 0.1
    assert dev_h < 5e-3 and dev_g < 5e-3


def test_brute_force_min_group_kl_is_group_score_topk():
    # Two query heads share a KV head and one selection.  Over every k-subset,
    # the subset with the smallest summed KL(p_hat_h || p_h) of the two heads
    # (token-level distributions) is the top-k of the exact group residual
    # sum_h R_h/Z_h, and, with exact variance estimates and small spreads,
    # the oracle's CompKV selection (review "Summary"; "Strengths" App. A.1).
    # The heads' logit scales differ by 5x: ranking by the unnormalised sum
    # of the heads' scores misses the best subset in some of the cases.
    d, b, M, kk, G = 8, 4, 8, 3, 2
    unnormalised_misses = 0
    for seed in range(12):
        rng = np.random.default_rng(800 + seed)
        q = rng.standard_normal((G, d)) * np.array([[0.5], [2.5]])
        base = rng.standard_normal((M, 1, d))
        k = np.repeat(base, b, axis=0).copy()
        for i in range(M):
            k[i * b:(i + 1) * b, 0, i % d] += rng.uniform(0.02, 0.4) * rng.standard_normal(b)
        v = rng.standard_normal((M * b, 1, d))
        summ = O.build_summaries(k, v, b, d, "f64")
        p = [softmax(token_logits(q, k, h, G)) for h in range(G)]
        kls = {}
        for sub in itertools.combinations(range(M), kk):
            kls[sub] = sum(O.kl_divergence(compensated_token_distribution(q, k, h, G, set(sub), b)[0], p[h])
                           for h in range(G))
        ranked = sorted(kls.items(), key=lambda t: t[1])
        best = ranked[0][0]
        assert ranked[1][1] - ranked[0][1] > 1e-3 * ranked[0][1], seed
        rho = sum(_exact_head_residuals(q, k, h, G, b) for h in range(G))
        assert tuple(sorted(np.argsort(-rho)[:kk])) == best, seed
        for mode in ("residual_exact", "compkv"):
            res = O.decode_step(q, k, v, summ, budget_tokens=kk * b, block_size=b, r=d, score_mode=mode)
            assert tuple(res.selected[0]) == best, (seed, mode)
        sc = O.block_scores(q, summ, d)
        raw = (sc.head_score * np.exp(sc.log_z_hat)[:, None]).sum(axis=0)
        unnormalised_misses += tuple(sorted(np.argsort(-raw)[:kk])) != best
    assert unnormalised_misses >= 2
