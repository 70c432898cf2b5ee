"""The seeded input generator: determinism, storage conversion, paged layout."""
import numpy as np
import torch

from compensated_kv_selection_amd import workloads as W


def test_bf16_conversion_matches_torch():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(100_000), rng.standard_normal(1000) * 1e-35,
                        rng.standard_normal(1000) * 1e35]).astype(np.float32)
    bits = W.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(bits, ref)
    back = W.bf16_bits_to_f32(bits)
    np.testing.assert_array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_generator_is_deterministic_and_seeded():
    a = W.make_decode_inputs(seq_lens=[100, 37], num_q_heads=4, num_kv_heads=2, head_dim=16,
                             n_needles=2, n_outliers=2, seed=3)
    b = W.make_decode_inputs(seq_lens=[100, 37], num_q_heads=4, num_kv_heads=2, head_dim=16,
                             n_needles=2, n_outliers=2, seed=3)
    c = W.make_decode_inputs(seq_lens=[100, 37], num_q_heads=4, num_kv_heads=2, head_dim=16,
                             n_needles=2, n_outliers=2, seed=4)
    np.testing.assert_array_equal(a.q, b.q)
    np.testing.assert_array_equal(a.k_tokens[1], b.k_tokens[1])
    np.testing.assert_array_equal(a.block_table, b.block_table)
    assert not np.array_equal(a.k_tokens[0], c.k_tokens[0])


def test_paged_cache_round_trip_and_nan_fill():
    w = W.make_decode_inputs(seq_lens=[100, 37, 16], num_q_heads=4, num_kv_heads=2, head_dim=16,
                             n_needles=1, n_outliers=1, seed=5, extra_capacity_tokens=20)
    kc, vc = w.paged_cache()
    assert kc.shape == (w.num_pages, 2, 16, 16)
    used = set()
    for b in range(w.batch):
        L = int(w.seq_lens[b])
        for t in range(L):
            p = w.block_table[b, t // 16]
            np.testing.assert_array_equal(kc[p, :, t % 16, :], w.k_tokens[b][t])
            np.testing.assert_array_equal(vc[p, :, t % 16, :], w.v_tokens[b][t])
        for i in range(-(-L // 16)):
            used.add(int(w.block_table[b, i]))
        tail = L % 16
        if tail:
            p = w.block_table[b, L // 16]
            assert np.all(kc[p, :, tail:, :] == W.BF16_NAN_BITS)
    # pages are a permutation: no page mapped twice
    mapped = w.block_table[w.block_table >= 0]
    assert len(set(mapped.tolist())) == mapped.size
    assert mapped.max() < w.num_pages


def test_needles_and_outliers_planted():
    w = W.make_decode_inputs(seq_lens=[512], num_q_heads=8, num_kv_heads=2, head_dim=32,
                             n_needles=4, n_outliers=4, seed=6)
    k = W.bf16_bits_to_f32(w.k_tokens[0]).astype(np.float64)
    q = W.bf16_bits_to_f32(w.q[0]).astype(np.float64)
    for g in range(2):
        for j, i in enumerate(w.needles[0][g]):
            h = g * 4 + j % 4
            blk = k[i * 16:(i + 1) * 16, g, :]
            # needle keys are 0.5 q_h + 0.3 noise: strongly aligned with q_h
            cos = (blk @ q[h]) / (np.linalg.norm(blk, axis=1) * np.linalg.norm(q[h]))
            assert cos.mean() > 0.7
        och = w.outlier_channels[0][g]
        non_needle = np.ones(512, bool)
        for i in w.needles[0][g]:
            non_needle[i * 16:(i + 1) * 16] = False
        std = k[non_needle, g, :].std(axis=0)
        assert np.all(std[och] > 5) and np.median(std) < 1.5


def test_presets_shapes():
    w = W.make_preset("tiny", seed=0)
    assert w.dtype == "f32" and w.q.dtype == np.float32
    assert w.num_q_heads == 1 and w.head_dim == 64 and int(w.seq_lens[0]) == 4096
    assert w.budget_tokens // w.block_size == 16 and len(w.needles[0][0]) == 4
    lens = W.ragged_lengths(16, seed=0)
    assert len(lens) == 16 and min(lens) >= 16384 and max(lens) <= 65536


def test_append_steps():
    w = W.make_decode_inputs(seq_lens=[32], num_q_heads=2, num_kv_heads=1, head_dim=16,
                             n_needles=0, n_outliers=1, seed=7, extra_capacity_tokens=17)
    steps = W.make_append_steps(w, 3, seed=8)
    for s in steps:
        W.append_tokens(w, s)
    assert int(w.seq_lens[0]) == 35 and w.k_tokens[0].shape[0] == 35
    np.testing.assert_array_equal(w.k_tokens[0][-1], steps[-1].k_new[0])
