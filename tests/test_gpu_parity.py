"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.  Needs an MI355X and the built library."""
import numpy as np
import pytest
import torch

from compensated_kv_selection_amd import compkv as C
from compensated_kv_selection_amd import workloads as W
from compensated_kv_selection_amd.tensors import dims_of, to_device
from oracle import compkv_oracle as O

from parity_util import (check_group_scores, check_outputs, check_selection_isolated,
                         check_selection_valid, check_selection_vs_oracle, check_summaries,
                         check_workspace_clean, concentrated_blocks_case, duplicated_blocks_case, run_gpu,
                         run_oracle)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests need an MI355X")
    C.load_library()  # raises if libcompkv.so is not built
    yield


def full_check(w, budget=None, score_mode=C.SCORE_COMPKV, compensate=True, fused=None, report=None):
    """Run the case through the three-launch path (fused=False), the
    single-launch step (fused=True) or both (None; the single-launch step
    always compensates) and check each against the oracle."""
    budget = w.budget_tokens if budget is None else budget
    ora = None
    g_first = None
    paths = [False, True] if fused is None else [fused]
    if not compensate:
        paths = [False]
    for fz in paths:
        print(f"[case] {w.name} seed={w.seed} B={w.batch} Hq={w.num_q_heads} Hkv={w.num_kv_heads} "
              f"d={w.head_dim} r={w.r_groups} {w.dtype} lens={list(w.seq_lens)[:6]} budget={budget} "
              f"mode={score_mode} comp={compensate} fused={fz}", flush=True)
        if fz:
            print(f"[case] decode_step launches: {C.decode_step_launches(dims_of(w), budget)}",
                  flush=True)
        g = run_gpu(w, budget, score_mode, compensate, fused=fz)
        if ora is None:
            ora = run_oracle(w, budget, score_mode, compensate)
        check_summaries(w, g, ora)
        if not fz:
            check_selection_isolated(w, g, budget)
            check_group_scores(w, g, ora)
        near = check_selection_vs_oracle(w, g, ora, report)
        err = check_outputs(w, g, ora, compensate)
        print(f"[case] ok: max |out - oracle| = {err:.2e}, near-ties {near}", flush=True)
        g_first = g_first or g
    return g_first, ora


def small_gqa(seed=0, **kw):
    cfg = dict(seq_lens=[1000, 777, 16, 1, 4097], num_q_heads=8, num_kv_heads=2, head_dim=128,
               r_groups=4, budget_tokens=128, dtype="bf16", n_needles=0, n_outliers=2, seed=seed)
    cfg.update(kw)
    return W.make_decode_inputs(name="small_gqa", **cfg)


@pytest.mark.parametrize("seed", range(5))
def test_tiny_single_head_f32(seed):
    full_check(W.make_preset("tiny", seed=seed))


@pytest.mark.parametrize("seed", range(3))
def test_small_gqa_ragged_bf16(seed):
    full_check(small_gqa(seed))


@pytest.mark.parametrize("r", [4, 8])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_every_kernel_instance(dtype, d, G, r):
    # Every instance the library builds - dtype x head_dim x query heads per
    # KV head x (r = 4, other r) - through the three-launch path and the
    # single launch, against the oracle.  Lengths give several chunks of 256
    # blocks, a ragged tail and a one-chunk sequence.
    w = W.make_decode_inputs(name=f"inst_{dtype}_d{d}_G{G}_r{r}", seq_lens=[70000, 2500, 333],
                             num_q_heads=2 * G, num_kv_heads=2, head_dim=d, r_groups=r, budget_tokens=160,
                             dtype=dtype, n_needles=3, n_outliers=1, seed=G * 10 + d + r)
    full_check(w)


@pytest.mark.parametrize("r", [1, 2, 8, 16, 64, 128])
def test_r_groups(r):
    full_check(small_gqa(seed=7, r_groups=r))


@pytest.mark.parametrize("budget", [0, 15, 16, 48, 4096, 100_000])
def test_budget_edges(budget):
    # 0 and 15: nothing selected, every block compensated; 4096+: every block
    # of the shorter sequences selected (dense); 100000: all blocks, all sequences.
    full_check(small_gqa(seed=3), budget=budget)


@pytest.mark.parametrize("budget", [0, 64, 100_000])
def test_without_compensation(budget):
    full_check(small_gqa(seed=4), budget=budget, compensate=False)


@pytest.mark.parametrize("budget", [64, 256])
def test_mass_score_mode(budget):
    full_check(small_gqa(seed=5), budget=budget, score_mode=C.SCORE_MASS)


def test_fused_step_matches():
    # One launch and the three-launch path select the same blocks; they split
    # the exact attention differently, so outputs agree to rounding.
    w = small_gqa(seed=6)
    g1, _ = full_check(w, fused=False)
    g2 = run_gpu(w, fused=True)
    np.testing.assert_array_equal(g1.selected, g2.selected)
    np.testing.assert_allclose(g1.out, g2.out, rtol=1e-5, atol=1e-6)
    np.testing.assert_allclose(g1.lse, g2.lse, rtol=1e-6, atol=1e-6)


@pytest.mark.parametrize("fused", [False, True])
def test_constant_key_blocks_give_dense_output(fused):
    # Zero within-block variance: every score is 0, ties go to the lowest ids,
    # and compensation is exact, so the output equals dense attention.  The
    # longer sequence spans two chunks of 256 blocks.
    w = small_gqa(seed=8, seq_lens=[6000, 100])
    for b in range(w.batch):
        k = w.k_tokens[b]
        L = k.shape[0]
        for i in range(0, L, 16):
            k[i:i + 16] = k[i]
    g = run_gpu(w, budget=64, fused=fused)
    for b in range(w.batch):
        M = w.num_blocks(b)
        if not fused:
            assert np.all(g.group_scores[b, :, :M] == 0)
        np.testing.assert_array_equal(g.selected[b, :, :4], np.tile(np.arange(4), (2, 1)))
        q, k, v = O.sequence_arrays(w.q[b], w.k_tokens[b], w.v_tokens[b], w.dtype)
        out, lse = O.dense_attention(q, k, v)
        assert np.abs(g.out[b] - out).max() <= 2e-3
        assert np.abs(g.lse[b] - lse).max() <= 1e-4


@pytest.mark.parametrize("fused", [False, True])
def test_duplicated_blocks_tie_to_the_lowest_index(fused):
    # Twelve copies of one hot block, three across chunk boundaries, a budget
    # of 8 blocks: the copies' scores are equal and straddle the k-th place,
    # so the lower block ids win, on both paths.
    w, copies = duplicated_blocks_case()
    g, ora = full_check(w, fused=fused)
    for h in range(2):
        rank = ora[0].step.rank_score[h]
        assert np.all(rank[copies] == rank[copies[0]])
        assert ora[0].step.gaps[h] == 0.0
        np.testing.assert_array_equal(g.selected[0, h, :8], copies[:8])


@pytest.mark.parametrize("fused", [True, False])
def test_selection_above_one_wave_with_a_concentrated_chunk(fused):
    # k = 96 blocks over 8 chunks: the single launch first reads each chunk's
    # 32 best candidates and its 33rd.  KV head 0 has 48 hot blocks in chunk 1,
    # more than 32 of its top k, so its pair needs every candidate; KV head 1's
    # pair is decided from the first 32 of every chunk.  Both against the
    # oracle, in one launch.
    w, hot = concentrated_blocks_case()
    g, ora = full_check(w, budget=96 * 16, fused=fused)
    rank = ora[0].step.rank_score[0]
    top = np.argsort(-rank, kind="stable")[:96]
    assert np.isin(hot, top).sum() > 32, "the hot chunk must hold more than 32 of the top k"
    sel0 = g.selected[0, 0, :96]
    assert np.isin(hot, sel0).sum() > 32


@pytest.mark.parametrize("fused", [True, False])
def test_selection_of_32_with_a_concentrated_chunk(fused):
    # k = 32 blocks over 16 chunks.  KV head 0 has 20 hot blocks in chunk 5,
    # more than 8 of its top k, so its chunk's candidates reach deep into the
    # pair's selection; KV head 1's selection is spread, no chunk holding
    # more than 8.  Both against the oracle, in one launch.
    w, hot = concentrated_blocks_case(seed=93, n_hot=20, hot_chunk=5, n_blocks=4096, budget_blocks=32)
    if fused:
        assert C.decode_step_launches(dims_of(w), 32 * 16) == 1
    g, ora = full_check(w, budget=32 * 16, fused=fused)
    top0 = np.argsort(-ora[0].step.rank_score[0], kind="stable")[:32]
    assert np.isin(hot, top0).sum() > 8, "the hot chunk must hold more than 8 of the top k"
    top1 = np.argsort(-ora[0].step.rank_score[1], kind="stable")[:32]
    assert np.bincount(top1 // 256, minlength=16).max() <= 8
    assert np.isin(hot, g.selected[0, 0, :32]).sum() > 8


def _dense_check(w):
    print(f"[case] dense {w.name} seed={w.seed} B={w.batch} Hq={w.num_q_heads} Hkv={w.num_kv_heads} "
          f"d={w.head_dim} {w.dtype} lens={list(w.seq_lens)[:6]}", flush=True)
    dev = to_device(w)
    ws = C.allocate_workspace(C.dense_workspace_bytes(dev.dims), "cuda:0")
    worst = 0.0
    for rep in range(2):  # the second call reuses the workspace (arrival counters reset)
        out, lse = C.dense_decode_attention(dev.dims, dev.q, dev.k_cache, dev.v_cache, dev.block_table,
                                            dev.seq_lens, ws)
        torch.cuda.synchronize()
        out, lse = out.cpu().numpy(), lse.cpu().numpy()
        for b in range(w.batch):
            q, k, v = O.sequence_arrays(w.q[b], w.k_tokens[b], w.v_tokens[b], w.dtype)
            ro, rl = O.dense_attention(q, k, v)
            err = float(np.abs(out[b] - ro).max())
            worst = max(worst, err)
            assert err <= 2e-3, (b, err)
            assert np.abs(lse[b] - rl).max() <= 1e-4
    print(f"[case] ok: dense max |out - oracle| = {worst:.2e}", flush=True)


@pytest.mark.parametrize("G,d,dtype", [(1, 128, "bf16"), (2, 64, "f32"), (4, 64, "bf16"), (8, 128, "bf16"),
                                       (8, 64, "f32"), (4, 128, "f32"), (2, 128, "bf16"), (8, 128, "f32")])
def test_dense_head_layouts(G, d, dtype):
    # lengths cover a split boundary (128 blocks = 2048 tokens), ragged tails
    # and a one-token sequence
    w = small_gqa(seed=10 + G, seq_lens=[2049, 2047, 17, 1, 5000], num_q_heads=2 * G, head_dim=d,
                  dtype=dtype)
    _dense_check(w)


def test_dense_llama_32k():
    _dense_check(W.make_preset("llama_32k", seed=1))


def test_dense_llama_128k():
    # the benchmarked launch: 128-block splits, one round of 512 workgroups
    _dense_check(W.make_preset("llama_128k", seed=2))


def test_dense_kernel_matches_oracle():
    w = small_gqa(seed=9)
    dev = to_device(w)
    ws = C.allocate_workspace(C.dense_workspace_bytes(dev.dims), "cuda:0")
    out, lse = C.dense_decode_attention(dev.dims, dev.q, dev.k_cache, dev.v_cache, dev.block_table,
                                        dev.seq_lens, ws)
    torch.cuda.synchronize()
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    for b in range(w.batch):
        q, k, v = O.sequence_arrays(w.q[b], w.k_tokens[b], w.v_tokens[b], w.dtype)
        ro, rl = O.dense_attention(q, k, v)
        assert np.abs(out[b] - ro).max() <= 2e-3
        assert np.abs(lse[b] - rl).max() <= 1e-4


def test_append_matches_bulk_bit_exact():
    # Decode-time append recomputes the tail block from raw tokens: after a
    # chain of appends the store equals a bulk build of the final cache.
    w = W.make_decode_inputs(name="append", seq_lens=[40, 16, 1], num_q_heads=4, num_kv_heads=2,
                             head_dim=128, r_groups=4, budget_tokens=32, dtype="bf16", n_needles=0,
                             n_outliers=1, seed=11, extra_capacity_tokens=40)
    steps = W.make_append_steps(w, 35, seed=12)
    full = W.make_decode_inputs(name="append", seq_lens=[40, 16, 1], num_q_heads=4, num_kv_heads=2,
                                head_dim=128, r_groups=4, budget_tokens=32, dtype="bf16", n_needles=0,
                                n_outliers=1, seed=11, extra_capacity_tokens=40)
    for s in steps:
        W.append_tokens(full, s)
    kc, vc = full.paged_cache()
    dev = to_device(full, k_cache=kc, v_cache=vc)
    dims = dev.dims
    bulk = C.allocate_summaries(dims, "cuda:0")
    C.build_summaries(dims, dev.k_cache, dev.v_cache, dev.block_table, dev.seq_lens, bulk)
    inc = C.allocate_summaries(dims, "cuda:0")
    lens = torch.tensor([40, 16, 1], dtype=torch.int32, device="cuda:0")
    C.build_summaries(dims, dev.k_cache, dev.v_cache, dev.block_table, lens, inc)
    for _ in steps:
        lens += 1
        C.build_summaries(dims, dev.k_cache, dev.v_cache, dev.block_table, lens, inc, append_only=True)
    torch.cuda.synchronize()
    for b in range(3):
        M = full.num_blocks(b)
        for name in ("mean_k", "mean_v", "gvar"):
            assert torch.equal(getattr(bulk, name)[b, :, :M], getattr(inc, name)[b, :, :M]), name
        assert torch.equal(bulk.count[b, :M], inc.count[b, :M])
    g = run_gpu(full, dev=dev, summaries=inc)
    ora = run_oracle(full)
    check_summaries(full, g, ora)
    check_selection_vs_oracle(full, g, ora)
    check_outputs(full, g, ora)


def test_many_fused_steps_on_one_workspace():
    # The step kernel's control words reset themselves: 25 launches in a row on
    # one workspace give identical results and leave the words at zero.
    w = small_gqa(seed=14)
    dev = to_device(w)
    dims = dev.dims
    summ = C.allocate_summaries(dims, "cuda:0")
    C.build_summaries(dims, dev.k_cache, dev.v_cache, dev.block_table, dev.seq_lens, summ)
    ws = C.allocate_workspace(C.workspace_bytes(dims, w.budget_tokens), "cuda:0")
    outs = []
    for _ in range(25):
        sel, nsel, out, lse = C.decode_step(dims, dev.q, dev.k_cache, dev.v_cache, summ, dev.block_table,
                                            dev.seq_lens, w.budget_tokens, ws)
        outs.append((sel.clone(), out.clone(), lse.clone()))
    torch.cuda.synchronize()
    for sel, out, lse in outs[1:]:
        assert torch.equal(sel, outs[0][0]) and torch.equal(out, outs[0][1]) and torch.equal(lse, outs[0][2])
    check_workspace_clean(ws, dims, w.budget_tokens)


def test_repeat_runs_are_bit_identical():
    w = small_gqa(seed=13)
    a = run_gpu(w)
    b = run_gpu(w)
    for name in ("mean_k", "mean_v", "gvar", "selected", "group_scores", "out", "lse"):
        np.testing.assert_array_equal(getattr(a, name), getattr(b, name), err_msg=name)


# ---- full-size workloads -------------------------------------------------------


def test_llama_32k():
    full_check(W.make_preset("llama_32k", seed=0), fused=True)


@pytest.mark.parametrize("preset,budget", [("llama_32k", 528), ("llama_32k", 1024), ("llama_128k", 1024)])
def test_selection_of_33_to_64_blocks(preset, budget):
    # 32 < k <= 64: the single launch publishes each chunk's 32 best
    # candidates and its 33rd first, and all of its top k only if some
    # chunk's 33rd lies above the pair's k-th; both paths against the oracle.
    w = W.make_preset(preset, seed=5)
    assert C.decode_step_launches(dims_of(w), budget) == 1
    full_check(w, budget=budget)


def test_max_context_length():
    # The widest page table the library takes (15872 blocks, 253952 tokens),
    # one token short so the last block is ragged: the single-launch step, the
    # three-launch path and dense decode, against the oracle.
    w = W.make_decode_inputs(name="max_ctx", seq_lens=[253951], num_q_heads=8, num_kv_heads=2, head_dim=128,
                             r_groups=4, budget_tokens=512, dtype="bf16", n_needles=8, n_outliers=4, seed=21)
    assert w.max_blocks == 15872
    full_check(w)
    _dense_check(w)


@pytest.mark.parametrize("across_xcds", [False, True])
def test_fused_step_both_placements(across_xcds, monkeypatch):
    # By default a pair's workgroups share one XCD and hand data over through
    # its L2; CKV_FUSED_ACROSS_XCDS=1 spreads them and uses device-scope
    # stores.  Both must match the oracle.
    if across_xcds:
        monkeypatch.setenv("CKV_FUSED_ACROSS_XCDS", "1")
    full_check(small_gqa(seed=4), fused=True)
    full_check(W.make_preset("llama_32k", seed=3), fused=True)


@pytest.mark.parametrize("across_xcds", [False, True])
def test_value_workgroups_take_several_chunks(across_xcds, monkeypatch):
    # 16 (sequence, KV head) pairs of 21 chunks do not fit on the device with
    # a value workgroup per chunk (16 x 42 > 2 x 256); with one value
    # workgroup per about two chunks they fit in one round.  The shorter
    # sequence leaves its last chunk empty.
    if across_xcds:
        monkeypatch.setenv("CKV_FUSED_ACROSS_XCDS", "1")
    w = W.make_decode_inputs(name="two_seq_86k", seq_lens=[86000, 80000], num_q_heads=32, num_kv_heads=8,
                             head_dim=128, r_groups=4, budget_tokens=512, dtype="bf16", n_needles=16,
                             n_outliers=4, seed=11)
    assert C.decode_step_launches(dims_of(w), 512) == 1
    full_check(w, fused=True)


def test_128k_with_spare_pages():
    # 131077 tokens in a page table with room for 64 more: 33 chunks per
    # pair, the last holding one block; two value workgroups take two chunks.
    w = W.make_preset("llama_128k", seed=2, seq_lens=[131077], extra_capacity_tokens=64)
    full_check(w, fused=True)


def test_headline_shape_runs_as_one_launch():
    # 128K tokens, Hq 32, Hkv 8, d 128, 16-token blocks, 512-token budget
    dims = C.Dims(batch=1, num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16, r_groups=4,
                  num_pages=8192, max_blocks_per_seq=8192, kv_dtype=C.CKV_BF16)
    assert C.decode_step_launches(dims, 512) == 1


def test_llama_128k_headline():
    report = []
    full_check(W.make_preset("llama_128k", seed=0), fused=True, report=report)
    print("near-ties:", report, flush=True)


def test_llama_128k_headline_unfused_scores():
    full_check(W.make_preset("llama_128k", seed=1), fused=False)


def test_batched_ragged():
    full_check(W.make_preset("batched_ragged", seed=0), fused=True)


@pytest.mark.parametrize("fused_append", [False, True])
def test_prefill_then_decode_loop(fused_append):
    # Bulk summaries over 128K tokens, then 64 decode steps that each append one
    # token (tail-block summary update) and run the compensated step with a
    # 2048-token budget; checked against the oracle at several steps.  The
    # append is a write plus the append-mode summary build, or it runs inside
    # the step (ckv_decode_step_append).
    w = W.make_preset("prefill_128k_loop", seed=0)
    steps = W.make_append_steps(w, 64, seed=21)
    kc, vc = w.paged_cache()
    dev = to_device(w, k_cache=kc, v_cache=vc)
    del kc, vc
    dims = dev.dims
    summ = C.allocate_summaries(dims, "cuda:0")
    C.build_summaries(dims, dev.k_cache, dev.v_cache, dev.block_table, dev.seq_lens, summ)
    L0 = int(w.seq_lens[0])
    _, k0, v0 = O.sequence_arrays(w.q[0], w.k_tokens[0], w.v_tokens[0], w.dtype)
    k64 = np.zeros((L0 + len(steps), 8, 128))
    v64 = np.zeros_like(k64)
    k64[:L0], v64[:L0] = k0, v0
    del k0, v0
    osumm = O.build_summaries(k64[:L0], v64[:L0], 16, 4, "bf16")
    ws = C.allocate_workspace(C.workspace_bytes(dims, w.budget_tokens), "cuda:0")
    checkpoints = {0, 1, 15, 16, 63}
    print(f"[case] decode loop fused_append={fused_append} launches per step "
          f"{C.decode_step_append_launches(dims, w.budget_tokens) if fused_append else 'append + step'}",
          flush=True)
    for t, st in enumerate(steps):
        L = L0 + t
        kn = torch.from_numpy(st.k_new[0].view(np.int16)).view(torch.bfloat16).cuda()
        vn = torch.from_numpy(st.v_new[0].view(np.int16)).view(torch.bfloat16).cuda()
        dev.seq_lens.fill_(L + 1)
        dev.q.copy_(torch.from_numpy(st.q.view(np.int16)).view(torch.bfloat16))
        if fused_append:
            sel, nsel, out, lse = C.decode_step_append(dims, dev.q, kn.unsqueeze(0), vn.unsqueeze(0), dev.k_cache,
                                                       dev.v_cache, summ, dev.block_table, dev.seq_lens,
                                                       w.budget_tokens, ws)
        else:
            p, slot = int(w.block_table[0, L // 16]), L % 16
            dev.k_cache[p, :, slot, :] = kn
            dev.v_cache[p, :, slot, :] = vn
            C.build_summaries(dims, dev.k_cache, dev.v_cache, dev.block_table, dev.seq_lens, summ,
                              append_only=True)
            sel, nsel, out, lse = C.decode_step(dims, dev.q, dev.k_cache, dev.v_cache, summ, dev.block_table,
                                                dev.seq_lens, w.budget_tokens, ws)
        k64[L] = O.widen(st.k_new[0], "bf16")
        v64[L] = O.widen(st.v_new[0], "bf16")
        osumm = O.append_summaries(osumm, k64[:L + 1], v64[:L + 1], 16, 4, "bf16")
        if t in checkpoints:
            torch.cuda.synchronize()
            print(f"[case] decode step {t}: L={L + 1}", flush=True)
            q = O.widen(st.q[0], "bf16")
            res = O.decode_step(q, k64[:L + 1], v64[:L + 1], osumm, budget_tokens=w.budget_tokens,
                                block_size=16, r=4)
            g_sel = sel.cpu().numpy()[0]
            kk = res.selected.shape[1]
            assert np.all(nsel.cpu().numpy()[0] == kk)
            C.workspace_status(ws)
            for h in range(8):
                check_selection_valid(res.rank_score[h], kk, g_sel[h, :kk], float(res.gaps[h]),
                                      res.selected[h], f"step {t} KV head {h}")
            o2, l2 = O.compensated_attention(q, k64[:L + 1], v64[:L + 1], osumm,
                                             g_sel[:, :kk].astype(np.int64), 16)
            assert np.abs(out.cpu().numpy()[0] - o2).max() <= 2e-3
            assert np.abs(lse.cpu().numpy()[0] - l2).max() <= 1e-4
            M = -(-(L + 1) // 16)
            assert summ.count[0, M - 1].item() == osumm.count[M - 1]


def test_decode_loop_graph_replays_match_eager():
    # Prefill over 128K tokens, then the 64-step appending loop (2048-token
    # budget) captured into one HIP graph: every replay, with eager work and
    # synchronisations between replays, gives the eager loop's outputs bit
    # for bit and leaves the workspace ready for the next call.
    from compensated_kv_selection_amd.decode_loop import DecodeLoop
    w = W.make_preset("prefill_128k_loop", seed=0)
    steps = W.make_append_steps(w, 64, seed=21)
    kc, vc = w.paged_cache()
    dev = to_device(w, k_cache=kc, v_cache=vc)
    del kc, vc
    dims = dev.dims
    summ = C.allocate_summaries(dims, "cuda:0")
    C.build_summaries(dims, dev.k_cache, dev.v_cache, dev.block_table, dev.seq_lens, summ)
    loop = DecodeLoop(dev, summ, w.block_table, w.seq_lens, steps, w.dtype)
    print(f"[case] decode loop eager: L0={int(w.seq_lens[0])} steps=64 budget={w.budget_tokens} "
          f"launches={C.decode_step_launches(dims, w.budget_tokens)}", flush=True)
    loop.run()
    torch.cuda.synchronize()
    outs = (loop.out, loop.lse, loop.num_selected, loop.selected)
    ref = [x.clone() for x in outs]
    assert torch.all(ref[2] == w.budget_tokens // 16)
    assert torch.isfinite(ref[0]).all() and torch.isfinite(ref[1]).all()
    print("[case] decode loop capture", flush=True)
    g = loop.capture()
    for rep in range(3):
        for x in outs:
            x.fill_(-7)
        junk = torch.randn(1 << 20, device="cuda:0")
        float(junk.square().sum())
        torch.cuda.synchronize()
        print(f"[case] decode loop replay {rep}", flush=True)
        g.replay()
        torch.cuda.synchronize()
        for name, x, r in zip(("out", "lse", "num_selected", "selected"), outs, ref):
            assert torch.equal(x, r), f"replay {rep}: {name} differs from the eager loop"
        check_workspace_clean(loop.ws, dims, w.budget_tokens)


def _oracle_check_paged(w, q_dev, k_cache, v_cache, lens, budget, result):
    """Check a decode step's (selected, num_selected, out, lse) against the
    oracle run on the given device caches, read back token by token through
    the page table for the given lengths."""
    from compensated_kv_selection_amd.tensors import torch_to_storage
    sel, nsel, out, lse = (x.cpu().numpy() for x in result)
    kc, vc = torch_to_storage(k_cache), torch_to_storage(v_cache)
    qs = torch_to_storage(q_dev)
    for b, L in enumerate(lens.tolist()):
        if L == 0:
            continue
        pages = w.block_table[b, np.arange(L) // 16]
        slots = np.arange(L) % 16
        q, k, v = O.sequence_arrays(qs[b], kc[pages, :, slots, :], vc[pages, :, slots, :], w.dtype)
        summ = O.build_summaries(k, v, 16, w.r_groups, w.dtype)
        res = O.decode_step(q, k, v, summ, budget_tokens=budget, block_size=16, r=w.r_groups)
        kk = res.selected.shape[1]
        assert np.all(nsel[b] == kk)
        for g in range(w.num_kv_heads):
            check_selection_valid(res.rank_score[g], kk, sel[b, g, :kk], float(res.gaps[g]), res.selected[g],
                                  f"seq {b} KV head {g}")
        o2, l2 = O.compensated_attention(q, k, v, summ, sel[b, :, :kk].astype(np.int64), 16)
        assert np.abs(out[b] - o2).max() <= 2e-3, (b, float(np.abs(out[b] - o2).max()))
        assert np.abs(lse[b] - l2).max() <= 1e-4


def _append_step_case(before, num_kv_heads, budget, seed, hot, steps=3, G=4, d=128, r=4, dtype="bf16"):
    """Inputs for `steps` appending decode steps: sequences of lengths
    `before` get one new token per step.  For sequences listed in `hot` the
    new keys point along the mean query of their KV head, with alternating
    sign and a large norm, so that the tail block (new tokens of very
    different logits) is selected and attended to from the page slots the
    steps just wrote."""
    w = W.make_decode_inputs(name="append_step", seq_lens=[max(L, 1) for L in before], num_q_heads=G * num_kv_heads,
                             num_kv_heads=num_kv_heads, head_dim=d, r_groups=r, budget_tokens=budget,
                             dtype=dtype, n_needles=0, n_outliers=2, extra_capacity_tokens=48, seed=seed)
    dev = to_device(w)
    rng = np.random.default_rng(seed + 100)
    B, H = len(before), num_kv_heads
    qf = dev.q.float().view(B, H, G, d).mean(dim=2).cpu().numpy()
    qf = qf / np.linalg.norm(qf, axis=-1, keepdims=True) * np.sqrt(d)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    kv = []
    for t in range(steps):
        k_new = rng.standard_normal((B, H, d), dtype=np.float32)
        v_new = rng.standard_normal((B, H, d), dtype=np.float32)
        for b in hot:
            k_new[b] = (6.0 if t % 2 == 0 else -6.0) * qf[b]
        kv.append((torch.from_numpy(k_new).to("cuda:0", tdt), torch.from_numpy(v_new).to("cuda:0", tdt)))
    return w, dev, kv


@pytest.mark.parametrize("before,num_kv_heads,budget,hot,shape", [
    # tails at slots 8, 0, 15, 1, 0 and 15 of their blocks (the fourth and
    # sixth sequences have every block selected), and one of length 0
    ([1000, 768, 15, 1, 4096, 31, 0], 2, 64, [0, 1, 4], {}),
    # one long sequence: 8 chunks per pair, the tail block's reader is
    # another chunk's workgroup
    ([32767], 8, 512, [0], {}),
    ([32768 + 5], 8, 512, [], {}),
    # the appending instances for 1, 2 and 8 query heads per KV head
    ([3000, 767, 16], 2, 128, [0, 1], {"G": 1}),
    ([3000, 767, 16], 2, 128, [0, 1], {"G": 2}),
    ([3000, 767, 16], 2, 128, [0, 1], {"G": 8}),
    # shapes the appending instance does not cover: append, then the step
    ([3000, 767, 16], 2, 128, [0, 1], {"r": 8}),
    ([3000, 767, 16], 2, 128, [0, 1], {"d": 64}),
    ([3000, 767, 16], 2, 128, [0, 1], {"dtype": "f32"}),
])
def test_decode_step_append_matches_append_then_step(before, num_kv_heads, budget, hot, shape):
    # ckv_decode_step_append against ckv_append_tokens + ckv_decode_step, from
    # the same state: outputs, selections, caches and summaries bit for bit,
    # over three steps in a row (each appending one more token).
    w, dev, kv = _append_step_case(before, num_kv_heads, budget, seed=41, hot=hot, **shape)
    dims = dev.dims
    summ = C.allocate_summaries(dims, "cuda:0")
    C.build_summaries(dims, dev.k_cache, dev.v_cache, dev.block_table, dev.seq_lens, summ)
    launches = C.decode_step_append_launches(dims, budget)
    print(f"[case] decode_step_append lens={before} Hkv={num_kv_heads} budget={budget} {shape} "
          f"launches={launches}", flush=True)
    fusable = shape.get("d", 128) == 128 and shape.get("r", 4) == 4 and shape.get("dtype", "bf16") == "bf16"
    assert launches == (1 if fusable else 1 + C.decode_step_launches(dims, budget))

    def state():
        return (dev.k_cache.clone(), dev.v_cache.clone(),
                C.Summaries(summ.mean_k.clone(), summ.mean_v.clone(), summ.gvar.clone(), summ.count.clone()))

    def bits(t):
        return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)

    ka, va, sa = state()
    kb, vb, sb = state()
    d = dims.head_dim
    wsa = C.allocate_workspace(C.workspace_bytes(dims, budget), "cuda:0")
    wsb = C.allocate_workspace(C.workspace_bytes(dims, budget), "cuda:0")
    for step, (k_new, v_new) in enumerate(kv):
        lens = torch.tensor([L + step + 1 if L > 0 else 0 for L in before], dtype=torch.int32, device="cuda:0")
        print(f"[case] step {step}: lens={lens.tolist()[:8]}", flush=True)
        C.append_tokens(dims, k_new, v_new, ka, va, dev.block_table, lens, sa)
        ra = C.decode_step(dims, dev.q, ka, va, sa, dev.block_table, lens, budget, wsa)
        rb = C.decode_step_append(dims, dev.q, k_new, v_new, kb, vb, sb, dev.block_table, lens, budget, wsb)
        torch.cuda.synchronize()
        for name, x, y in zip(("selected", "num_selected", "out", "lse"), ra, rb):
            if name == "selected":
                kk = ra[1].unsqueeze(-1)
                ar = torch.arange(x.shape[-1], device=x.device)
                x, y = x.masked_fill(ar >= kk, -1), y.masked_fill(ar >= kk, -1)
            assert torch.equal(bits(x), bits(y)), f"step {step}: {name} differs"
        assert torch.equal(bits(ka), bits(kb)) and torch.equal(bits(va), bits(vb)), f"step {step}: caches differ"
        for name, x, y in zip(("mean_k", "mean_v", "gvar", "count"), (sa.mean_k, sa.mean_v, sa.gvar, sa.count),
                              (sb.mean_k, sb.mean_v, sb.gvar, sb.count)):
            assert torch.equal(bits(x), bits(y)), f"step {step}: summary {name} differs"
        check_workspace_clean(wsb, dims, budget)
    # the appending step's last results against the oracle, on the caches
    # it wrote (read back from the device through the page table)
    _oracle_check_paged(w, dev.q, kb, vb, lens, budget, rb)
    # the hot sequences did attend to their tail block
    for b in hot:
        L = int(lens[b])
        for g in range(num_kv_heads):
            assert int((L - 1) // 16) in ra[0][b, g, : int(ra[1][b, g])].tolist(), (b, g)


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64)])
def test_append_tokens_matches_write_then_append(dtype, d):
    # New tokens landing at slot 8, 0, 15, 1, 0 and 15 of their blocks, and
    # a sequence of length 0 that must be left alone: ckv_append_tokens gives
    # the caches and summaries of writing the token and then running the
    # append-mode summary build, bit for bit.
    before = [1000, 768, 15, 1, 4096, 31]
    w = W.make_decode_inputs(name="append", seq_lens=before, num_q_heads=8, num_kv_heads=2, head_dim=d,
                             r_groups=4, budget_tokens=64, dtype=dtype, n_needles=0, n_outliers=2,
                             extra_capacity_tokens=16, seed=31)
    dev = to_device(w)
    dims = dev.dims
    summ = C.allocate_summaries(dims, "cuda:0")
    C.build_summaries(dims, dev.k_cache, dev.v_cache, dev.block_table, dev.seq_lens, summ)
    rng = np.random.default_rng(32)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    k_new = torch.from_numpy(rng.standard_normal((6, 2, d), dtype=np.float32)).to("cuda:0", tdt)
    v_new = torch.from_numpy(rng.standard_normal((6, 2, d), dtype=np.float32)).to("cuda:0", tdt)
    after = torch.tensor([L + 1 for L in before[:-1]] + [0], dtype=torch.int32, device="cuda:0")

    def state():
        return (dev.k_cache.clone(), dev.v_cache.clone(),
                C.Summaries(summ.mean_k.clone(), summ.mean_v.clone(), summ.gvar.clone(), summ.count.clone()))

    ka, va, sa = state()
    for b, L in enumerate(before[:-1]):
        p, slot = int(w.block_table[b, L // 16]), L % 16
        ka[p, :, slot, :] = k_new[b]
        va[p, :, slot, :] = v_new[b]
    C.build_summaries(dims, ka, va, dev.block_table, after, sa, append_only=True)
    kb, vb, sb = state()
    print(f"[case] append_tokens {dtype} d={d} lens={before}", flush=True)
    C.append_tokens(dims, k_new, v_new, kb, vb, dev.block_table, after, sb)
    torch.cuda.synchronize()

    def bits(t):
        return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)

    assert torch.equal(bits(ka), bits(kb)) and torch.equal(bits(va), bits(vb))
    assert torch.equal(bits(dev.k_cache[int(w.block_table[5, 1])]), bits(kb[int(w.block_table[5, 1])]))
    for x, y in zip((sa.mean_k, sa.mean_v, sa.gvar, sa.count), (sb.mean_k, sb.mean_v, sb.gvar, sb.count)):
        assert torch.equal(bits(x), bits(y))
    # the tail blocks did change
    assert not torch.equal(bits(summ.mean_k), bits(sb.mean_k))
