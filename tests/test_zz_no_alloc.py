"""ckv_decode_step_noalloc (the step in the library's built-in workspace)
against ckv_decode_step with a workspace of its own, through the C ABI:
selections, outputs and log-sum-exps bit for bit, over consecutive calls
whose layouts change (a large batch, then a smaller one, then the large one
again, and a repeat of it that reuses the built-in workspace as left)."""
import numpy as np
import pytest
import torch

from compensated_kv_selection_amd import compkv as C
from compensated_kv_selection_amd import workloads as W
from compensated_kv_selection_amd.tensors import to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests need an MI355X")
    C.load_library()  # raises if libcompkv.so is not built
    yield


CASES = {
    # GQA 4:1 at d = 128 with one long sequence: the single launch, several
    # chunks per pair, a ragged tail
    "large": dict(seq_lens=[70000, 2500, 333, 81], num_q_heads=32, num_kv_heads=8, head_dim=128, r_groups=4,
                  budget_tokens=512, dtype="bf16", n_needles=4, n_outliers=2),
    # fewer pairs and blocks, another budget: a smaller layout
    "small": dict(seq_lens=[5000, 900], num_q_heads=8, num_kv_heads=2, head_dim=128, r_groups=4,
                  budget_tokens=256, dtype="bf16", n_needles=2, n_outliers=2),
}


def _setup(name, seed):
    w = W.make_decode_inputs(name=name, seed=seed, **CASES[name])
    dev = to_device(w, "cuda:0")
    summ = C.allocate_summaries(dev.dims, "cuda:0")
    C.build_summaries(dev.dims, dev.k_cache, dev.v_cache, dev.block_table, dev.seq_lens, summ)
    return w, dev, summ


def _compare(name, w, dev, summ):
    budget = w.budget_tokens
    print(f"[case] noalloc {name}: lens={list(w.seq_lens)} Hq={w.num_q_heads} Hkv={w.num_kv_heads} "
          f"budget={budget} launches={C.decode_step_launches(dev.dims, budget)}", flush=True)
    ws = C.allocate_workspace(C.workspace_bytes(dev.dims, budget), "cuda:0")
    ref = C.decode_step(dev.dims, dev.q, dev.k_cache, dev.v_cache, summ, dev.block_table, dev.seq_lens,
                        budget, ws)
    got = C.decode_step_noalloc(dev.dims, dev.q, dev.k_cache, dev.v_cache, summ, dev.block_table,
                                dev.seq_lens, budget)
    torch.cuda.synchronize()
    C.workspace_status(ws)
    C.noalloc_status("cuda:0")  # raises if the call's workgroups left the error word set
    sel_r, n_r, out_r, lse_r = (t.cpu() for t in ref)
    sel_g, n_g, out_g, lse_g = (t.cpu() for t in got)
    assert torch.equal(n_r, n_g), f"{name}: num_selected differs"
    kk = n_r.unsqueeze(-1)
    ar = torch.arange(sel_r.shape[-1])
    assert torch.equal(sel_r.masked_fill(ar >= kk, -1), sel_g.masked_fill(ar >= kk, -1)), f"{name}: selection differs"
    assert torch.equal(out_r.view(torch.int32), out_g.view(torch.int32)), (
        f"{name}: out differs, max abs {float((out_r - out_g).abs().max()):.3e}")
    assert torch.equal(lse_r.view(torch.int32), lse_g.view(torch.int32)), f"{name}: lse differs"
    assert np.isfinite(out_g.numpy()).all()
    print(f"[case] noalloc {name}: identical to ckv_decode_step", flush=True)


def test_noalloc_step_matches_decode_step_across_layouts():
    large = _setup("large", 5)
    small = _setup("small", 6)
    _compare("large", *large)   # first call on the device: the built-in workspace is looked up and cleared
    _compare("small", *small)   # a smaller layout: cleared again
    _compare("large", *large)   # back to the large layout
    _compare("large", *large)   # same layout: runs on the state the last call left


def test_noalloc_step_rejects_an_oversized_layout():
    dims = C.Dims(32, 32, 8, 128, 16, 4, 32 * 8192, 8192, C.CKV_BF16)
    assert C.workspace_bytes(dims, 512) > C.CKV_NOALLOC_WORKSPACE_BYTES
    t = torch.zeros(16, dtype=torch.int32, device="cuda:0")
    summ = C.Summaries(t, t, t, t)
    with pytest.raises(C.CompKVError) as e:
        C.decode_step_noalloc(dims, t, t, t, summ, t, t, 512, selected=t, num_selected=t,
                              out=t.float(), lse=t.float())
    assert e.value.name == "CKV_ERR_WORKSPACE"
