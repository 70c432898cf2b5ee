"""Host-side checks of the C ABI: the library loads, exports every declared
symbol, and rejects invalid arguments with the documented status before
anything is enqueued.  Pointers passed here are never dereferenced because
every call fails validation first; no GPU is needed."""
import ctypes
import os
import re

import pytest

from compensated_kv_selection_amd import compkv as C
from ws_layout import workspace_regions

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "compkv.h")

OK, INVALID, UNSUPPORTED, WORKSPACE, HIP, INCOMPLETE = range(6)
FAKE = ctypes.c_void_p(0x100000)   # never dereferenced: validation fails first


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(C.LIB_PATH):
        from compensated_kv_selection_amd import build
        build.build()
    return C.load_library()


def header_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\*?\s+\*?(ckv_[a-z_]+)\(", text, re.M)))


def test_header_declares_the_exports():
    assert sorted(C.EXPORTS) == header_functions()


def test_library_exports_every_declared_symbol(lib):
    for name in header_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    names = ["CKV_OK", "CKV_ERR_INVALID_ARG", "CKV_ERR_UNSUPPORTED", "CKV_ERR_WORKSPACE", "CKV_ERR_HIP",
             "CKV_ERR_INCOMPLETE"]
    for code, name in enumerate(names):
        assert lib.ckv_status_string(code).decode() == name


def good_dims(**kw):
    d = dict(batch=1, num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16, r_groups=4,
             num_pages=8192, max_blocks_per_seq=8192, kv_dtype=C.CKV_BF16)
    d.update(kw)
    return C.CkvDims(**d)


def summ():
    return C.CkvSummaries(0x100000, 0x100000, 0x100000, 0x100000)


def ws_bytes(lib, dims, budget=512):
    return lib.ckv_workspace_bytes(ctypes.byref(dims), budget)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(batch=0), INVALID, "batch"),
    (dict(num_q_heads=0), INVALID, "head"),
    (dict(num_q_heads=12, num_kv_heads=8), INVALID, "num_q_heads"),
    (dict(num_q_heads=24, num_kv_heads=8), UNSUPPORTED, "query heads per KV head"),
    (dict(num_q_heads=32 * 16, num_kv_heads=32), UNSUPPORTED, "query heads per KV head"),
    (dict(num_kv_heads=128, num_q_heads=128), UNSUPPORTED, "num_kv_heads"),
    (dict(head_dim=96), UNSUPPORTED, "head_dim"),
    (dict(head_dim=0), INVALID, "head_dim"),
    (dict(block_size=32), UNSUPPORTED, "block_size"),
    (dict(block_size=0), INVALID, "block_size"),
    (dict(r_groups=3), INVALID, "r_groups"),
    (dict(r_groups=0), INVALID, "r_groups"),
    (dict(num_pages=0), INVALID, "num_pages"),
    (dict(max_blocks_per_seq=0), INVALID, "max_blocks"),
    (dict(max_blocks_per_seq=20000), UNSUPPORTED, "max_blocks"),
    (dict(max_blocks_per_seq=15873, num_pages=15873), UNSUPPORTED, "max_blocks"),  # one past the widest table
    (dict(kv_dtype=7), INVALID, "kv_dtype"),
])
def test_bad_dims_rejected_everywhere(lib, kw, status, needle):
    d = good_dims(**kw)
    s = summ()
    calls = [
        lambda: lib.ckv_build_summaries(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, 0, ctypes.byref(s), None),
        lambda: lib.ckv_append_tokens(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ctypes.byref(s), None),
        lambda: lib.ckv_score_select(ctypes.byref(d), FAKE, ctypes.byref(s), FAKE, FAKE, 512, 0, FAKE,
                                     FAKE, None, FAKE, 1 << 40, None),
        lambda: lib.ckv_compensated_decode_attention(ctypes.byref(d), FAKE, FAKE, FAKE, ctypes.byref(s),
                                                     FAKE, FAKE, 512, FAKE, FAKE, 1, FAKE, None, FAKE,
                                                     1 << 40, None),
        lambda: lib.ckv_decode_step(ctypes.byref(d), FAKE, FAKE, FAKE, ctypes.byref(s), FAKE, FAKE, 512, 0,
                                    FAKE, FAKE, FAKE, None, FAKE, 1 << 40, None),
        lambda: lib.ckv_dense_decode_attention(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None,
                                               FAKE, 1 << 40, None),
        lambda: lib.ckv_decode_step_noalloc(ctypes.byref(d), FAKE, FAKE, FAKE, ctypes.byref(s), FAKE, FAKE, 512,
                                            0, FAKE, FAKE, FAKE, None, None),
    ]
    for call in calls:
        assert call() == status
        assert needle in lib.ckv_last_error().decode()
    assert lib.ckv_workspace_bytes(ctypes.byref(d), 512) == 0
    assert lib.ckv_dense_workspace_bytes(ctypes.byref(d)) == 0
    assert lib.ckv_decode_step_launches(ctypes.byref(d), 512) == 0


def test_null_dims(lib):
    assert lib.ckv_build_summaries(None, FAKE, FAKE, FAKE, FAKE, 0, ctypes.byref(summ()), None) == INVALID
    assert lib.ckv_workspace_bytes(None, 512) == 0
    assert lib.ckv_decode_step_launches(None, 512) == 0
    assert lib.ckv_decode_step_launches(ctypes.byref(good_dims()), -1) == 0


def test_null_pointers_rejected(lib):
    d = good_dims()
    s = summ()
    n = None
    W = ws_bytes(lib, d)
    assert lib.ckv_build_summaries(ctypes.byref(d), n, FAKE, FAKE, FAKE, 0, ctypes.byref(s), None) == INVALID
    assert lib.ckv_build_summaries(ctypes.byref(d), FAKE, FAKE, n, FAKE, 0, ctypes.byref(s), None) == INVALID
    assert lib.ckv_build_summaries(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, 0, None, None) == INVALID
    bad_s = C.CkvSummaries(0x100000, 0, 0x100000, 0x100000)
    assert lib.ckv_build_summaries(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, 0, ctypes.byref(bad_s), None) == INVALID
    for i in range(6):  # k_new, v_new, k_cache, v_cache, block_table, seq_lens
        args = [FAKE] * 6
        args[i] = n
        assert lib.ckv_append_tokens(ctypes.byref(d), *args, ctypes.byref(s), None) == INVALID
    assert lib.ckv_append_tokens(ctypes.byref(d), *([FAKE] * 6), None, None) == INVALID
    assert lib.ckv_append_tokens(None, *([FAKE] * 6), ctypes.byref(s), None) == INVALID
    assert lib.ckv_score_select(ctypes.byref(d), n, ctypes.byref(s), FAKE, FAKE, 512, 0, FAKE, FAKE, None,
                                FAKE, W, None) == INVALID
    assert lib.ckv_score_select(ctypes.byref(d), FAKE, ctypes.byref(s), FAKE, FAKE, 512, 0, n, FAKE, None,
                                FAKE, W, None) == INVALID
    assert lib.ckv_compensated_decode_attention(ctypes.byref(d), FAKE, FAKE, FAKE, ctypes.byref(s), FAKE,
                                                FAKE, 512, FAKE, FAKE, 1, n, None, FAKE, W, None) == INVALID
    assert lib.ckv_dense_decode_attention(ctypes.byref(d), FAKE, n, FAKE, FAKE, FAKE, FAKE, None, FAKE,
                                          1 << 40, None) == INVALID


def test_budget_and_mode_checked(lib):
    d = good_dims()
    s = summ()
    W = ws_bytes(lib, d)
    assert lib.ckv_score_select(ctypes.byref(d), FAKE, ctypes.byref(s), FAKE, FAKE, -1, 0, FAKE, FAKE, None,
                                FAKE, W, None) == INVALID
    assert "budget" in lib.ckv_last_error().decode()
    assert lib.ckv_score_select(ctypes.byref(d), FAKE, ctypes.byref(s), FAKE, FAKE, 512, 5, FAKE, FAKE, None,
                                FAKE, W, None) == INVALID
    assert "score_mode" in lib.ckv_last_error().decode()
    assert lib.ckv_workspace_bytes(ctypes.byref(d), -16) == 0


def test_workspace_checked(lib):
    d = good_dims()
    s = summ()
    W = ws_bytes(lib, d)
    assert W > 0
    assert lib.ckv_score_select(ctypes.byref(d), FAKE, ctypes.byref(s), FAKE, FAKE, 512, 0, FAKE, FAKE, None,
                                FAKE, W - 1, None) == WORKSPACE
    assert lib.ckv_score_select(ctypes.byref(d), FAKE, ctypes.byref(s), FAKE, FAKE, 512, 0, FAKE, FAKE, None,
                                None, W, None) == WORKSPACE
    assert lib.ckv_score_select(ctypes.byref(d), FAKE, ctypes.byref(s), FAKE, FAKE, 512, 0, FAKE, FAKE, None,
                                ctypes.c_void_p(0x100010), W, None) == INVALID
    assert "aligned" in lib.ckv_last_error().decode()
    dw = lib.ckv_dense_workspace_bytes(ctypes.byref(d))
    assert lib.ckv_dense_decode_attention(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE,
                                          dw - 1, None) == WORKSPACE


def test_workspace_size_formula(lib):
    d = good_dims()
    for budget in (0, 15, 16, 512, 2048, 10 ** 9):
        expect = sum(workspace_regions(1, 32, 8, 128, 8192, budget))
        assert ws_bytes(lib, d, budget) == expect, budget
    ctrl = workspace_regions(1, 32, 8, 128, 8192, 0)[0]
    # dense: 8192 blocks per pair in splits of 128 blocks (the cap) -> 64 splits
    assert lib.ckv_dense_workspace_bytes(ctypes.byref(d)) == ctrl + (8 * 64 * 4 * 132 * 4 + 255) // 256 * 256


@pytest.mark.parametrize("batch,kv_heads,max_blocks,splits", [
    (1, 8, 8192, 64),    # 128-block splits (the cap)
    (1, 8, 2048, 32),    # 64-block splits: about 256 workgroups
    (1, 1, 256, 32),     # 8-block splits (the floor)
    (1, 1, 15872, 248),  # at most 256 splits per pair: 64-block splits
    (16, 8, 4096, 32),   # a large batch: 128-block splits
])
def test_dense_split_rule(lib, batch, kv_heads, max_blocks, splits):
    d = good_dims(batch=batch, num_q_heads=4 * kv_heads, num_kv_heads=kv_heads, max_blocks_per_seq=max_blocks)
    ctrl = workspace_regions(batch, 4 * kv_heads, kv_heads, 128, max_blocks, 0)[0]
    part = batch * kv_heads * splits * 4 * 132 * 4
    assert lib.ckv_dense_workspace_bytes(ctypes.byref(d)) == ctrl + (part + 255) // 256 * 256


def test_errors_leave_no_stale_message_after_success_path_text(lib):
    d = good_dims(head_dim=96)
    assert lib.ckv_build_summaries(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, 0, ctypes.byref(summ()), None) \
        == UNSUPPORTED
    assert lib.ckv_last_error().decode().startswith("head_dim")


def test_workspace_status_rejects_a_missing_or_short_workspace(lib):
    # checked before any HIP call: the error word is uint32 word 2
    word = ctypes.c_uint32(7)
    assert lib.ckv_workspace_status(None, 4096, ctypes.byref(word), None) == INVALID
    assert "NULL" in lib.ckv_last_error().decode()
    assert word.value == 0
    assert lib.ckv_workspace_status(FAKE, 11, ctypes.byref(word), None) == INVALID
    assert "12" in lib.ckv_last_error().decode()


def test_noalloc_step_checks_its_arguments_first(lib):
    # every argument check of ckv_decode_step, before any HIP call
    d = good_dims()
    s = summ()
    args = [FAKE, FAKE, FAKE, ctypes.byref(s), FAKE, FAKE, 512, 0, FAKE, FAKE, FAKE, None, None]
    for i in (0, 1, 2, 3, 4, 5, 8, 9, 10):  # q, k, v, summaries, block_table, seq_lens, selected, num, out
        a = list(args)
        a[i] = None
        assert lib.ckv_decode_step_noalloc(ctypes.byref(d), *a) == INVALID
    a = list(args)
    a[6] = -1
    assert lib.ckv_decode_step_noalloc(ctypes.byref(d), *a) == INVALID
    assert "budget" in lib.ckv_last_error().decode()
    a = list(args)
    a[7] = 9
    assert lib.ckv_decode_step_noalloc(ctypes.byref(d), *a) == INVALID
    assert "score_mode" in lib.ckv_last_error().decode()


def test_noalloc_step_rejects_a_layout_beyond_its_workspace(lib):
    s = summ()
    limit = C.CKV_NOALLOC_WORKSPACE_BYTES
    # 16 sequences of 64K tokens with a 1024-token budget fit; 32 of 128K do not
    fits = good_dims(batch=16, max_blocks_per_seq=4096, num_pages=16 * 4096)
    assert 0 < lib.ckv_workspace_bytes(ctypes.byref(fits), 1024) <= limit
    big = good_dims(batch=32, max_blocks_per_seq=8192, num_pages=32 * 8192)
    need = lib.ckv_workspace_bytes(ctypes.byref(big), 512)
    assert need > limit
    assert lib.ckv_decode_step_noalloc(ctypes.byref(big), FAKE, FAKE, FAKE, ctypes.byref(s), FAKE, FAKE, 512, 0,
                                       FAKE, FAKE, FAKE, None, None) == WORKSPACE
    msg = lib.ckv_last_error().decode()
    assert str(need) in msg and str(limit) in msg
