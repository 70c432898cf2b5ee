"""Python binding of libcompkv.so (ctypes): argument marshalling only.

Every step of the decode path runs in the library's HIP kernels; this module
turns torch device tensors into pointers and the current torch stream into a
hipStream_t, and raises on a non-OK status.  There is no fallback: without
the built library every call raises.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional

import torch

LIB_NAME = "libcompkv.so"
# The in-tree build; CKV_LIBRARY names another build of the same library.
LIB_PATH = os.environ.get("CKV_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)), LIB_NAME)

CKV_BF16, CKV_F32 = 0, 1
SCORE_COMPKV, SCORE_MASS = 0, 1

# Every symbol include/compkv.h declares.
EXPORTS = (
    "ckv_build_summaries",
    "ckv_append_tokens",
    "ckv_workspace_bytes",
    "ckv_score_select",
    "ckv_compensated_decode_attention",
    "ckv_decode_step",
    "ckv_decode_step_launches",
    "ckv_decode_step_append",
    "ckv_decode_step_append_launches",
    "ckv_dense_workspace_bytes",
    "ckv_dense_decode_attention",
    "ckv_workspace_status",
    "ckv_decode_step_noalloc",
    "ckv_status_string",
    "ckv_last_error",
)
CKV_ERR_INCOMPLETE = 5
CKV_NOALLOC_WORKSPACE_BYTES = 64 << 20


class CompKVError(RuntimeError):
    def __init__(self, status: int, name: str, detail: str):
        super().__init__(f"{name}: {detail}" if detail else name)
        self.status = status
        self.name = name
        self.detail = detail


class CkvDims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "num_q_heads", "num_kv_heads", "head_dim", "block_size", "r_groups",
        "num_pages", "max_blocks_per_seq", "kv_dtype")]


class CkvSummaries(ctypes.Structure):
    _fields_ = [("mean_k", ctypes.c_void_p), ("mean_v", ctypes.c_void_p),
                ("gvar", ctypes.c_void_p), ("count", ctypes.c_void_p)]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libcompkv.so and declare its signatures; raise if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m compensated_kv_selection_amd.build`")
    lib = ctypes.CDLL(path)
    P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    D = ctypes.POINTER(CkvDims)
    S = ctypes.POINTER(CkvSummaries)
    sig = {
        "ckv_build_summaries": (I32, [D, P, P, P, P, I32, S, P]),
        "ckv_append_tokens": (I32, [D, P, P, P, P, P, P, S, P]),
        "ckv_workspace_bytes": (SZ, [D, I32]),
        "ckv_score_select": (I32, [D, P, S, P, P, I32, I32, P, P, P, P, SZ, P]),
        "ckv_compensated_decode_attention": (I32, [D, P, P, P, S, P, P, I32, P, P, I32, P, P, P, SZ, P]),
        "ckv_decode_step": (I32, [D, P, P, P, S, P, P, I32, I32, P, P, P, P, P, SZ, P]),
        "ckv_decode_step_launches": (I32, [D, I32]),
        "ckv_decode_step_append": (I32, [D, P, P, P, P, P, S, P, P, I32, I32, P, P, P, P, P, SZ, P]),
        "ckv_decode_step_append_launches": (I32, [D, I32]),
        "ckv_dense_workspace_bytes": (SZ, [D]),
        "ckv_dense_decode_attention": (I32, [D, P, P, P, P, P, P, P, P, SZ, P]),
        "ckv_workspace_status": (I32, [P, SZ, ctypes.POINTER(ctypes.c_uint32), P]),
        "ckv_decode_step_noalloc": (I32, [D, P, P, P, S, P, P, I32, I32, P, P, P, P, P]),
        "ckv_status_string": (ctypes.c_char_p, [I32]),
        "ckv_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != 0:
        lib = load_library()
        raise CompKVError(status, lib.ckv_status_string(status).decode(),
                          lib.ckv_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libcompkv must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


@dataclasses.dataclass
class Dims:
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    r_groups: int
    num_pages: int
    max_blocks_per_seq: int
    kv_dtype: int

    def c(self) -> CkvDims:
        return CkvDims(*dataclasses.astuple(self))

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.kv_dtype == CKV_BF16 else torch.float32

    def kmax(self, budget_tokens: int) -> int:
        return min(self.max_blocks_per_seq, max(0, budget_tokens) // self.block_size)


@dataclasses.dataclass
class Summaries:
    """Block summaries by (sequence, KV head, logical block)."""
    mean_k: torch.Tensor  # [B, Hkv, max_blocks, d] kv dtype
    mean_v: torch.Tensor  # [B, Hkv, max_blocks, d] kv dtype
    gvar: torch.Tensor    # [B, Hkv, max_blocks, r] float32
    count: torch.Tensor   # [B, max_blocks] int32

    def c(self) -> CkvSummaries:
        return CkvSummaries(self.mean_k.data_ptr(), self.mean_v.data_ptr(),
                            self.gvar.data_ptr(), self.count.data_ptr())


def allocate_summaries(dims: Dims, device) -> Summaries:
    B, H, M = dims.batch, dims.num_kv_heads, dims.max_blocks_per_seq
    d, r = dims.head_dim, dims.r_groups
    return Summaries(torch.zeros((B, H, M, d), dtype=dims.torch_dtype, device=device),
                     torch.zeros((B, H, M, d), dtype=dims.torch_dtype, device=device),
                     torch.zeros((B, H, M, r), dtype=torch.float32, device=device),
                     torch.zeros((B, M), dtype=torch.int32, device=device))


def build_summaries(dims: Dims, k_cache, v_cache, block_table, seq_lens, summaries: Summaries,
                    append_only: bool = False) -> None:
    lib = load_library()
    d = dims.c()
    s = summaries.c()
    _check(lib.ckv_build_summaries(ctypes.byref(d), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
                                   _ptr(seq_lens), 1 if append_only else 0, ctypes.byref(s),
                                   _stream(k_cache.device)))


def append_tokens(dims: Dims, k_new, v_new, k_cache, v_cache, block_table, seq_lens,
                  summaries: Summaries) -> None:
    """Write every sequence's new last token (k_new, v_new: [B, Hkv, d]) into
    its page and refresh that block's summary, in one launch; seq_lens
    already count the new token."""
    lib = load_library()
    d = dims.c()
    s = summaries.c()
    _check(lib.ckv_append_tokens(ctypes.byref(d), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
                                 _ptr(block_table), _ptr(seq_lens), ctypes.byref(s), _stream(k_cache.device)))


def workspace_bytes(dims: Dims, budget_tokens: int) -> int:
    d = dims.c()
    return int(load_library().ckv_workspace_bytes(ctypes.byref(d), budget_tokens))


def decode_step_launches(dims: Dims, budget_tokens: int) -> int:
    """Kernel launches decode_step makes for these dims on the current
    device: 1 (one persistent launch) or 3 (score, select, attend)."""
    d = dims.c()
    n = int(load_library().ckv_decode_step_launches(ctypes.byref(d), budget_tokens))
    if n == 0:
        raise ValueError("invalid dims or budget")
    return n


def decode_step_append_launches(dims: Dims, budget_tokens: int) -> int:
    """Kernel launches decode_step_append makes for these dims on the current
    device: 1 when the append runs inside the single-launch step, else the
    append's launch plus decode_step's."""
    d = dims.c()
    n = int(load_library().ckv_decode_step_append_launches(ctypes.byref(d), budget_tokens))
    if n == 0:
        raise ValueError("invalid dims or budget")
    return n


def dense_workspace_bytes(dims: Dims) -> int:
    d = dims.c()
    return int(load_library().ckv_dense_workspace_bytes(ctypes.byref(d)))


def allocate_workspace(nbytes: int, device) -> torch.Tensor:
    """Zero-filled workspace (the step kernel's control words must start at
    zero; every call leaves them zero).  torch's caching allocator returns
    blocks aligned to at least 512 bytes."""
    return torch.zeros((max(nbytes, 256),), dtype=torch.uint8, device=device)


CTRL_WORDS_HEADER = 64
CTRL_WORDS_PER_PAIR = 8
CTRL_EPOCH = 3   # per-pair word that counts single-launch steps


def workspace_control(ws: torch.Tensor, batch: int, num_kv_heads: int) -> torch.Tensor:
    """The workspace's control words as int32 (host copy): 64 header words
    (word 2: error flag) then eight words per (sequence, KV head).  Between
    calls every word is zero except each pair's step counter (word 3 of the
    pair); the error flag is set if a bounded wait ever ran out."""
    n = CTRL_WORDS_HEADER + CTRL_WORDS_PER_PAIR * batch * num_kv_heads
    return ws[: 4 * n].view(torch.int32).cpu()


def workspace_status(workspace: torch.Tensor) -> None:
    """Wait for the work queued on the current stream, then read and clear the
    workspace's error word; raise CompKVError (status CKV_ERR_INCOMPLETE) if
    a call since the last check left it set (its outputs are unspecified)."""
    word = ctypes.c_uint32(0)
    _check(load_library().ckv_workspace_status(_ptr(workspace), workspace.numel() * workspace.element_size(),
                                                ctypes.byref(word), _stream(workspace.device)))


def noalloc_status(device) -> None:
    """workspace_status for the built-in workspace of decode_step_noalloc on
    `device` (made current for the call)."""
    word = ctypes.c_uint32(0)
    with torch.cuda.device(device):
        _check(load_library().ckv_workspace_status(None, 0, ctypes.byref(word), _stream(torch.device(device))))


def score_select(dims: Dims, q, summaries: Summaries, block_table, seq_lens, budget_tokens: int,
                 workspace: torch.Tensor, score_mode: int = SCORE_COMPKV, selected=None,
                 num_selected=None, group_scores=None):
    lib = load_library()
    dev = q.device
    B, H = dims.batch, dims.num_kv_heads
    kmax = dims.kmax(budget_tokens)
    if selected is None:
        selected = torch.empty((B, H, max(kmax, 1)), dtype=torch.int32, device=dev)
    if num_selected is None:
        num_selected = torch.empty((B, H), dtype=torch.int32, device=dev)
    d = dims.c()
    s = summaries.c()
    _check(lib.ckv_score_select(ctypes.byref(d), _ptr(q), ctypes.byref(s), _ptr(block_table),
                                _ptr(seq_lens), budget_tokens, score_mode, _ptr(selected),
                                _ptr(num_selected), _ptr(group_scores), _ptr(workspace),
                                workspace.numel() * workspace.element_size(), _stream(dev)))
    return selected, num_selected


def compensated_decode_attention(dims: Dims, q, k_cache, v_cache, summaries: Summaries,
                                 block_table, seq_lens, budget_tokens: int, selected, num_selected,
                                 workspace: torch.Tensor, compensate: bool = True, out=None, lse=None):
    lib = load_library()
    dev = q.device
    if out is None:
        out = torch.empty((dims.batch, dims.num_q_heads, dims.head_dim), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((dims.batch, dims.num_q_heads), dtype=torch.float32, device=dev)
    d = dims.c()
    s = summaries.c()
    _check(lib.ckv_compensated_decode_attention(
        ctypes.byref(d), _ptr(q), _ptr(k_cache), _ptr(v_cache), ctypes.byref(s), _ptr(block_table),
        _ptr(seq_lens), budget_tokens, _ptr(selected), _ptr(num_selected), 1 if compensate else 0,
        _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(dev)))
    return out, lse


def decode_step(dims: Dims, q, k_cache, v_cache, summaries: Summaries, block_table, seq_lens,
                budget_tokens: int, workspace: torch.Tensor, score_mode: int = SCORE_COMPKV,
                selected=None, num_selected=None, out=None, lse=None):
    lib = load_library()
    dev = q.device
    B, H = dims.batch, dims.num_kv_heads
    kmax = dims.kmax(budget_tokens)
    if selected is None:
        selected = torch.empty((B, H, max(kmax, 1)), dtype=torch.int32, device=dev)
    if num_selected is None:
        num_selected = torch.empty((B, H), dtype=torch.int32, device=dev)
    if out is None:
        out = torch.empty((B, dims.num_q_heads, dims.head_dim), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((B, dims.num_q_heads), dtype=torch.float32, device=dev)
    d = dims.c()
    s = summaries.c()
    _check(lib.ckv_decode_step(
        ctypes.byref(d), _ptr(q), _ptr(k_cache), _ptr(v_cache), ctypes.byref(s), _ptr(block_table),
        _ptr(seq_lens), budget_tokens, score_mode, _ptr(selected), _ptr(num_selected), _ptr(out),
        _ptr(lse), _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(dev)))
    return selected, num_selected, out, lse


def decode_step_noalloc(dims: Dims, q, k_cache, v_cache, summaries: Summaries, block_table, seq_lens,
                        budget_tokens: int, score_mode: int = SCORE_COMPKV, selected=None, num_selected=None,
                        out=None, lse=None):
    """decode_step in the library's built-in workspace (the library
    allocates nothing; outputs not passed in are allocated here by torch)."""
    lib = load_library()
    dev = q.device
    B, H = dims.batch, dims.num_kv_heads
    kmax = dims.kmax(budget_tokens)
    if selected is None:
        selected = torch.empty((B, H, max(kmax, 1)), dtype=torch.int32, device=dev)
    if num_selected is None:
        num_selected = torch.empty((B, H), dtype=torch.int32, device=dev)
    if out is None:
        out = torch.empty((B, dims.num_q_heads, dims.head_dim), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((B, dims.num_q_heads), dtype=torch.float32, device=dev)
    d = dims.c()
    s = summaries.c()
    with torch.cuda.device(dev):
        _check(lib.ckv_decode_step_noalloc(
            ctypes.byref(d), _ptr(q), _ptr(k_cache), _ptr(v_cache), ctypes.byref(s), _ptr(block_table),
            _ptr(seq_lens), budget_tokens, score_mode, _ptr(selected), _ptr(num_selected), _ptr(out),
            _ptr(lse), _stream(dev)))
    return selected, num_selected, out, lse


def decode_step_append(dims: Dims, q, k_new, v_new, k_cache, v_cache, summaries: Summaries, block_table,
                       seq_lens, budget_tokens: int, workspace: torch.Tensor, score_mode: int = SCORE_COMPKV,
                       selected=None, num_selected=None, out=None, lse=None):
    """append_tokens followed by decode_step, as one call (one launch where
    the library can fuse them); seq_lens already count the new token."""
    lib = load_library()
    dev = q.device
    B, H = dims.batch, dims.num_kv_heads
    kmax = dims.kmax(budget_tokens)
    if selected is None:
        selected = torch.empty((B, H, max(kmax, 1)), dtype=torch.int32, device=dev)
    if num_selected is None:
        num_selected = torch.empty((B, H), dtype=torch.int32, device=dev)
    if out is None:
        out = torch.empty((B, dims.num_q_heads, dims.head_dim), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((B, dims.num_q_heads), dtype=torch.float32, device=dev)
    d = dims.c()
    s = summaries.c()
    _check(lib.ckv_decode_step_append(
        ctypes.byref(d), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), ctypes.byref(s),
        _ptr(block_table), _ptr(seq_lens), budget_tokens, score_mode, _ptr(selected), _ptr(num_selected),
        _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(dev)))
    return selected, num_selected, out, lse


def dense_decode_attention(dims: Dims, q, k_cache, v_cache, block_table, seq_lens,
                           workspace: torch.Tensor, out=None, lse=None):
    lib = load_library()
    dev = q.device
    if out is None:
        out = torch.empty((dims.batch, dims.num_q_heads, dims.head_dim), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((dims.batch, dims.num_q_heads), dtype=torch.float32, device=dev)
    d = dims.c()
    _check(lib.ckv_dense_decode_attention(
        ctypes.byref(d), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(seq_lens),
        _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(dev)))
    return out, lse
