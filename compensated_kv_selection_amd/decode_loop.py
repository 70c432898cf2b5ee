"""A generation loop over one paged attention layer: every step appends one
token per sequence and runs the compensated decode step on the grown context.

Per step, one ckv_decode_step_append call writes every sequence's new key
and value into the page slot its block table gives for the new position,
recomputes that block's summary, then scores, selects and attends.  Where
the library fuses the two that is one launch; otherwise (and with
``fused=False``) it is ckv_append_tokens followed by ckv_decode_step.  All
per-step inputs (queries, new keys and values, lengths) are staged on the
device up front and passed to the calls in place, and every step writes its
own output buffers, so any run of steps can be captured into one HIP graph
and replayed.
"""
from __future__ import annotations

from typing import Sequence

import numpy as np
import torch

from . import compkv as C
from .tensors import DeviceInputs, storage_to_torch


class DecodeLoop:
    def __init__(self, dev: DeviceInputs, summaries: C.Summaries, block_table: np.ndarray,
                 start_lens: Sequence[int], steps, dtype: str, workspace: torch.Tensor = None,
                 fused: bool = True):
        """``steps`` holds per-step ``q`` [B, Hq, d], ``k_new`` and ``v_new``
        [B, Hkv, d] in storage form; ``start_lens`` are the lengths before the
        first step.  Raises if a sequence runs out of pages."""
        dims = dev.dims
        device = dev.q.device
        B, T, bs = dims.batch, len(steps), dims.block_size
        self.dev, self.summ, self.dims, self.T, self.fused = dev, summaries, dims, T, fused
        self.budget = dev.budget_tokens
        lens = np.zeros((T, B), dtype=np.int32)
        for t in range(T):
            for b in range(B):
                pos = int(start_lens[b]) + t
                if pos // bs >= block_table.shape[1] or block_table[b, pos // bs] < 0:
                    raise ValueError(f"sequence {b} has no page for position {pos}")
                lens[t, b] = pos + 1
        self.lens = torch.from_numpy(lens).to(device)
        self.q = torch.stack([storage_to_torch(s.q, dtype) for s in steps]).to(device)
        self.k_new = torch.stack([storage_to_torch(s.k_new, dtype) for s in steps]).to(device)
        self.v_new = torch.stack([storage_to_torch(s.v_new, dtype) for s in steps]).to(device)
        kmax = max(1, dims.kmax(self.budget))
        self.selected = torch.empty((T, B, dims.num_kv_heads, kmax), dtype=torch.int32, device=device)
        self.num_selected = torch.empty((T, B, dims.num_kv_heads), dtype=torch.int32, device=device)
        self.out = torch.empty((T, B, dims.num_q_heads, dims.head_dim), dtype=torch.float32, device=device)
        self.lse = torch.empty((T, B, dims.num_q_heads), dtype=torch.float32, device=device)
        self.ws = workspace if workspace is not None else \
            C.allocate_workspace(C.workspace_bytes(dims, self.budget), device)

    def step(self, t: int) -> None:
        """Step t: lengths self.lens[t] (they count the new token), query
        self.q[t]; the device inputs' own q and seq_lens are not used."""
        d = self.dev
        if self.fused:
            C.decode_step_append(self.dims, self.q[t], self.k_new[t], self.v_new[t], d.k_cache, d.v_cache,
                                 self.summ, d.block_table, self.lens[t], self.budget, self.ws,
                                 selected=self.selected[t], num_selected=self.num_selected[t],
                                 out=self.out[t], lse=self.lse[t])
            return
        C.append_tokens(self.dims, self.k_new[t], self.v_new[t], d.k_cache, d.v_cache, d.block_table,
                        self.lens[t], self.summ)
        C.decode_step(self.dims, self.q[t], d.k_cache, d.v_cache, self.summ, d.block_table, self.lens[t],
                      self.budget, self.ws, selected=self.selected[t], num_selected=self.num_selected[t],
                      out=self.out[t], lse=self.lse[t])

    def run(self, first: int = 0, last: int = None) -> None:
        for t in range(first, self.T if last is None else last):
            self.step(t)

    def capture(self) -> torch.cuda.CUDAGraph:
        """All steps in one HIP graph (the caller replays it)."""
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.run()
        return g
