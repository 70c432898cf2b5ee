"""Move generated decode-step inputs (numpy storage arrays) to device tensors."""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

from .compkv import CKV_BF16, CKV_F32, Dims
from .workloads import DecodeInputs


def storage_to_torch(x: np.ndarray, dtype: str) -> torch.Tensor:
    """uint16 bf16 bits -> torch.bfloat16 (same bits); float32 -> torch.float32."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))


def torch_to_storage(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


@dataclasses.dataclass
class DeviceInputs:
    dims: Dims
    q: torch.Tensor
    k_cache: torch.Tensor
    v_cache: torch.Tensor
    block_table: torch.Tensor
    seq_lens: torch.Tensor
    budget_tokens: int


def dims_of(w: DecodeInputs) -> Dims:
    return Dims(batch=w.batch, num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads,
                head_dim=w.head_dim, block_size=w.block_size, r_groups=w.r_groups,
                num_pages=w.num_pages, max_blocks_per_seq=w.max_blocks,
                kv_dtype=CKV_BF16 if w.dtype == "bf16" else CKV_F32)


def to_device(w: DecodeInputs, device="cuda:0", k_cache=None, v_cache=None) -> DeviceInputs:
    if k_cache is None or v_cache is None:
        k_cache, v_cache = w.paged_cache()
    return DeviceInputs(
        dims=dims_of(w),
        q=storage_to_torch(w.q, w.dtype).to(device),
        k_cache=storage_to_torch(k_cache, w.dtype).to(device),
        v_cache=storage_to_torch(v_cache, w.dtype).to(device),
        block_table=torch.from_numpy(w.block_table).to(device),
        seq_lens=torch.from_numpy(w.seq_lens.astype(np.int32)).to(device),
        budget_tokens=w.budget_tokens,
    )
