"""Seeded synthetic inputs for one compensated block-sparse decode step.

Shapes and value distributions follow the workloads the CompKV pages speak
of: a Llama-3.1-8B-shaped attention layer (32 query heads, 8 KV heads,
head_dim 128), 32K and 128K contexts, token budgets of 512 and more (CompKV
review, evolve.pub: "Summary" and the FAQ on speed).  The pages measure
accuracy on RULER and LongBench-Pro; those suites are not available here, so
planted "needle" blocks (keys aligned with a query) stand in for retrieval
targets.  No item of any benchmark is reproduced.

This module holds none of the method's arithmetic.  It draws random numbers
with numpy's seeded generator, converts them to the storage format (bf16 by
round-to-nearest-even, or f32), and lays the tokens out in a paged KV cache
with a shuffled page table.  Both the GPU path and the CPU oracle consume the
same bits from here.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Sequence

import numpy as np

BF16_NAN_BITS = np.uint16(0x7FC0)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return raw bits.

    Inputs must be finite.  The 16 dropped bits are rounded by adding
    0x7FFF plus the lowest kept bit, which carries into the kept half exactly
    when the dropped part is above one half, or equal to it with an odd kept
    part.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen raw bfloat16 bits to float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass
class DecodeInputs:
    """One decode step's inputs for a batch of sequences.

    Storage arrays hold raw bf16 bits (``np.uint16``) when ``dtype == "bf16"``
    and ``np.float32`` values when ``dtype == "f32"``.
    """

    name: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    r_groups: int
    budget_tokens: int
    dtype: str
    seq_lens: np.ndarray          # int32 [B]
    q: np.ndarray                 # [B, Hq, d] storage
    k_tokens: List[np.ndarray]    # per sequence [L_b, Hkv, d] storage, logical order
    v_tokens: List[np.ndarray]
    block_table: np.ndarray       # int32 [B, max_blocks]; -1 where no page is mapped
    num_pages: int
    needles: List[np.ndarray]     # per sequence int [Hkv, n_needles] logical block ids
    outlier_channels: List[np.ndarray]  # per sequence int [Hkv, n_outliers]
    seed: int = 0

    @property
    def batch(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def max_blocks(self) -> int:
        return int(self.block_table.shape[1])

    def num_blocks(self, b: int) -> int:
        return -(-int(self.seq_lens[b]) // self.block_size)

    def storage_dtype(self):
        return np.uint16 if self.dtype == "bf16" else np.float32

    def paged_cache(self, fill_unused: bool = True):
        """Scatter tokens into ``[num_pages, Hkv, block_size, d]`` K and V caches.

        Slots past a sequence's length are filled with NaN so that a kernel
        reading them would poison its output.
        """
        P, H, bs, d = self.num_pages, self.num_kv_heads, self.block_size, self.head_dim
        if self.dtype == "bf16":
            k_cache = np.full((P, H, bs, d), BF16_NAN_BITS, dtype=np.uint16)
            v_cache = np.full((P, H, bs, d), BF16_NAN_BITS, dtype=np.uint16)
        else:
            k_cache = np.full((P, H, bs, d), np.nan, dtype=np.float32)
            v_cache = np.full((P, H, bs, d), np.nan, dtype=np.float32)
        if not fill_unused:
            k_cache[...] = 0
            v_cache[...] = 0
        for b in range(self.batch):
            self._scatter(b, self.k_tokens[b], k_cache)
            self._scatter(b, self.v_tokens[b], v_cache)
        return k_cache, v_cache

    def _scatter(self, b: int, tok: np.ndarray, cache: np.ndarray) -> None:
        L = tok.shape[0]
        bs = self.block_size
        full = L // bs
        pages = self.block_table[b]
        if full:
            tiles = tok[: full * bs].reshape(full, bs, self.num_kv_heads, self.head_dim)
            cache[pages[:full]] = tiles.transpose(0, 2, 1, 3)
        rem = L - full * bs
        if rem:
            cache[pages[full], :, :rem, :] = tok[full * bs:].transpose(1, 0, 2)


@dataclasses.dataclass
class AppendStep:
    """One decode step of a generation loop: the new token's K/V and the query."""

    q: np.ndarray      # [B, Hq, d] storage
    k_new: np.ndarray  # [B, Hkv, d] storage
    v_new: np.ndarray  # [B, Hkv, d] storage


def _to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    raise ValueError(f"unknown storage dtype {dtype!r}")


def make_decode_inputs(
    *,
    name: str = "custom",
    seq_lens: Sequence[int],
    num_q_heads: int,
    num_kv_heads: int,
    head_dim: int,
    block_size: int = 16,
    r_groups: int = 4,
    budget_tokens: int = 512,
    dtype: str = "bf16",
    n_needles: int = 16,
    n_outliers: int = 4,
    outlier_scale: float = 8.0,
    needle_q_scale: float = 0.5,
    needle_noise: float = 0.3,
    extra_capacity_tokens: int = 0,
    seed: int = 0,
) -> DecodeInputs:
    """Draw one decode step's inputs.

    q, K and V are i.i.d. N(0, 1) in float32.  Per (sequence, KV head),
    ``n_outliers`` distinct key channels are scaled by ``outlier_scale`` and
    then ``n_needles`` distinct full blocks are overwritten with keys
    ``needle_q_scale * q[h*] + needle_noise * N(0, 1)``, where ``h*`` cycles
    over the query heads sharing that KV head.  Values are then rounded to
    the storage dtype.  Physical pages are a seeded random permutation, with
    ``extra_capacity_tokens`` of spare pages per sequence for appends.
    """
    rng = np.random.default_rng(seed)
    B = len(seq_lens)
    Hq, Hkv, d, bs = num_q_heads, num_kv_heads, head_dim, block_size
    if Hq % Hkv:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    G = Hq // Hkv
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    q32 = rng.standard_normal((B, Hq, d), dtype=np.float32)
    k_tokens, v_tokens, needles, outliers = [], [], [], []
    for b in range(B):
        L = int(seq_lens[b])
        k = rng.standard_normal((L, Hkv, d), dtype=np.float32)
        och = np.zeros((Hkv, n_outliers), dtype=np.int64)
        for g in range(Hkv):
            if n_outliers:
                och[g] = np.sort(rng.choice(d, n_outliers, replace=False))
                k[:, g, och[g]] *= np.float32(outlier_scale)
        nd = np.zeros((Hkv, n_needles), dtype=np.int64)
        full_blocks = L // bs
        for g in range(Hkv):
            if n_needles:
                if n_needles > full_blocks:
                    raise ValueError("more needles than full blocks")
                nd[g] = np.sort(rng.choice(full_blocks, n_needles, replace=False))
                for j, i in enumerate(nd[g]):
                    hstar = g * G + (j % G)
                    noise = rng.standard_normal((bs, d), dtype=np.float32)
                    k[i * bs:(i + 1) * bs, g, :] = (np.float32(needle_q_scale) * q32[b, hstar][None, :]
                                                    + np.float32(needle_noise) * noise)
        v = rng.standard_normal((L, Hkv, d), dtype=np.float32)
        k_tokens.append(_to_storage(k, dtype))
        v_tokens.append(_to_storage(v, dtype))
        needles.append(nd)
        outliers.append(och)
        del k, v
    caps = [-(-(int(L) + extra_capacity_tokens) // bs) for L in seq_lens]
    P = int(sum(caps))
    perm = rng.permutation(P).astype(np.int32)
    max_blocks = max(caps) if caps else 0
    table = np.full((B, max_blocks), -1, dtype=np.int32)
    off = 0
    for b, c in enumerate(caps):
        table[b, :c] = perm[off:off + c]
        off += c
    return DecodeInputs(
        name=name, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d, block_size=bs,
        r_groups=r_groups, budget_tokens=budget_tokens, dtype=dtype, seq_lens=seq_lens,
        q=_to_storage(q32, dtype), k_tokens=k_tokens, v_tokens=v_tokens, block_table=table,
        num_pages=P, needles=needles, outlier_channels=outliers, seed=seed)


def make_append_steps(inputs: DecodeInputs, steps: int, seed: int = 1) -> List[AppendStep]:
    """Fresh q, k, v per decode step, same distributions as ``inputs``
    (the new keys get the same outlier-channel scaling)."""
    rng = np.random.default_rng(seed)
    B, Hq, Hkv, d = inputs.batch, inputs.num_q_heads, inputs.num_kv_heads, inputs.head_dim
    out = []
    scale = np.float32(8.0)
    for _ in range(steps):
        q = rng.standard_normal((B, Hq, d), dtype=np.float32)
        k = rng.standard_normal((B, Hkv, d), dtype=np.float32)
        for b in range(B):
            for g in range(Hkv):
                och = inputs.outlier_channels[b][g]
                if och.size:
                    k[b, g, och] *= scale
        v = rng.standard_normal((B, Hkv, d), dtype=np.float32)
        out.append(AppendStep(_to_storage(q, inputs.dtype), _to_storage(k, inputs.dtype),
                              _to_storage(v, inputs.dtype)))
    return out


def append_tokens(inputs: DecodeInputs, step: AppendStep) -> None:
    """Append one token per sequence to ``inputs`` in place (logical arrays,
    lengths and query).  Pages must have spare capacity."""
    for b in range(inputs.batch):
        L = int(inputs.seq_lens[b])
        if (L + 1 + inputs.block_size - 1) // inputs.block_size > inputs.max_blocks or \
                inputs.block_table[b, L // inputs.block_size] < 0:
            raise ValueError("no spare page capacity for append")
        inputs.k_tokens[b] = np.concatenate([inputs.k_tokens[b], step.k_new[b][None]], axis=0)
        inputs.v_tokens[b] = np.concatenate([inputs.v_tokens[b], step.v_new[b][None]], axis=0)
        inputs.seq_lens[b] = L + 1
    inputs.q = step.q.copy()


# Named workloads.  "tiny" is the parity case the oracle finishes in well
# under a second; "llama_128k" is the headline decode step (128K context,
# 512-token budget); the others are parity and coverage cases.
PRESETS = {
    "tiny": dict(seq_lens=[4096], num_q_heads=1, num_kv_heads=1, head_dim=64, block_size=16,
                 r_groups=4, budget_tokens=256, dtype="f32", n_needles=4, n_outliers=0),
    "llama_32k": dict(seq_lens=[32768], num_q_heads=32, num_kv_heads=8, head_dim=128,
                      block_size=16, r_groups=4, budget_tokens=512, dtype="bf16",
                      n_needles=16, n_outliers=4),
    "llama_128k": dict(seq_lens=[131072], num_q_heads=32, num_kv_heads=8, head_dim=128,
                       block_size=16, r_groups=4, budget_tokens=512, dtype="bf16",
                       n_needles=16, n_outliers=4),
    "prefill_128k_loop": dict(seq_lens=[131072], num_q_heads=32, num_kv_heads=8, head_dim=128,
                              block_size=16, r_groups=4, budget_tokens=2048, dtype="bf16",
                              n_needles=16, n_outliers=4, extra_capacity_tokens=64),
}


def ragged_lengths(batch: int = 16, lo: int = 16384, hi: int = 65536, seed: int = 0) -> List[int]:
    """Sequence lengths uniform on the integers [lo, hi]."""
    rng = np.random.default_rng(10_000 + seed)
    return [int(x) for x in rng.integers(lo, hi + 1, size=batch)]


def make_preset(name: str, seed: int = 0, **overrides) -> DecodeInputs:
    if name == "batched_ragged":
        cfg = dict(seq_lens=ragged_lengths(16, seed=seed), num_q_heads=32, num_kv_heads=8,
                   head_dim=128, block_size=16, r_groups=4, budget_tokens=1024, dtype="bf16",
                   n_needles=16, n_outliers=4)
    else:
        cfg = dict(PRESETS[name])
    cfg.update(overrides)
    return make_decode_inputs(name=name, seed=seed, **cfg)
