"""Seeded inputs for the paged FP8 KV append: a cache state before the
append and the new tokens' K/V rows (input generation only; the quantiser
used to fill the cached part is the one the attention inputs use).

Recipe: numpy ``default_rng(seed)``; draw order pool permutation -> cached K
-> cached V -> new K -> new V.  Cached values ~ N(0,1) fp32 quantised per
(page, kv head) over the cached slots only; pages with no cached slot are
fresh pool pages (every byte the poison code 0x7F, scales NaN), as are the
unreferenced ones.  New values ~ N(0, sigma_b^2) with sigma_b drawn per
sequence from ``new_sigmas`` (values above 1 make pages' scales grow, so
cached tokens are requantised), rounded to nearest-even into the new-row
dtype.  Sequence b caches ctx_b - q_b tokens and appends q_b.
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np
import torch

from .workloads import (PAGE_SIZE, POISON_BYTE, _quantise_pages, _quantise_pages_int8, empty_pages, k_to_layout,
                        v_to_layout)


@dataclass
class AppendCase:
    name: str
    num_kv_heads: int
    head_dim: int
    new_dtype: str  # "bf16" or "f32"
    q_lens: np.ndarray  # int32 [B] tokens appended
    ctx_lens: np.ndarray  # int32 [B] tokens after the append
    block_table: np.ndarray  # int32 [B][max_pages_per_seq]
    k_pages: np.ndarray  # uint8 pools before the append (ABI layouts)
    v_pages: np.ndarray
    kv_scales: np.ndarray  # float32 [2][P][Hkv]
    k_new: torch.Tensor  # [sum Q][Hkv][D] new_dtype (CPU)
    v_new: torch.Tensor
    seed: int = 0
    kv_format: str = "e4m3"  # or "int8" (cached part quantised to two's-complement bytes, absmax / 127)

    @property
    def num_seqs(self) -> int:
        return int(self.q_lens.shape[0])

    @property
    def num_pages(self) -> int:
        return int(self.k_pages.shape[0])

    @property
    def max_pages_per_seq(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def max_ctx_len(self) -> int:
        return int(self.ctx_lens.max())

    @property
    def max_q_len(self) -> int:
        return int(self.q_lens.max())

    @property
    def total_q(self) -> int:
        return int(self.q_lens.sum())


def _round(x: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    if dtype == "bf16":
        return t.to(torch.bfloat16)
    if dtype == "f32":
        return t
    raise ValueError(dtype)


def append_case(q_lens, ctx_lens, *, num_kv_heads=8, head_dim=128, new_dtype="bf16", seed=0,
                new_sigmas=(0.5, 1.0, 2.0), num_pages=None, max_pages_per_seq=None, name="append",
                kv_format="e4m3") -> AppendCase:
    S = PAGE_SIZE
    q_lens = np.asarray(q_lens, dtype=np.int32)
    ctx_lens = np.asarray(ctx_lens, dtype=np.int32)
    if np.any(q_lens < 1) or np.any(ctx_lens < q_lens):
        raise ValueError("need 1 <= q_len <= ctx_len")
    rng = np.random.default_rng(seed)
    B = q_lens.size
    npages = (ctx_lens + S - 1) // S
    used = int(npages.sum())
    if max_pages_per_seq is None:
        max_pages_per_seq = int(npages.max())
    if num_pages is None:
        num_pages = int(math.ceil(1.125 * used))
    phys = rng.permutation(num_pages).astype(np.int32)
    block_table = np.full((B, max_pages_per_seq), -1, dtype=np.int32)
    first = np.concatenate([[0], np.cumsum(npages)[:-1]]).astype(np.int64)
    cached_slots = np.zeros(used, dtype=np.int64)
    for b in range(B):
        block_table[b, : npages[b]] = phys[first[b] : first[b] + npages[b]]
        cached = int(ctx_lens[b] - q_lens[b])
        for pi in range(int(npages[b])):
            cached_slots[first[b] + pi] = max(0, min(S, cached - pi * S))

    k_pages, v_pages = empty_pages(num_pages, num_kv_heads, head_dim)
    kv_scales = np.full((2, num_pages, num_kv_heads), np.nan, dtype=np.float32)
    has = cached_slots > 0
    idx = np.nonzero(has)[0]
    for which in range(2):
        x = rng.standard_normal((used, num_kv_heads, S, head_dim), dtype=np.float32)
        if idx.size:
            quantise = _quantise_pages_int8 if kv_format == "int8" else _quantise_pages
            codes, scale = quantise(x[idx], cached_slots[idx])
            pool = k_pages if which == 0 else v_pages
            pool[phys[idx]] = k_to_layout(codes) if which == 0 else v_to_layout(codes)
            kv_scales[which, phys[idx]] = scale
        del x

    sig = np.asarray(new_sigmas, dtype=np.float32)[rng.integers(0, len(new_sigmas), size=B)]
    total_q = int(q_lens.sum())
    rows_sigma = np.repeat(sig, q_lens)[:, None, None]
    k_new = rng.standard_normal((total_q, num_kv_heads, head_dim), dtype=np.float32) * rows_sigma
    v_new = rng.standard_normal((total_q, num_kv_heads, head_dim), dtype=np.float32) * rows_sigma
    return AppendCase(name=name, num_kv_heads=num_kv_heads, head_dim=head_dim, new_dtype=new_dtype, q_lens=q_lens,
                      ctx_lens=ctx_lens, block_table=block_table, k_pages=k_pages, v_pages=v_pages,
                      kv_scales=kv_scales, k_new=_round(k_new, new_dtype), v_new=_round(v_new, new_dtype), seed=seed,
                      kv_format=kv_format)


# Append steps of the measured serving shapes: the decode step of the
# LLaMA-3-8B-shaped batch (one token per sequence) and the prefill chunk
# (512 tokens per sequence on top of 0..8192 cached ones).
APPEND_CONFIGS = {"append_decode": dict(seed=12), "append_prefill": dict(seed=15)}


def make_append_case(name: str, seed: int | None = None, *, batch: int | None = None,
                     ctx_range: tuple | None = None, new_dtype: str = "bf16", q_len: int | None = None,
                     kv_format: str = "e4m3") -> AppendCase:
    if name not in APPEND_CONFIGS:
        raise KeyError(name)
    seed = APPEND_CONFIGS[name]["seed"] if seed is None else seed
    rng = np.random.default_rng(seed)
    if name == "append_decode":
        B = batch or 32
        lo, hi = ctx_range or (512, 4096)
        ctx = rng.integers(lo, hi + 1, size=B).astype(np.int32)
        q = np.ones(B, np.int32)
        mpps = (hi + PAGE_SIZE - 1) // PAGE_SIZE
    else:
        B = batch or 8
        chunk = q_len or 512
        lo, hi = ctx_range or (0, 8192)  # cached tokens
        cached = rng.integers(lo, hi + 1, size=B).astype(np.int32)
        ctx = cached + chunk
        q = np.full(B, chunk, np.int32)
        mpps = (hi + chunk + PAGE_SIZE - 1) // PAGE_SIZE
    return append_case(q, ctx, num_kv_heads=8, head_dim=128, new_dtype=new_dtype,
                       seed=int(rng.integers(0, 2**31)), max_pages_per_seq=mpps, name=name, kv_format=kv_format)


__all__ = ["AppendCase", "append_case", "make_append_case", "APPEND_CONFIGS", "POISON_BYTE"]
