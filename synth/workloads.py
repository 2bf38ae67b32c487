"""Seeded synthetic workloads shaped like the pages' serving scenarios.

This module only *generates inputs*: sequence lengths, a shuffled physical page
pool with its block table, Q, and K/V quantised to OCP FP8 E4M3 with one fp32
scale per (page, kv head).  It holds none of the attention arithmetic, and
both the CPU oracle and the GPU path consume what it produces without it
importing either of them.

Sources of the shapes:
  * Atlas engine article (ainews.cool, "技术深度解析" and its benchmark table):
    LLaMA-3-8B decode at batch 1 and 32 -> 32 query heads / 8 KV heads /
    head_dim 128 decode batches.
  * "Atlas Takes On vLLM ... on a Single GB10" (ainews.surl.tw): paged FP8 KV
    cache, 128-token prompts with 1024 generated tokens and MTP with K=4 ->
    verification batches of 1+4 query tokens over 128..1152 cached tokens.
  * Long-context split decode, a chunked-prefill tile and MQA decode complete
    the set of shapes the kernels are measured on.

Recipe (every config): numpy ``default_rng(seed)``; draw order lengths ->
pool permutation -> Q -> K -> V.  Q ~ N(0,1) rounded to nearest-even into the
Q dtype.  K, V ~ N(0,1) in fp32, quantised per (page, kv head): scale =
fp32(absmax over the page's valid tokens) / 448 (1.0 if absmax is 0), byte =
round-to-nearest-even E4M3 of fp32(x / scale), saturated to +-448.  Slots past
a sequence's length and every unreferenced page hold the NaN code 0x7F; the
scales of unreferenced pages are NaN; unused block-table entries are -1.

Memory layouts (the library's ABI; S = 16 slots, D a multiple of 64):
  k_pages   uint8 [P][Hkv][D/16][S][16]   inside a (page, head): 16-byte blocks
                                          of d, slot-major within a block; the
                                          byte of (slot s, d) is
                                          k[p][h][d/16][s][d%16]
  v_pages   uint8 [P][Hkv][S/4][D/64][16][4][4]
                                          inside a (page, head): four
                                          consecutive slots interleaved per d;
                                          with NVB = D/16, d = NVB*a + 4*i + e,
                                          the byte of (slot s, d) is
                                          v[p][h][s/4][i][a][e][s%4]
  kv_scales fp32  [2][P][Hkv]             [0] = K scale, [1] = V scale
  block_table int32 [B][max_pages_per_seq]
  q         [sum(q_lens)][Hq][D]          sequences concatenated in order
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

PAGE_SIZE = 16
E4M3_MAX = 448.0
POISON_BYTE = 0x7F
INT4_POISON = 0x8  # the 4-bit code of -8: never produced by the INT4 quantiser


@dataclass
class Workload:
    name: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    q_dtype: str  # "f32" or "bf16"
    out_dtype: str  # "f32" or "bf16"
    q_lens: np.ndarray  # int32 [B]
    ctx_lens: np.ndarray  # int32 [B]; keys visible to the last query row, new tokens included
    block_table: np.ndarray  # int32 [B][max_pages_per_seq]
    k_pages: np.ndarray  # uint8 [P][Hkv][D/16][S][16]
    v_pages: np.ndarray  # uint8 [P][Hkv][S/4][D/64][16][4][4]
    kv_scales: np.ndarray  # float32 [2][P][Hkv]
    q: torch.Tensor  # CPU tensor [sum Q][Hq][D], float32 or bfloat16
    max_q_len: int
    max_ctx_len: int
    num_kv_splits: int = 0  # 0: the plan chooses
    sm_scale: float = 0.0  # 0: 1/sqrt(head_dim)
    seed: int = 0
    # Per-sequence logical (unpaged) copies of the quantised K/V, for tests.
    logical: list = field(default_factory=list, repr=False)
    kv_format: str = "e4m3"  # "int8": two's-complement bytes, scale = absmax / 127; "int4": 4-bit codes,
    # two per byte, scale = absmax / 7 (the logical copies then hold one code per uint8)

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
    def total_q(self) -> int:
        return int(self.q_lens.sum())

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads


def _round_q(x: np.ndarray, q_dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    if q_dtype == "bf16":
        return t.to(torch.bfloat16)  # round to nearest even
    if q_dtype == "f32":
        return t
    raise ValueError(q_dtype)


def _quantise_pages(x: np.ndarray, valid_slots: np.ndarray):
    """x: float32 [N][Hkv][S][D]; valid_slots: int [N] tokens used per page.

    Returns (bytes uint8 [N][Hkv][S][D] with poison in unused slots,
    scales float32 [N][Hkv]).
    """
    n, hkv, s, d = x.shape
    slot_ok = np.arange(s)[None, :] < valid_slots[:, None]  # [N][S]
    masked = np.where(slot_ok[:, None, :, None], np.abs(x), np.float32(0))
    absmax = masked.reshape(n, hkv, s * d).max(axis=2).astype(np.float32)
    scale = (absmax / np.float32(E4M3_MAX)).astype(np.float32)
    scale = np.where(absmax > 0, scale, np.float32(1.0)).astype(np.float32)
    y = (x / scale[:, :, None, None]).astype(np.float32)
    y = np.clip(y, -E4M3_MAX, E4M3_MAX)
    codes = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    codes = np.where(slot_ok[:, None, :, None], codes, np.uint8(POISON_BYTE)).astype(np.uint8)
    return codes, scale


def _quantise_pages_int8(x: np.ndarray, valid_slots: np.ndarray):
    """INT8 variant of _quantise_pages: scale = fp32(absmax) / 127 (1.0 if
    absmax is 0), byte = round-half-even of fp32(x / scale) clipped to +-127,
    stored two's complement; poison in unused slots."""
    n, hkv, s, d = x.shape
    slot_ok = np.arange(s)[None, :] < valid_slots[:, None]
    masked = np.where(slot_ok[:, None, :, None], np.abs(x), np.float32(0))
    absmax = masked.reshape(n, hkv, s * d).max(axis=2).astype(np.float32)
    scale = (absmax / np.float32(127.0)).astype(np.float32)
    scale = np.where(absmax > 0, scale, np.float32(1.0)).astype(np.float32)
    y = (x / scale[:, :, None, None]).astype(np.float32)
    codes = np.clip(np.rint(y), -127, 127).astype(np.int8).view(np.uint8)
    codes = np.where(slot_ok[:, None, :, None], codes, np.uint8(POISON_BYTE)).astype(np.uint8)
    return codes, scale


def _quantise_pages_int4(x: np.ndarray, valid_slots: np.ndarray):
    """INT4 variant of _quantise_pages: scale = fp32(absmax) / 7 (1.0 if
    absmax is 0), code = round-half-even of fp32(x / scale) clipped to +-7,
    kept as its 4-bit two's complement (0..15, one per uint8); unused slots
    hold the code of -8, which the quantiser never produces."""
    n, hkv, s, d = x.shape
    slot_ok = np.arange(s)[None, :] < valid_slots[:, None]
    masked = np.where(slot_ok[:, None, :, None], np.abs(x), np.float32(0))
    absmax = masked.reshape(n, hkv, s * d).max(axis=2).astype(np.float32)
    scale = (absmax / np.float32(7.0)).astype(np.float32)
    scale = np.where(absmax > 0, scale, np.float32(1.0)).astype(np.float32)
    y = (x / scale[:, :, None, None]).astype(np.float32)
    codes = (np.clip(np.rint(y), -7, 7).astype(np.int8).view(np.uint8) & 0x0F).astype(np.uint8)
    codes = np.where(slot_ok[:, None, :, None], codes, np.uint8(INT4_POISON)).astype(np.uint8)
    return codes, scale


def empty_pages4(num_pages: int, num_kv_heads: int, head_dim: int):
    """INT4 K and V pools in the ABI layouts (two codes per byte), every code -8."""
    if head_dim != 128:
        raise ValueError("INT4 pools are laid out for head_dim 128")
    S = PAGE_SIZE
    byte = np.uint8(INT4_POISON | (INT4_POISON << 4))
    k = np.full((num_pages, num_kv_heads, 4, S, head_dim // 8), byte, dtype=np.uint8)
    v = np.full((num_pages, num_kv_heads, S // 4, 16, head_dim // 16, 2), byte, dtype=np.uint8)
    return k, v


def k4_to_layout(codes: np.ndarray) -> np.ndarray:
    """[N][Hkv][S][D] 4-bit codes -> [N][Hkv][4][S][D/8] bytes: quarter c of d
    (d = c D/4 + u) holds u = 2 j (low nibble) and u = 2 j + 1 (high) in byte j."""
    n, hkv, s, d = codes.shape
    x = codes.reshape(n, hkv, s, 4, d // 8, 2).transpose(0, 1, 3, 2, 4, 5)  # [n][h][c][s][j][bit]
    return np.ascontiguousarray((x[..., 0] | (x[..., 1] << 4)).astype(np.uint8))


def v4_to_layout(codes: np.ndarray) -> np.ndarray:
    """[N][Hkv][S][D] 4-bit codes -> [N][Hkv][S/4][16][D/16][2] bytes: slot
    s = 4 g + 2 k + bit, d = (D/16) a + r; byte [g][a][r][k] holds bit 0 low."""
    n, hkv, s, d = codes.shape
    nvb = d // 16
    x = codes.reshape(n, hkv, s // 4, 2, 2, 16, nvb)  # [n][h][g][k][bit][a][r]
    x = x.transpose(0, 1, 2, 5, 6, 3, 4)  # [n][h][g][a][r][k][bit]
    return np.ascontiguousarray((x[..., 0] | (x[..., 1] << 4)).astype(np.uint8))


def empty_pages(num_pages: int, num_kv_heads: int, head_dim: int):
    """K and V pools in the ABI layouts, every byte the poison code."""
    if head_dim % 64:
        raise ValueError("head_dim must be a multiple of 64")
    S = PAGE_SIZE
    k = np.full((num_pages, num_kv_heads, head_dim // 16, S, 16), POISON_BYTE, dtype=np.uint8)
    v = np.full((num_pages, num_kv_heads, S // 4, head_dim // 64, 16, 4, 4), POISON_BYTE, dtype=np.uint8)
    return k, v


def k_to_layout(codes: np.ndarray) -> np.ndarray:
    """[N][Hkv][S][D] bytes -> [N][Hkv][D/16][S][16]."""
    n, hkv, s, d = codes.shape
    return np.ascontiguousarray(codes.reshape(n, hkv, s, d // 16, 16).transpose(0, 1, 3, 2, 4))


def v_to_layout(codes: np.ndarray) -> np.ndarray:
    """[N][Hkv][S][D] bytes -> [N][Hkv][S/4][D/64][16][4][4]."""
    n, hkv, s, d = codes.shape
    # slot = 4*g + r; d = (D/16)*a + 4*i + e
    x = codes.reshape(n, hkv, s // 4, 4, 16, d // 64, 4)  # [n][h][g][r][a][i][e]
    return np.ascontiguousarray(x.transpose(0, 1, 2, 5, 4, 6, 3))  # [n][h][g][i][a][e][r]


def build_workload(
    name: str,
    rng: np.random.Generator,
    *,
    q_lens,
    ctx_lens,
    num_q_heads: int,
    num_kv_heads: int,
    head_dim: int,
    q_dtype: str = "bf16",
    out_dtype: str = "bf16",
    max_q_len: int | None = None,
    max_ctx_len: int | None = None,
    num_pages: int | None = None,
    max_pages_per_seq: int | None = None,
    num_kv_splits: int = 0,
    seed: int = 0,
    keep_logical: bool = True,
    kv_format: str = "e4m3",
) -> Workload:
    """Build a workload from drawn lengths, continuing the rng's draw order."""
    S = PAGE_SIZE
    q_lens = np.asarray(q_lens, dtype=np.int32)
    ctx_lens = np.asarray(ctx_lens, dtype=np.int32)
    B = q_lens.shape[0]
    if num_q_heads % num_kv_heads:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    if np.any(q_lens < 1) or np.any(ctx_lens < q_lens):
        raise ValueError("need 1 <= q_len <= ctx_len for every sequence")
    max_q_len = int(max_q_len if max_q_len is not None else q_lens.max())
    max_ctx_len = int(max_ctx_len if max_ctx_len is not None else ctx_lens.max())
    npages = (ctx_lens + S - 1) // S
    used = int(npages.sum())
    if max_pages_per_seq is None:
        max_pages_per_seq = (max_ctx_len + S - 1) // S
    if num_pages is None:
        num_pages = int(math.ceil(1.125 * used))
    if num_pages < used:
        raise ValueError("pool too small")

    # pool permutation: logical page k (sequence-major order) -> physical id
    phys = rng.permutation(num_pages).astype(np.int32)
    block_table = np.full((B, max_pages_per_seq), -1, dtype=np.int32)
    first = np.concatenate([[0], np.cumsum(npages)[:-1]]).astype(np.int64)
    for b in range(B):
        block_table[b, : npages[b]] = phys[first[b] : first[b] + npages[b]]

    total_q = int(q_lens.sum())
    q = _round_q(rng.standard_normal((total_q, num_q_heads, head_dim), dtype=np.float32), q_dtype)

    # valid tokens in each logical page
    valid = np.empty(used, dtype=np.int64)
    for b in range(B):
        n = int(npages[b])
        v = np.full(n, S, dtype=np.int64)
        v[-1] = int(ctx_lens[b]) - (n - 1) * S
        valid[first[b] : first[b] + n] = v

    k_f = rng.standard_normal((used, num_kv_heads, S, head_dim), dtype=np.float32)
    quantise = {"int8": _quantise_pages_int8, "int4": _quantise_pages_int4}.get(kv_format, _quantise_pages)
    k_codes, k_scale = quantise(k_f, valid)
    del k_f
    v_f = rng.standard_normal((used, num_kv_heads, S, head_dim), dtype=np.float32)
    v_codes, v_scale = quantise(v_f, valid)
    del v_f

    int4 = kv_format == "int4"
    k_pages, v_pages = (empty_pages4 if int4 else empty_pages)(num_pages, num_kv_heads, head_dim)
    kv_scales = np.full((2, num_pages, num_kv_heads), np.nan, dtype=np.float32)
    used_phys = phys[:used]
    k_pages[used_phys] = (k4_to_layout if int4 else k_to_layout)(k_codes)
    v_pages[used_phys] = (v4_to_layout if int4 else v_to_layout)(v_codes)
    kv_scales[0, used_phys] = k_scale
    kv_scales[1, used_phys] = v_scale

    logical = []
    if keep_logical:
        for b in range(B):
            n, L = int(npages[b]), int(ctx_lens[b])
            sl = slice(int(first[b]), int(first[b]) + n)
            kb = k_codes[sl].transpose(1, 0, 2, 3).reshape(num_kv_heads, n * S, head_dim)[:, :L]
            vb = v_codes[sl].transpose(1, 0, 2, 3).reshape(num_kv_heads, n * S, head_dim)[:, :L]
            ks = np.repeat(k_scale[sl].T, S, axis=1)[:, :L]
            vs = np.repeat(v_scale[sl].T, S, axis=1)[:, :L]
            logical.append(
                dict(k_bytes=np.ascontiguousarray(kb), v_bytes=np.ascontiguousarray(vb),
                     k_scale=np.ascontiguousarray(ks), v_scale=np.ascontiguousarray(vs))
            )
    del k_codes, v_codes

    return Workload(
        name=name,
        num_q_heads=num_q_heads,
        num_kv_heads=num_kv_heads,
        head_dim=head_dim,
        page_size=S,
        q_dtype=q_dtype,
        out_dtype=out_dtype,
        q_lens=q_lens,
        ctx_lens=ctx_lens,
        block_table=block_table,
        k_pages=k_pages,
        v_pages=v_pages,
        kv_scales=kv_scales,
        q=q,
        max_q_len=max_q_len,
        max_ctx_len=max_ctx_len,
        num_kv_splits=num_kv_splits,
        seed=seed,
        logical=logical,
        kv_format=kv_format,
    )


# ---------------------------------------------------------------------------
# The measured shapes.  Keys are the names used by tests and the bench.
# ---------------------------------------------------------------------------

CONFIGS = {
    # batch 1, 4 query heads on 1 KV head, d=64, 256 tokens in 16 pages of a
    # 32-page permuted pool, fp32 Q and output
    "tiny_decode": dict(seed=1),
    # LLaMA-3-8B-shaped decode: batch 32, 32/8 heads, d=128, ctx U{512..4096}
    "llama3_8b_decode": dict(seed=2),
    # MTP verification: batch 128, 1+4 query tokens, 40/8 heads, ctx U{128..1152}
    "mtp_verify": dict(seed=3),
    # long-context split decode: batch 4, ctx 32768, 64 KV partitions
    "long_ctx_split": dict(seed=4),
    # chunked prefill: 8 x 512 new tokens appended to U{0..8192} cached tokens
    "prefill_chunk": dict(seed=5),
    # MQA decode: 64 sequences, 64 query heads on 1 KV head, ctx log-U[256, 16384]
    "mqa_decode": dict(seed=6),
}


def make_workload(name: str, seed: int | None = None, *, batch: int | None = None,
                  ctx_range: tuple | None = None, keep_logical: bool = True, **over) -> Workload:
    """Generate one of the named workloads.

    ``batch`` and ``ctx_range`` shrink a workload for fast tests (same recipe,
    smaller sizes); ``over`` overrides heads/head_dim/dtypes/q_len.
    """
    if name not in CONFIGS:
        raise KeyError(name)
    seed = CONFIGS[name]["seed"] if seed is None else seed
    rng = np.random.default_rng(seed)
    kw = dict(keep_logical=keep_logical, seed=seed, kv_format=over.get("kv_format", "e4m3"))

    if name == "tiny_decode":
        B = batch or 1
        L = 256 if ctx_range is None else int(ctx_range[1])
        ctx = np.full(B, L, dtype=np.int32)
        pool = 32 if B == 1 and L == 256 else None
        return build_workload(name, rng, q_lens=np.ones(B, np.int32), ctx_lens=ctx,
                              num_q_heads=over.get("num_q_heads", 4), num_kv_heads=over.get("num_kv_heads", 1),
                              head_dim=over.get("head_dim", 64), q_dtype=over.get("q_dtype", "f32"),
                              out_dtype=over.get("out_dtype", "f32"), num_pages=pool, **kw)

    if name == "llama3_8b_decode":
        B = batch or 32
        lo, hi = ctx_range or (512, 4096)
        ctx = rng.integers(lo, hi + 1, size=B).astype(np.int32)
        return build_workload(name, rng, q_lens=np.ones(B, np.int32), ctx_lens=ctx,
                              num_q_heads=over.get("num_q_heads", 32), num_kv_heads=over.get("num_kv_heads", 8),
                              head_dim=over.get("head_dim", 128), q_dtype=over.get("q_dtype", "bf16"),
                              out_dtype=over.get("out_dtype", "bf16"), max_ctx_len=hi,
                              num_kv_splits=over.get("num_kv_splits", 0), **kw)

    if name == "mtp_verify":
        B = batch or 128
        qlen = over.get("q_len", 5)
        lo, hi = ctx_range or (128, 1152)
        ctx = rng.integers(lo, hi + 1, size=B).astype(np.int32)
        return build_workload(name, rng, q_lens=np.full(B, qlen, np.int32), ctx_lens=ctx,
                              num_q_heads=over.get("num_q_heads", 40), num_kv_heads=over.get("num_kv_heads", 8),
                              head_dim=over.get("head_dim", 128), q_dtype=over.get("q_dtype", "bf16"),
                              out_dtype=over.get("out_dtype", "bf16"), max_ctx_len=hi, max_q_len=qlen, **kw)

    if name == "long_ctx_split":
        B = batch or 4
        L = 32768 if ctx_range is None else int(ctx_range[1])
        ctx = np.full(B, L, dtype=np.int32)
        return build_workload(name, rng, q_lens=np.ones(B, np.int32), ctx_lens=ctx,
                              num_q_heads=over.get("num_q_heads", 32), num_kv_heads=over.get("num_kv_heads", 8),
                              head_dim=over.get("head_dim", 128), q_dtype=over.get("q_dtype", "bf16"),
                              out_dtype=over.get("out_dtype", "bf16"),
                              num_kv_splits=over.get("num_kv_splits", 64), **kw)

    if name == "prefill_chunk":
        B = batch or 8
        chunk = over.get("q_len", 512)
        lo, hi = ctx_range or (0, 8192)  # range of *cached* tokens
        cached = rng.integers(lo, hi + 1, size=B).astype(np.int32)
        ctx = cached + chunk
        return build_workload(name, rng, q_lens=np.full(B, chunk, np.int32), ctx_lens=ctx,
                              num_q_heads=over.get("num_q_heads", 32), num_kv_heads=over.get("num_kv_heads", 8),
                              head_dim=over.get("head_dim", 128), q_dtype=over.get("q_dtype", "bf16"),
                              out_dtype=over.get("out_dtype", "bf16"), max_ctx_len=hi + chunk,
                              max_q_len=chunk, **kw)

    if name == "mqa_decode":
        B = batch or 64
        lo, hi = ctx_range or (256, 16384)
        u = rng.uniform(math.log(lo), math.log(hi), size=B)
        ctx = np.clip(np.rint(np.exp(u)), lo, hi).astype(np.int32)
        return build_workload(name, rng, q_lens=np.ones(B, np.int32), ctx_lens=ctx,
                              num_q_heads=over.get("num_q_heads", 64), num_kv_heads=over.get("num_kv_heads", 1),
                              head_dim=over.get("head_dim", 128), q_dtype=over.get("q_dtype", "bf16"),
                              out_dtype=over.get("out_dtype", "bf16"), max_ctx_len=hi, **kw)

    raise KeyError(name)


def custom_workload(q_lens, ctx_lens, *, num_q_heads=8, num_kv_heads=2, head_dim=128, seed=0,
                    q_dtype="bf16", out_dtype="bf16", num_kv_splits=0, max_ctx_len=None,
                    max_q_len=None, num_pages=None, keep_logical=True, name="custom",
                    kv_format="e4m3") -> Workload:
    """Explicit lengths (edge cases): same recipe, lengths given instead of drawn."""
    rng = np.random.default_rng(seed)
    return build_workload(name, rng, q_lens=q_lens, ctx_lens=ctx_lens, num_q_heads=num_q_heads,
                          num_kv_heads=num_kv_heads, head_dim=head_dim, q_dtype=q_dtype,
                          out_dtype=out_dtype, num_kv_splits=num_kv_splits, max_ctx_len=max_ctx_len,
                          max_q_len=max_q_len, num_pages=num_pages, keep_logical=keep_logical, seed=seed,
                          kv_format=kv_format)
