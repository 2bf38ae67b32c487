"""Plain fp64 paged FP8-KV attention -- TEST INFRASTRUCTURE ONLY.

The definition followed:
  * Atlas engine article (ainews.cool), "技术深度解析":
      - memory section: the KV cache lives in fixed-size blocks taken from a
        preallocated pool; a sequence's blocks are found through its block
        table (the paged KV cache of the GB10 article);
      - quantisation section: FP8 storage with per-group scale factors; here
        one fp32 scale per (page, kv head), separate for K and V, and
        value = decoded byte * scale;
      - attention section: a FlashAttention-2 variant with native MQA/GQA.
        FA2's online softmax computes exactly softmax(Q K^T / sqrt(d)) V, so
        the oracle is that formula, evaluated directly in fp64.
  * GB10 article (ainews.surl.tw): MTP with K=4 draft tokens -> a sequence
    may bring several new query tokens; they attend causally (token i of
    Q new tokens sees keys 0 .. L-Q+i, where L counts every key including
    the new ones).

Readings where the pages are silent (each listed in the design notes):
  * GQA grouping: query head hq uses kv head hq // (Hq / Hkv).
  * Layouts (the library's ABI, S = 16 slots per page):
      k_pages [P][Hkv][D/16][S][16]: the K byte of slot s, dim d of a (page,
        head) is k[p][h][d // 16][s][d % 16];
      v_pages [P][Hkv][S/4][D/64][16][4][4]: with NVB = D/16 and
        d = NVB*a + 4*i + e, the V byte of slot s, dim d is
        v[p][h][s // 4][i][a][e][s % 4].
  * INT4 pools (two 4-bit codes per byte, D = 128), the library's layouts:
      k_pages [P][Hkv][4][S][D/8]: with u = d % (D/4), the K code of slot s,
        dim d is nibble u % 2 (0: bits 0-3, 1: bits 4-7) of
        k[p][h][d // (D/4)][s][u // 2];
      v_pages [P][Hkv][S/4][16][D/16][2]: with NVB = D/16 and d = NVB*a + r,
        the V code of slot s, dim d is nibble s % 2 of
        v[p][h][s // 4][a][r][(s % 4) // 2].
  * Scale 1/sqrt(D) unless given; no soft-cap, ALiBi, window or sinks.
  * Bytes past a sequence's length and unreferenced pages are never read.

The small helpers below name each reading separately, so the tests can
replace one of them with a plausible mistake and check that a pin fails.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import e4m3


def kv_head_of(hq: int, num_q_heads: int, num_kv_heads: int) -> int:
    """GQA/MQA: consecutive groups of Hq/Hkv query heads share one kv head."""
    return hq // (num_q_heads // num_kv_heads)


def last_visible_key(ctx_len: int, q_len: int, i: int) -> int:
    """Causal limit of new token i: keys 0..L-Q+i (bottom-right alignment)."""
    return ctx_len - q_len + i


def token_location(block_table_row: np.ndarray, t: np.ndarray, page_size: int):
    """Logical token t -> (physical page, slot inside the page)."""
    return block_table_row[t // page_size], t % page_size


def k_token_bytes(k_pages: np.ndarray, pages: np.ndarray, h: int, slots: np.ndarray) -> np.ndarray:
    """K bytes of (page, head h, slot) for each token: [T][D]."""
    blocks = k_pages[pages, h, :, slots, :]  # [T][D/16][16]: d = 16 * block + offset
    return blocks.reshape(blocks.shape[0], -1)


def v_token_bytes(v_pages: np.ndarray, pages: np.ndarray, h: int, slots: np.ndarray) -> np.ndarray:
    """V bytes of (page, head h, slot) for each token: [T][D] (4-slot interleave)."""
    parts = v_pages[pages, h, slots // 4, :, :, :, slots % 4]  # [T][i][a][e]
    # d = NVB * a + 4 * i + e: order the axes (a, i, e)
    return parts.transpose(0, 2, 1, 3).reshape(parts.shape[0], -1)


def k4_token_codes(k_pages: np.ndarray, pages: np.ndarray, h: int, slots: np.ndarray) -> np.ndarray:
    """INT4 K codes (0..15) of (page, head h, slot) for each token: [T][D]."""
    quarters = k_pages[pages, h, :, slots, :]  # [T][4][D/8] bytes
    lo = quarters & 0x0F  # even u
    hi = quarters >> 4  # odd u
    codes = np.stack([lo, hi], axis=-1)  # [T][4][D/8][2]: u = 2 * byte + nibble
    return codes.reshape(codes.shape[0], -1)


def v4_token_codes(v_pages: np.ndarray, pages: np.ndarray, h: int, slots: np.ndarray) -> np.ndarray:
    """INT4 V codes (0..15) of (page, head h, slot) for each token: [T][D]."""
    pairs = v_pages[pages, h, slots // 4, :, :, (slots % 4) // 2]  # [T][16][NVB]: d = NVB * a + r
    shift = (4 * (slots % 2)).astype(np.uint8)[:, None, None]
    codes = (pairs >> shift) & 0x0F
    return codes.reshape(codes.shape[0], -1)


def softmax_scale(head_dim: int, sm_scale: float | None) -> float:
    return 1.0 / np.sqrt(head_dim) if not sm_scale else float(sm_scale)


@dataclass
class GatheredSequence:
    k_bytes: np.ndarray  # uint8 [Hkv][L][D]
    v_bytes: np.ndarray  # uint8 [Hkv][L][D]
    k_scale: np.ndarray  # float64 [Hkv][L]
    v_scale: np.ndarray  # float64 [Hkv][L]
    page_of_token: np.ndarray  # int64 [L]


def gather_sequence(k_pages, v_pages, kv_scales, block_table_row, ctx_len: int,
                    kv_format: str = "e4m3") -> GatheredSequence:
    """Follow one sequence's block table and collect its L tokens' codes
    (bytes, or 4-bit codes for INT4) and scales."""
    k_pages = np.asarray(k_pages)
    v_pages = np.asarray(v_pages)
    if kv_format == "int4":
        _, hkv, _, page_size, half_quarter = k_pages.shape
        d = 8 * half_quarter
        k_codes, v_codes = k4_token_codes, v4_token_codes
    else:
        _, hkv, d_blocks, page_size, _ = k_pages.shape
        d = 16 * d_blocks
        k_codes, v_codes = k_token_bytes, v_token_bytes
    t = np.arange(int(ctx_len))
    pages, slots = token_location(np.asarray(block_table_row).astype(np.int64), t, page_size)
    kb = np.empty((hkv, t.size, d), dtype=np.uint8)
    vb = np.empty((hkv, t.size, d), dtype=np.uint8)
    ks = np.empty((hkv, t.size), dtype=np.float64)
    vs = np.empty((hkv, t.size), dtype=np.float64)
    for h in range(hkv):
        kb[h] = k_codes(k_pages, pages, h, slots)
        vb[h] = v_codes(v_pages, pages, h, slots)
        ks[h] = kv_scales[0][pages, h]
        vs[h] = kv_scales[1][pages, h]
    return GatheredSequence(kb, vb, ks, vs, pages)


def decode_int8(codes) -> np.ndarray:
    """INT8 KV bytes (two's complement) -> fp64: byte c is c for c < 128,
    c - 256 otherwise (the quantisation section of the Atlas article lists
    INT8 beside FP8, with the same per-group scales)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    return np.where(c < 128, c, c - 256).astype(np.float64)


def decode_int4(codes) -> np.ndarray:
    """INT4 KV codes (two's complement in 4 bits) -> fp64: code c is c for
    c < 8, c - 16 otherwise (the quantisation section lists INT4 beside INT8
    and FP8, with the same per-group scales)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64) & 0x0F
    return np.where(c < 8, c, c - 16).astype(np.float64)


def decode_kv(codes, kv_format: str = "e4m3") -> np.ndarray:
    """KV codes -> fp64 values before the page scale."""
    if kv_format == "e4m3":
        return e4m3.decode(codes)
    if kv_format == "int8":
        return decode_int8(codes)
    if kv_format == "int4":
        return decode_int4(codes)
    raise ValueError(kv_format)


def paged_attention(q, k_pages, v_pages, kv_scales, block_table, ctx_lens, q_lens, *,
                    num_kv_heads: int, sm_scale: float | None = None, rows=None,
                    kv_format: str = "e4m3") -> np.ndarray:
    """out[r][hq][:] = sum_t softmax_t(z) * V~[t], z_t = scale * <q[r][hq], K~[t]>.

    q: [sum Q][Hq][D] (any real dtype; read exactly into fp64).
    rows: optional iterable of global query rows to evaluate (others stay 0).
    Returns fp64 [sum Q][Hq][D].
    """
    if hasattr(q, "detach"):  # torch tensor
        q = q.detach().to("cpu").double().numpy()
    q = np.asarray(q, dtype=np.float64)
    total_q, num_q_heads, d = q.shape
    ctx_lens = np.asarray(ctx_lens).astype(np.int64)
    q_lens = np.asarray(q_lens).astype(np.int64)
    scale = softmax_scale(d, sm_scale)
    want = None if rows is None else set(int(r) for r in rows)
    out = np.zeros((total_q, num_q_heads, d), dtype=np.float64)

    row0 = 0
    for b in range(len(q_lens)):
        L, Q = int(ctx_lens[b]), int(q_lens[b])
        mine = [i for i in range(Q) if want is None or (row0 + i) in want]
        if mine:
            g = gather_sequence(k_pages, v_pages, kv_scales, block_table[b], L, kv_format)
            k_deq = [decode_kv(g.k_bytes[h], kv_format) * g.k_scale[h][:, None] for h in range(num_kv_heads)]
            v_deq = [decode_kv(g.v_bytes[h], kv_format) * g.v_scale[h][:, None] for h in range(num_kv_heads)]
            idx = np.array(mine)
            lim = np.array([last_visible_key(L, Q, i) for i in mine])  # [n]
            visible = np.arange(L)[None, :] <= lim[:, None]  # [n][L]
            for hq in range(num_q_heads):
                h = kv_head_of(hq, num_q_heads, num_kv_heads)
                z = (q[row0 + idx, hq, :] @ k_deq[h].T) * scale  # [n][L]
                z = np.where(visible, z, -np.inf)
                z = z - z.max(axis=1, keepdims=True)
                w = np.exp(z)
                w = w / w.sum(axis=1, keepdims=True)
                out[row0 + idx, hq, :] = w @ v_deq[h]
        row0 += Q
    return out
