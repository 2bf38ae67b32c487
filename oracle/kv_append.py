"""Plain paged FP8 KV append (quantise new tokens into the pool) -- TEST
INFRASTRUCTURE ONLY.

What it follows:
  * Atlas engine article (ainews.cool), "技术深度解析": the memory section
    (the KV cache lives in fixed-size blocks from a preallocated pool) and
    the quantisation section (FP8 storage with per-group scale factors).
  * "Atlas Takes On vLLM ... on a Single GB10" (ainews.surl.tw): the paged
    FP8 KV cache that decode, MTP verification and prefill append to.

Readings where the pages are silent (each listed in the design notes):
  * One fp32 scale per (page, kv head), separate for K and V, equal to
    fp32(absmax of the page's valid values) / 448 (1 when that absmax is 0):
    the same rule the inputs of the attention tests are quantised with.
  * A page that already holds tokens is read back as decoded byte * old
    scale (an fp32 product); the absmax covers those values and the new
    ones, and every valid slot of the page is encoded again with the new
    scale.  Where the scale does not change this reproduces the old bytes.
  * Encoding: the finite E4M3 code nearest to fp32(value / scale), ties to
    the code with an even mantissa, magnitudes above 448 saturated to 448,
    the sign kept (a negative value that rounds to zero gives -0, 0x80).
  * INT8 pools (the quantisation section lists INT8 beside FP8): the same
    steps with scale = fp32(absmax) / 127 and the integer nearest to
    fp32(value / scale), ties to even, clipped to +-127, stored two's
    complement.
  * Slots at or past the sequence's new length keep whatever they held;
    pages the sequence does not touch are not written.
  * New token i of sequence b (0 <= i < Q_b) is key L_b - Q_b + i; its K/V
    row is k_new[r_b + i], r_b = sum of the earlier Q.
"""

from __future__ import annotations

import numpy as np

from . import e4m3
from .attention import k_token_bytes, v_token_bytes

E4M3_MAX = 448.0


def _finite_magnitudes():
    """(values, codes) of the non-negative finite E4M3 codes 0x00..0x7E,
    increasing in value."""
    codes = np.arange(0x7F, dtype=np.uint8)
    return e4m3.decode(codes), codes


def encode(y) -> np.ndarray:
    """fp32 values -> OCP E4M3 bytes, round to nearest, ties to even.

    The magnitude is clipped to 448, its two neighbouring finite codes are
    found by a search in the table of code values, and the nearer one is
    taken (on a tie the one whose mantissa bit 0 is clear).  The sign bit is
    the sign bit of y."""
    y = np.asarray(y, dtype=np.float32)
    vals, codes = _finite_magnitudes()
    mag = np.minimum(np.abs(y).astype(np.float64), E4M3_MAX)
    hi = np.searchsorted(vals, mag, side="left")  # first code value >= mag
    hi = np.minimum(hi, vals.size - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = mag - vals[lo]
    d_hi = vals[hi] - mag
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((codes[hi] & 1) == 0))
    code = np.where(take_hi, codes[hi], codes[lo]).astype(np.uint8)
    sign = np.signbit(y).astype(np.uint8) << 7
    return (code | sign).astype(np.uint8)


INT8_MAX = 127.0


def encode_int8(y) -> np.ndarray:
    """fp32 values -> INT8 bytes (two's complement): round half to even,
    clipped to +-127."""
    y = np.asarray(y, dtype=np.float32)
    q = np.clip(np.rint(y.astype(np.float64)), -INT8_MAX, INT8_MAX).astype(np.int64)
    return (q & 0xFF).astype(np.uint8)


def page_scale_int8(absmax) -> np.float32:
    """fp32(absmax) / 127 in fp32; 1 for an all-zero page."""
    a = np.float32(absmax)
    if a == 0:
        return np.float32(1.0)
    return np.float32(a / np.float32(INT8_MAX))


def page_scale(absmax) -> np.float32:
    """fp32(absmax) / 448 in fp32; 1 for an all-zero page."""
    a = np.float32(absmax)
    if a == 0:
        return np.float32(1.0)
    return np.float32(a / np.float32(E4M3_MAX))


def _set_k_bytes(k_pages, page, h, slot, row):
    """Write the D bytes of (page, head, slot) into the K layout
    [P][Hkv][D/16][S][16]: byte d sits at [d // 16][slot][d % 16]."""
    k_pages[page, h, :, slot, :] = np.asarray(row, dtype=np.uint8).reshape(-1, 16)


def _set_v_bytes(v_pages, page, h, slot, row):
    """Write the D bytes of (page, head, slot) into the V layout
    [P][Hkv][S/4][D/64][16][4][4]: with NVB = D / 16 and d = NVB*a + 4*i + e
    the byte sits at [slot // 4][i][a][e][slot % 4]."""
    d = row.size
    a_i_e = np.asarray(row, dtype=np.uint8).reshape(16, d // 64, 4)  # [a][i][e]
    v_pages[page, h, slot // 4, :, :, :, slot % 4] = a_i_e.transpose(1, 0, 2)


def kv_append(k_new, v_new, k_pages, v_pages, kv_scales, block_table, ctx_lens, q_lens, *, page_size: int = 16,
              kv_format: str = "e4m3"):
    """Quantise the new tokens' K and V into copies of the pools.

    k_new, v_new: [sum Q][Hkv][D] (any real dtype; read exactly as fp32).
    kv_format "int8": the same steps with scale = fp32(absmax)/127 and
    round-half-even integer codes clipped to +-127 (two's complement).
    Returns (k_pages, v_pages, kv_scales) after the append."""
    from .attention import decode_kv

    if kv_format == "int8":
        scale_of, encode_fn = page_scale_int8, encode_int8
    elif kv_format == "e4m3":
        scale_of, encode_fn = page_scale, encode
    else:
        raise ValueError(kv_format)
    if hasattr(k_new, "detach"):
        k_new = k_new.detach().to("cpu").float().numpy()
    if hasattr(v_new, "detach"):
        v_new = v_new.detach().to("cpu").float().numpy()
    k_new = np.asarray(k_new, dtype=np.float32)
    v_new = np.asarray(v_new, dtype=np.float32)
    k_pages = np.array(k_pages, copy=True)
    v_pages = np.array(v_pages, copy=True)
    kv_scales = np.array(kv_scales, copy=True)
    hkv = k_pages.shape[1]
    ctx_lens = np.asarray(ctx_lens).astype(np.int64)
    q_lens = np.asarray(q_lens).astype(np.int64)
    S = page_size

    row0 = 0
    for b in range(len(q_lens)):
        L, Q = int(ctx_lens[b]), int(q_lens[b])
        first_new = L - Q
        for pi in range(first_new // S, (L - 1) // S + 1):
            page = int(block_table[b][pi])
            valid = min(S, L - pi * S)  # slots holding keys after the append
            n_old = max(0, min(S, first_new - pi * S))  # of which already cached
            slots = np.arange(valid)
            for h in range(hkv):
                for which, pool, new_rows, read_bytes, write_bytes in (
                        (0, k_pages, k_new, k_token_bytes, _set_k_bytes),
                        (1, v_pages, v_new, v_token_bytes, _set_v_bytes)):
                    vals = np.empty((valid, new_rows.shape[2]), dtype=np.float32)
                    if n_old:
                        old = read_bytes(pool, np.full(n_old, page), h, slots[:n_old])
                        vals[:n_old] = (decode_kv(old, kv_format) * np.float64(kv_scales[which][page, h])).astype(
                            np.float32)
                    for s in range(n_old, valid):
                        vals[s] = new_rows[row0 + (pi * S + s - first_new), h]
                    scale = scale_of(np.max(np.abs(vals)))
                    kv_scales[which][page, h] = scale
                    codes = encode_fn((vals / scale).astype(np.float32))
                    for s in range(valid):
                        write_bytes(pool, page, h, s, codes[s])
        row0 += Q
    return k_pages, v_pages, kv_scales
