"""Independent re-derivations used to pin the oracle (tests only).

Nothing here is imported by the oracle or the library.  Each function
re-states a fact in a different way from the oracle's own code:
  * e4m3_by_bits: builds the IEEE fp32 bit pattern of an E4M3 code by
    normalising its mantissa bit by bit (no closed-form power expression);
  * e4m3_by_torch: the library decode of torch.float8_e4m3fn;
  * brute_force_attention: pure-Python loops over flat byte offsets and
    math.exp, for tiny inputs;
  * sdpa_attention: torch's scaled_dot_product_attention in fp64 on the
    unpaged logical K/V with an explicit bottom-right causal mask and the
    library's own GQA head expansion.
"""

from __future__ import annotations

import math
import struct

import numpy as np
import torch


def e4m3_by_bits(x: int) -> float:
    sign = (x >> 7) & 1
    e = (x >> 3) & 0xF
    m = x & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0 and m == 0:
        return -0.0 if sign else 0.0
    if e == 0:
        # subnormal: shift the mantissa left until its leading one reaches
        # bit 3 (the implicit-one position), lowering the exponent each time
        exp_unbiased = -6
        while not (m & 0x8):
            m <<= 1
            exp_unbiased -= 1
        m &= 0x7
    else:
        exp_unbiased = e - 7
    bits = (sign << 31) | ((exp_unbiased + 127) << 23) | (m << 20)
    return struct.unpack("<f", struct.pack("<I", bits))[0]


def int8_by_torch(codes) -> np.ndarray:
    """The library reading of INT8 bytes (torch's int8 view)."""
    t = torch.as_tensor(np.ascontiguousarray(codes, dtype=np.uint8))
    return t.view(torch.int8).to(torch.float64).numpy()


def int4_by_shift(codes) -> np.ndarray:
    """4-bit two's-complement codes read by moving the nibble to the top of
    an int8 and shifting it back arithmetically (sign extension)."""
    c = np.asarray(codes, dtype=np.uint8)
    return (((c & 0x0F) << 4).astype(np.uint8).view(np.int8) >> 4).astype(np.float64)


def e4m3_by_torch(codes) -> np.ndarray:
    t = torch.as_tensor(np.asarray(codes, dtype=np.uint8))
    return t.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def brute_force_attention(w) -> np.ndarray:
    """Pure-Python triple loop over a (tiny) workload's flat buffers."""
    S, D = w.page_size, w.head_dim
    Hq, Hkv = w.num_q_heads, w.num_kv_heads
    kflat = w.k_pages.reshape(-1).tolist()
    vflat = w.v_pages.reshape(-1).tolist()
    ksc = w.kv_scales[0].reshape(-1).tolist()
    vsc = w.kv_scales[1].reshape(-1).tolist()
    q = w.q.double().numpy()
    fmt = getattr(w, "kv_format", "e4m3")
    if fmt == "int8":
        dec = [float(c - 256 if c & 0x80 else c) for c in range(256)]  # two's complement
    elif fmt == "int4":
        dec = [float(c - 16 if c & 0x8 else c) for c in range(16)]
    else:
        dec = [e4m3_by_bits(c) for c in range(256)]

    def k_code(p, h, s, d):
        if fmt != "int4":
            return kflat[(((p * Hkv + h) * (D // 16) + d // 16) * S + s) * 16 + d % 16]
        # [P][Hkv][4][S][D/8], nibble u % 2 of byte u // 2 with u = d % (D/4)
        u = d % (D // 4)
        byte = kflat[(((p * Hkv + h) * 4 + d // (D // 4)) * S + s) * (D // 8) + u // 2]
        return (byte >> (4 * (u % 2))) & 0xF

    def v_code(p, h, s, d):
        nvb = D // 16
        if fmt != "int4":
            va, vi, ve = d // nvb, (d % nvb) // 4, d % 4
            return vflat[(((((p * Hkv + h) * (S // 4) + s // 4) * (D // 64) + vi) * 16 + va) * 4 + ve) * 4 + s % 4]
        # [P][Hkv][S/4][16][D/16][2], nibble s % 2 of byte (s % 4) // 2, d = nvb a + r
        byte = vflat[(((((p * Hkv + h) * (S // 4) + s // 4) * 16 + d // nvb) * nvb + d % nvb) * 2 + (s % 4) // 2)]
        return (byte >> (4 * (s % 2))) & 0xF
    scale = w.sm_scale if w.sm_scale else 1.0 / math.sqrt(D)
    out = np.zeros(q.shape, dtype=np.float64)
    row = 0
    for b in range(w.num_seqs):
        L, Q = int(w.ctx_lens[b]), int(w.q_lens[b])
        for i in range(Q):
            position = (L - Q) + i  # absolute position of this new token
            for hq in range(Hq):
                h = (hq * Hkv) // Hq
                zs = []
                for t in range(position + 1):
                    p = int(w.block_table[b][t // S])
                    s = t % S
                    acc = 0.0
                    for d in range(D):
                        acc += float(q[row + i, hq, d]) * dec[k_code(p, h, s, d)] * ksc[p * Hkv + h]
                    zs.append(acc * scale)
                zmax = max(zs)
                ws = [math.exp(z - zmax) for z in zs]
                tot = sum(ws)
                for d in range(D):
                    acc = 0.0
                    for t in range(position + 1):
                        p = int(w.block_table[b][t // S])
                        s = t % S
                        acc += ws[t] * dec[v_code(p, h, s, d)] * vsc[p * Hkv + h]
                    out[row + i, hq, d] = acc / tot
        row += Q
    return out


def sdpa_attention(w) -> np.ndarray:
    """Library attention in fp64 on the generator's logical (unpaged) K/V."""
    D = w.head_dim
    scale = w.sm_scale if w.sm_scale else 1.0 / math.sqrt(D)
    q_all = w.q.double()
    out = torch.zeros(q_all.shape, dtype=torch.float64)
    row = 0
    for b in range(w.num_seqs):
        L, Q = int(w.ctx_lens[b]), int(w.q_lens[b])
        lg = w.logical[b]
        dec = {"int8": int8_by_torch, "int4": int4_by_shift}.get(getattr(w, "kv_format", "e4m3"), e4m3_by_torch)
        k = torch.from_numpy(dec(lg["k_bytes"]) * lg["k_scale"][:, :, None].astype(np.float64))
        v = torch.from_numpy(dec(lg["v_bytes"]) * lg["v_scale"][:, :, None].astype(np.float64))
        qb = q_all[row : row + Q].permute(1, 0, 2).contiguous()  # [Hq][Q][D]
        # bottom-right causal mask: query i sits at position L-Q+i
        qpos = torch.arange(Q)[:, None] + (L - Q)
        kpos = torch.arange(L)[None, :]
        mask = kpos <= qpos
        o = torch.nn.functional.scaled_dot_product_attention(
            qb[None], k[None], v[None], attn_mask=mask, scale=scale, enable_gqa=True
        )[0]
        out[row : row + Q] = o.permute(1, 0, 2)
        row += Q
    return out.numpy()


def e4m3_encode_brute(y: float) -> int:
    """Nearest finite E4M3 code to fp32 y by trying all 127 magnitudes (ties
    to the code with mantissa bit 0 clear), magnitude clipped to 448, sign
    bit from y's sign bit."""
    mag = min(abs(y), 448.0)
    best, best_d = 0, None
    for c in range(0x7F):
        d = abs(e4m3_by_bits(c) - mag)
        if best_d is None or d < best_d or (d == best_d and (c & 1) == 0 and (best & 1) == 1):
            best, best_d = c, d
    return best | (0x80 if math.copysign(1.0, y) < 0 else 0)


def _f32(x: float) -> float:
    return struct.unpack("<f", struct.pack("<f", x))[0]


def int8_encode_brute(y: float) -> int:
    """The integer nearest to y (ties to the even one) clipped to +-127, as a
    two's-complement byte."""
    f = math.floor(y)
    d = y - f
    q = f + 1 if d > 0.5 or (d == 0.5 and f % 2 == 1) else f
    q = max(-127, min(127, int(q)))
    return q & 0xFF


def brute_force_append(c, kv_format: str = "e4m3"):
    """Pure-Python loops over flat byte offsets: quantise an AppendCase's new
    rows into copies of its pools (tiny cases only)."""
    int8 = kv_format == "int8"
    qmax = 127.0 if int8 else 448.0
    dec_tab = [float(b - 256 if b & 0x80 else b) for b in range(256)] if int8 else [e4m3_by_bits(b) for b in range(256)]
    enc = int8_encode_brute if int8 else e4m3_encode_brute
    S, D, Hkv = 16, c.head_dim, c.num_kv_heads
    kflat = c.k_pages.reshape(-1).copy()
    vflat = c.v_pages.reshape(-1).copy()
    scales = c.kv_scales.copy()
    kn = c.k_new.float().numpy()
    vn = c.v_new.float().numpy()
    nvb = D // 16

    def k_off(p, h, s, d):
        return (((p * Hkv + h) * (D // 16) + d // 16) * S + s) * 16 + d % 16

    def v_off(p, h, s, d):
        a, i, e = d // nvb, (d % nvb) // 4, d % 4
        return (((((p * Hkv + h) * (S // 4) + s // 4) * (D // 64) + i) * 16 + a) * 4 + e) * 4 + s % 4

    row = 0
    for b in range(c.num_seqs):
        L, Q = int(c.ctx_lens[b]), int(c.q_lens[b])
        for t0 in range(((L - Q) // S) * S, L, S):  # first slot of each touched page
            p = int(c.block_table[b][t0 // S])
            for h in range(Hkv):
                for which, flat, new, off in ((0, kflat, kn, k_off), (1, vflat, vn, v_off)):
                    old_scale = float(scales[which][p, h])
                    vals = {}
                    for s in range(S):
                        t = t0 + s
                        if t >= L:
                            break
                        for d in range(D):
                            if t < L - Q:
                                vals[(s, d)] = _f32(dec_tab[int(flat[off(p, h, s, d)])] * old_scale)
                            else:
                                vals[(s, d)] = float(new[row + t - (L - Q), h, d])
                    amax = max(abs(x) for x in vals.values())
                    sc = 1.0 if amax == 0 else _f32(amax / qmax)
                    scales[which][p, h] = sc
                    for (s, d), x in vals.items():
                        flat[off(p, h, s, d)] = enc(_f32(x / sc))
        row += Q
    return kflat.reshape(c.k_pages.shape), vflat.reshape(c.v_pages.shape), scales
