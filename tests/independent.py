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
    dec = [e4m3_by_bits(c) for c in range(256)]
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
                        kb = kflat[(((p * Hkv + h) * (D // 16) + d // 16) * S + s) * 16 + d % 16]
                        acc += float(q[row + i, hq, d]) * dec[kb] * ksc[p * Hkv + h]
                    zs.append(acc * scale)
                zmax = max(zs)
                ws = [math.exp(z - zmax) for z in zs]
                tot = sum(ws)
                for d in range(D):
                    acc = 0.0
                    for t in range(position + 1):
                        p = int(w.block_table[b][t // S])
                        s = t % S
                        nvb = D // 16
                        va, vi, ve = d // nvb, (d % nvb) // 4, d % 4
                        vb = vflat[(((((p * Hkv + h) * (S // 4) + s // 4) * (D // 64) + vi) * 16 + va) * 4 + ve) * 4
                                   + s % 4]
                        acc += ws[t] * dec[vb] * vsc[p * Hkv + h]
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
        k = torch.from_numpy(e4m3_by_torch(lg["k_bytes"]) * lg["k_scale"][:, :, None].astype(np.float64))
        v = torch.from_numpy(e4m3_by_torch(lg["v_bytes"]) * lg["v_scale"][:, :, None].astype(np.float64))
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
