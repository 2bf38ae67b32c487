"""Pins of the oracle's INT8 KV reading (CPU only): every byte against
torch's int8 view and the two's-complement closed form; attention on INT8
workloads against pure-Python loops and torch's fp64
scaled_dot_product_attention; the generator's INT8 quantiser within half a
step; and a planted mistake (bytes read as unsigned) that fails a pin."""

import numpy as np
import pytest

import oracle.attention as pa
from synth import custom_workload
from tests.independent import brute_force_attention, int8_by_torch, sdpa_attention


def test_decode_every_byte():
    codes = np.arange(256, dtype=np.uint8)
    got = pa.decode_int8(codes)
    assert np.array_equal(got, int8_by_torch(codes))
    assert got[0] == 0 and got[127] == 127 and got[128] == -128 and got[255] == -1


def _run(w, **kw):
    return pa.paged_attention(w.q, w.k_pages, w.v_pages, w.kv_scales, w.block_table, w.ctx_lens, w.q_lens,
                              num_kv_heads=w.num_kv_heads, sm_scale=w.sm_scale, kv_format=w.kv_format, **kw)


def test_brute_force_tiny():
    w = custom_workload([1, 3], [20, 9], num_q_heads=4, num_kv_heads=2, head_dim=64, seed=21, kv_format="int8")
    np.testing.assert_allclose(_run(w), brute_force_attention(w), rtol=0, atol=1e-12)


@pytest.mark.parametrize("shape", [([1, 1, 5], [300, 47, 90], 8, 2), ([40, 7], [100, 300], 4, 1)])
def test_sdpa(shape):
    ql, cl, hq, hkv = shape
    w = custom_workload(ql, cl, num_q_heads=hq, num_kv_heads=hkv, head_dim=128, seed=22, kv_format="int8")
    np.testing.assert_allclose(_run(w), sdpa_attention(w), rtol=0, atol=1e-12)


def test_quantiser_within_half_step():
    w = custom_workload([1], [64], num_q_heads=2, num_kv_heads=2, head_dim=64, seed=23, kv_format="int8")
    lg = w.logical[0]
    vals = int8_by_torch(lg["k_bytes"])
    assert np.abs(vals).max() == 127  # the absmax element maps to 127
    assert np.all(np.abs(vals) <= 127)


def test_planted_unsigned_reading_fails(monkeypatch):
    w = custom_workload([1, 2], [40, 33], num_q_heads=4, num_kv_heads=1, head_dim=64, seed=24, kv_format="int8")
    good = _run(w)
    monkeypatch.setattr(pa, "decode_int8", lambda c: np.asarray(c, dtype=np.uint8).astype(np.float64))
    bad = _run(w)
    assert not np.allclose(bad, sdpa_attention(w), rtol=0, atol=1e-6)
    assert np.allclose(good, sdpa_attention(w), rtol=0, atol=1e-12)
