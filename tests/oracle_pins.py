"""The oracle's pins, as plain functions (used by the tests and by the
planted-mistake tests, which swap one oracle helper for a wrong one and
require that at least one pin fails).

Every pin compares the oracle with something other than itself: the OCP
spec values, an independent bit-level decode, torch's FP8 decode, a
pure-Python brute force, torch's fp64 scaled_dot_product_attention on the
unpaged data, and closed forms.
"""

from __future__ import annotations

import math
import os

import numpy as np

import oracle
from oracle import e4m3
from synth import custom_workload
from tests.independent import brute_force_attention, e4m3_by_bits, e4m3_by_torch, sdpa_attention

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _same(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return np.array_equal(np.isnan(a), np.isnan(b)) and np.array_equal(
        np.where(np.isnan(a), 0, a), np.where(np.isnan(b), 0, b)
    ) and np.array_equal(np.signbit(np.where(np.isnan(a), 0, a)), np.signbit(np.where(np.isnan(b), 0, b)))


# --- decode table ---------------------------------------------------------

def pin_table_vs_spec_values():
    t = e4m3.decode_table()
    with open(os.path.join(GOLDEN, "e4m3_ocp_spot_values.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            code, val = line.split()
            code = int(code, 16)
            want = float(val)
            got = t[code]
            if math.isnan(want):
                assert math.isnan(got), (hex(code), got)
            else:
                assert got == want and math.copysign(1, got) == math.copysign(1, want), (hex(code), got, want)


def pin_table_vs_bit_assembly():
    t = e4m3.decode_table()
    ref = np.array([e4m3_by_bits(c) for c in range(256)])
    assert _same(t, ref)


def pin_table_vs_torch():
    t = e4m3.decode_table()
    assert _same(t, e4m3_by_torch(np.arange(256)))


def pin_table_structure():
    t = e4m3.decode_table()
    pos = t[:0x7F]
    assert np.all(np.diff(pos) > 0), "positive codes must increase strictly"
    assert _same(t[0x80:0xFF], -t[0x00:0x7F]), "sign bit must negate"
    assert np.isnan(t).sum() == 2


# --- attention --------------------------------------------------------------

def _tiny_cases():
    return [
        custom_workload([1, 3, 2], [1, 20, 33], num_q_heads=4, num_kv_heads=2, head_dim=64, seed=11),
        custom_workload([2], [17], num_q_heads=3, num_kv_heads=1, head_dim=64, seed=12, q_dtype="f32"),
        custom_workload([1, 1], [16, 40], num_q_heads=6, num_kv_heads=3, head_dim=64, seed=13),
    ]


def _oracle(w, **kw):
    return oracle.paged_attention(w.q, w.k_pages, w.v_pages, w.kv_scales, w.block_table, w.ctx_lens,
                                  w.q_lens, num_kv_heads=w.num_kv_heads, sm_scale=w.sm_scale, **kw)


def pin_brute_force():
    for w in _tiny_cases():
        got = _oracle(w)
        ref = brute_force_attention(w)
        np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def pin_sdpa():
    cases = _tiny_cases() + [
        custom_workload([5, 5, 1], [5, 70, 130], num_q_heads=10, num_kv_heads=2, head_dim=64, seed=21),
        custom_workload([1, 4], [300, 64], num_q_heads=8, num_kv_heads=8, head_dim=128, seed=22),
        custom_workload([3], [35], num_q_heads=16, num_kv_heads=1, head_dim=64, seed=23),
    ]
    for w in cases:
        got = _oracle(w)
        ref = sdpa_attention(w)
        np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def pin_single_key():
    # one key: softmax weight 1, out = V~[0] for every head of the group
    w = custom_workload([1, 1], [1, 1], num_q_heads=4, num_kv_heads=2, head_dim=64, seed=31)
    got = _oracle(w)
    for b in range(2):
        lg = w.logical[b]
        for hq in range(4):
            h = hq // 2
            want = e4m3_by_torch(lg["v_bytes"][h, 0]) * float(lg["v_scale"][h, 0])
            np.testing.assert_array_equal(got[b, hq], want)


def pin_zero_keys_mean_of_visible():
    # K bytes all zero -> every visible key has score 0 -> out = mean of the
    # visible V~ rows; pins the causal limit and the per-sequence length.
    w = custom_workload([3, 1, 4], [7, 18, 21], num_q_heads=4, num_kv_heads=2, head_dim=64, seed=32)
    used = np.unique(w.block_table[w.block_table >= 0])
    w.k_pages[used] = 0
    got = _oracle(w)
    row = 0
    for b in range(w.num_seqs):
        L, Q = int(w.ctx_lens[b]), int(w.q_lens[b])
        lg = w.logical[b]
        for i in range(Q):
            n_visible = L - Q + i + 1
            for hq in range(4):
                h = hq // 2
                vals = e4m3_by_torch(lg["v_bytes"][h, :n_visible]) * lg["v_scale"][h, :n_visible, None]
                np.testing.assert_allclose(got[row + i, hq], vals.mean(axis=0), rtol=0, atol=1e-14)
        row += Q


def pin_constant_v():
    # every visible V~ equal -> out equals it whatever the weights
    w = custom_workload([2, 1], [19, 40], num_q_heads=6, num_kv_heads=2, head_dim=64, seed=33)
    used = np.unique(w.block_table[w.block_table >= 0])
    w.v_pages[used] = 0x44  # 3.0
    w.kv_scales[1][used] = 0.25
    got = _oracle(w)
    np.testing.assert_allclose(got, 0.75, rtol=0, atol=1e-14)


def pin_scale_changes_result():
    # sm_scale is honoured: with 1/sqrt(D) replaced the result moves, and a
    # tiny explicit scale tends to the uniform mean (brute force agrees).
    w = custom_workload([1], [30], num_q_heads=2, num_kv_heads=1, head_dim=64, seed=34)
    w.sm_scale = 1e-9
    got = _oracle(w)
    lg = w.logical[0]
    vals = e4m3_by_torch(lg["v_bytes"][0]) * lg["v_scale"][0][:, None]
    np.testing.assert_allclose(got[0, 0], vals.mean(axis=0), rtol=0, atol=1e-6)
    np.testing.assert_allclose(got, brute_force_attention(w), rtol=0, atol=1e-12)


ALL_TABLE_PINS = [pin_table_vs_spec_values, pin_table_vs_bit_assembly, pin_table_vs_torch, pin_table_structure]
ALL_ATTENTION_PINS = [pin_brute_force, pin_sdpa, pin_single_key, pin_zero_keys_mean_of_visible,
                      pin_constant_v, pin_scale_changes_result]
