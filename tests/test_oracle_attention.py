"""Pins of the oracle's attention: brute force on tiny inputs, torch fp64
SDPA on the unpaged data, closed forms, and invariances of the paged form."""

import numpy as np
import pytest

import oracle
from synth import custom_workload, make_workload
from tests import oracle_pins as pins
from tests.independent import e4m3_by_torch


def test_brute_force():
    pins.pin_brute_force()


def test_library_sdpa():
    pins.pin_sdpa()


def test_single_key_closed_form():
    pins.pin_single_key()


def test_zero_keys_give_mean_of_visible_values():
    pins.pin_zero_keys_mean_of_visible()


def test_constant_values_closed_form():
    pins.pin_constant_v()


def test_softmax_scale_is_honoured():
    pins.pin_scale_changes_result()


def _run(w, **kw):
    return oracle.paged_attention(w.q, w.k_pages, w.v_pages, w.kv_scales, w.block_table, w.ctx_lens,
                                  w.q_lens, num_kv_heads=w.num_kv_heads, sm_scale=w.sm_scale, **kw)


def test_pool_permutation_invariance():
    w = custom_workload([1, 5, 2], [37, 64, 9], num_q_heads=8, num_kv_heads=2, head_dim=64, seed=41)
    ref = _run(w)
    rng = np.random.default_rng(7)
    perm = rng.permutation(w.num_pages)  # new physical id of old page p is perm[p]
    k2 = np.empty_like(w.k_pages)
    v2 = np.empty_like(w.v_pages)
    s2 = np.empty_like(w.kv_scales)
    k2[perm] = w.k_pages
    v2[perm] = w.v_pages
    s2[:, perm] = w.kv_scales
    bt2 = np.where(w.block_table >= 0, perm[np.maximum(w.block_table, 0)], -1).astype(np.int32)
    got = oracle.paged_attention(w.q, k2, v2, s2, bt2, w.ctx_lens, w.q_lens, num_kv_heads=2)
    np.testing.assert_array_equal(got, ref)


def test_poison_independence():
    # bytes past each length and unreferenced pages never influence the result
    w = custom_workload([1, 3], [21, 50], num_q_heads=4, num_kv_heads=1, head_dim=64, seed=42)
    ref = _run(w)
    rng = np.random.default_rng(8)
    used = set(int(p) for p in w.block_table[w.block_table >= 0])
    for p in range(w.num_pages):
        if p not in used:
            w.k_pages[p] = rng.integers(0, 256, w.k_pages[p].shape)
            w.v_pages[p] = rng.integers(0, 256, w.v_pages[p].shape)
            w.kv_scales[:, p] = rng.standard_normal(2)[:, None]
    for b in range(w.num_seqs):
        L = int(w.ctx_lens[b])
        last = int(w.block_table[b][(L - 1) // 16])
        for s in range(L % 16 or 16, 16):
            w.k_pages[last, :, :, s, :] = 0x7F
            w.v_pages[last, :, s // 4, :, :, :, s % 4] = 0xFF
    np.testing.assert_array_equal(_run(w), ref)


def test_shared_prefix_pages():
    # two sequences whose block tables point at the same physical pages and
    # whose query rows are equal produce equal outputs
    w = custom_workload([1, 1], [40, 40], num_q_heads=4, num_kv_heads=2, head_dim=64, seed=43)
    w.block_table[1] = w.block_table[0]
    w.q[1] = w.q[0]
    got = _run(w)
    np.testing.assert_array_equal(got[1], got[0])


def test_rows_subset_matches_full():
    w = custom_workload([4, 2], [30, 70], num_q_heads=4, num_kv_heads=2, head_dim=64, seed=44)
    full = _run(w)
    part = _run(w, rows=[1, 4])
    np.testing.assert_allclose(part[[1, 4]], full[[1, 4]], rtol=0, atol=1e-14)
    assert np.all(part[[0, 2, 3, 5]] == 0)


@pytest.mark.parametrize("name", ["tiny_decode", "mtp_verify", "prefill_chunk", "mqa_decode"])
def test_named_workloads_reduced_vs_sdpa(name):
    # the named shapes at reduced batch/length, oracle vs library SDPA
    ctx = {"tiny_decode": None, "mtp_verify": (128, 300), "prefill_chunk": (0, 100),
           "mqa_decode": (256, 600)}[name]
    over = {"prefill_chunk": dict(q_len=48)}.get(name, {})
    w = make_workload(name, batch=2, ctx_range=ctx, **over)
    np.testing.assert_allclose(_run(w), pins.sdpa_attention(w), rtol=0, atol=1e-12)


def test_gather_round_trip():
    # logical bytes scattered by hand into a permuted pool come back unchanged
    rng = np.random.default_rng(45)
    P, Hkv, S, D = 12, 2, 16, 128
    L = 70
    logical_k = rng.integers(0, 256, (Hkv, L, D), dtype=np.uint8)
    logical_v = rng.integers(0, 256, (Hkv, L, D), dtype=np.uint8)
    phys = rng.permutation(P)[: (L + S - 1) // S]
    # written byte by byte at the flat offsets of the ABI layouts
    k_flat = np.zeros(P * Hkv * S * D, np.uint8)
    v_flat = np.zeros(P * Hkv * S * D, np.uint8)
    scales = rng.standard_normal((2, P, Hkv)).astype(np.float32)
    nvb = D // 16
    for t in range(L):
        p, s = phys[t // S], t % S
        for h in range(Hkv):
            for d in range(D):
                k_flat[(((p * Hkv + h) * (D // 16) + d // 16) * S + s) * 16 + d % 16] = logical_k[h, t, d]
                a, i, e = d // nvb, (d % nvb) // 4, d % 4
                v_flat[(((((p * Hkv + h) * (S // 4) + s // 4) * (D // 64) + i) * 16 + a) * 4 + e) * 4 + s % 4] = \
                    logical_v[h, t, d]
    k_pages = k_flat.reshape(P, Hkv, D // 16, S, 16)
    v_pages = v_flat.reshape(P, Hkv, S // 4, D // 64, 16, 4, 4)
    bt = np.full(8, -1, np.int32)
    bt[: phys.size] = phys
    g = oracle.gather_sequence(k_pages, v_pages, scales, bt, L)
    np.testing.assert_array_equal(g.k_bytes, logical_k)
    np.testing.assert_array_equal(g.v_bytes, logical_v)
    np.testing.assert_array_equal(g.page_of_token, phys[np.arange(L) // S])
    np.testing.assert_array_equal(g.k_scale, scales[0][phys[np.arange(L) // S]].T)
    np.testing.assert_array_equal(g.v_scale, scales[1][phys[np.arange(L) // S]].T)
