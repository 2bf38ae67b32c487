"""Pins of the append oracle (oracle/kv_append.py), CPU only.

* encoder: brute-force nearest code over every finite magnitude (ties to
  even), torch's float8_e4m3fn conversion, and the round trip of every
  finite code; ties and their neighbours are covered explicitly;
* append: pure-Python loops over flat byte offsets on tiny cases (cached
  prefixes, pages whose scale grows, ragged tails, fp32 and bf16 rows);
* fresh pages: the generator's own page quantiser (torch conversion) on the
  same fp32 values;
* unchanged scale: cached bytes come back unchanged;
* error bound: every written value is within half an E4M3 spacing (times the
  page scale) of its input;
* planted mistakes in the oracle each fail one of these.
"""

import numpy as np
import pytest
import torch

import oracle.kv_append as ka
from oracle import e4m3
from synth import append as sa
from synth.workloads import _quantise_pages, k_to_layout, v_to_layout
from tests.independent import brute_force_append, e4m3_encode_brute


def _probe_values():
    vals = e4m3.decode(np.arange(0x7F, dtype=np.uint8))
    mids = (vals[:-1] + vals[1:]) / 2  # exact ties (5 significant bits)
    f = np.float32
    ys = [vals, mids, np.nextafter(mids.astype(f), f(0)), np.nextafter(mids.astype(f), f(1000)),
          np.array([0.0, 2.0 ** -10, 2.0 ** -11, 3 * 2.0 ** -11, 447.99, 448.0, 448.01, 464.0, 464.01, 500.0, 1e6])]
    rng = np.random.default_rng(7)
    ys.append(np.exp(rng.uniform(np.log(2.0 ** -12), np.log(600.0), 400)))
    y = np.concatenate([np.asarray(a, dtype=np.float64) for a in ys]).astype(np.float32)
    return np.concatenate([y, -y, np.array([-0.0], dtype=np.float32)])


def test_encode_brute_force():
    y = _probe_values()
    got = ka.encode(y)
    want = np.array([e4m3_encode_brute(float(v)) for v in y], dtype=np.uint8)
    assert np.array_equal(got, want)


def test_encode_matches_torch():
    y = _probe_values()
    t = torch.from_numpy(y).clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ka.encode(y), t)


def test_encode_round_trip_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(ka.encode(e4m3.decode(codes).astype(np.float32)), codes)


TINY = [
    # (q_lens, ctx_lens, Hkv, D, new_dtype, sigmas)
    ([3], [20], 1, 64, "f32", (4.0,)),        # scale grows: cached slots requantised
    ([1, 2], [17, 16], 2, 64, "bf16", (1.0,)),  # a fresh page; a page filled to the end
    ([5, 1], [5, 33], 1, 64, "f32", (0.25,)),   # no cache; cache with an unchanged scale
    ([18], [40], 1, 64, "bf16", (2.0, 0.5)),    # three pages touched, ragged tail
]


def _oracle(c):
    return ka.kv_append(c.k_new, c.v_new, c.k_pages, c.v_pages, c.kv_scales, c.block_table, c.ctx_lens, c.q_lens)


@pytest.mark.parametrize("idx", range(len(TINY)))
def test_append_brute_force(idx):
    ql, cl, hkv, d, dt, sig = TINY[idx]
    c = sa.append_case(ql, cl, num_kv_heads=hkv, head_dim=d, new_dtype=dt, seed=40 + idx, new_sigmas=sig)
    k, v, s = _oracle(c)
    bk, bv, bs = brute_force_append(c)
    assert np.array_equal(k, bk) and np.array_equal(v, bv)
    assert np.array_equal(s.view(np.uint32), bs.view(np.uint32))


def test_fresh_pages_match_generator_quantiser():
    # all tokens new: every page is quantised from scratch, as the generator does
    c = sa.append_case([37, 16], [37, 16], num_kv_heads=2, head_dim=128, new_dtype="f32", seed=3)
    k, v, s = _oracle(c)
    S = 16
    row = 0
    for b in range(c.num_seqs):
        L = int(c.ctx_lens[b])
        n = (L + S - 1) // S
        for which, new, pool in ((0, c.k_new, k), (1, c.v_new, v)):
            x = np.zeros((n, c.num_kv_heads, S, c.head_dim), dtype=np.float32)
            xs = new[row:row + L].numpy()  # [L][H][D]
            for t in range(L):
                x[t // S, :, t % S] = xs[t]
            valid = np.minimum(S, L - np.arange(n) * S)
            codes, scale = _quantise_pages(x, valid)
            phys = c.block_table[b, :n]
            want = k_to_layout(codes) if which == 0 else v_to_layout(codes)
            assert np.array_equal(pool[phys], want)
            assert np.array_equal(s[which, phys], scale)
        row += L


def test_unchanged_scale_keeps_cached_bytes():
    c = sa.append_case([1, 1, 1], [100, 65, 200], num_kv_heads=2, head_dim=64, new_dtype="f32", seed=5,
                       new_sigmas=(1e-3,))
    k, v, s = _oracle(c)
    for b in range(c.num_seqs):
        L = int(c.ctx_lens[b])
        p = c.block_table[b, (L - 1) // 16]
        cached = (L - 1) % 16
        for pool_new, pool_old in ((k, c.k_pages), (v, c.v_pages)):
            got = e4m3.decode(pool_new[p]).ravel()
            old = e4m3.decode(pool_old[p]).ravel()
            # every byte of the cached slots is unchanged (poisoned tail aside)
            mask = np.zeros(pool_old[p].shape, dtype=bool)
            if pool_new is k:
                mask[:, :, :cached, :] = True
            else:
                for sl in range(cached):
                    mask[:, sl // 4, :, :, :, sl % 4] = True
            assert np.array_equal(pool_new[p][mask], pool_old[p][mask])
            del got, old


def test_dequantisation_within_half_spacing():
    c = sa.append_case([40, 9], [40, 9], num_kv_heads=1, head_dim=64, new_dtype="f32", seed=9, new_sigmas=(3.0,))
    k, _, s = _oracle(c)
    from oracle.attention import k_token_bytes
    vals = e4m3.decode(np.arange(0x7F, dtype=np.uint8))
    row = 0
    for b in range(c.num_seqs):
        L = int(c.ctx_lens[b])
        t = np.arange(L)
        pages = c.block_table[b][t // 16]
        got = e4m3.decode(k_token_bytes(k, pages, 0, t % 16)) * s[0, pages, 0][:, None]
        x = c.k_new[row:row + L, 0].double().numpy()
        sc = s[0, pages, 0][:, None].astype(np.float64)
        mag = np.minimum(np.abs(x) / sc, 448.0)
        hi = np.minimum(np.searchsorted(vals, mag), vals.size - 1)
        spacing = vals[hi] - vals[np.maximum(hi - 1, 0)]
        assert np.all(np.abs(got - x) <= (spacing / 2 + 1e-6 * mag) * sc + 1e-12)
        row += L


def _encode_ties_up(y):
    y = np.asarray(y, dtype=np.float32)
    vals, codes = ka._finite_magnitudes()
    mag = np.minimum(np.abs(y).astype(np.float64), 448.0)
    hi = np.minimum(np.searchsorted(vals, mag), vals.size - 1)
    lo = np.maximum(hi - 1, 0)
    take_hi = (vals[hi] - mag) <= (mag - vals[lo])
    return (np.where(take_hi, codes[hi], codes[lo]) | (np.signbit(y).astype(np.uint8) << 7)).astype(np.uint8)


_ENCODE = ka.encode


def _encode_no_saturation(y):
    # magnitudes past 448 become the NaN code instead of saturating
    return np.where(np.abs(np.asarray(y, np.float32)) > 448.0, np.uint8(0x7F), _ENCODE(y)).astype(np.uint8)


PLANTED = {
    "ties_away_from_even": ("encode", _encode_ties_up),
    "no_saturation": ("encode", _encode_no_saturation),
    "scale_one_ulp_high": ("page_scale", lambda a: np.float32(1.0) if a == 0 else np.nextafter(
        np.float32(np.float32(a) / np.float32(448.0)), np.float32(np.inf))),
    "zero_page_scale_448": ("page_scale", lambda a: np.float32(448.0) if a == 0 else np.float32(
        np.float32(a) / np.float32(448.0))),
}


@pytest.mark.parametrize("name", sorted(PLANTED))
def test_planted_mistake_fails_a_pin(name, monkeypatch):
    attr, fn = PLANTED[name]
    monkeypatch.setattr(ka, attr, fn)
    failed = False
    for idx in range(len(TINY)):
        try:
            test_append_brute_force(idx)
        except AssertionError:
            failed = True
            break
    if not failed:
        try:
            test_encode_brute_force()
            test_append_zero_rows_pin()
        except AssertionError:
            failed = True
    assert failed, f"planted mistake {name} passed every pin"


def test_append_zero_rows_pin():
    # all-zero new rows on fresh pages: scale 1, bytes 0 (0x80 for -0)
    c = sa.append_case([16], [16], num_kv_heads=1, head_dim=64, new_dtype="f32", seed=1, new_sigmas=(0.0,))
    k, v, s = ka.kv_append(c.k_new, c.v_new, c.k_pages, c.v_pages, c.kv_scales, c.block_table, c.ctx_lens,
                           c.q_lens)
    p = c.block_table[0, 0]
    assert s[0, p, 0] == 1.0 and s[1, p, 0] == 1.0
    assert np.all((k[p] & 0x7F) == 0) and np.all((v[p] & 0x7F) == 0)


@pytest.mark.parametrize("idx", range(len(TINY)))
def test_append_int8_brute_force(idx):
    ql, cl, hkv, d, dt, sig = TINY[idx]
    c = sa.append_case(ql, cl, num_kv_heads=hkv, head_dim=d, new_dtype=dt, seed=80 + idx, new_sigmas=sig,
                       kv_format="int8")
    k, v, s = ka.kv_append(c.k_new, c.v_new, c.k_pages, c.v_pages, c.kv_scales, c.block_table, c.ctx_lens,
                           c.q_lens, kv_format="int8")
    bk, bv, bs = brute_force_append(c, kv_format="int8")
    assert np.array_equal(k, bk) and np.array_equal(v, bv)
    assert np.array_equal(s.view(np.uint32), bs.view(np.uint32))


def test_int8_encoder_ties_and_clip():
    y = np.array([0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 126.5, 127.4, 130.0, -200.0, 0.49999997, -0.0], dtype=np.float32)
    got = ka.encode_int8(y).view(np.int8).tolist()
    assert got == [0, 2, 2, 0, -2, -2, 126, 127, 127, -127, 0, 0]


def test_int8_fresh_pages_match_generator_quantiser():
    from synth.workloads import _quantise_pages_int8

    c = sa.append_case([37, 16], [37, 16], num_kv_heads=2, head_dim=128, new_dtype="f32", seed=3, kv_format="int8")
    k, v, s = ka.kv_append(c.k_new, c.v_new, c.k_pages, c.v_pages, c.kv_scales, c.block_table, c.ctx_lens,
                           c.q_lens, kv_format="int8")
    S = 16
    row = 0
    for b in range(c.num_seqs):
        L = int(c.ctx_lens[b])
        n = (L + S - 1) // S
        for which, new, pool in ((0, c.k_new, k), (1, c.v_new, v)):
            x = np.zeros((n, c.num_kv_heads, S, c.head_dim), dtype=np.float32)
            xs = new[row:row + L].numpy()
            for t in range(L):
                x[t // S, :, t % S] = xs[t]
            valid = np.minimum(S, L - np.arange(n) * S)
            codes, scale = _quantise_pages_int8(x, valid)
            phys = c.block_table[b, :n]
            want = k_to_layout(codes) if which == 0 else v_to_layout(codes)
            assert np.array_equal(pool[phys], want)
            assert np.array_equal(s[which, phys], scale)
        row += L
