"""The seeded input generator: quantiser rounding, poison placement, block
tables and determinism.  (The generator feeds both the oracle and the GPU
path; these checks make sure its inputs follow the stated recipe.)"""

import numpy as np
import torch

from synth import POISON_BYTE, custom_workload, make_workload
from synth.workloads import _quantise_pages
from tests.independent import e4m3_by_bits


def _finite_codes():
    vals = np.array([e4m3_by_bits(c) for c in range(256)])
    codes = np.array([c for c in range(256) if not np.isnan(vals[c])])
    return codes, vals


def test_quantiser_is_nearest_even_saturating():
    codes, vals = _finite_codes()
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(3000) * 100, rng.standard_normal(3000) * 1e-2,
                        np.array([448.0, 460.0, 464.0, 470.0, 1e6, -1e6, 0.0, 2.0 ** -10, 3 * 2.0 ** -11])]).astype(np.float32)
    got = torch.from_numpy(np.clip(x, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    for xi, gi in zip(x, got):
        xc = float(np.clip(xi, -448, 448))
        d = np.abs(vals[codes] - xc)
        best = d.min()
        cands = codes[d == best]
        if len(cands) > 1:  # tie: the even mantissa (code LSB 0) wins; +-0 both fine
            cands = [c for c in cands if c & 1 == 0]
        assert vals[gi] == vals[cands[0]] or (vals[gi] == 0 and vals[cands[0]] == 0), (xi, gi, cands)


def test_page_scale_is_absmax_over_valid_slots():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((3, 2, 16, 8)).astype(np.float32)
    x[1, :, 5:, :] = 1000.0  # invalid slots must not enter the absmax
    codes, scale = _quantise_pages(x, np.array([16, 5, 16]))
    np.testing.assert_array_equal(scale[0], np.abs(x[0]).reshape(2, -1).max(1) / np.float32(448))
    np.testing.assert_array_equal(scale[1], np.abs(x[1, :, :5]).reshape(2, -1).max(1) / np.float32(448))
    assert np.all(codes[1, :, 5:] == POISON_BYTE)
    # the absmax element maps to +-448 exactly
    assert np.abs(codes[0].astype(np.int32) & 0x7F).max() == 0x7E


def test_pool_structure_and_poison():
    w = custom_workload([1, 2], [17, 40], num_q_heads=4, num_kv_heads=2, head_dim=64, seed=3)
    npages = (w.ctx_lens + 15) // 16
    used = np.concatenate([w.block_table[b, : npages[b]] for b in range(2)])
    assert len(set(used.tolist())) == used.size  # distinct physical pages
    assert np.all(w.block_table[0, npages[0]:] == -1)
    unused = np.setdiff1d(np.arange(w.num_pages), used)
    assert np.all(w.k_pages[unused] == POISON_BYTE) and np.all(np.isnan(w.kv_scales[:, unused]))
    last = w.block_table[0, npages[0] - 1]  # seq 0 has 17 tokens -> 1 valid slot in page 2
    assert np.all(w.k_pages[last, :, :, 1:] == POISON_BYTE)
    assert np.all(w.v_pages[last, :, 0, :, :, :, 1:] == POISON_BYTE)
    assert np.all(w.v_pages[last, :, 1:] == POISON_BYTE)
    assert not np.any(w.k_pages[last, :, :, 0] == POISON_BYTE)


def test_logical_copy_matches_pool():
    w = custom_workload([1, 1], [33, 16], num_q_heads=2, num_kv_heads=2, head_dim=64, seed=4)
    for b in range(2):
        lg = w.logical[b]
        for t in range(int(w.ctx_lens[b])):
            p, s = w.block_table[b, t // 16], t % 16
            D = w.head_dim
            for d in (0, 1, 5, 15, 16, 17, 33, D - 1):
                # flat-offset reading of the ABI layouts
                np.testing.assert_array_equal(lg["k_bytes"][:, t, d], w.k_pages[p, :, d // 16, s, d % 16])
                nvb = D // 16
                np.testing.assert_array_equal(lg["v_bytes"][:, t, d],
                                              w.v_pages[p, :, s // 4, (d % nvb) // 4, d // nvb, d % 4, s % 4])
            np.testing.assert_array_equal(lg["k_scale"][:, t], w.kv_scales[0, p])


def test_named_workloads_follow_their_shapes():
    w = make_workload("tiny_decode")
    assert (w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim, w.num_pages) == (1, 4, 1, 64, 32)
    assert w.ctx_lens.tolist() == [256] and w.q.dtype == torch.float32
    w = make_workload("llama3_8b_decode", keep_logical=False)
    assert w.num_seqs == 32 and w.ctx_lens.min() >= 512 and w.ctx_lens.max() <= 4096
    assert w.max_pages_per_seq == 256 and w.q.dtype == torch.bfloat16
    w = make_workload("mtp_verify", batch=4, ctx_range=(128, 200))
    assert np.all(w.q_lens == 5) and w.num_q_heads == 40


def test_determinism():
    a = make_workload("mtp_verify", batch=3, ctx_range=(128, 160))
    b = make_workload("mtp_verify", batch=3, ctx_range=(128, 160))
    assert np.array_equal(a.k_pages, b.k_pages) and np.array_equal(a.block_table, b.block_table)
    assert torch.equal(a.q, b.q)
