"""GPU invariances: pool permutation, shared prefix pages, poison bytes,
run-to-run determinism (all bit-identical), and partition counts."""

import numpy as np
import pytest
import torch

from synth import custom_workload, make_workload
from tests.gpu_helpers import check_contract, device_inputs, log, plan_for, run_gpu, run_oracle

pytestmark = pytest.mark.gpu


def test_pool_permutation_bit_identical():
    w = make_workload("mtp_verify", batch=6, ctx_range=(128, 300))
    log("invariance: permutation (mtp_verify reduced)")
    ref = run_gpu(w)
    perm = np.random.default_rng(3).permutation(w.num_pages)
    k2 = np.empty_like(w.k_pages)
    v2 = np.empty_like(w.v_pages)
    s2 = np.empty_like(w.kv_scales)
    k2[perm], v2[perm], s2[:, perm] = w.k_pages, w.v_pages, w.kv_scales
    w.block_table = np.where(w.block_table >= 0, perm[np.maximum(w.block_table, 0)], -1).astype(np.int32)
    w.k_pages, w.v_pages, w.kv_scales = k2, v2, s2
    assert np.array_equal(run_gpu(w), ref)


def test_shared_prefix_pages():
    # Two sequences reading the same physical pages with the same queries.
    # Both match the oracle; they may sit at different cut points of the
    # balanced chunk schedule (which depends on the whole batch), so they
    # agree to fp32 rounding: at most one bf16 ulp apart.
    w = custom_workload([1, 1, 1], [500, 500, 120], num_q_heads=8, num_kv_heads=2, head_dim=128, seed=301)
    log("invariance: shared prefix pages")
    w.block_table[1] = w.block_table[0]
    w.q[1] = w.q[0]
    got = run_gpu(w)
    ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(got[0]), 2.0 ** -126))) - 7)
    assert np.all(np.abs(got[1] - got[0]) <= ulp)
    check_contract(got, run_oracle(w), "bf16", "shared-prefix")
    # with one workgroup per sequence-sized share the cut points coincide
    got1 = run_gpu(w, num_kv_splits=1)
    check_contract(got1, run_oracle(w), "bf16", "shared-prefix, 1 split")


def test_poison_does_not_leak():
    w = make_workload("llama3_8b_decode", batch=4, ctx_range=(500, 700))
    log("invariance: poison")
    ref = run_gpu(w)
    used = set(int(p) for p in w.block_table[w.block_table >= 0])
    unused = [p for p in range(w.num_pages) if p not in used]
    assert unused
    for p in range(w.num_pages):
        if p not in used:
            w.k_pages[p] = 0xFF
            w.v_pages[p] = 0x7F
            w.kv_scales[:, p] = np.nan
    for b in range(w.num_seqs):
        L = int(w.ctx_lens[b])
        last = int(w.block_table[b][(L - 1) // 16])
        for s in range(L % 16 or 16, 16):
            w.k_pages[last, :, :, s, :] = 0x7F
            w.v_pages[last, :, s // 4, :, :, :, s % 4] = 0xFF
        # entries past the last page name a poisoned page: were one read,
        # NaN scales and codes would fail the comparison (no wild address)
        w.block_table[b, (L + 15) // 16:] = unused[b % len(unused)]
    assert np.array_equal(run_gpu(w), ref)


def test_run_to_run_bit_identical():
    w = make_workload("long_ctx_split", batch=2, ctx_range=(0, 8192), num_kv_splits=16)
    log("invariance: determinism")
    plan = plan_for(w)
    x = device_inputs(w)
    outs = []
    for _ in range(3):
        out = torch.empty((w.total_q, w.num_q_heads, w.head_dim), dtype=torch.bfloat16, device="cuda")
        plan.forward(x["q"], x["k_pages"], x["v_pages"], x["kv_scales"], x["block_table"], x["ctx_lens"],
                     x["q_lens"], out)
        outs.append(out)
    torch.cuda.synchronize()
    assert all(torch.equal(outs[0], o) for o in outs[1:])
    plan.close()


def test_partition_count_agreement():
    w = custom_workload([1, 1], [3000, 1500], num_q_heads=32, num_kv_heads=8, head_dim=128, seed=302)
    log("invariance: partition counts")
    ref = run_oracle(w)
    outs = [run_gpu(w, num_kv_splits=s) for s in (1, 4, 47)]
    for o in outs:
        check_contract(o, ref, "bf16", "partitions")
    # different partitionings differ only by fp32 rounding: at most one bf16 ulp apart
    assert np.max(np.abs(outs[0] - outs[2])) < 4e-3
