"""GPU parity of the attention kernels on an INT8 KV cache (two's-complement
bytes times the page scale) with the fp64 oracle, through the C ABI: every
kernel family (packed decode, single tile, shared-KV tile), forced
partitions, ragged tails, D 64 and 128."""

import numpy as np
import pytest

from synth import custom_workload, make_workload
from tests.gpu_helpers import (check_contract, log, plan_for, run_gpu, takes_whole_schedule,
                                whole_schedule_workload)

import oracle

pytestmark = pytest.mark.gpu


def _parity(w, rows=None, **over):
    log(f"int8 parity: {w.name} seed={w.seed} B={w.num_seqs} Hq={w.num_q_heads} Hkv={w.num_kv_heads} "
        f"D={w.head_dim} q_lens={sorted(set(w.q_lens.tolist()))[:4]} ctx=[{w.ctx_lens.min()},{w.ctx_lens.max()}]")
    plan = plan_for(w, kv_format="int8", **over)
    got = run_gpu(w, plan=plan)
    plan.close()
    ref = oracle.paged_attention(w.q, w.k_pages, w.v_pages, w.kv_scales, w.block_table, w.ctx_lens, w.q_lens,
                                 num_kv_heads=w.num_kv_heads, sm_scale=w.sm_scale, kv_format="int8", rows=rows)
    if rows is not None:
        got, ref = got[rows], ref[rows]
    return check_contract(got, ref, w.out_dtype, what=f"int8 {w.name}")


REDUCED = {
    "llama3_8b_decode": dict(batch=5, ctx_range=(512, 1100)),
    "mtp_verify": dict(batch=9, ctx_range=(128, 400)),
    "long_ctx_split": dict(batch=2, ctx_range=(0, 4096), num_kv_splits=8),
    "prefill_chunk": dict(batch=3, ctx_range=(0, 300), q_len=96),
    "mqa_decode": dict(batch=6, ctx_range=(256, 2000)),
}


@pytest.mark.parametrize("name", sorted(REDUCED))
def test_int8_reduced(name):
    _parity(make_workload(name, kv_format="int8", **REDUCED[name]))


def test_int8_llama3_full():
    _parity(make_workload("llama3_8b_decode", kv_format="int8", keep_logical=False))


@pytest.mark.parametrize("name", ["mtp_verify", "mqa_decode", "long_ctx_split"])
def test_int8_full(name):
    w = make_workload(name, kv_format="int8", keep_logical=False)
    stats = _parity(w)
    assert stats["n"] == w.total_q * w.num_q_heads * w.head_dim


def test_int8_prefill_full_sampled_rows():
    # every sequence's first, page-edge and last new tokens, plus random rows
    w = make_workload("prefill_chunk", kv_format="int8", keep_logical=False)
    rng = np.random.default_rng(1)
    starts = np.concatenate([[0], np.cumsum(w.q_lens)[:-1]])
    rows = sorted(set(int(s + i) for s in starts for i in [0, 15, 16, 255, 511])
                  | set(rng.integers(0, w.total_q, 48).tolist()))
    _parity(w, rows=rows)


EDGE = [
    ([1, 1, 1], [16, 17, 15], 8, 2, 128),
    ([1, 1], [31, 33], 8, 8, 64),
    ([2, 1], [70, 9], 16, 2, 128),  # single 16-column tile
    ([1, 3, 5, 2], [40, 3, 90, 2], 10, 2, 128),
    ([33, 20], [33, 100], 4, 2, 128),
]


@pytest.mark.parametrize("idx", range(len(EDGE)))
def test_int8_edges(idx):
    ql, cl, hq, hkv, d = EDGE[idx]
    _parity(custom_workload(ql, cl, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, seed=400 + idx,
                            kv_format="int8", name=f"int8_edge{idx}"))


def test_int8_forced_partitions():
    w = custom_workload([1, 1, 1], [1000, 37, 2048], num_q_heads=8, num_kv_heads=2, head_dim=128, seed=410,
                        num_kv_splits=7, kv_format="int8", name="int8_splits7")
    _parity(w)


def test_int8_whole_segment_schedule():
    # every unit takes one (sequence, kv head) segment whole
    w = whole_schedule_workload(128, 300, 600, seed=950, kv_format="int8")
    plan = plan_for(w, kv_format="int8")
    info = plan.info()
    plan.close()
    assert takes_whole_schedule(w, info), info
    _parity(w)
