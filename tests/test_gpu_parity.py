"""GPU parity with the fp64 oracle, element by element, through the C ABI.

The named workloads run at reduced sizes (full oracle, several tiles and a
ragged tail) and at their full sizes (full oracle where it finishes in
seconds, sampled rows for the prefill chunk), plus edge cases: single key,
ctx == q_len, ctx % 16 in {0, 1, 15}, group sizes 1..64, head_dim 64/128,
mixed q_lens, fp32/bf16 in/out, forced partitions."""

import numpy as np
import pytest

from synth import custom_workload, make_workload
from tests.gpu_helpers import (check_contract, log, plan_for, record, run_gpu, run_oracle, takes_whole_schedule,
                                whole_schedule_workload)

pytestmark = pytest.mark.gpu


def _parity(w, rows=None, **plan_over):
    log(f"parity: {w.name} seed={w.seed} B={w.num_seqs} Hq={w.num_q_heads} Hkv={w.num_kv_heads} D={w.head_dim} "
        f"q_lens={sorted(set(w.q_lens.tolist()))[:6]} ctx=[{w.ctx_lens.min()},{w.ctx_lens.max()}] "
        f"q={w.q_dtype} out={w.out_dtype} over={plan_over}")
    plan = plan_for(w, **plan_over)
    info = plan.info()
    got = run_gpu(w, plan=plan)
    plan.close()
    ref = run_oracle(w, rows=rows)
    if rows is not None:
        got, ref = got[rows], ref[rows]
    stats = check_contract(got, ref, w.out_dtype, what=w.name)
    log(f"  plan={info} stats={stats}")
    record(dict(case=w.name, seed=w.seed, B=w.num_seqs, Hq=w.num_q_heads, Hkv=w.num_kv_heads, D=w.head_dim,
                q_dtype=w.q_dtype, out_dtype=w.out_dtype, plan=info, **stats))
    return stats


REDUCED = {
    "tiny_decode": dict(),
    "llama3_8b_decode": dict(batch=5, ctx_range=(512, 1100)),
    "mtp_verify": dict(batch=9, ctx_range=(128, 400)),
    "long_ctx_split": dict(batch=2, ctx_range=(0, 4096), num_kv_splits=8),
    "prefill_chunk": dict(batch=3, ctx_range=(0, 300), q_len=96),
    "mqa_decode": dict(batch=6, ctx_range=(256, 2000)),
}


@pytest.mark.parametrize("name", sorted(REDUCED))
def test_named_workload_reduced(name):
    _parity(make_workload(name, **REDUCED[name]))


@pytest.mark.parametrize("name", ["tiny_decode", "llama3_8b_decode", "mtp_verify", "mqa_decode"])
def test_named_workload_full(name):
    _parity(make_workload(name, keep_logical=False))


def test_long_context_split_full():
    # 4 x 32768 keys, 64 partitions merged by log-sum-exp
    w = make_workload("long_ctx_split", keep_logical=False)
    stats = _parity(w)
    assert stats["n"] == 4 * 32 * 128


def test_prefill_chunk_full_sampled_rows():
    w = make_workload("prefill_chunk", keep_logical=False)
    rng = np.random.default_rng(0)
    starts = np.concatenate([[0], np.cumsum(w.q_lens)[:-1]])
    rows = sorted(set(int(s + i) for s in starts for i in [0, 1, 2, 15, 16, 17, 63, 64, 255, 256, 510, 511])
                  | set(rng.integers(0, w.total_q, 256).tolist()))
    _parity(w, rows=rows)


EDGE = [
    # (q_lens, ctx_lens, Hq, Hkv, D, q_dtype, out_dtype)
    ([1], [1], 4, 1, 128, "bf16", "bf16"),
    ([1, 1, 1], [16, 17, 15], 8, 2, 128, "bf16", "bf16"),
    ([1, 1], [31, 33], 8, 8, 64, "bf16", "bf16"),
    ([5, 5], [5, 6], 40, 8, 128, "bf16", "bf16"),
    ([1, 3, 5, 2], [40, 3, 90, 2], 10, 2, 128, "bf16", "bf16"),
    ([1, 1], [300, 47], 64, 1, 128, "bf16", "bf16"),
    ([1, 1], [250, 1000], 64, 1, 64, "bf16", "bf16"),
    ([2, 1], [70, 9], 16, 2, 128, "bf16", "bf16"),  # 16 columns per group
    ([1, 1], [129, 500], 8, 1, 128, "f32", "f32"),
    ([1, 4], [129, 64], 4, 1, 64, "f32", "bf16"),
    ([3, 1], [200, 333], 12, 4, 128, "bf16", "f32"),
    ([33, 20], [33, 100], 4, 2, 128, "bf16", "bf16"),  # prefill from empty cache
    # shared-KV tile kernels with fp32 Q and/or output
    ([5, 2], [400, 70], 40, 8, 128, "f32", "f32"),  # 25 columns
    ([1, 1, 1], [700, 64, 2100], 64, 1, 128, "f32", "bf16"),  # 64 columns, split segments
    ([40, 7], [300, 800], 4, 2, 64, "bf16", "f32"),  # 80 columns, D = 64
]


@pytest.mark.parametrize("idx", range(len(EDGE)))
def test_edge_cases(idx):
    ql, cl, hq, hkv, d, qd, od = EDGE[idx]
    w = custom_workload(ql, cl, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, q_dtype=qd, out_dtype=od,
                        seed=100 + idx, name=f"edge{idx}")
    _parity(w)


# Batches beyond 128 sequences: the kernels hold the lengths of sequences
# 0..127 in lanes and read the others from memory while they count chunks,
# locate a unit's first sequence and step to the next one; the merge needs
# every sequence's first query row.
MANY = [
    # (B, q_len, ctx range, Hq, Hkv, forced splits): kernel family exercised
    (300, 1, (1, 300), 8, 2, 0),     # packed decode, short and split sequences
    (300, 1, (1, 300), 8, 2, 3),     # packed decode, forced partitions beyond one resident round
    (260, 2, (2, 200), 8, 2, 0),     # single tile with the low halves of P in spare columns (8 columns)
    (260, 2, (2, 200), 16, 2, 0),    # single tile (16 columns)
    (150, 5, (5, 400), 40, 8, 0),    # shared-KV tile, two waves (25 columns)
    (200, 1, (1, 600), 64, 1, 0),    # shared-KV tile, four waves (64 columns)
    (140, 16, (16, 300), 32, 2, 0),  # shared-KV tile, eight waves (256-column blocks)
]


@pytest.mark.parametrize("idx", range(len(MANY)))
def test_many_sequences(idx):
    B, ql, (lo, hi), hq, hkv, splits = MANY[idx]
    rng = np.random.default_rng(700 + idx)
    ctx = rng.integers(max(lo, ql), hi + 1, size=B).tolist()
    w = custom_workload([ql] * B, ctx, num_q_heads=hq, num_kv_heads=hkv, head_dim=128, seed=700 + idx,
                        num_kv_splits=splits, name=f"many{idx}")
    assert w.num_seqs > 128
    _parity(w)


# Shapes on which the shared-KV tile kernel gives every unit one segment
# whole (about as many (sequence, kv head) segments as units, none longer
# than twice the mean): the two-wave tile on 25-column blocks, 4 resident
# workgroups per compute unit.
WHOLE = [
    # (B, ctx range, q dtype, out dtype); 5 new tokens, 40 query heads / 8 kv heads
    (128, (300, 600), "bf16", "bf16"),
    (128, (500, 500), "bf16", "bf16"),   # equal lengths: ranked by sequence index
    (128, (300, 600), "f32", "f32"),
    (100, (300, 600), "bf16", "bf16"),   # 800 segments: some units idle
]


@pytest.mark.parametrize("idx", range(len(WHOLE)))
def test_whole_segment_schedule(idx):
    B, (lo, hi), qd, od = WHOLE[idx]
    w = whole_schedule_workload(B, lo, hi, seed=900 + idx, q_dtype=qd, out_dtype=od)
    plan = plan_for(w)
    info = plan.info()
    plan.close()
    assert takes_whole_schedule(w, info), info
    _parity(w)


@pytest.mark.parametrize("splits", [1, 2, 3, 7, 64])
def test_forced_partitions(splits):
    w = custom_workload([1, 1, 1], [1000, 37, 2048], num_q_heads=8, num_kv_heads=2, head_dim=128, seed=200,
                        num_kv_splits=splits, name=f"splits{splits}")
    _parity(w)
