"""The bench's algorithmic byte counts for the append and the acceptance,
against direct counts written differently (per touched page and per row),
CPU only."""

import numpy as np

import bench
from synth.accept import accept_case
from synth.append import append_case


def test_append_counts_direct():
    c = append_case([1, 5, 40, 16], [300, 133, 90, 16], num_kv_heads=4, head_dim=128, new_dtype="bf16", seed=3)
    got = bench.append_counts(c)["bytes"]
    want = 0
    hd = c.num_kv_heads * c.head_dim
    for b in range(c.num_seqs):
        L, Q = int(c.ctx_lens[b]), int(c.q_lens[b])
        want += Q * hd * 2 * 2  # new K and V rows, bf16
        want += Q * hd * 2  # their bytes written
        pages = range((L - Q) // 16, (L - 1) // 16 + 1)
        for pi in pages:
            cached = max(0, min(16, (L - Q) - 16 * pi))
            want += cached * hd * 2  # cached bytes of the touched page, K and V
            want += c.num_kv_heads * 2 * 8  # K and V scales read and written
            want += 4  # block-table entry
        want += 8  # lengths
    assert got == want


def test_accept_counts_direct():
    c = accept_case(3, 4, 64, dtype="bf16", seed=1)
    got = bench.accept_counts(c)["bytes"]
    B, K, V = 3, 4, 64
    assert got == B * (K + 1) * V * 2 + B * K * 4 + B * (K + 1) * 4 + B * 4


def test_int8_runs_read_their_own_counter_summary():
    class W:
        name = "llama3_8b_decode"
        kv_format = "int8"
    assert bench.profile_name(W()) == "llama3_8b_decode_int8"
    W.kv_format = "e4m3"
    assert bench.profile_name(W()) == "llama3_8b_decode"
