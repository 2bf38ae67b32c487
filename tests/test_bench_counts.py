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


def test_attention_counts_direct():
    from synth.workloads import make_workload
    w = make_workload("mtp_verify", batch=5, ctx_range=(7, 90))
    got = bench.algorithmic_counts(w)
    pairs = 0
    kv = scales = bt = 0
    for b in range(w.num_seqs):
        L, Q = int(w.ctx_lens[b]), int(w.q_lens[b])
        for i in range(Q):  # query i sees the cached keys and drafts 0..i
            pairs += L - Q + i + 1
        for key in range(L):
            kv += w.num_kv_heads * w.head_dim * 2  # one K and one V byte per (head, dim)
        for pg in range(-(-L // w.page_size)):
            scales += w.num_kv_heads * 2 * 4
            bt += 4
    qo = int(w.q_lens.sum()) * w.num_q_heads * w.head_dim * 2 * 2  # bf16 Q in, bf16 out
    assert got["pairs"] == pairs
    assert got["flops"] == 2 * 2 * w.head_dim * w.num_q_heads * pairs  # QK and PV, a multiply-add each
    assert got["kv_bytes"] == kv
    assert got["bytes"] == kv + scales + bt + qo + 8 * w.num_seqs


def _summary(tmp_path, sha, fetch_kib, write_kib, copy_kib):
    p = tmp_path / "attn_stream_kernel_demo_hbm_counters.txt"
    p.write_text(f"# test summary\nkernel_source_sha256_16: {sha}\nattn_FETCH_SIZE_KiB_per_dispatch: {fetch_kib}\n"
                 f"attn_WRITE_SIZE_KiB_per_dispatch: {write_kib}\ncopy_bytes: {1 << 30}\n"
                 f"copy_FETCH_SIZE_KiB_per_dispatch: {copy_kib}\ncopy_WRITE_SIZE_KiB_per_dispatch: {copy_kib / 2}\n")


def test_traffic_scaled_by_the_copy_and_dropped_for_another_source(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    # a 1 GiB copy read as 2^21 KiB fetched and 2^20 KiB written: factors 1/2 and 1
    _summary(tmp_path, bench.source_hash(bench.KERNEL_SOURCE), 1000.0, 10.0, float(1 << 21))
    assert bench.committed_traffic("demo") == 1000.0 * 1024 / 2 + 10.0 * 1024
    _summary(tmp_path, "0000000000000000", 1000.0, 10.0, float(1 << 21))
    assert bench.committed_traffic("demo") is None
    assert bench.committed_traffic("absent") is None


def test_source_hash_follows_local_includes(tmp_path):
    (tmp_path / "k.hip").write_text('#include <hip/hip_runtime.h>\n#include "a.h"\n__global__ void k() {}\n')
    (tmp_path / "a.h").write_text('#include "b.h"\n#include "a.h"\n')  # a cycle is followed once
    (tmp_path / "b.h").write_text("constexpr int kB = 1;\n")
    h0 = bench.source_hash(str(tmp_path / "k.hip"))
    assert h0 == bench.source_hash(str(tmp_path / "k.hip"))
    (tmp_path / "b.h").write_text("constexpr int kB = 2;\n")  # a change two includes down
    h1 = bench.source_hash(str(tmp_path / "k.hip"))
    assert h1 != h0
    (tmp_path / "b.h").write_text("constexpr int kB = 1;\n")
    assert bench.source_hash(str(tmp_path / "k.hip")) == h0
