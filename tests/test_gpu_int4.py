"""GPU parity of the attention kernels on an INT4 KV cache (two 4-bit
two's-complement codes per byte times the page scale, head_dim 128) with the
fp64 oracle, through the C ABI: the kernels' widening of every code and the
block-table gather of codes, scales and pages bit for bit; every kernel family
(packed decode, single tile, shared-KV tile) on reduced and full-size
workloads, ragged tails, forced partitions; and output independent of the
codes of unused slots and pages."""

import numpy as np
import pytest
import torch

import oracle
import oracle.attention as oracle_attention
import paged_fp8_kv_attn_amd as pa
from synth import custom_workload, make_workload
from tests.gpu_helpers import (check_contract, device_inputs, log, plan_for, run_gpu, takes_whole_schedule,
                                whole_schedule_workload)

pytestmark = pytest.mark.gpu


def test_int4_decode_all_codes_bit_exact():
    log("int4 decode: 256 bytes x 3 (512 codes each), ragged length")
    codes = torch.arange(256, dtype=torch.uint8).repeat(3)
    for n in (768, 767, 5):
        c = codes[:n].cuda()
        out = torch.full((2 * n,), float("nan"), dtype=torch.float32, device="cuda")
        pa.debug_decode_int4(c, out)
        torch.cuda.synchronize()
        got = out.double().cpu().numpy()
        b = codes[:n].numpy()
        ref = np.stack([oracle_attention.decode_int4(b & 0x0F), oracle_attention.decode_int4(b >> 4)], axis=1)
        assert np.array_equal(got, ref.reshape(-1))


@pytest.mark.parametrize("case", ["gqa", "mqa"])
def test_int4_gather_bit_exact(case):
    w = {
        "gqa": lambda: custom_workload([1, 2, 1], [37, 16, 90], num_q_heads=8, num_kv_heads=2, head_dim=128,
                                       seed=501, kv_format="int4"),
        "mqa": lambda: custom_workload([1, 1], [100, 17], num_q_heads=16, num_kv_heads=1, head_dim=128, seed=502,
                                       kv_format="int4"),
    }[case]()
    log(f"int4 gather: {case} B={w.num_seqs} Hkv={w.num_kv_heads} max_ctx={w.max_ctx_len}")
    x = device_inputs(w)
    plan = plan_for(w, kv_format="int4")
    B, H, T, D = w.num_seqs, w.num_kv_heads, w.max_ctx_len, w.head_dim
    k_out = torch.full((B, H, T, D), 0xAA, dtype=torch.uint8, device="cuda")
    v_out = torch.full((B, H, T, D), 0xAA, dtype=torch.uint8, device="cuda")
    s_out = torch.full((2, B, H, T), -7.0, dtype=torch.float32, device="cuda")
    p_out = torch.full((B, T), -7, dtype=torch.int32, device="cuda")
    pa.debug_gather(plan, x["k_pages"], x["v_pages"], x["kv_scales"], x["block_table"], x["ctx_lens"], k_out,
                    v_out, s_out, p_out)
    torch.cuda.synchronize()
    plan.close()
    k_out, v_out, s_out, p_out = (t.cpu().numpy() for t in (k_out, v_out, s_out, p_out))
    for b in range(B):
        L = int(w.ctx_lens[b])
        g = oracle.gather_sequence(w.k_pages, w.v_pages, w.kv_scales, w.block_table[b], L, "int4")
        assert np.array_equal(k_out[b, :, :L], g.k_bytes)
        assert np.array_equal(v_out[b, :, :L], g.v_bytes)
        assert np.array_equal(s_out[0, b, :, :L], g.k_scale.astype(np.float32))
        assert np.array_equal(s_out[1, b, :, :L], g.v_scale.astype(np.float32))
        assert np.array_equal(p_out[b, :L], g.page_of_token)
        assert np.all(k_out[b, :, L:] == 0) and np.all(p_out[b, L:] == -1)


def _parity(w, rows=None, **over):
    log(f"int4 parity: {w.name} seed={w.seed} B={w.num_seqs} Hq={w.num_q_heads} Hkv={w.num_kv_heads} "
        f"q_lens={sorted(set(w.q_lens.tolist()))[:4]} ctx=[{w.ctx_lens.min()},{w.ctx_lens.max()}]")
    plan = plan_for(w, kv_format="int4", **over)
    got = run_gpu(w, plan=plan)
    plan.close()
    ref = oracle.paged_attention(w.q, w.k_pages, w.v_pages, w.kv_scales, w.block_table, w.ctx_lens, w.q_lens,
                                 num_kv_heads=w.num_kv_heads, sm_scale=w.sm_scale, kv_format="int4", rows=rows)
    if rows is not None:
        got, ref = got[rows], ref[rows]
    return check_contract(got, ref, w.out_dtype, what=f"int4 {w.name}")


REDUCED = {
    "llama3_8b_decode": dict(batch=5, ctx_range=(512, 1100)),
    "mtp_verify": dict(batch=9, ctx_range=(128, 400)),
    "long_ctx_split": dict(batch=2, ctx_range=(0, 4096), num_kv_splits=8),
    "prefill_chunk": dict(batch=3, ctx_range=(0, 300), q_len=96),
    "mqa_decode": dict(batch=6, ctx_range=(256, 2000)),
}


@pytest.mark.parametrize("name", sorted(REDUCED))
def test_int4_reduced(name):
    _parity(make_workload(name, kv_format="int4", **REDUCED[name]))


def test_int4_llama3_full():
    _parity(make_workload("llama3_8b_decode", kv_format="int4", keep_logical=False))


@pytest.mark.parametrize("name", ["mtp_verify", "mqa_decode", "long_ctx_split"])
def test_int4_full(name):
    w = make_workload(name, kv_format="int4", keep_logical=False)
    stats = _parity(w)
    assert stats["n"] == w.total_q * w.num_q_heads * w.head_dim


def test_int4_prefill_full_sampled_rows():
    # every sequence's first, page-edge and last new tokens, plus random rows
    w = make_workload("prefill_chunk", kv_format="int4", keep_logical=False)
    rng = np.random.default_rng(1)
    starts = np.concatenate([[0], np.cumsum(w.q_lens)[:-1]])
    rows = sorted(set(int(s + i) for s in starts for i in [0, 15, 16, 255, 511])
                  | set(rng.integers(0, w.total_q, 48).tolist()))
    _parity(w, rows=rows)


EDGE = [
    ([1, 1, 1], [16, 17, 15], 8, 2),
    ([1, 1], [31, 33], 8, 8),
    ([2, 1], [70, 9], 16, 2),  # single 16-column tile
    ([1, 3, 5, 2], [40, 3, 90, 2], 10, 2),  # at most 8 columns: low parts in spare columns
    ([33, 20], [33, 100], 4, 2),  # prefill from an empty cache, shared-KV tile
]


@pytest.mark.parametrize("idx", range(len(EDGE)))
def test_int4_edges(idx):
    ql, cl, hq, hkv = EDGE[idx]
    _parity(custom_workload(ql, cl, num_q_heads=hq, num_kv_heads=hkv, head_dim=128, seed=510 + idx,
                            kv_format="int4", name=f"int4_edge{idx}"))


def test_int4_forced_partitions():
    w = custom_workload([1, 1, 1], [1000, 37, 2048], num_q_heads=8, num_kv_heads=2, head_dim=128, seed=520,
                        num_kv_splits=7, kv_format="int4", name="int4_splits7")
    _parity(w)


def test_int4_garbage_does_not_leak():
    w = make_workload("mtp_verify", batch=6, ctx_range=(130, 500), kv_format="int4")
    log("int4 invariance: garbage codes in unused slots and pages")
    ref = run_gpu(w, plan=plan_for(w, kv_format="int4"))
    rng = np.random.default_rng(530)
    used = set(int(p) for p in w.block_table[w.block_table >= 0])
    for p in range(w.num_pages):
        if p not in used:
            w.k_pages[p] = rng.integers(0, 256, size=w.k_pages[p].shape, dtype=np.uint8)
            w.v_pages[p] = rng.integers(0, 256, size=w.v_pages[p].shape, dtype=np.uint8)
            w.kv_scales[:, p] = np.nan
    for b in range(w.num_seqs):
        L = int(w.ctx_lens[b])
        last = int(w.block_table[b][(L - 1) // 16])
        for s in range(L % 16 or 16, 16):
            # K codes of slot s: every byte of row s of each quarter
            w.k_pages[last, :, :, s, :] = rng.integers(0, 256, size=w.k_pages[last, :, :, s, :].shape,
                                                       dtype=np.uint8)
            # V code of slot s: nibble s % 2 of byte (s % 4) // 2 in group s // 4
            sub = w.v_pages[last, :, s // 4, :, :, (s % 4) // 2]
            keep = np.uint8(0xF0 if s % 2 == 0 else 0x0F)
            noise = rng.integers(0, 256, size=sub.shape, dtype=np.uint8) & np.uint8(~keep & 0xFF)
            w.v_pages[last, :, s // 4, :, :, (s % 4) // 2] = (sub & keep) | noise
    got = run_gpu(w, plan=plan_for(w, kv_format="int4"))
    assert np.array_equal(got, ref)


def test_int4_whole_segment_schedule():
    # every unit takes one (sequence, kv head) segment whole
    w = whole_schedule_workload(128, 300, 600, seed=960, kv_format="int4")
    plan = plan_for(w, kv_format="int4")
    info = plan.info()
    plan.close()
    assert takes_whole_schedule(w, info), info
    _parity(w)
