"""GPU checks of the shared device helpers, bit for bit: the FP8 and INT8
decodes over all 256 codes and the block-table gather (bytes, scales, page
ids)."""

import numpy as np
import pytest
import torch

import oracle
import oracle.attention as oracle_attention
import paged_fp8_kv_attn_amd as pa
from synth import custom_workload, make_workload
from tests.gpu_helpers import device_inputs, log, plan_for

pytestmark = pytest.mark.gpu


def test_decode_all_codes_bit_exact():
    log("decode: 256 codes x 3 (contiguous, ragged length)")
    codes = torch.arange(256, dtype=torch.uint8).repeat(3)
    for n in (768, 767, 5):
        c = codes[:n].cuda()
        out = torch.empty(n, dtype=torch.float32, device="cuda")
        pa.debug_decode_fp8(c, out)
        torch.cuda.synchronize()
        got = out.double().cpu().numpy()
        ref = oracle.decode(codes[:n].numpy())
        nan = np.isnan(ref)
        assert np.array_equal(np.isnan(got), nan)
        assert np.array_equal(got[~nan], ref[~nan])
        assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_int8_decode_all_codes_bit_exact():
    log("int8 decode: 256 codes x 3 (contiguous, ragged length)")
    codes = torch.arange(256, dtype=torch.uint8).repeat(3)
    for n in (768, 767, 5):
        c = codes[:n].cuda()
        out = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
        pa.debug_decode_int8(c, out)
        torch.cuda.synchronize()
        got = out.double().cpu().numpy()
        ref = oracle_attention.decode_int8(codes[:n].numpy())
        assert np.array_equal(got, ref)
        assert not np.any(np.signbit(got[ref == 0]))  # code 0 widens to +0


@pytest.mark.parametrize("case", ["tiny", "ragged", "llama_reduced", "d64_mqa"])
def test_gather_bit_exact(case):
    w = {
        "tiny": lambda: make_workload("tiny_decode"),
        "ragged": lambda: custom_workload([1, 3, 1], [1, 33, 47], num_q_heads=8, num_kv_heads=4, head_dim=128,
                                          seed=5, max_ctx_len=64),
        "llama_reduced": lambda: make_workload("llama3_8b_decode", batch=3, ctx_range=(512, 700)),
        "d64_mqa": lambda: custom_workload([1, 1], [100, 17], num_q_heads=16, num_kv_heads=1, head_dim=64, seed=6),
    }[case]()
    log(f"gather: {case} B={w.num_seqs} Hkv={w.num_kv_heads} D={w.head_dim} max_ctx={w.max_ctx_len}")
    x = device_inputs(w)
    plan = plan_for(w)
    B, H, T, D = w.num_seqs, w.num_kv_heads, w.max_ctx_len, w.head_dim
    k_out = torch.full((B, H, T, D), 0xAA, dtype=torch.uint8, device="cuda")
    v_out = torch.full((B, H, T, D), 0xAA, dtype=torch.uint8, device="cuda")
    s_out = torch.full((2, B, H, T), -7.0, dtype=torch.float32, device="cuda")
    p_out = torch.full((B, T), -7, dtype=torch.int32, device="cuda")
    pa.debug_gather(plan, x["k_pages"], x["v_pages"], x["kv_scales"], x["block_table"], x["ctx_lens"], k_out,
                    v_out, s_out, p_out)
    torch.cuda.synchronize()
    k_out, v_out, s_out, p_out = (t.cpu().numpy() for t in (k_out, v_out, s_out, p_out))
    for b in range(B):
        L = int(w.ctx_lens[b])
        g = oracle.gather_sequence(w.k_pages, w.v_pages, w.kv_scales, w.block_table[b], L)
        assert np.array_equal(k_out[b, :, :L], g.k_bytes)
        assert np.array_equal(v_out[b, :, :L], g.v_bytes)
        assert np.array_equal(s_out[0, b, :, :L], g.k_scale.astype(np.float32))
        assert np.array_equal(s_out[1, b, :, :L], g.v_scale.astype(np.float32))
        assert np.array_equal(p_out[b, :L], g.page_of_token)
        assert np.all(k_out[b, :, L:] == 0) and np.all(v_out[b, :, L:] == 0) and np.all(p_out[b, L:] == -1)
    plan.close()
