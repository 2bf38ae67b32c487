"""attn_paged_forward_static, the allocation-free forward: through the C ABI it
gives the same bits as attn_paged_forward with a plan made from the same
descriptor, and both meet the accuracy contract against the fp64 oracle, on
two calls in a row whose second input is smaller (the per-GPU scratch array
keeps the first call's contents).  Shapes too large for the array are
refused before any launch."""

import ctypes

import numpy as np
import pytest
import torch

from paged_fp8_kv_attn_amd import AttnError, forward_static, make_desc, static_scratch_bytes
from paged_fp8_kv_attn_amd import _binding
from synth import make_workload
from tests.gpu_helpers import check_contract, device_inputs, log, out_tensor, plan_for, run_oracle

pytestmark = pytest.mark.gpu


def _desc(w, **over):
    return make_desc(num_seqs=w.num_seqs, num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads,
                     head_dim=w.head_dim, num_pages=w.num_pages, max_pages_per_seq=w.max_pages_per_seq,
                     max_q_len=w.max_q_len, max_ctx_len=w.max_ctx_len, q_dtype=w.q_dtype, out_dtype=w.out_dtype,
                     sm_scale=w.sm_scale, num_kv_splits=w.num_kv_splits, **over)


def _both(w, **over):
    """The static forward's output and the plan forward's output."""
    x = device_inputs(w)
    args = (x["q"], x["k_pages"], x["v_pages"], x["kv_scales"], x["block_table"], x["ctx_lens"], x["q_lens"])
    out_s = out_tensor(w)
    forward_static(_desc(w, **over), *args, out_s)
    torch.cuda.synchronize()
    plan = plan_for(w, **over)
    info = plan.info()
    out_p = out_tensor(w)
    plan.forward(*args, out_p)
    torch.cuda.synchronize()
    plan.close()
    return out_s.double().cpu().numpy(), out_p.double().cpu().numpy(), info


# (first call, second call with a smaller input): every pair splits its
# segments, so the partials go through the scratch array
CASES = {
    "decode": (dict(name="llama3_8b_decode", batch=16, ctx_range=(512, 2048)),
               dict(name="llama3_8b_decode", batch=5, ctx_range=(300, 900))),
    "mtp": (dict(name="mtp_verify", batch=24, ctx_range=(128, 700)),
            dict(name="mtp_verify", batch=6, ctx_range=(128, 300))),
    "mqa": (dict(name="mqa_decode", batch=8, ctx_range=(256, 4096)),
            dict(name="mqa_decode", batch=3, ctx_range=(256, 1024))),
    "split": (dict(name="long_ctx_split", batch=2, ctx_range=(0, 4096)),
              dict(name="long_ctx_split", batch=1, ctx_range=(0, 2048))),
    # fixed pieces of 256 keys (batch-invariant split)
    "pieces": (dict(name="mqa_decode", batch=8, ctx_range=(256, 4096), kv_piece_len=256),
               dict(name="llama3_8b_decode", batch=5, ctx_range=(300, 900), kv_piece_len=256)),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_static_forward_matches_plan_forward(case):
    for i, spec in enumerate(CASES[case]):
        spec = dict(spec)
        over = {"kv_piece_len": spec.pop("kv_piece_len")} if "kv_piece_len" in spec else {}
        w = make_workload(spec.pop("name"), **spec)
        log(f"no-alloc: {case} call {i} B={w.num_seqs} ctx={int(w.ctx_lens.min())}..{int(w.ctx_lens.max())} {over}")
        got_s, got_p, info = _both(w, **over)
        assert info["workspace_bytes"] <= static_scratch_bytes()
        assert info["merge_grid_size"] > 0, "the case should split keys (and use the scratch partials)"
        assert np.array_equal(got_s, got_p, equal_nan=True), f"{case} call {i}: static forward differs"
        check_contract(got_s, run_oracle(w), w.out_dtype, what=f"no-alloc {case} call {i}")


def test_static_forward_refuses_oversized_workspace():
    # the 8 x 512-token prefill chunk (32 query / 8 kv heads) needs ~100 MB of partials
    d = make_desc(num_seqs=8, num_q_heads=32, num_kv_heads=8, head_dim=128, num_pages=5000,
                  max_pages_per_seq=544, max_q_len=512, max_ctx_len=8704)
    buf = torch.zeros(1 << 16, dtype=torch.uint8, device="cuda")
    p = ctypes.c_void_p(buf.data_ptr())
    lib = _binding.load_library()
    log("no-alloc: oversized descriptor")
    st = lib.attn_paged_forward_static(ctypes.byref(d), p, p, p, p, p, p, p, p,
                                       ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert st == 2, AttnError(st, "attn_paged_forward_static")
