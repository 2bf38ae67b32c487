"""The forward captured in a HIP graph: every replay equals the eager result
(with eager work and synchronisations between replays).  Uses partitioned
workloads so the arrival counters must re-arm between forwards."""

import numpy as np
import pytest
import torch

from synth import custom_workload, make_workload
from tests.gpu_helpers import device_inputs, log, out_tensor, plan_for

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("case", ["decode_splits", "mqa_splits", "mtp"])
def test_graph_replays_match_eager(case):
    w = {
        "decode_splits": lambda: make_workload("llama3_8b_decode", batch=6, ctx_range=(512, 3000)),
        "mqa_splits": lambda: make_workload("mqa_decode", batch=5, ctx_range=(256, 5000)),
        "mtp": lambda: make_workload("mtp_verify", batch=7, ctx_range=(128, 600)),
    }[case]()
    log(f"graph: {case}")
    plan = plan_for(w)
    x = device_inputs(w)
    eager = out_tensor(w)
    plan.forward(x["q"], x["k_pages"], x["v_pages"], x["kv_scales"], x["block_table"], x["ctx_lens"],
                 x["q_lens"], eager)
    torch.cuda.synchronize()
    ref = eager.clone()

    out = out_tensor(w)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        g.capture_begin()
        for _ in range(3):  # three forwards per replay
            plan.forward(x["q"], x["k_pages"], x["v_pages"], x["kv_scales"], x["block_table"], x["ctx_lens"],
                         x["q_lens"], out, stream=s)
        g.capture_end()
    torch.cuda.current_stream().wait_stream(s)
    for r in range(4):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {r} differs"
        # eager forwards between replays
        plan.forward(x["q"], x["k_pages"], x["v_pages"], x["kv_scales"], x["block_table"], x["ctx_lens"],
                     x["q_lens"], eager)
        torch.cuda.synchronize()
        assert torch.equal(eager, ref)
    plan.close()


def test_graph_append_replays_match_eager():
    from synth.append import append_case

    c = append_case([1, 5, 40, 1], [300, 133, 90, 16], num_kv_heads=4, head_dim=128, new_dtype="bf16", seed=77,
                    new_sigmas=(0.5, 2.0))
    log("graph: append")
    plan = plan_for_append(c)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    k0, v0, s0 = t(c.k_pages), t(c.v_pages), t(c.kv_scales)
    kn, vn = c.k_new.cuda().contiguous(), c.v_new.cuda().contiguous()
    bt, cl, ql = t(c.block_table), t(c.ctx_lens), t(c.q_lens)
    k, v, s = k0.clone(), v0.clone(), s0.clone()
    plan.kv_append(kn, vn, k, v, s, bt, cl, ql)
    torch.cuda.synchronize()
    ref = (k.clone(), v.clone(), s.clone())

    k.copy_(k0), v.copy_(v0), s.copy_(s0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        g.capture_begin()
        plan.kv_append(kn, vn, k, v, s, bt, cl, ql, stream=st)
        g.capture_end()
    torch.cuda.current_stream().wait_stream(st)
    for r in range(4):
        k.copy_(k0), v.copy_(v0), s.copy_(s0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(k, ref[0]) and torch.equal(v, ref[1]), f"replay {r}: pools differ"
        assert torch.equal(s.view(torch.int32), ref[2].view(torch.int32)), f"replay {r}: scales differ"
    plan.close()


def plan_for_append(c):
    from paged_fp8_kv_attn_amd import Plan

    return Plan(num_seqs=c.num_seqs, num_q_heads=c.num_kv_heads, num_kv_heads=c.num_kv_heads, head_dim=c.head_dim,
                num_pages=c.num_pages, max_pages_per_seq=c.max_pages_per_seq, max_q_len=c.max_q_len,
                max_ctx_len=c.max_ctx_len)


def test_graph_accept_replays_match_eager():
    from paged_fp8_kv_attn_amd import mtp_accept, mtp_accept_workspace_size
    from synth.accept import accept_case

    c = accept_case(24, 4, 65536, dtype="bf16", seed=78)
    log("graph: accept")
    B, K, V = c.num_seqs, c.num_drafts, c.vocab
    logits = c.logits.cuda().contiguous()
    drafts = torch.from_numpy(c.drafts).cuda()
    ws = torch.empty(mtp_accept_workspace_size(B, K, V), dtype=torch.uint8, device="cuda")
    t_ref = torch.empty((B, K + 1), dtype=torch.int32, device="cuda")
    n_ref = torch.empty((B,), dtype=torch.int32, device="cuda")
    mtp_accept(logits, drafts, t_ref, n_ref, ws)
    torch.cuda.synchronize()
    t_out = torch.full_like(t_ref, -1)
    n_out = torch.full_like(n_ref, -1)
    g = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        g.capture_begin()
        mtp_accept(logits, drafts, t_out, n_out, ws, stream=st)
        g.capture_end()
    torch.cuda.current_stream().wait_stream(st)
    for r in range(4):
        t_out.fill_(-1)
        n_out.fill_(-1)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(t_out, t_ref) and torch.equal(n_out, n_ref), f"replay {r} differs"
        mtp_accept(logits, drafts, t_ref, n_ref, ws)  # eager work between replays
        torch.cuda.synchronize()
