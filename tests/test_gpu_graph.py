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
