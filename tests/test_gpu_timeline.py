"""The per-wave timeline hook (attn_plan_set_timeline): recording changes no
output bit, every wave that ran leaves a well-formed row (start, range
known, pieces of start / chunk steps / end, wave end, times in order), and
the chunk steps of the tile kernels' first waves add up to the schedule's
chunks."""

import numpy as np
import pytest
import torch

from paged_fp8_kv_attn_amd import TIMELINE_WORDS
from synth import custom_workload, make_workload
from tests.gpu_helpers import device_inputs, log, out_tensor, plan_for

pytestmark = pytest.mark.gpu

CASES = {
    # packed decode: one wave per unit, a step per group of chunks
    "decode": lambda: make_workload("llama3_8b_decode", batch=5, ctx_range=(512, 1100)),
    # shared-KV tile kernel, balanced split (MQA decode, 64 columns)
    "mqa": lambda: make_workload("mqa_decode", batch=6, ctx_range=(256, 2000)),
    # shared-KV tile kernel, one segment per unit
    "mtp_whole": lambda: custom_workload([5] * 128, np.random.default_rng(970).integers(300, 601, 128).tolist(),
                                         num_q_heads=40, num_kv_heads=8, head_dim=128, seed=970),
}


def _forward(plan, w, x, rows=None):
    out = out_tensor(w)
    if rows is not None:
        rows.zero_()
    plan.set_timeline(rows)
    plan.forward(x["q"], x["k_pages"], x["v_pages"], x["kv_scales"], x["block_table"], x["ctx_lens"],
                 x["q_lens"], out)
    plan.set_timeline(None)
    torch.cuda.synchronize()
    return out.cpu()


@pytest.mark.parametrize("case", sorted(CASES))
def test_timeline_rows(case):
    w = CASES[case]()
    log(f"timeline: {case} B={w.num_seqs} Hq={w.num_q_heads} Hkv={w.num_kv_heads}")
    x = device_inputs(w)
    plan = plan_for(w)
    info = plan.info()
    nrows = info["grid_size"] * info["waves_per_group"]
    rows = torch.zeros(nrows * TIMELINE_WORDS, dtype=torch.int64, device="cuda")
    ref = _forward(plan, w, x)
    got = _forward(plan, w, x, rows)
    with pytest.raises(ValueError):
        plan.set_timeline(torch.zeros(nrows * TIMELINE_WORDS - 1, dtype=torch.int64, device="cuda"))
    plan.close()
    assert torch.equal(ref.view(torch.int16) if ref.dtype == torch.bfloat16 else ref,
                       got.view(torch.int16) if got.dtype == torch.bfloat16 else got)
    assert info["wallclock_khz"] > 0

    a = rows.view(nrows, TIMELINE_WORDS).cpu().numpy().view(np.uint64)
    typ = (a & np.uint64(15)).astype(np.int64)
    tim = (a >> np.uint64(4)).astype(np.int64)
    ran = typ[:, 0] == 1
    assert ran.any()
    steps_first_waves = 0
    for r in np.nonzero(ran)[0]:
        assert typ[r, -1] == 7, (case, r)
        ev = [(int(typ[r, i]), int(tim[r, i])) for i in range(TIMELINE_WORDS - 1) if typ[r, i] != 0]
        types = [t for t, _ in ev]
        times = [t for _, t in ev] + [int(tim[r, -1])]
        assert all(b >= a_ for a_, b in zip(times, times[1:])), (case, r)
        assert types[:3] == [1, 6, 2], (case, r, types[:4])
        # pieces: 3, then 4s, then 5, repeated (the row may end early when full)
        state = 5
        for t in types[3:]:
            if t == 3:
                assert state == 5
            elif t == 4:
                assert state in (3, 4)
            else:
                assert t == 5 and state in (3, 4)
            state = t
        if len(types) < TIMELINE_WORDS - 1:
            assert state == 5 or len(types) == 3, (case, r)
        if not info["packed"] and r % info["waves_per_group"] == 0:
            steps_first_waves += types.count(4)
    if not info["packed"]:
        # every chunk of every segment is stepped once by each wave of the workgroup holding it
        G = w.num_q_heads // w.num_kv_heads
        cpb = info["cols_per_block"]
        total = 0
        for L, Q in zip(w.ctx_lens.tolist(), w.q_lens.tolist()):
            for cb in range(info["col_blocks"]):
                col0 = cb * cpb
                if col0 >= G * Q:
                    continue
                i_hi = (min(col0 + cpb, G * Q) - 1) // G
                total += w.num_kv_heads * -(-(L - Q + i_hi + 1) // 32)
        assert steps_first_waves == total, (case, steps_first_waves, total)
