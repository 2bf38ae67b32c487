"""The Python binding rejects tensors that do not fit the plan before any
library call: a CPU tensor, a wrong dtype, a non-contiguous view or a buffer
shorter than the descriptor implies never reaches a kernel as a device
pointer.  Runs without a GPU: the plan object is built around a descriptor
only, and the library entry points are replaced by a recorder that fails the
test if it is reached."""

import pytest
import torch

from paged_fp8_kv_attn_amd import _binding
from paged_fp8_kv_attn_amd._binding import Plan, PlanDesc

B, HQ, HKV, D, P, MPS, MAXQ, MAXL = 3, 8, 2, 128, 20, 4, 2, 64


class _NoLibrary:
    def __getattr__(self, name):
        raise AssertionError(f"library entry point {name} reached with tensors the binding should reject")


@pytest.fixture
def plan(monkeypatch):
    monkeypatch.setattr(_binding, "load_library", lambda: _NoLibrary())
    d = PlanDesc()
    d.num_seqs, d.num_q_heads, d.num_kv_heads, d.head_dim = B, HQ, HKV, D
    d.page_size, d.num_pages, d.max_pages_per_seq = 16, P, MPS
    d.max_q_len, d.max_ctx_len = MAXQ, MAXL
    d.q_dtype, d.out_dtype = _binding.ATTN_DTYPE_BF16, _binding.ATTN_DTYPE_BF16
    p = Plan.__new__(Plan)
    p.desc = d
    p._h = None
    # a plan made on the GPU; these tests hand it CPU tensors unless they
    # pretend the plan lives on the CPU to reach the later checks
    p.device = torch.device("cuda", 0)
    yield p
    p._h = None


def _inputs(rows=B, dev="cpu"):
    return dict(
        q=torch.zeros(rows, HQ, D, dtype=torch.bfloat16, device=dev),
        k_pages=torch.zeros(P * HKV * 16 * D, dtype=torch.uint8, device=dev),
        v_pages=torch.zeros(P * HKV * 16 * D, dtype=torch.uint8, device=dev),
        kv_scales=torch.ones(2, P, HKV, dtype=torch.float32, device=dev),
        block_table=torch.zeros(B, MPS, dtype=torch.int32, device=dev),
        ctx_lens=torch.full((B,), 16, dtype=torch.int32, device=dev),
        q_lens=torch.ones(B, dtype=torch.int32, device=dev),
        out=torch.zeros(rows, HQ, D, dtype=torch.bfloat16, device=dev),
    )


def _call(plan, x):
    plan.forward(x["q"], x["k_pages"], x["v_pages"], x["kv_scales"], x["block_table"], x["ctx_lens"],
                 x["q_lens"], x["out"])


def test_cpu_tensor_rejected(plan):
    with pytest.raises(ValueError, match="on cuda:0"):
        _call(plan, _inputs())


@pytest.mark.parametrize("name,bad,match", [
    ("q", lambda x: x["q"].to(torch.float16), "dtype"),
    ("q", lambda x: x["q"].float(), "dtype"),           # an fp32 q given to a bf16 plan
    ("out", lambda x: x["out"].float(), "dtype"),
    ("k_pages", lambda x: x["k_pages"].to(torch.int8), "dtype"),
    ("kv_scales", lambda x: x["kv_scales"].double(), "dtype"),
    ("block_table", lambda x: x["block_table"].long(), "dtype"),
    ("ctx_lens", lambda x: x["ctx_lens"].long(), "dtype"),
    ("out", lambda x: x["out"][:-1], "elements"),        # a short out
    ("out", lambda x: torch.zeros(B + 1, HQ, D, dtype=torch.bfloat16), "elements"),
    ("q", lambda x: x["q"][:, :, : D // 2], "contiguous"),
    ("block_table", lambda x: x["block_table"][:, :2].contiguous(), "at least"),  # shorter than B * stride
    ("k_pages", lambda x: x["k_pages"][:-1], "at least"),
    ("kv_scales", lambda x: x["kv_scales"][0].contiguous(), "at least"),        # only the K scales
    ("q_lens", lambda x: x["q_lens"][:1], "at least"),
])
def test_bad_tensor_rejected(plan, name, bad, match):
    plan.device = torch.device("cpu")  # reach the checks after the device one
    x = _inputs()
    x[name] = bad(x)
    with pytest.raises(ValueError, match=match):
        _call(plan, x)


def test_rows_bounded_by_max_q_len(plan):
    plan.device = torch.device("cpu")
    with pytest.raises(ValueError, match="rows"):
        _call(plan, _inputs(rows=B * MAXQ + 1))
    with pytest.raises(ValueError, match="at least"):
        _call(plan, _inputs(rows=B - 1))


def test_good_tensors_reach_the_library(plan):
    plan.device = torch.device("cpu")
    with pytest.raises(AssertionError, match="attn_paged_forward"):
        _call(plan, _inputs(rows=B * MAXQ))


def test_append_guards(plan):
    plan.device = torch.device("cpu")
    x = _inputs()
    kn = torch.zeros(B, HKV, D, dtype=torch.bfloat16)
    args = (x["k_pages"], x["v_pages"], x["kv_scales"], x["block_table"], x["ctx_lens"], x["q_lens"])
    with pytest.raises(ValueError, match="dtype"):
        plan.kv_append(kn, kn.float(), *args)
    with pytest.raises(ValueError, match="dtype"):
        plan.kv_append(kn.half(), kn.half(), *args)
    with pytest.raises(ValueError, match="elements"):
        plan.kv_append(kn, kn[:-1], *args)
    plan.device = torch.device("cuda", 0)
    with pytest.raises(ValueError, match="on cuda:0"):
        plan.kv_append(kn, kn, *args)


def test_accept_and_codec_guards(monkeypatch):
    monkeypatch.setattr(_binding, "load_library", lambda: _NoLibrary())
    monkeypatch.setattr(_binding, "mtp_accept_workspace_size", lambda b, k, v: 64)
    logits = torch.zeros(2, 5, 64, dtype=torch.bfloat16)
    i32 = lambda *s: torch.zeros(*s, dtype=torch.int32)  # noqa: E731
    with pytest.raises(ValueError, match="GPU tensor"):
        _binding.mtp_accept(logits, i32(2, 4), i32(2, 5), i32(2), torch.zeros(64, dtype=torch.uint8))
    with pytest.raises(ValueError, match="GPU tensor"):
        _binding.debug_decode_fp8(torch.zeros(8, dtype=torch.uint8), torch.zeros(8))
    with pytest.raises(ValueError, match="GPU tensor"):
        _binding.calib_stream_read(torch.zeros(4096, dtype=torch.uint8), i32(1), 1024, 1, i32(64))
