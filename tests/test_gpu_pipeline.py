"""The steps chained on the GPU as a verification step runs them: the new
tokens' K/V are appended to the paged pool, then the new tokens attend over
the updated pages; the output must meet the accuracy contract against the
oracle's append followed by the oracle's attention (E4M3 and INT8 pools)."""

import numpy as np
import pytest
import torch

import oracle
import oracle.kv_append as ka
from paged_fp8_kv_attn_amd import Plan
from synth.append import append_case
from tests.gpu_helpers import check_contract, log

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kv_format", ["e4m3", "int8"])
def test_append_then_verify(kv_format):
    q_len, hq, hkv, d = 5, 40, 8, 128
    c = append_case([q_len] * 6, [133, 700, 16, 301, 5, 1024], num_kv_heads=hkv, head_dim=d, new_dtype="bf16",
                    seed=500, new_sigmas=(0.5, 2.0), kv_format=kv_format, name=f"pipeline_{kv_format}")
    log(f"pipeline: {c.name} B={c.num_seqs} ctx={c.ctx_lens.tolist()}")
    rng = np.random.default_rng(501)
    q = torch.from_numpy(rng.standard_normal((c.total_q, hq, d), dtype=np.float32)).to(torch.bfloat16)
    dev = "cuda"
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731
    k, v, s = t(c.k_pages), t(c.v_pages), t(c.kv_scales)
    bt, cl, ql = t(c.block_table), t(c.ctx_lens), t(c.q_lens)
    plan = Plan(num_seqs=c.num_seqs, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, num_pages=c.num_pages,
                max_pages_per_seq=c.max_pages_per_seq, max_q_len=c.max_q_len, max_ctx_len=c.max_ctx_len,
                kv_format=kv_format)
    plan.kv_append(c.k_new.to(dev).contiguous(), c.v_new.to(dev).contiguous(), k, v, s, bt, cl, ql)
    out = torch.full((c.total_q, hq, d), float("nan"), dtype=torch.bfloat16, device=dev)
    plan.forward(q.to(dev), k, v, s, bt, cl, ql, out)
    torch.cuda.synchronize()
    plan.close()

    k2, v2, s2 = ka.kv_append(c.k_new, c.v_new, c.k_pages, c.v_pages, c.kv_scales, c.block_table, c.ctx_lens,
                              c.q_lens, kv_format=kv_format)
    assert np.array_equal(k.cpu().numpy(), k2) and np.array_equal(v.cpu().numpy(), v2)
    ref = oracle.paged_attention(q, k2, v2, s2, c.block_table, c.ctx_lens, c.q_lens, num_kv_heads=hkv,
                                 kv_format=kv_format)
    check_contract(out.double().cpu().numpy(), ref, "bf16", what=c.name)
