"""GPU parity of greedy MTP acceptance (attn_mtp_accept) with the oracle,
through the C ABI: every target token and accepted count must be equal."""

import numpy as np
import pytest
import torch

import oracle.mtp_accept as ma
from paged_fp8_kv_attn_amd import mtp_accept, mtp_accept_workspace_size
from synth.accept import accept_case, make_accept_case
from tests.gpu_helpers import log

pytestmark = pytest.mark.gpu


def _parity(c):
    B, K, V = c.num_seqs, c.num_drafts, c.vocab
    log(f"accept: {c.name} seed={c.seed} B={B} K={K} V={V} dtype={c.logits.dtype}")
    dev = "cuda"
    logits = c.logits.to(dev).contiguous()
    drafts = torch.from_numpy(np.ascontiguousarray(c.drafts)).to(dev)
    targets = torch.full((B, K + 1), -7, dtype=torch.int32, device=dev)
    n = torch.full((B,), -7, dtype=torch.int32, device=dev)
    ws = torch.empty(mtp_accept_workspace_size(B, K, V), dtype=torch.uint8, device=dev)
    mtp_accept(logits, drafts, targets, n, ws)
    torch.cuda.synchronize()
    want_t, want_n = ma.accept(c.logits, c.drafts)
    got_t, got_n = targets.cpu().numpy(), n.cpu().numpy()
    assert np.array_equal(got_t, want_t), f"{c.name}: {int((got_t != want_t).sum())} target tokens differ"
    assert np.array_equal(got_n, want_n), f"{c.name}: accepted counts differ"
    log(f"  accepted histogram {np.bincount(got_n, minlength=K + 1).tolist()}")


CASES = [
    # (B, K, V, dtype, seed)
    (1, 4, 8, "bf16", 1),
    (3, 4, 64, "f32", 2),
    (7, 1, 1000, "bf16", 3),
    (5, 0, 4096, "bf16", 4),  # no drafts: one target token, nothing to accept
    (33, 4, 40000, "f32", 5),
    (64, 4, 131072, "bf16", 6),  # several segments per row
    (2, 4, 151936 * 2, "bf16", 7),
]


@pytest.mark.parametrize("idx", range(len(CASES)))
def test_accept_cases(idx):
    B, K, V, dt, seed = CASES[idx]
    _parity(accept_case(B, K, V, dtype=dt, seed=seed, name=f"accept_edge{idx}"))


def test_accept_all_equal_logits():
    # every logit equal: token 0 everywhere
    c = accept_case(4, 4, 512, dtype="bf16", seed=8, name="accept_flat")
    c.logits.fill_(0.5)
    c.drafts[:] = 0
    c.drafts[1, 2] = 3
    _parity(c)


def test_mtp_accept_full():
    _parity(make_accept_case("mtp_accept"))
