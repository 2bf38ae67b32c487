"""Seeded inputs for greedy MTP acceptance (input generation only): target
logits for the K + 1 positions of each sequence and its K draft tokens.

Recipe: numpy ``default_rng(seed)``; logits ~ N(0, 1) in fp32; each row
gets a planted token p whose logit is set to 6 + |N(0,1)| (far above the
rest on N(0,1) rows, without the generator computing an argmax); a quarter
of the rows also get a second planted token carrying exactly the same
value (a tie) and a few rows a planted +0 / -0 pair as their only
non-negative entries; the rows are rounded to nearest-even into the logits
dtype.  Draft j of a sequence is the planted token of row j with
probability p_match, else a uniformly drawn token.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch


@dataclass
class AcceptCase:
    name: str
    logits: torch.Tensor  # [B][K+1][V] bf16 or fp32 (CPU)
    drafts: np.ndarray  # int32 [B][K]
    seed: int = 0

    @property
    def num_seqs(self) -> int:
        return int(self.drafts.shape[0])

    @property
    def num_drafts(self) -> int:
        return int(self.drafts.shape[1])

    @property
    def vocab(self) -> int:
        return int(self.logits.shape[2])


def accept_case(batch: int, num_drafts: int, vocab: int, *, dtype="bf16", seed=0, p_match=0.8,
                name="accept") -> AcceptCase:
    rng = np.random.default_rng(seed)
    B, K, V = batch, num_drafts, vocab
    x = rng.standard_normal((B, K + 1, V), dtype=np.float32)
    planted = rng.integers(0, V, size=(B, K + 1))
    top = (6.0 + np.abs(rng.standard_normal((B, K + 1)))).astype(np.float32)
    tie = rng.random((B, K + 1)) < 0.25
    other = rng.integers(0, V, size=(B, K + 1))
    zeros = rng.random((B, K + 1)) < 0.02
    for b in range(B):
        for i in range(K + 1):
            if zeros[b, i]:
                row = x[b, i]
                np.negative(np.abs(row), out=row)
                row[row == 0] = -1.0
                row[planted[b, i]] = -0.0
                row[other[b, i]] = 0.0
                continue
            x[b, i, planted[b, i]] = top[b, i]
            if tie[b, i]:
                x[b, i, other[b, i]] = top[b, i]
    if dtype == "bf16":
        logits = torch.from_numpy(x).to(torch.bfloat16)
    elif dtype == "f32":
        logits = torch.from_numpy(x)
    else:
        raise ValueError(dtype)
    match = rng.random((B, K)) < p_match
    rand_tok = rng.integers(0, V, size=(B, K))
    drafts = np.where(match, planted[:, :K], rand_tok).astype(np.int32)
    return AcceptCase(name=name, logits=logits, drafts=drafts, seed=seed)


# The acceptance step of the MTP verification batch: 128 sequences, K = 4
# drafts, a 151936-token vocabulary (the Qwen3 family served on the GB10).
ACCEPT_CONFIGS = {"mtp_accept": dict(batch=128, num_drafts=4, vocab=151936, seed=13)}


def make_accept_case(name: str = "mtp_accept", *, batch=None, vocab=None, dtype="bf16") -> AcceptCase:
    c = dict(ACCEPT_CONFIGS[name])
    return accept_case(batch or c["batch"], c["num_drafts"], vocab or c["vocab"], dtype=dtype, seed=c["seed"],
                       name=name)
