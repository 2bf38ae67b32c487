"""Greedy acceptance of multi-token-prediction drafts -- TEST
INFRASTRUCTURE ONLY.

What it follows: the GB10 article (ainews.surl.tw) serves with
multi-token prediction, K = 4 draft tokens, under deterministic decoding.
After the verification attention the target model scores the K + 1
positions (the last accepted token and the K drafts); with deterministic
(greedy) decoding the target's token at position i is the argmax of its
logits row, and the drafts are accepted while they equal those tokens.

Readings where the pages are silent (listed in the design notes):
  * greedy: target token t_i = the lowest index holding the largest logit
    of row i (+0 and -0 compare equal; logits are finite);
  * accepted count n = the length of the longest prefix with
    draft[j] == t_j for every j < n (0 <= n <= K); the tokens emitted are
    t_0 .. t_n (the accepted drafts, then the target's own token).
"""

from __future__ import annotations

import numpy as np


def greedy_tokens(logits) -> np.ndarray:
    """[..., V] logits (any real dtype, read exactly) -> int64 [...] argmax,
    first occurrence of the maximum."""
    if hasattr(logits, "detach"):
        logits = logits.detach().to("cpu").double().numpy()
    x = np.asarray(logits, dtype=np.float64)
    return np.argmax(x, axis=-1)


def accept(logits, drafts):
    """logits [B][K+1][V], drafts [B][K] -> (targets int32 [B][K+1],
    accepted int32 [B])."""
    t = greedy_tokens(logits)
    drafts = np.asarray(drafts)
    B, K = drafts.shape
    n = np.zeros(B, dtype=np.int32)
    for b in range(B):
        while n[b] < K and int(drafts[b, n[b]]) == int(t[b, n[b]]):
            n[b] += 1
    return t.astype(np.int32), n
