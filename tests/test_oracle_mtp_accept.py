"""Pins of the greedy MTP acceptance oracle (oracle/mtp_accept.py), CPU only:
pure-Python loops, torch's argmax, the planted structure of the inputs
(largest logit at a known token, exact ties, +0/-0 rows), closed forms, and
planted mistakes that must each fail a pin."""

import numpy as np
import pytest
import torch

import oracle.mtp_accept as ma
from synth.accept import accept_case


def _brute(logits, drafts):
    x = logits.double().numpy()
    B, K1, V = x.shape
    t = np.zeros((B, K1), dtype=np.int64)
    for b in range(B):
        for i in range(K1):
            best = 0
            for v in range(1, V):
                if x[b, i, v] > x[b, i, best]:
                    best = v
            t[b, i] = best
    n = np.zeros(B, dtype=np.int64)
    for b in range(B):
        k = 0
        for j in range(K1 - 1):
            if drafts[b, j] != t[b, j]:
                break
            k += 1
        n[b] = k
    return t, n


CASES = [(3, 4, 50, "f32", 1), (5, 4, 64, "bf16", 2), (4, 2, 7, "bf16", 3), (6, 4, 300, "f32", 4)]


@pytest.mark.parametrize("idx", range(len(CASES)))
def test_brute_force(idx):
    B, K, V, dt, seed = CASES[idx]
    c = accept_case(B, K, V, dtype=dt, seed=seed, p_match=0.7)
    t, n = ma.accept(c.logits, c.drafts)
    bt, bn = _brute(c.logits, c.drafts)
    assert np.array_equal(t, bt) and np.array_equal(n, bn)


def test_torch_argmax():
    c = accept_case(8, 4, 5000, dtype="bf16", seed=5)
    assert np.array_equal(ma.greedy_tokens(c.logits), torch.argmax(c.logits.float(), dim=-1).numpy())


def test_planted_structure():
    # rebuild the generator's planted tokens from its seed order: compare the
    # oracle with what was planted, row by row
    B, K, V, seed = 16, 4, 1000, 9
    c = accept_case(B, K, V, dtype="bf16", seed=seed)
    rng = np.random.default_rng(seed)
    rng.standard_normal((B, K + 1, V), dtype=np.float32)
    planted = rng.integers(0, V, size=(B, K + 1))
    rng.standard_normal((B, K + 1))
    tie = rng.random((B, K + 1)) < 0.25
    other = rng.integers(0, V, size=(B, K + 1))
    zeros = rng.random((B, K + 1)) < 0.02
    t = ma.greedy_tokens(c.logits)
    for b in range(B):
        for i in range(K + 1):
            if zeros[b, i] or tie[b, i]:
                assert t[b, i] == min(planted[b, i], other[b, i])
            else:
                assert t[b, i] == planted[b, i]


def test_closed_forms():
    c = accept_case(6, 4, 200, dtype="f32", seed=11)
    t = ma.greedy_tokens(c.logits)
    all_match = t[:, :4].astype(np.int32)
    _, n = ma.accept(c.logits, all_match)
    assert np.all(n == 4)
    first_wrong = all_match.copy()
    first_wrong[:, 0] = (first_wrong[:, 0] + 1) % 200
    _, n = ma.accept(c.logits, first_wrong)
    assert np.all(n == 0)
    third_wrong = all_match.copy()
    third_wrong[:, 2] = (third_wrong[:, 2] + 1) % 200
    third_wrong[:, 3] = (third_wrong[:, 3] + 1) % 200  # later mismatches do not matter
    _, n = ma.accept(c.logits, third_wrong)
    assert np.all(n == 2)


def test_signed_zero_tie():
    x = torch.tensor([[[-1.0, -0.0, 0.0, -2.0], [-3.0, 0.0, -0.0, -0.5]]])
    t = ma.greedy_tokens(x)
    assert t.tolist() == [[1, 1]]


def _all_pins():
    for idx in range(len(CASES)):
        test_brute_force(idx)
    test_torch_argmax()
    test_planted_structure()
    test_closed_forms()
    test_signed_zero_tie()


def _last_occurrence(logits):
    x = logits.detach().double().numpy() if hasattr(logits, "detach") else np.asarray(logits, np.float64)
    return x.shape[-1] - 1 - np.argmax(x[..., ::-1], axis=-1)


def _zero_sign_ordered(logits):
    x = logits.detach().double().numpy() if hasattr(logits, "detach") else np.asarray(logits, np.float64)
    x = np.where((x == 0) & np.signbit(x), -1e-300, x)
    return np.argmax(x, axis=-1)


def _accept_all_matches(logits, drafts):
    t = ma.greedy_tokens(logits)
    return t.astype(np.int32), (np.asarray(drafts) == t[:, :-1]).sum(axis=1).astype(np.int32)


def _accept_one_more(logits, drafts):
    t, n = _ORIG_ACCEPT(logits, drafts)
    return t, np.minimum(n + 1, np.asarray(drafts).shape[1]).astype(np.int32)


_ORIG_ACCEPT = ma.accept

PLANTED = {
    "argmax_last_occurrence": ("greedy_tokens", _last_occurrence),
    "minus_zero_below_plus_zero": ("greedy_tokens", _zero_sign_ordered),
    "count_every_match": ("accept", _accept_all_matches),
    "accept_one_more": ("accept", _accept_one_more),
}


@pytest.mark.parametrize("name", sorted(PLANTED))
def test_planted_mistake_fails_a_pin(name, monkeypatch):
    attr, fn = PLANTED[name]
    monkeypatch.setattr(ma, attr, fn)
    with pytest.raises(AssertionError):
        _all_pins()
