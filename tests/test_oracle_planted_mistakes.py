"""Each plausible mistake planted in the oracle (on the CPU) must make at
least one pin fail; the unmodified oracle passes them all."""

import numpy as np
import pytest

import oracle.e4m3 as e4m3_mod
import oracle.attention as pa
from tests import oracle_pins as pins


def _all_pins_pass():
    for pin in pins.ALL_TABLE_PINS + pins.ALL_ATTENTION_PINS:
        try:
            pin()
        except AssertionError:
            return False, pin.__name__
    return True, None


def _wrong_table(bias):
    vals = []
    for x in range(256):
        s = -1.0 if x >> 7 else 1.0
        e, m = (x >> 3) & 15, x & 7
        if e == 15 and m == 7:
            vals.append(np.nan)
        elif e == 0:
            vals.append(s * m * 2.0 ** (1 - bias - 3))
        else:
            vals.append(s * (1 + m / 8) * 2.0 ** (e - bias))
    return np.array(vals)


MUTATIONS = {
    "gqa_head_modulo": ("kv_head_of", lambda hq, nq, nkv: hq % nkv),
    "causal_off_by_one_low": ("last_visible_key", lambda L, Q, i: L - Q + i - 1),
    "causal_off_by_one_high": ("last_visible_key", lambda L, Q, i: min(L - Q + i + 1, L - 1)),
    "no_causal_mask": ("last_visible_key", lambda L, Q, i: L - 1),
    "slot_shift": ("token_location", lambda row, t, S: (row[t // S], (t + 1) % S)),
    # V read as if it had K's layout
    "v_read_with_k_layout": ("v_token_bytes",
                             lambda v, pages, h, slots: v.reshape(v.shape[0], v.shape[1], -1, 16, 16)
                             [pages, h, :, slots, :].reshape(len(slots), -1)),
    # the two slot digits of the 4-slot interleave exchanged
    "v_interleave_swapped": ("v_token_bytes",
                             lambda v, pages, h, slots: v[pages, h, slots % 4, :, :, :, slots // 4]
                             .transpose(0, 2, 1, 3).reshape(len(slots), -1)),
    # d taken in (i, a, e) order instead of (a, i, e)
    "v_d_order_wrong": ("v_token_bytes",
                        lambda v, pages, h, slots: v[pages, h, slots // 4, :, :, :, slots % 4].reshape(len(slots), -1)),
    "k_d_reversed": ("k_token_bytes",
                     lambda k, pages, h, slots: k[pages, h, :, slots, :].reshape(len(slots), -1)[:, ::-1]),
    # K read token-major, as [S][D] inside a (page, head)
    "k_token_major": ("k_token_bytes",
                      lambda k, pages, h, slots: k.reshape(k.shape[0], k.shape[1], 16, -1)[pages, h, slots, :]),
    "scale_1_over_d": ("softmax_scale", lambda d, s: 1.0 / d if not s else s),
}


def test_unmodified_oracle_passes_every_pin():
    ok, which = _all_pins_pass()
    assert ok, which


@pytest.mark.filterwarnings("ignore::RuntimeWarning")
@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_attention_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(pa, attr, fn)
    ok, _ = _all_pins_pass()
    assert not ok, f"mistake {name} went unnoticed"


@pytest.mark.parametrize("bias", [6, 8])
def test_planted_table_bias_is_caught(bias, monkeypatch):
    monkeypatch.setattr(e4m3_mod, "_TABLE", _wrong_table(bias))
    ok, _ = _all_pins_pass()
    assert not ok


def test_planted_swapped_scales_are_caught(monkeypatch):
    real = pa.gather_sequence

    def swapped(k_pages, v_pages, kv_scales, row, L, *fmt):
        return real(k_pages, v_pages, kv_scales[::-1], row, L, *fmt)

    monkeypatch.setattr(pa, "gather_sequence", swapped)
    ok, _ = _all_pins_pass()
    assert not ok


def test_planted_dropped_scale_is_caught(monkeypatch):
    real = pa.gather_sequence

    def unscaled(k_pages, v_pages, kv_scales, row, L, *fmt):
        return real(k_pages, v_pages, np.ones_like(kv_scales), row, L, *fmt)

    monkeypatch.setattr(pa, "gather_sequence", unscaled)
    ok, _ = _all_pins_pass()
    assert not ok
