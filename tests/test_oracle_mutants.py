"""Planted mistakes in the oracle must each be caught by at least one pin.

Each mutant patches one step of ``oracle.attention`` with a plausible error (a
dropped term, a wrong sign or index, a swapped operand, an off-by-one, a
missing guard) and runs every pin against it.  CPU only.
"""

import math

import numpy as np
import pytest

import oracle.attention as orc
from oracle_pins import ALL_PINS


def _softmax_state_sign(s, vg):
    if s.shape[1] == 0:
        return orc.Carry(np.full(s.shape[0], -np.inf), np.zeros(s.shape[0]),
                         np.zeros((s.shape[0], vg.shape[1])))
    m = s.max(axis=1)
    e = np.exp(m[:, None] - s)                      # wrong sign
    return orc.Carry(m, e.sum(axis=1), e @ vg.astype(np.float64))


def _softmax_state_no_shift(s, vg):
    if s.shape[1] == 0:
        return orc.Carry(np.full(s.shape[0], -np.inf), np.zeros(s.shape[0]),
                         np.zeros((s.shape[0], vg.shape[1])))
    e = np.exp(s)                                   # no max taken out
    return orc.Carry(np.zeros(s.shape[0]), e.sum(axis=1),
                     e @ vg.astype(np.float64))


def _merge_swapped(a, b):
    m_a, l_a, acc_a = (np.asarray(x, dtype=np.float64) for x in a)
    m_b, l_b, acc_b = (np.asarray(x, dtype=np.float64) for x in b)
    m = np.maximum(m_a, m_b)
    out_m, out_l, out_acc = m.copy(), np.zeros_like(l_a), np.zeros_like(acc_a)
    for r in range(len(m)):
        if l_a[r] == 0.0:
            out_m[r], out_l[r], out_acc[r] = m_b[r], l_b[r], acc_b[r]
            continue
        if l_b[r] == 0.0:
            out_m[r], out_l[r], out_acc[r] = m_a[r], l_a[r], acc_a[r]
            continue
        alpha, beta = math.exp(m_b[r] - m[r]), math.exp(m_a[r] - m[r])  # swap
        out_l[r] = alpha * l_a[r] + beta * l_b[r]
        out_acc[r] = alpha * acc_a[r] + beta * acc_b[r]
    return orc.Carry(out_m, out_l, out_acc)


def _finalize_no_guard(c):
    with np.errstate(invalid="ignore", divide="ignore"):
        return c.acc / c.l[:, None]


def _finalize_unnormalised(c):
    return np.array(c.acc, copy=True)


def _attend_ignores_carry(q, k, v, lens, scale=0.0, carry_in=None):
    return _real_attend(q, k, v, lens, scale)


def _attend_wrong_value_group(q, k, v, lens, scale=0.0, carry_in=None):
    Hkv = k.shape[2]
    v_shift = np.roll(np.asarray(v), 1, axis=2)     # value rows of group g-1
    if Hkv == 1:
        v_shift = np.asarray(v)[::-1].copy()
    return _real_attend(q, k, v_shift, lens, scale, carry_in)


def _kv_append_no_increment(k_cache, v_cache, k_new, v_new, lens):
    k, v, lens_out, dropped = _real_append(k_cache, v_cache, k_new, v_new, lens)
    return k, v, np.asarray(lens, dtype=np.int32), dropped


def _softmax_state_unguarded(s, vg):
    if s.shape[1] == 0:
        return orc.Carry(np.full(s.shape[0], -np.inf), np.zeros(s.shape[0]),
                         np.zeros((s.shape[0], vg.shape[1])))
    m = s.max(axis=1)                               # -inf rows give NaN
    with np.errstate(invalid="ignore"):
        e = np.exp(s - m[:, None])
    return orc.Carry(m, e.sum(axis=1), e @ vg.astype(np.float64))


def _biased_logits_scaled(qg, kg, scale, bias_row):
    s = qg.astype(np.float64) @ kg.astype(np.float64).T
    if bias_row is not None:
        s = s + np.asarray(bias_row)[None, :]
    return scale * s                                # bias scaled too


def _biased_logits_ignored(qg, kg, scale, bias_row):
    return _real_group_logits(qg, kg, scale)


_real_attend = orc.attend
_real_append = orc.kv_append
_real_group_logits = orc.group_logits

MUTANTS = {
    "scale_dropped": ("group_logits",
                      lambda qg, kg, scale: qg.astype(np.float64) @
                      kg.astype(np.float64).T),
    "scale_from_wrong_power": ("resolve_scale",
                               lambda scale, dk: scale if scale else 1.0 / dk),
    "head_map_modulo": ("kv_head_of", lambda h, hpk: h % hpk),
    "exp_sign_flipped": ("softmax_state", _softmax_state_sign),
    "max_not_subtracted": ("softmax_state", _softmax_state_no_shift),
    "length_off_by_one_short": ("live_length",
                                lambda n, T: max(min(int(n), T) - 1, 0)),
    "length_off_by_one_long": ("live_length",
                               lambda n, T: max(min(int(n) + 1, T), 0)),
    "length_not_clamped": ("live_length", lambda n, T: int(n)),
    "merge_weights_swapped": ("merge", _merge_swapped),
    "empty_gives_nan": ("finalize", _finalize_no_guard),
    "not_divided_by_partition": ("finalize", _finalize_unnormalised),
    "carry_in_ignored": ("attend", _attend_ignores_carry),
    "values_of_wrong_group": ("attend", _attend_wrong_value_group),
    "append_keeps_length": ("kv_append", _kv_append_no_increment),
    "removed_keys_give_nan": ("softmax_state", _softmax_state_unguarded),
    "bias_scaled_with_logits": ("biased_logits", _biased_logits_scaled),
    "bias_ignored": ("biased_logits", _biased_logits_ignored),
    "bias_of_wrong_sequence": ("bias_row_of",
                               lambda bias, b, n: np.asarray(
                                   bias[b - 1][:n], dtype=np.float64)),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(orc, attr, fn)
    caught = []
    for pin in ALL_PINS:
        try:
            pin(orc)
        except AssertionError:
            caught.append(pin.__name__)
        except (ValueError, IndexError, FloatingPointError, TypeError):
            caught.append(pin.__name__ + " (error)")
    assert caught, f"no pin catches mutant {name}"
