"""The multi-branch and streaming-layout oracle against its pins, and planted
mistakes in it, each caught.  CPU only."""

import numpy as np
import pytest

import oracle.streaming as st
from oracle_pins import STREAM_PINS


@pytest.mark.parametrize("pin", STREAM_PINS, ids=lambda p: p.__name__)
def test_stream_pin(pin):
    pin(st)


_real_append = st.stream_append
_real_lengths = st.stream_lengths
_real_mask = st.selection_mask


def _mask_counts_dups(row, n):
    """a duplicated entry selects the next key too (no collapse)"""
    m = _real_mask(row, n)
    seen = set()
    for i in np.asarray(row).ravel():
        i = int(i)
        if 0 <= i < n:
            if i in seen and i + 1 < n:
                m[i + 1] = True
            seen.add(i)
    return m


def _ring_slot_shifted(sk, sv, rk, rv, mk, mv, kn, vn, count):
    """new tokens land one ring slot late"""
    out = _real_append(sk, sv, rk, rv, mk, mv, kn, vn, count)
    rk2, rv2 = np.roll(out[2], 1, axis=1), np.roll(out[3], 1, axis=1)
    return (out[0], out[1], rk2, rv2) + tuple(out[4:])


def _evicts_new_token(sk, sv, rk, rv, mk, mv, kn, vn, count):
    """main receives the new token instead of the evicted one"""
    res = list(_real_append(sk, sv, rk, rv, mk, mv, kn, vn, count))
    if mk is None:
        return tuple(res)
    S = 0 if sk is None else sk.shape[1]
    W = rk.shape[1]
    for b in range(rk.shape[0]):
        t = int(count[b])
        if t >= 0 and t - S >= W and t - S - W < mk.shape[1]:
            res[4][b, t - S - W] = kn[b]
            res[5][b, t - S - W] = vn[b]
    return tuple(res)


MUTANTS = {
    "ring_slot_shifted": ("stream_append", _ring_slot_shifted),
    "evicts_new_token": ("stream_append", _evicts_new_token),
    "window_not_clamped": ("stream_lengths",
                           lambda c, s, w, m: (min(max(c, 0), s),
                                               max(c - s, 0),
                                               min(max(c - s - w, 0), m))),
    "main_off_by_one": ("stream_lengths",
                        lambda c, s, w, m: _real_lengths(c, s, w, m)[:2] +
                        (max(_real_lengths(c, s, w, m)[2] - 1, 0),)),
    "selection_keeps_duplicates": ("selection_mask", _mask_counts_dups),
    "selection_ignores_length": ("selection_mask",
                                 lambda row, n: _real_mask(row, 10 ** 6)),
    "branches_drop_carry": ("attend_branches",
                            lambda q, brs, scale=0.0, carry_in=None:
                            _real_branches(q, brs, scale)),
}
_real_branches = st.attend_branches


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_stream_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(st, attr, fn)
    caught = []
    for pin in STREAM_PINS:
        try:
            pin(st)
        except AssertionError:
            caught.append(pin.__name__)
        except (ValueError, IndexError, TypeError):
            caught.append(pin.__name__ + " (error)")
    assert caught, f"no pin catches mutant {name}"
