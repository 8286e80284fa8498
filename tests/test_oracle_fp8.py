"""The fp8 KV oracle against its pins, and planted mistakes in it, each
caught.  CPU only."""

import math

import numpy as np
import pytest

import oracle.fp8 as f8
from oracle_pins import FP8_PINS


@pytest.mark.parametrize("pin", FP8_PINS, ids=lambda p: p.__name__)
def test_fp8_pin(pin):
    pin(f8)


_real_decode1 = f8.e4m3_decode
_real_encode = f8.encode
_real_quantize = f8.quantize
_real_dequant = f8.dequantize_cache
_real_attend = f8.attend_fp8
_real_append = f8.kv_append_fp8
_real_stream = f8.stream_append_fp8


def _decode_bias8(code):
    """exponent bias 8 instead of 7"""
    v = _real_decode1(code)
    return v if (code & 0x78) == 0 else v / 2


def _decode_no_subnormals(code):
    """exponent field 0 read as a normal binade"""
    code = int(code) & 0xFF
    if (code >> 3) & 0xF:
        return _real_decode1(code)
    s = -1.0 if code & 0x80 else 1.0
    return s * (1 + (code & 7) / 8) * 2.0 ** -6 if code & 7 else s * 0.0


def _encode_ties_up(x):
    """ties go to the larger magnitude"""
    c = _real_encode(x)
    a = np.abs(np.asarray(x, dtype=np.float64))
    up = np.minimum((c & 0x7F).astype(np.int64) + 1, 0x7E)
    lo, hi = f8.decode(c & 0x7F), f8.decode(up)
    tie = (a < 448) & (np.abs(hi - a) == np.abs(a - lo))
    return np.where(tie, (c & 0x80) | up, c).astype(np.uint8)


def _encode_truncate(x):
    """rounds toward zero"""
    x = np.asarray(x, dtype=np.float64)
    c = _real_encode(x).astype(np.int64)
    over = np.abs(f8.decode(c)) > np.minimum(np.abs(x), 448)
    return np.where(over, c - 1, c).astype(np.uint8)


def _encode_overflow_nan(x):
    """magnitudes above 448 give NaN"""
    x = np.asarray(x, dtype=np.float64)
    c = _real_encode(x)
    return np.where(np.abs(x) > 448, c | 0x7F, c).astype(np.uint8)


def _encode_unsigned_zero(x):
    """a zero result loses its sign"""
    c = _real_encode(x)
    return np.where((c & 0x7F) == 0, 0, c).astype(np.uint8)


MUTANTS = {
    "exponent_bias_8": ("e4m3_decode", _decode_bias8),
    "no_subnormals": ("e4m3_decode", _decode_no_subnormals),
    "ties_up": ("encode", _encode_ties_up),
    "truncate": ("encode", _encode_truncate),
    "overflow_nan": ("encode", _encode_overflow_nan),
    "unsigned_zero": ("encode", _encode_unsigned_zero),
    "scale_multiplied": ("quantize",
                         lambda x, s: _real_encode(
                             np.asarray(x, np.float32) *
                             np.asarray(s, np.float32))),
    "quotient_not_reciprocal": ("quantize",
                                lambda x, s: _real_encode(
                                    (np.asarray(x, np.float32) /
                                     np.asarray(s, np.float32)).astype(
                                         np.float32))),
    "scales_swapped": ("attend_fp8",
                       lambda q, kc, vc, ks, vs, *a, **kw:
                       _real_attend(q, kc, vc, vs, ks, *a, **kw)),
    "v_scale_dropped": ("attend_fp8",
                        lambda q, kc, vc, ks, vs, *a, **kw:
                        _real_attend(q, kc, vc, ks, np.ones_like(vs), *a,
                                     **kw)),
    "scale_rows_reversed": ("dequantize_cache",
                            lambda c, s: _real_dequant(c, np.asarray(s)[::-1])),
    "append_k_with_v_scale": ("kv_append_fp8",
                              lambda k, v, kn, vn, ks, vs, lens:
                              _real_append(k, v, kn, vn, vs, vs, lens)),
    "stream_k_with_v_scale": ("stream_append_fp8",
                              lambda *a: _real_stream(*a[:8], a[9], a[9],
                                                      a[10])),
    "stream_scales_of_next_sequence": (
        "stream_append_fp8",
        lambda *a: _real_stream(*a[:8], np.roll(a[8], 1, axis=0),
                                np.roll(a[9], 1, axis=0), a[10])),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_fp8_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(f8, attr, fn)
    caught = []
    for pin in FP8_PINS:
        try:
            pin(f8)
        except AssertionError:
            caught.append(pin.__name__)
        except (ValueError, IndexError, TypeError):
            caught.append(pin.__name__ + " (error)")
    assert caught, f"no pin catches mutant {name}"
