"""CPU oracle for fp8 KV caches.

TEST INFRASTRUCTURE ONLY (like the rest of ``oracle``): plain numpy, fp64
arithmetic except where the format fixes a narrower step.

The pages fix no 8-bit format.  usearch "linear-algebra" (section Attention)
hands back each value row in whatever quantised form the index keeps it,
and qualiaDB ``KvDictionary`` (its decode of code words) serves a
compressed-cache read path; neither names a scheme, so this module takes one
reading, listed in the design notes:

* element format: OCP 8-bit floating point E4M3 (E4M3FN): a sign bit, a
  4-bit exponent with bias 7 and a 3-bit mantissa; exponent field 0 holds the
  subnormals m * 2^-9; S.1111.111 is NaN; there are no infinities, and the
  largest finite magnitude is 448 (S.1111.110);
* one fp32 scale per (sequence, KV head) for K and another for V: a stored
  code c stands for decode(c) * scale;
* quantisation (the quantising append): x times the fp32 reciprocal of the
  scale (1 / scale correctly rounded to fp32, then the product correctly
  rounded to fp32), then the nearest E4M3 value, ties to the even mantissa,
  magnitudes above 448 saturating to 448, the sign kept (also on zero);
* attention over fp8 caches is exact attention over the decoded values.

``e4m3_decode`` is the format's definition written out; ``encode`` picks the
nearest finite value by exhaustive search over the 127 non-negative finite
codes.  The pins check both against values the definition fixes.
"""

from __future__ import annotations

import math
from typing import Optional

import numpy as np

from .attention import Carry, attend, kv_append
from .streaming import stream_append

E4M3_MAX = 448.0


def e4m3_decode(code: int) -> float:
    """Value of one E4M3 code (NaN for S.1111.111)."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return sign * m * 2.0 ** -9
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def decode(codes) -> np.ndarray:
    """Element-wise decode of uint8 codes to fp64."""
    table = np.array([e4m3_decode(c) for c in range(256)])
    return table[np.asarray(codes, dtype=np.uint8)]


def encode(x) -> np.ndarray:
    """Nearest E4M3 code to each element of x (fp64 arithmetic on the given
    values), ties to the even mantissa, saturating at +-448, sign kept.
    NaN is not accepted."""
    x = np.asarray(x, dtype=np.float64)
    assert not np.isnan(x).any(), "NaN has no nearest finite code"
    finite = decode(np.arange(0x7F))        # 0, subnormals, ..., 448
    even = (np.arange(0x7F) % 2) == 0
    flat = np.minimum(np.abs(x.ravel()), E4M3_MAX)
    codes = np.empty(flat.size, dtype=np.int64)
    for s in range(0, flat.size, 1 << 15):
        a = flat[s:s + (1 << 15)]
        d = np.abs(finite[None, :] - a[:, None])
        near = d == d.min(axis=1, keepdims=True)
        tie_even = near & even[None, :]
        codes[s:s + a.size] = np.where(tie_even.any(axis=1),
                                       tie_even.argmax(axis=1),
                                       near.argmax(axis=1))
    codes |= np.signbit(x.ravel()).astype(np.int64) << 7
    return codes.astype(np.uint8).reshape(x.shape)


def quantize(x, scale) -> np.ndarray:
    """Codes of x with a broadcast fp32 scale: x times the fp32 reciprocal of
    the scale, rounded to fp32, then ``encode``."""
    inv = (np.float32(1.0) / np.asarray(scale, dtype=np.float32)).astype(np.float32)
    prod = np.asarray(x, dtype=np.float32) * inv
    return encode(prod.astype(np.float32))


def dequantize_cache(codes, scale) -> np.ndarray:
    """[B, T, Hkv, d] codes with scales [B, Hkv] -> fp64 values."""
    s = np.asarray(scale, dtype=np.float64)
    return decode(codes) * s[:, None, :, None]


def attend_fp8(q, k_codes, v_codes, k_scale, v_scale, lens,
               scale: float = 0.0, carry_in: Optional[Carry] = None,
               bias=None):
    """Attention over the decoded caches; slots at or past each length are
    never read (they may hold any code, NaN included).  Returns (out, Carry)
    as ``attend``."""
    k = dequantize_cache(k_codes, k_scale)
    v = dequantize_cache(v_codes, v_scale)
    T = k.shape[1]
    for b in range(k.shape[0]):
        n = int(min(max(int(lens[b]), 0), T))
        k[b, n:] = np.nan
        v[b, n:] = np.nan
    return attend(q, k, v, lens, scale, carry_in=carry_in, bias=bias)


def kv_append_fp8(k_cache, v_cache, k_new, v_new, k_scale, v_scale, lens):
    """needle-core ``push_kv`` into fp8 caches: the new rows [B, Hkv, d]
    (values exact in fp32, e.g. bf16) are quantised with their sequence's
    per-KV-head scales [B, Hkv], then appended as for any cache (a full cache
    drops the token).  Returns (k_codes, v_codes, lens, dropped)."""
    ks = np.asarray(k_scale, dtype=np.float32)[:, :, None]
    vs = np.asarray(v_scale, dtype=np.float32)[:, :, None]
    return kv_append(k_cache, v_cache, quantize(k_new, ks),
                     quantize(v_new, vs), lens)


def stream_append_fp8(sink_k, sink_v, ring_k, ring_v, main_k, main_v,
                      k_new, v_new, k_scale, v_scale, count):
    """The sink / ring / main layout of ``oracle.streaming.stream_append``
    (cortiq-engine ``NystromState``) over fp8 code caches whose three parts
    share one K and one V scale per (sequence, KV head), [B, Hkv]: the new
    rows (values exact in fp32, e.g. bf16) are quantised with those scales,
    then placed as any cache row; a ring row a full ring evicts moves to main
    as its codes, so it keeps its value.  Returns as ``stream_append``."""
    ks = np.asarray(k_scale, dtype=np.float32)[:, :, None]
    vs = np.asarray(v_scale, dtype=np.float32)[:, :, None]
    return stream_append(sink_k, sink_v, ring_k, ring_v, main_k, main_v,
                         quantize(k_new, ks), quantize(v_new, vs), count)
