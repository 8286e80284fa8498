"""CPU oracle for exact grouped-query decode attention over a KV cache.

TEST INFRASTRUCTURE ONLY.  The tests, the smoke check and the benchmark's CPU
baseline leg are the only callers; the product path never imports this
package, and it imports nothing from the product.

Everything here is plain numpy in float64.  Inputs are read as stored (bf16 and
fp32 values convert to float64 exactly), the full logit vector is formed, and
the softmax is taken in two passes: first the maximum, then the exponentials
against it, their sum and the weighted value sum.  The passages followed:

* needle-core ``attn.rs``, ``self_attn_incremental``: query head ``hi`` reads
  KV head ``hi / kv_repeat`` (contiguous grouping); every cached position is
  given the logit ``scale * <q_h, k_h>``, the scale being ``head_dim^-0.5``;
  the scores are softmaxed and the value rows are summed with those weights.
  Decode needs no causal mask: the query attends to exactly the cached rows.
* usearch "linear-algebra", section Attention: every scored key updates three
  per-head quantities (largest logit so far, sum of exponentials, weighted
  value sum); the outputs are
  normalised by the partition; a carry per query row lets one branch resume
  where another left off on the same query rows.  Struct ``DenseSoftmaxState``:
  ``maximum_score`` holds the maximum logit so far (m), ``partition`` the sum
  of exponentials relative to it (l).  A zero ``score_scale`` is replaced by
  the derived one, 1/sqrt of the key width by convention.
* cortiq-engine ``NystromState``, example ``o1_recovery.rs`` ``trial()``: the
  exact reference takes the maximum logit first and then the exponentials
  ``exp(l - mx)`` in double precision.
* metrale DSA reference, ``pool_states``: a softmax over an empty set
  contributes zero weight (a zero result) rather than a NaN.
* needle-core ``self_attn_incremental``, argument ``attn_bias``: an optional
  additive term per cached position, added to the scaled dot product of every
  head before the softmax.

Readings taken where the pages are silent (each listed in the design notes):
the carry is ``(m, l, acc)`` with ``acc`` the *unnormalised* weighted value sum
``sum_j exp(s_j - m) v_j``; ``m`` is in natural-log units of the scaled logit;
a state with ``l == 0`` is empty whatever its ``m``; an empty result has output
0 and carry ``(-inf, 0, 0)``; lengths are clamped to ``[0, max_len]``; the
scale defaults to ``1/sqrt(dk)`` (the key width) when given as 0; the bias
is one fp32 value per (sequence, position), shared by the sequence's heads, and
a bias of -inf removes the key, so a row whose every key is removed is empty.
"""

from __future__ import annotations

import math
from typing import NamedTuple, Optional

import numpy as np


class Carry(NamedTuple):
    """Online-softmax state per query row: m [R], l [R], acc [R, dv]."""

    m: np.ndarray
    l: np.ndarray
    acc: np.ndarray


def resolve_scale(scale: float, dk: int) -> float:
    """usearch DenseAttendConfig.score_scale: a zero scale is replaced by
    1/sqrt(head width).

    The head width used is the key width dk (it is the width of the dot
    product being scaled)."""
    return float(scale) if scale != 0.0 else 1.0 / math.sqrt(dk)


def kv_head_of(h: int, heads_per_kv: int) -> int:
    """needle-core self_attn_incremental: kv_hi = hi / kv_repeat."""
    return h // heads_per_kv


def live_length(length: int, max_len: int) -> int:
    """Keys attended are slots [0, n) with n clamped into [0, max_len]."""
    return int(min(max(int(length), 0), max_len))


def group_logits(qg: np.ndarray, kg: np.ndarray, scale: float) -> np.ndarray:
    """Full logit matrix of one KV group: s[i, j] = scale * <q_i, k_j>.

    qg [heads, dk], kg [n, dk] -> [heads, n], float64."""
    return scale * (qg.astype(np.float64) @ kg.astype(np.float64).T)


def bias_row_of(bias, b: int, n: int) -> np.ndarray:
    """The additive bias of sequence b's first n positions (fp64)."""
    return np.asarray(bias[b][:n], dtype=np.float64)


def biased_logits(qg: np.ndarray, kg: np.ndarray, scale: float,
                  bias_row) -> np.ndarray:
    """needle-core self_attn_incremental: score = dot(q, k) * scale, then
    score += bias[t] when a bias is given (the same term for every head)."""
    s = group_logits(qg, kg, scale)
    if bias_row is not None:
        s = s + np.asarray(bias_row, dtype=np.float64)[None, :]
    return s


def softmax_state(s: np.ndarray, vg: np.ndarray) -> Carry:
    """Two-pass softmax state of a logit matrix s [heads, n] over values vg [n, dv].

    Pass 1: m = max_j s_j.  Pass 2: l = sum_j exp(s_j - m),
    acc = sum_j exp(s_j - m) v_j.  With no keys, or no key with a finite
    logit (all removed by a -inf bias), the state is empty."""
    heads, n = s.shape
    dv = vg.shape[1]
    m = np.full(heads, -np.inf)
    l = np.zeros(heads)
    acc = np.zeros((heads, dv))
    if n == 0:
        return Carry(m, l, acc)
    mx = s.max(axis=1)
    for h in range(heads):
        if mx[h] == -np.inf:
            continue
        e = np.exp(s[h] - mx[h])
        m[h] = mx[h]
        l[h] = e.sum()
        acc[h] = e @ vg.astype(np.float64)
    return Carry(m, l, acc)


def merge(a: Carry, b: Carry) -> Carry:
    """Fold two online-softmax states over the same query rows.

    usearch DenseAttendConfig.carry (partial softmaxes rescaled to a common
    maximum): with
    m = max(m_a, m_b), alpha = exp(m_a - m), beta = exp(m_b - m):
    l = alpha l_a + beta l_b and acc = alpha acc_a + beta acc_b.
    An empty state (l == 0) is the identity."""
    m_a, l_a, acc_a = (np.asarray(x, dtype=np.float64) for x in a)
    m_b, l_b, acc_b = (np.asarray(x, dtype=np.float64) for x in b)
    m = np.empty_like(m_a)
    l = np.empty_like(l_a)
    acc = np.empty_like(acc_a)
    for r in range(m_a.shape[0]):
        if l_a[r] == 0.0 and l_b[r] == 0.0:
            m[r], l[r], acc[r] = -np.inf, 0.0, 0.0
        elif l_a[r] == 0.0:
            m[r], l[r], acc[r] = m_b[r], l_b[r], acc_b[r]
        elif l_b[r] == 0.0:
            m[r], l[r], acc[r] = m_a[r], l_a[r], acc_a[r]
        else:
            mm = max(m_a[r], m_b[r])
            alpha = math.exp(m_a[r] - mm)
            beta = math.exp(m_b[r] - mm)
            m[r] = mm
            l[r] = alpha * l_a[r] + beta * l_b[r]
            acc[r] = alpha * acc_a[r] + beta * acc_b[r]
    return Carry(m, l, acc)


def finalize(c: Carry) -> np.ndarray:
    """Output rows normalised by the partition; 0 for an empty state."""
    out = np.zeros_like(c.acc)
    live = c.l > 0.0
    out[live] = c.acc[live] / c.l[live][:, None]
    return out


def empty_carry(rows: int, dv: int) -> Carry:
    return Carry(np.full(rows, -np.inf), np.zeros(rows), np.zeros((rows, dv)))


def attend(q, k, v, lens, scale: float = 0.0,
           carry_in: Optional[Carry] = None, bias=None):
    """Exact GQA decode attention of one query token per sequence.

    q [B, Hq, dk]; k [B, max_len, Hkv, dk]; v [B, max_len, Hkv, dv];
    lens [B] (live keys per sequence); bias None or [B, >= n] additive
    logit terms.  Rows of the result are b * Hq + h.
    With ``carry_in`` the result is merge(carry_in, this branch).
    Returns (out [B, Hq, dv], Carry with m [B*Hq], l [B*Hq], acc [B*Hq, dv]).
    """
    q = np.asarray(q)
    B, Hq, dk = q.shape
    _, max_len, Hkv, _ = k.shape
    dv = v.shape[3]
    if Hq % Hkv != 0:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    hpk = Hq // Hkv
    s_scale = resolve_scale(scale, dk)
    m = np.empty(B * Hq)
    l = np.empty(B * Hq)
    acc = np.empty((B * Hq, dv))
    for b in range(B):
        n = live_length(lens[b], max_len)
        for g in range(Hkv):
            heads = [h for h in range(Hq) if kv_head_of(h, hpk) == g]
            kg = np.asarray(k[b, :n, g, :])
            vg = np.asarray(v[b, :n, g, :])
            brow = None if bias is None else bias_row_of(bias, b, n)
            st = softmax_state(biased_logits(q[b, heads, :], kg, s_scale,
                                             brow), vg)
            rows = [b * Hq + h for h in heads]
            m[rows], l[rows], acc[rows] = st.m, st.l, st.acc
    c = Carry(m, l, acc)
    if carry_in is not None:
        c = merge(carry_in, c)
    return finalize(c).reshape(B, Hq, dv), c


def kv_append(k_cache, v_cache, k_new, v_new, lens):
    """needle-core KvCache::push_kv, batched over sequences.

    For each sequence b with n = lens[b]: if 0 <= n < max_len, slot n of every
    KV head receives the new K and V rows and the length becomes n + 1;
    otherwise nothing is written, the length is unchanged and the sequence
    counts as dropped (the page warns and returns without writing).
    Works on any element type (a bit copy).  Returns (k, v, lens, dropped)."""
    k = np.array(k_cache, copy=True)
    v = np.array(v_cache, copy=True)
    lens_out = np.array(lens, dtype=np.int64, copy=True)
    dropped = 0
    max_len = k.shape[1]
    for b in range(k.shape[0]):
        n = int(lens_out[b])
        if n < 0 or n >= max_len:
            dropped += 1
            continue
        k[b, n] = k_new[b]
        v[b, n] = v_new[b]
        lens_out[b] = n + 1
    return k, v, lens_out.astype(np.int32), dropped
