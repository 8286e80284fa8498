"""CPU oracle for multi-branch decode: several caches attended as one, and the
sink / ring-window / main cache layout a streaming decoder keeps.

TEST INFRASTRUCTURE ONLY (like ``oracle.attention``, which it builds on):
plain numpy, fp64 arithmetic, bit copies for cache data.

Passages followed:

* usearch "linear-algebra", section Attention: a carry per query row lets one
  branch resume where another left off on the same query rows.  Attending
  several caches
  is therefore the carry of each branch folded in turn; it equals one pass
  over the concatenated keys.
* cortiq-engine ``NystromState`` (struct doc, ``new``, ``step_group``): per
  KV group an exact window ring of width w (128 validated) and a buffer of
  permanent exact sink keys (4 by default), shared by the group's query
  heads; each decode step adds the group's new key/value row a single time
  and drops the oldest window key.  The page's far field (landmarks) is an approximation and is
  not modelled: here the evicted key moves, exactly, into a main cache.

Readings (listed in the design notes): the first ``S`` tokens of a sequence
go to the sink; token ``t >= S`` goes to ring slot ``(t - S) % W``; when the
ring is full, the token it evicts (the one ``W`` positions older, in the same
slot) is first appended to the main cache at ``t - S - W``; with no main
cache the evicted token is dropped from attention (sink + window only).  A
full main cache (or a negative count) drops the new token: nothing changes
and the drop is counted, as a full needle-core cache does.
"""

from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

from .attention import Carry, attend, finalize


def attend_branches(q, branches: Sequence, scale: float = 0.0,
                    carry_in: Optional[Carry] = None):
    """Attention over the union of the branches' live keys.

    ``branches``: (k, v, lens) or (k, v, lens, bias) per cache, as for
    ``attend``.  Each branch's state continues the previous one's (usearch
    carry), starting from ``carry_in``.  Returns (out, Carry)."""
    c = carry_in
    for br in branches:
        k, v, lens = br[:3]
        bias = br[3] if len(br) > 3 else None
        _, c = attend(q, k, v, lens, scale, carry_in=c, bias=bias)
    B, Hq = np.asarray(q).shape[:2]
    return finalize(c).reshape(B, Hq, -1), c


def stream_lengths(count, sink: int, window: int, main: int):
    """Live keys of each part after ``count`` tokens: (sink, window, main)."""
    t = max(int(count), 0)
    return (min(t, sink), min(max(t - sink, 0), window),
            min(max(t - sink - window, 0), main))


def stream_append(sink_k, sink_v, ring_k, ring_v, main_k, main_v,
                  k_new, v_new, count):
    """One token per sequence into the sink / ring / main layout.

    Caches are [B, slots, Hkv, d] (any element type: bit copies); sink or
    main may be None (no sink; no main cache).  ``count`` [B] is the tokens
    seen so far.  Returns (sink_k, sink_v, ring_k, ring_v, main_k, main_v,
    count_out, dropped), new arrays, inputs untouched."""
    cp = lambda a: None if a is None else np.array(a, copy=True)
    sk, sv, rk, rv, mk, mv = map(cp, (sink_k, sink_v, ring_k, ring_v,
                                      main_k, main_v))
    S = 0 if sk is None else sk.shape[1]
    W = rk.shape[1]
    M = 0 if mk is None else mk.shape[1]
    out = np.array(count, dtype=np.int64, copy=True)
    dropped = 0
    for b in range(rk.shape[0]):
        t = int(out[b])
        if t < 0:
            dropped += 1
            continue
        if t < S:
            sk[b, t] = k_new[b]
            sv[b, t] = v_new[b]
            out[b] = t + 1
            continue
        r = (t - S) % W
        if t - S >= W and mk is not None:
            j = t - S - W          # the evicted token's place in main
            if j >= M:
                dropped += 1
                continue
            mk[b, j] = rk[b, r]
            mv[b, j] = rv[b, r]
        rk[b, r] = k_new[b]
        rv[b, r] = v_new[b]
        out[b] = t + 1
    return sk, sv, rk, rv, mk, mv, out.astype(np.int32), dropped


def selection_mask(idx_row, kv_len: int) -> np.ndarray:
    """metrale DSA ``topk_to_mask`` for one query row: key i is visible when
    some entry equals i with 0 <= i < kv_len; duplicates collapse to one
    visible key and out-of-range or INVALID (negative) entries are dropped."""
    mask = np.zeros(max(int(kv_len), 0), dtype=bool)
    for i in np.asarray(idx_row).ravel():
        i = int(i)
        if 0 <= i < kv_len:
            mask[i] = True
    return mask


def attend_gathered(q, k, v, lens, idx, scale: float = 0.0,
                    carry_in: Optional[Carry] = None):
    """Attention of each sequence's query over the keys its index row
    selects (``selection_mask`` with kv_len = the sequence's live length),
    taken in ascending position order.  idx [B, width] int."""
    B = np.asarray(q).shape[0]
    T = np.asarray(k).shape[1]
    kc = np.full_like(np.asarray(k, dtype=np.float64), np.nan)
    vc = np.full_like(np.asarray(v, dtype=np.float64), np.nan)
    n_sel = np.zeros(B, dtype=np.int64)
    for b in range(B):
        n = int(min(max(int(lens[b]), 0), T))
        sel = np.nonzero(selection_mask(idx[b], n))[0]
        n_sel[b] = len(sel)
        kc[b, :len(sel)] = np.asarray(k[b], dtype=np.float64)[sel]
        vc[b, :len(sel)] = np.asarray(v[b], dtype=np.float64)[sel]
    return attend(q, kc, vc, n_sel, scale, carry_in=carry_in)
