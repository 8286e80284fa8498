"""Pins for the CPU oracle: checks against what the pages and the mathematics fix.

Each ``pin_*`` takes an oracle module (``oracle.attention`` or a copy of it with
a planted mistake) and raises ``AssertionError`` when the oracle breaks the
property.  None of them re-types the oracle's two-pass formula: they use
closed forms (equal keys give the plain mean; a dominant key returns its own
value row), a library routine (torch's fp64 ``scaled_dot_product_attention`` on
repeat-copied heads), exact 50-digit evaluation of the softmax definition
without a max shift, the carry algebra (any split merged equals one pass), the
a planted key's exact weight, and special cases.
"""

from __future__ import annotations

import itertools
import json
import math
from decimal import Decimal, localcontext
from pathlib import Path

import numpy as np
import torch

GOLDEN = Path(__file__).parent / "golden"


def _problem(seed, B, Hq, Hkv, dk, dv, T, lens=None, poison=True,
             dyadic=False):
    """Random problem; padding slots past each length are NaN-poisoned."""
    rng = np.random.default_rng(seed)
    if dyadic:
        q = rng.integers(-16, 17, (B, Hq, dk)) / 16.0
        k = rng.integers(-16, 17, (B, T, Hkv, dk)) / 16.0
        v = rng.integers(-16, 17, (B, T, Hkv, dv)) / 16.0
    else:
        q = rng.uniform(-1, 1, (B, Hq, dk))
        k = rng.uniform(-1, 1, (B, T, Hkv, dk))
        v = rng.uniform(-1, 1, (B, T, Hkv, dv))
    lens = np.full(B, T) if lens is None else np.asarray(lens)
    if poison:
        for b in range(B):
            n = int(min(max(lens[b], 0), T))
            k[b, n:] = np.nan
            v[b, n:] = np.nan
    return q, k, v, lens


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    assert np.all(np.isfinite(a) == np.isfinite(b)), f"{what}: finiteness"
    fin = np.isfinite(b)
    assert np.array_equal(a[~fin], b[~fin]), f"{what}: non-finite entries"
    err = np.max(np.abs(a[fin] - b[fin])) if fin.any() else 0.0
    assert err <= tol, f"{what}: max err {err:.3e} > {tol:.3e}"


# --- closed forms ---------------------------------------------------------

def pin_equal_keys(orc):
    """All live keys of a group equal (or q = 0): every weight is 1/n, so the
    output is the plain mean of the group's live value rows (math.fsum)."""
    B, Hq, Hkv, dk, dv, T = 3, 8, 4, 16, 8, 37
    q, k, v, lens = _problem(1, B, Hq, Hkv, dk, dv, T, lens=[37, 20, 1])
    for b in range(B):
        n = int(lens[b])
        k[b, :n] = k[b, :1]
    q[1] = 0.0                       # q = 0: any keys give the mean too
    rng = np.random.default_rng(2)
    k[1, :20] = rng.uniform(-1, 1, (20, Hkv, dk))
    out, c = orc.attend(q, k, v, lens, scale=0.3)
    hpk = Hq // Hkv
    for b in range(B):
        n = int(lens[b])
        for h in range(Hq):
            g = h // hpk             # needle-core: kv_hi = hi / kv_repeat
            want = [math.fsum(v[b, :n, g, c_]) / n for c_ in range(dv)]
            _close(out[b, h], want, 1e-14, f"mean b={b} h={h}")
            _close(c.l[b * Hq + h], float(n), 1e-12, "partition of equal keys")


def pin_dominant_key(orc):
    """One key per group leads every other logit by > 800: its weight is 1 to
    far below fp64 rounding, so the output is that key's value row, and the
    running max is its logit.  Logits near 1000 also overflow exp() unless the
    maximum is taken out first."""
    B, Hq, Hkv, dk, dv, T = 2, 4, 2, 8, 5, 50
    q, k, v, lens = _problem(3, B, Hq, Hkv, dk, dv, T, lens=[50, 33])
    q[:, :, 0] = 1.0
    pos = {(0, 0): 7, (0, 1): 49, (1, 0): 0, (1, 1): 32}
    for (b, g), p in pos.items():
        k[b, p, g, 0] = 1000.0
    out, c = orc.attend(q, k, v, lens, scale=1.0)
    hpk = Hq // Hkv
    for b in range(B):
        for h in range(Hq):
            g = h // hpk
            p = pos[(b, g)]
            _close(out[b, h], v[b, p, g], 1e-13, f"dominant b={b} h={h}")
            s_p = math.fsum(q[b, h, c_] * k[b, p, g, c_] for c_ in range(dk))
            _close(c.m[b * Hq + h], s_p, 1e-9, "max logit")
            _close(c.l[b * Hq + h], 1.0, 1e-14, "partition of dominant key")


def pin_planted_key(orc):
    """A planted key along the query returns its value row (cortiq-engine,
    NystromState page, example o1_recovery: a key pushed along the unit
    query with channel 0 of the values zero everywhere else).

    With V[j][0] = 0 for j != p and V[p][0] = 1, channel 0 of the exact
    output is the planted key's softmax weight
        w_p = 1 / sum_j exp(s_j - s_p),   s_j = <q, k_j> / sqrt(d),
    evaluated here at 50 digits from the stored float64 values (every
    float64 converts to a Decimal exactly), independently of the oracle.
    The other channels are the same weights applied to the background value
    rows.  Raising the amplitude must raise w_p towards 1 (recovery)."""
    spec = json.loads((GOLDEN / "planted_key.json").read_text())
    d, dv, n = spec["d"], spec["dv"], spec["n"]
    for case in spec["cases"]:
        rng = np.random.default_rng(case["seed"])
        u = rng.uniform(-1.0, 1.0, d)
        q_hat = u / np.linalg.norm(u)
        q = math.sqrt(d) * q_hat
        keys = spec["key_spread"] * rng.uniform(-1.0, 1.0, (n, d))
        vals = rng.uniform(-1.0, 1.0, (n, dv))
        vals[:, 0] = 0.0
        p = n - case["depth"]
        weights = []
        for amp in case["amps"]:
            k = keys.copy()
            v = vals.copy()
            k[p] += amp * q_hat
            v[p, 0] = 1.0
            out, c = orc.attend(q[None, None], k[None, :, None],
                                v[None, :, None], [n], scale=0.0)
            with localcontext() as ctx:
                ctx.prec = 50
                rs = Decimal(d).sqrt()
                s = [sum(Decimal(float(q[i])) * Decimal(float(k[j, i]))
                         for i in range(d)) / rs for j in range(n)]
                e = [(sj - s[p]).exp() for sj in s]
                den = sum(e)
                want = [float(sum(e[j] * Decimal(float(v[j, ch]))
                                  for j in range(n)) / den)
                        for ch in range(dv)]
                w_p = float(1 / den)
            assert abs(want[0] - w_p) <= 1e-15
            _close(out[0, 0, 0], w_p, 1e-13 * max(w_p, 1e-300),
                   f"planted weight amp={amp} depth={case['depth']}")
            _close(out[0, 0], np.array(want), 1e-13,
                   f"planted output amp={amp}")
            # m is the largest logit: the planted one once it leads
            if w_p > 0.5:
                _close(c.m[0], float(s[p]), 1e-12, "m at the planted key")
            weights.append(w_p)
        assert all(a < b for a, b in zip(weights, weights[1:])), \
            f"weight must grow with the amplitude: {weights}"
        assert weights[-1] > 0.99, "a large amplitude recovers the key"


# --- library routine ------------------------------------------------------

def pin_gqa_is_repeated_mha(orc):
    """GQA broadcasts each KV head to its group (needle-core module doc:
    each KV head serves its query heads without per-head copies).  It must
    equal plain multi-head attention on
    K/V repeat-copied per query head, which torch's fp64 CPU
    scaled_dot_product_attention computes independently.  scale = 0 must give
    torch's default 1/sqrt(key width) (dk != dv here)."""
    B, Hq, Hkv, dk, dv, T = 2, 12, 3, 24, 40, 29
    q, k, v, lens = _problem(4, B, Hq, Hkv, dk, dv, T, lens=[29, 11])
    hpk = Hq // Hkv
    out, _ = orc.attend(q, k, v, lens, scale=0.0)
    out_mha, _ = orc.attend(q, np.repeat(k, hpk, axis=2),
                            np.repeat(v, hpk, axis=2), lens, scale=0.0)
    _close(out, out_mha, 1e-14, "gqa vs repeated mha (oracle)")
    for b in range(B):
        n = int(lens[b])
        qt = torch.from_numpy(q[b]).reshape(1, Hq, 1, dk)
        kt = torch.from_numpy(np.ascontiguousarray(k[b, :n])).permute(1, 0, 2)
        vt = torch.from_numpy(np.ascontiguousarray(v[b, :n])).permute(1, 0, 2)
        kt = kt.repeat_interleave(hpk, dim=0).unsqueeze(0).contiguous()
        vt = vt.repeat_interleave(hpk, dim=0).unsqueeze(0).contiguous()
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt)
        _close(out[b], ref[0, :, 0].numpy(), 1e-13, f"vs torch sdpa b={b}")


# --- exact evaluation of the definition -----------------------------------

def pin_brute_force(orc):
    """Tiny dyadic inputs (exact in binary) evaluated at 50 digits straight
    from the softmax definition w_j = exp(s_j) / sum_i exp(s_i), with no max
    shift; m is the largest logit and l the sum of exp(s_j - m)."""
    B, Hq, Hkv, dk, dv, T = 2, 4, 2, 3, 3, 6
    q, k, v, lens = _problem(5, B, Hq, Hkv, dk, dv, T, lens=[6, 4],
                             dyadic=True)
    scale = 0.75
    out, c = orc.attend(q, k, v, lens, scale=scale)
    hpk = Hq // Hkv
    with localcontext() as ctx:
        ctx.prec = 50
        for b in range(B):
            n = int(lens[b])
            for h in range(Hq):
                g = h // hpk
                s = [Decimal(scale) * sum(Decimal(float(q[b, h, i])) *
                                          Decimal(float(k[b, j, g, i]))
                                          for i in range(dk))
                     for j in range(n)]
                ex = [x.exp() for x in s]
                z = sum(ex)
                for ch in range(dv):
                    want = sum(e * Decimal(float(v[b, j, g, ch]))
                               for j, e in enumerate(ex)) / z
                    got = Decimal(float(out[b, h, ch]))
                    assert abs(got - want) <= Decimal("1e-14"), \
                        f"brute force out b={b} h={h} c={ch}: {got} vs {want}"
                mx = max(s)
                lw = sum((x - mx).exp() for x in s)
                r = b * Hq + h
                assert abs(Decimal(float(c.m[r])) - mx) <= Decimal("1e-14"), \
                    "brute force m"
                assert abs(Decimal(float(c.l[r])) - lw) <= Decimal("1e-13"), \
                    "brute force l"
                for ch in range(dv):
                    wa = sum((x - mx).exp() * Decimal(float(v[b, j, g, ch]))
                             for j, x in enumerate(s))
                    assert abs(Decimal(float(c.acc[r, ch])) - wa) <= \
                        Decimal("1e-13"), "brute force acc"


# --- carry algebra --------------------------------------------------------

def pin_split_merge(orc):
    """Folding the carries of any split of the keys equals one pass over all
    of them (usearch carry: partial softmaxes rescaled to a common maximum).
    Checked for every
    split point, through merge() and through carry_in, and for every order of
    a three-way merge; the empty state is the identity."""
    B, Hq, Hkv, dk, dv, T = 2, 4, 2, 8, 6, 23
    q, k, v, lens = _problem(6, B, Hq, Hkv, dk, dv, T, lens=[23, 9])
    scale = 0.5
    out_all, c_all = orc.attend(q, k, v, lens, scale=scale)

    def part(lo, hi):
        ln = [max(0, min(int(x), hi) - lo) for x in lens]
        return orc.attend(q, k[:, lo:hi], v[:, lo:hi], ln, scale=scale)

    def same(c, what):
        _close(c.m, c_all.m, 1e-13, what + " m")
        _close(c.l, c_all.l, 1e-12, what + " l")
        _close(c.acc, c_all.acc, 1e-12, what + " acc")
        _close(orc.finalize(c).reshape(out_all.shape), out_all, 1e-13,
               what + " out")

    for s in range(T + 1):
        a, b_ = part(0, s)[1], part(s, T)[1]
        same(orc.merge(a, b_), f"split {s}")
        same(orc.merge(b_, a), f"split {s} swapped")
        ln = [max(0, int(x) - s) for x in lens]
        out2, c2 = orc.attend(q, k[:, s:], v[:, s:], ln, scale=scale,
                              carry_in=a)
        same(c2, f"carry_in split {s}")
    pieces = [part(0, 5)[1], part(5, 14)[1], part(14, T)[1]]
    for p in itertools.permutations(range(3)):
        x, y, z = (pieces[i] for i in p)
        same(orc.merge(orc.merge(x, y), z), f"three-way {p} left")
        same(orc.merge(x, orc.merge(y, z)), f"three-way {p} right")
    rows = B * Hq
    same(orc.merge(orc.empty_carry(rows, dv), c_all), "empty left")
    same(orc.merge(c_all, orc.empty_carry(rows, dv)), "empty right")
    zero_default = orc.Carry(np.zeros(rows), np.zeros(rows),
                             np.zeros((rows, dv)))
    same(orc.merge(zero_default, c_all), "default (0, 0) state is empty")


# --- special cases --------------------------------------------------------

def pin_special_cases(orc):
    """n = 1 returns its value row with l = 1; a vanishing scale gives the
    mean; permuting the live (K, V) rows changes nothing; the output is linear
    in V; an empty key set gives 0 and an empty carry, never NaN (DSA
    pool_states guard); lengths clamp into [0, max_len]."""
    B, Hq, Hkv, dk, dv, T = 2, 6, 3, 10, 7, 19
    q, k, v, lens = _problem(7, B, Hq, Hkv, dk, dv, T, lens=[1, 19])
    out, c = orc.attend(q, k, v, lens, scale=0.9)
    hpk = Hq // Hkv
    for h in range(Hq):
        g = h // hpk
        _close(out[0, h], v[0, 0, g], 0.0, "n = 1 output")
        _close(c.l[h], 1.0, 0.0, "n = 1 partition")
        s0 = 0.9 * math.fsum(q[0, h, i] * k[0, 0, g, i] for i in range(dk))
        _close(c.m[h], s0, 1e-14, "n = 1 max")

    out_tiny, _ = orc.attend(q, k, v, lens, scale=1e-30)
    for h in range(Hq):
        g = h // hpk
        want = [math.fsum(v[1, :19, g, ch]) / 19 for ch in range(dv)]
        _close(out_tiny[1, h], want, 1e-14, "vanishing scale mean")

    perm = np.random.default_rng(8).permutation(19)
    kp, vp = k.copy(), v.copy()
    kp[1, :19], vp[1, :19] = k[1, perm], v[1, perm]
    outp, cp = orc.attend(q, kp, vp, lens, scale=0.9)
    _close(outp, out, 1e-14, "permutation invariance")
    _close(cp.m, c.m, 0.0, "permutation invariance of m")

    rng = np.random.default_rng(9)
    v2 = rng.uniform(-1, 1, v.shape)
    out2, _ = orc.attend(q, k, v2, lens, scale=0.9)
    out3, _ = orc.attend(q, k, 2.0 * v - 3.0 * v2, lens, scale=0.9)
    _close(out3, 2.0 * out - 3.0 * out2, 1e-13, "linearity in V")

    oute, ce = orc.attend(q, k, v, [0, -5], scale=0.9)
    assert np.all(oute == 0.0), "empty key set must give 0"
    assert np.all(ce.l == 0.0) and np.all(ce.acc == 0.0), "empty carry"
    assert np.all(np.isneginf(ce.m)), "empty carry max is -inf"

    outc, _ = orc.attend(q, k, v, [1, 10 ** 6], scale=0.9)
    _close(outc, out, 0.0, "length clamps to max_len")


def pin_kv_append(orc):
    """needle-core KvCache::push_kv: a full cache is left untouched (the page
    warns and returns); otherwise slot `len` receives the token's rows for
    every KV head and the length grows by one.  Bit copy on uint16 words."""
    B, T, Hkv, dk, dv = 5, 4, 3, 6, 2
    rng = np.random.default_rng(10)
    k = rng.integers(0, 65536, (B, T, Hkv, dk), dtype=np.uint16)
    v = rng.integers(0, 65536, (B, T, Hkv, dv), dtype=np.uint16)
    kn = rng.integers(0, 65536, (B, Hkv, dk), dtype=np.uint16)
    vn = rng.integers(0, 65536, (B, Hkv, dv), dtype=np.uint16)
    lens = np.array([0, 2, 4, 3, 7], dtype=np.int32)
    k2, v2, lens2, dropped = orc.kv_append(k, v, kn, vn, lens)
    assert list(lens2) == [1, 3, 4, 4, 7], f"lens after append {lens2}"
    assert dropped == 2, f"dropped {dropped}"
    for b, slot in [(0, 0), (1, 2), (3, 3)]:
        assert np.array_equal(k2[b, slot], kn[b]) and \
            np.array_equal(v2[b, slot], vn[b]), f"written row b={b}"
        keep = [s for s in range(T) if s != slot]
        assert np.array_equal(k2[b, keep], k[b, keep]), "other slots kept"
        assert np.array_equal(v2[b, keep], v[b, keep]), "other slots kept"
    for b in (2, 4):
        assert np.array_equal(k2[b], k[b]) and np.array_equal(v2[b], v[b]), \
            "full cache untouched"


ALL_PINS = [pin_equal_keys, pin_dominant_key, pin_planted_key,
            pin_gqa_is_repeated_mha, pin_brute_force, pin_split_merge,
            pin_special_cases, pin_kv_append]


# --- additive logit bias (needle-core attn_bias) ---------------------------

def pin_bias(orc):
    """The additive bias of needle-core self_attn_incremental, one value per
    (sequence, position) shared by all heads and added to the scaled dot
    product:
    * bias_j = ln w_j (w_j > 0) weights key j by w_j: checked at 50 digits
      straight from out = sum_j w_j e^(s_j) v_j / sum_j w_j e^(s_j), with m
      the largest biased logit and l the partition against it;
    * a constant bias leaves out and l unchanged and shifts m by it;
    * a bias of -inf on a set of keys equals attending over the other keys
      (a cache with those rows taken out);
    * a row whose every key is removed is empty (out 0, carry (-inf, 0, 0)),
      and with a carry_in it returns the carry_in."""
    B, Hq, Hkv, dk, dv, T = 2, 4, 2, 3, 3, 6
    q, k, v, lens = _problem(11, B, Hq, Hkv, dk, dv, T, lens=[6, 5],
                             dyadic=True)
    scale = 0.75
    rng = np.random.default_rng(12)
    w = rng.uniform(0.2, 3.0, (B, T))
    bias = np.log(w)
    out, c = orc.attend(q, k, v, lens, scale=scale, bias=bias)
    hpk = Hq // Hkv
    with localcontext() as ctx:
        ctx.prec = 50
        for b in range(B):
            n = int(lens[b])
            for h in range(Hq):
                g = h // hpk
                s = [Decimal(scale) * sum(Decimal(float(q[b, h, i])) *
                                          Decimal(float(k[b, j, g, i]))
                                          for i in range(dk))
                     for j in range(n)]
                ww = [Decimal(float(w[b, j])) for j in range(n)]
                ex = [wj * x.exp() for wj, x in zip(ww, s)]
                z = sum(ex)
                for ch in range(dv):
                    want = sum(e * Decimal(float(v[b, j, g, ch]))
                               for j, e in enumerate(ex)) / z
                    assert abs(Decimal(float(out[b, h, ch])) - want) <= \
                        Decimal("1e-13"), f"weighted keys b={b} h={h}"
                sb = [x + Decimal(float(bias[b, j])) for j, x in enumerate(s)]
                mx = max(sb)
                r = b * Hq + h
                assert abs(Decimal(float(c.m[r])) - mx) <= Decimal("1e-13"), \
                    "m is the largest biased logit"
                lw = sum((x - mx).exp() for x in sb)
                assert abs(Decimal(float(c.l[r])) - lw) <= Decimal("1e-12"), \
                    "l against the biased maximum"

    # constant bias: shift invariance
    q, k, v, lens = _problem(13, 2, 8, 4, 16, 8, 29, lens=[29, 11])
    out0, c0 = orc.attend(q, k, v, lens, scale=0.4)
    outc, cc = orc.attend(q, k, v, lens, scale=0.4,
                          bias=np.full((2, 29), 2.5))
    _close(outc, out0, 1e-13, "constant bias: out")
    _close(cc.l, c0.l, 1e-11, "constant bias: l")
    _close(cc.m, c0.m + 2.5, 1e-13, "constant bias: m shifts")

    # -inf on a key set == the cache without those keys; one row all removed
    q, k, v, lens = _problem(14, 3, 8, 4, 16, 8, 21, lens=[21, 13, 7])
    keep = np.ones((3, 21), dtype=bool)
    keep[0, [0, 5, 6, 20]] = False
    keep[1, 3:9] = False
    keep[2, :7] = False            # every key of sequence 2 removed
    bias = np.where(keep, 0.0, -np.inf)
    outm, cm = orc.attend(q, k, v, lens, scale=0.3, bias=bias)
    for b in range(3):
        n = int(lens[b])
        idx = [j for j in range(n) if keep[b, j]]
        kk = np.full_like(k[b:b + 1], np.nan)
        vv = np.full_like(v[b:b + 1], np.nan)
        kk[0, :len(idx)] = k[b, idx]
        vv[0, :len(idx)] = v[b, idx]
        want, cw = orc.attend(q[b:b + 1], kk, vv, [len(idx)], scale=0.3)
        _close(outm[b], want[0], 1e-14, f"masked keys b={b}")
        rows = slice(b * 8, (b + 1) * 8)
        _close(cm.m[rows], cw.m, 1e-14, f"masked m b={b}")
        _close(cm.l[rows], cw.l, 1e-12, f"masked l b={b}")
    assert np.all(outm[2] == 0.0) and np.all(np.isneginf(cm.m[16:24])) and \
        np.all(cm.l[16:24] == 0.0), "all keys removed: empty"
    cin = orc.Carry(np.full(24, 0.7), np.full(24, 2.0), np.ones((24, 8)))
    outi, ci = orc.attend(q, k, v, lens, scale=0.3, bias=bias, carry_in=cin)
    _close(outi[2], np.full((8, 8), 0.5), 1e-15, "removed row returns carry_in")
    _close(ci.m[16:24], np.full(8, 0.7), 0.0, "removed row keeps carry_in m")


ALL_PINS.append(pin_bias)


# --- several caches as one; the sink / ring / main layout -----------------

def pin_branches(orc_stream):
    """attend_branches over caches of different lengths (some empty) equals
    one pass over each sequence's concatenated live keys, in any order, and
    folds carry_in like a single branch does."""
    import oracle.attention as att
    rng = np.random.default_rng(21)
    B, Hq, Hkv, dk, dv = 3, 8, 4, 16, 8
    q = rng.uniform(-1, 1, (B, Hq, dk))
    branches = []
    for T, lens in ((5, [5, 0, 3]), (9, [2, 9, 0]), (13, [13, 7, 0])):
        k = rng.uniform(-1, 1, (B, T, Hkv, dk))
        v = rng.uniform(-1, 1, (B, T, Hkv, dv))
        branches.append((k, v, np.array(lens)))
    out, c = orc_stream.attend_branches(q, branches, scale=0.4)
    for perm in ((0, 1, 2), (2, 0, 1)):
        total = [sum(int(branches[i][2][b]) for i in range(3))
                 for b in range(B)]
        T = max(total)
        kc = np.full((B, T, Hkv, dk), np.nan)
        vc = np.full((B, T, Hkv, dv), np.nan)
        for b in range(B):
            rows_k = [branches[i][0][b, :branches[i][2][b]] for i in perm]
            rows_v = [branches[i][1][b, :branches[i][2][b]] for i in perm]
            n = total[b]
            if n:
                kc[b, :n] = np.concatenate(rows_k)
                vc[b, :n] = np.concatenate(rows_v)
        want, cw = att.attend(q, kc, vc, total, scale=0.4)
        _close(out, want, 1e-14, f"branches = one pass, order {perm}")
        _close(c.m, cw.m, 1e-14, "branches m")
        _close(c.l, cw.l, 1e-12, "branches l")
    cin = att.Carry(rng.uniform(-1, 1, B * Hq), rng.uniform(0.5, 2, B * Hq),
                    rng.uniform(-1, 1, (B * Hq, dv)))
    out2, c2 = orc_stream.attend_branches(q, branches, scale=0.4,
                                          carry_in=cin)
    want2 = att.finalize(att.merge(cin, c)).reshape(B, Hq, dv)
    _close(out2, want2, 1e-13, "branches fold carry_in")


def pin_stream(orc_stream):
    """The sink / ring / main layout over a run of decode steps: the sink
    holds the first S tokens, ring slot (p - S) % W holds token p for the
    last W tokens, main holds the evicted tokens in order; attending the
    three parts equals attending the whole history; a full main cache drops
    the new token; with no main cache the evicted tokens leave attention;
    with no sink the ring starts at token 0."""
    import oracle.attention as att
    rng = np.random.default_rng(22)
    B, Hq, Hkv, dk, dv = 3, 4, 2, 8, 8
    for S, W, M, use_main in ((4, 8, 20, True), (0, 6, 10, True),
                              (3, 5, 0, False)):
        sk = np.zeros((B, max(S, 1), Hkv, dk)) if S else None
        sv = np.zeros((B, max(S, 1), Hkv, dv)) if S else None
        rk = np.zeros((B, W, Hkv, dk))
        rv = np.zeros((B, W, Hkv, dv))
        mk = np.zeros((B, max(M, 1), Hkv, dk)) if use_main else None
        mv = np.zeros((B, max(M, 1), Hkv, dv)) if use_main else None
        count = np.array([0, 0, -1])           # sequence 2 is invalid
        hist_k = [[] for _ in range(B)]
        hist_v = [[] for _ in range(B)]
        for step in range(S + W + M + 3):
            kn = rng.uniform(-1, 1, (B, Hkv, dk))
            vn = rng.uniform(-1, 1, (B, Hkv, dv))
            before = count.copy()
            sk, sv, rk, rv, mk, mv, count, dropped = orc_stream.stream_append(
                sk, sv, rk, rv, mk, mv, kn, vn, count)
            exp_drop = 1                       # the invalid sequence
            for b in range(2):
                full = use_main and before[b] - S - W >= M
                if full:
                    exp_drop += 1
                    assert count[b] == before[b], "full main: no change"
                else:
                    assert count[b] == before[b] + 1, "count advances"
                    hist_k[b].append(kn[b])
                    hist_v[b].append(vn[b])
            assert count[2] == -1 and dropped == exp_drop, "drop count"
            q = rng.uniform(-1, 1, (B, Hq, dk))
            for b in range(2):
                t = int(count[b])
                ns, nw, nm = orc_stream.stream_lengths(t, S, W, M)
                assert ns + nw + nm == (t if use_main else min(t, S + W))
                for p in range(min(t, S)):
                    assert np.array_equal(sk[b, p], hist_k[b][p]), "sink"
                for p in range(max(S, t - W), t):
                    assert np.array_equal(rk[b, (p - S) % W], hist_k[b][p]) \
                        and np.array_equal(rv[b, (p - S) % W], hist_v[b][p]), \
                        "ring slot"
                for j in range(nm):
                    assert np.array_equal(mk[b, j], hist_k[b][S + j]) and \
                        np.array_equal(mv[b, j], hist_v[b][S + j]), "main"
                kept = list(range(min(t, S))) + \
                    list(range(max(S, t - W), t)) + \
                    (list(range(S, S + nm)) if use_main else [])
                if not kept:
                    continue
                kc = np.stack([hist_k[b][p] for p in kept])[None]
                vc = np.stack([hist_v[b][p] for p in kept])[None]
                want, _ = att.attend(q[b:b + 1], kc, vc, [len(kept)], 0.5)
                parts = [(rk[b:b + 1], rv[b:b + 1], [nw])]
                if S:
                    parts.insert(0, (sk[b:b + 1], sv[b:b + 1], [ns]))
                if use_main and nm:
                    parts.append((mk[b:b + 1], mv[b:b + 1], [nm]))
                got, _ = orc_stream.attend_branches(q[b:b + 1], parts, 0.5)
                _close(got, want, 1e-14, f"stream S={S} W={W} t={t}")


STREAM_PINS = [pin_branches, pin_stream]


def pin_gathered(orc_stream):
    """Index-gathered decode (metrale DSA topk_to_mask): equals attention
    with a -inf bias on every unselected key (the bias path is pinned on its
    own); duplicates collapse (a row with repeats equals the deduplicated
    row); order does not matter; INVALID and out-of-range entries drop; a
    row selecting [0, n) equals plain attention over n keys; a row selecting
    nothing is empty."""
    import oracle.attention as att
    rng = np.random.default_rng(23)
    B, Hq, Hkv, dk, dv, T = 4, 8, 4, 16, 8, 40
    q, k, v, lens = _problem(24, B, Hq, Hkv, dk, dv, T, lens=[40, 25, 7, 30])
    width = 12
    idx = rng.integers(0, 40, (B, width))
    idx[0, :3] = -1                  # INVALID padding
    idx[1, 4] = idx[1, 5] = 3        # a duplicate
    idx[1, 6] = 38                   # past the live length (25)
    idx[2] = -1                      # selects nothing
    idx[3] = np.r_[np.arange(10), -1, -1]   # the prefix [0, 10)
    out, c = orc_stream.attend_gathered(q, k, v, lens, idx, scale=0.4)
    bias = np.full((B, T), -np.inf)
    for b in range(B):
        for i in idx[b]:
            if 0 <= i < min(lens[b], T):
                bias[b, i] = 0.0
    want, cw = att.attend(q, k, v, lens, scale=0.4, bias=bias)
    _close(out, want, 1e-14, "gathered = masked by a -inf bias")
    _close(c.l, cw.l, 1e-12, "gathered l")
    assert np.all(out[2] == 0.0) and np.all(c.l[16:24] == 0.0), \
        "nothing selected: empty"
    want3, _ = att.attend(q[3:4], k[3:4], v[3:4], [10], scale=0.4)
    _close(out[3], want3[0], 1e-14, "prefix selection = plain attention")
    dedup = idx.copy()
    dedup[1, 5] = -1
    perm = rng.permutation(width)
    out2, _ = orc_stream.attend_gathered(q, k, v, lens, dedup[:, perm],
                                         scale=0.4)
    _close(out2, out, 1e-14, "duplicates collapse; order is free")


STREAM_PINS.append(pin_gathered)


# --- fp8 (E4M3) KV caches -----------------------------------------------------
# The format's definition fixes every value below: bias 7, 3 mantissa bits,
# subnormals m * 2^-9, NaN at S.1111.111 only, 448 the largest finite value.

_E4M3_KNOWN = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9,
               0x08: 2.0 ** -6, 0x38: 1.0, 0x39: 1.125, 0x3A: 1.25,
               0x3C: 1.5, 0x40: 2.0, 0x48: 4.0, 0x4B: 5.5, 0x77: 240.0,
               0x78: 256.0, 0x7E: 448.0, 0xB8: -1.0, 0xFE: -448.0}


def pin_fp8_format(orc8):
    """E4M3 decode: the known codes, NaN exactly at 0x7F and 0xFF, sign
    symmetry (0x80 is -0), and the spacing of consecutive non-negative codes:
    2^-9 through the subnormals and the first binade, then doubling with each
    exponent step (so the values rise strictly up to 448)."""
    vals = [orc8.e4m3_decode(c) for c in range(256)]
    for c, want in _E4M3_KNOWN.items():
        assert vals[c] == want, f"code {c:#04x}: {vals[c]} != {want}"
    assert [c for c in range(256) if math.isnan(vals[c])] == [0x7F, 0xFF]
    assert vals[0x80] == 0.0 and math.copysign(1.0, vals[0x80]) < 0, "-0"
    for c in range(0x7F):
        assert vals[c | 0x80] == -vals[c], f"sign of {c:#04x}"
    for c in range(0x7E):
        step = vals[c + 1] - vals[c]
        assert step == 2.0 ** (max(c >> 3, 1) - 10), f"spacing at {c:#04x}"
    assert np.array_equal(orc8.decode(np.arange(256, dtype=np.uint8)),
                          np.array(vals), equal_nan=True), "array decode"


def pin_fp8_encode(orc8):
    """Nearest finite code, ties to the even mantissa, saturation at 448, sign
    kept: every finite code round-trips; midpoints of adjacent codes go to
    the even one; the error of any value is at most half the local spacing."""
    finite = [c for c in range(256) if c not in (0x7F, 0xFF)]
    vals = orc8.decode(np.array(finite, dtype=np.uint8))
    assert orc8.encode(vals).tolist() == finite, "round trip of every code"
    cases = [(1.0625, 0x38), (1.1875, 0x3A), (2.0 ** -10, 0x00),
             (3 * 2.0 ** -10, 0x02), (5 * 2.0 ** -10, 0x02),
             (2.0 ** -6 + 2.0 ** -10, 0x08), (464.0, 0x7E), (-1.0625, 0xB8),
             (1.07, 0x39), (1.05, 0x38), (5.75, 0x4C), (449.0, 0x7E),
             (1e6, 0x7E), (-1e30, 0xFE), (np.inf, 0x7E),
             (-2.0 ** -12, 0x80), (-0.0, 0x80), (0.0, 0x00)]
    got = orc8.encode(np.array([x for x, _ in cases]))
    for (x, want), c in zip(cases, got.tolist()):
        assert c == want, f"encode({x}) = {c:#04x}, want {want:#04x}"
    rng = np.random.default_rng(31)
    x = np.exp2(rng.uniform(-12, np.log2(448.0), 4000))
    c = orc8.encode(x)
    err = np.abs(orc8.decode(c) - x)
    e = np.maximum(np.floor(np.log2(x)), -6)
    assert np.all(err <= np.exp2(e - 3) / 2), "more than half a spacing off"
    assert np.array_equal(orc8.encode(-x), c | 0x80), "sign symmetry"


def pin_fp8_quantize(orc8):
    """quantize(x, s) encodes x times the fp32 reciprocal of s: with s a power
    of two every code round-trips from its scaled value; 3 * fl(1 / 0.75)
    rounds to 4 and 17 * fl(1 / 3) to 5.5 (its nearest code).  Two inputs
    whose exact quotient is an E4M3 midpoint (1.0625, 1.1875) but whose
    product with the rounded reciprocal lands one fp32 step off it decide
    the reading: both give code 0x39 (the quotient would give 0x38, 0x3A)."""
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)],
                      dtype=np.uint8)
    for s in (0.125, 1.0, 32.0):
        x = (orc8.decode(finite) * s).astype(np.float32)
        assert np.array_equal(orc8.quantize(x, np.float32(s)), finite), \
            f"scale {s}"
    assert orc8.quantize(np.float32(3.0), np.float32(0.75)) == 0x48
    assert orc8.quantize(np.float32(17.0), np.float32(3.0)) == 0x4B
    assert orc8.quantize(np.float32(0.20383667945861816),
                         np.float32(0.19184628129005432)) == 0x39
    assert orc8.quantize(np.float32(0.5486176013946533),
                         np.float32(0.4619937837123871)) == 0x39


def _fp8_codes(rng, shape):
    """Random finite E4M3 codes of magnitude up to 4."""
    c = rng.integers(0, 0x49, shape)          # 0 .. 4.0
    return (c | (rng.integers(0, 2, shape) << 7)).astype(np.uint8)


def pin_fp8_attend(orc8):
    """Attention over fp8 caches, in closed form: (1) equal keys give each
    head the plain mean of its group's decoded values times the group's V
    scale; (2) two keys with known codes give sigmoid weights of the logit gap
    scale * k_scale * (q . (k1 - k0)).  Scales differ per (sequence, KV head)
    and between K and V; slots past each length hold NaN codes."""
    rng = np.random.default_rng(32)
    B, Hkv, hpk, dk, dv, T = 2, 3, 2, 16, 8, 10
    lens = np.array([7, 4])
    ks = np.array([[0.5, 1.5, 3.0], [0.25, 2.0, 5.0]])
    vs = np.array([[1.25, 0.5, 4.0], [3.0, 0.125, 1.5]])
    q = rng.uniform(-1, 1, (B, Hkv * hpk, dk))
    kc = np.repeat(_fp8_codes(rng, (B, 1, Hkv, dk)), T, axis=1)
    vc = _fp8_codes(rng, (B, T, Hkv, dv))
    for b in range(B):
        kc[b, lens[b]:] = 0x7F
        vc[b, lens[b]:] = 0xFF
    out, _ = orc8.attend_fp8(q, kc, vc, ks, vs, lens, scale=0.7)
    for b in range(B):
        for h in range(Hkv * hpk):
            g = h // hpk
            want = vs[b, g] * orc8.decode(vc[b, :lens[b], g]).mean(axis=0)
            _close(out[b, h], want, 1e-14, f"equal keys b{b} h{h}")
    # two keys: k0 = (1, 0, 0, 0), k1 = (2, 1, 0, 0)
    B, Hkv, hpk, d = 2, 3, 2, 4
    kc = np.zeros((B, 2, Hkv, d), dtype=np.uint8)
    kc[:, 0, :, 0] = 0x38
    kc[:, 1, :, 0] = 0x40
    kc[:, 1, :, 1] = 0x38
    vc = _fp8_codes(rng, (B, 2, Hkv, d))
    q = rng.uniform(-1, 1, (B, Hkv * hpk, d))
    out, _ = orc8.attend_fp8(q, kc, vc, ks, vs, [2, 2], scale=0.5)
    for b in range(B):
        for h in range(Hkv * hpk):
            g = h // hpk
            gap = 0.5 * ks[b, g] * (q[b, h, 0] + q[b, h, 1])
            w1 = 1.0 / (1.0 + math.exp(-gap))
            v0, v1 = orc8.decode(vc[b, 0, g]), orc8.decode(vc[b, 1, g])
            want = vs[b, g] * ((1 - w1) * v0 + w1 * v1)
            _close(out[b, h], want, 1e-14, f"two keys b{b} h{h}")


def pin_fp8_append(orc8):
    """Quantising append: rows whose values are codes times power-of-two
    scales (different for K and V and per KV head) land as those codes in
    slot lens[b]; a full cache drops the token; nothing else changes."""
    rng = np.random.default_rng(33)
    B, T, Hkv, d = 3, 5, 2, 8
    k = _fp8_codes(rng, (B, T, Hkv, d))
    v = _fp8_codes(rng, (B, T, Hkv, d))
    lens = np.array([0, 4, 5])
    ks = np.array([[0.25, 2.0], [8.0, 0.5], [1.0, 4.0]], dtype=np.float32)
    vs = np.array([[16.0, 0.125], [1.0, 2.0], [0.5, 0.25]], dtype=np.float32)
    kcode = _fp8_codes(rng, (B, Hkv, d))
    vcode = _fp8_codes(rng, (B, Hkv, d))
    kn = (orc8.decode(kcode) * ks[:, :, None]).astype(np.float32)
    vn = (orc8.decode(vcode) * vs[:, :, None]).astype(np.float32)
    k2, v2, l2, dropped = orc8.kv_append_fp8(k, v, kn, vn, ks, vs, lens)
    assert l2.tolist() == [1, 5, 5] and dropped == 1, "lengths, drops"
    for b, slot in ((0, 0), (1, 4)):
        assert np.array_equal(k2[b, slot], kcode[b]), f"K codes b{b}"
        assert np.array_equal(v2[b, slot], vcode[b]), f"V codes b{b}"
    keep = np.ones((B, T), dtype=bool)
    keep[0, 0] = keep[1, 4] = False
    assert np.array_equal(k2[keep], k[keep]) and \
        np.array_equal(v2[keep], v[keep]), "other slots untouched"


def pin_fp8_stream(orc8):
    """The streaming layout over fp8 caches whose parts share the scales:
    rows whose values are codes times power-of-two scales (per sequence and
    KV head, different for K and V) land in sink / ring / main exactly as
    those codes over a run of steps (the evicted ring rows move to main as
    codes); a full main cache drops the token; attending the three decoded
    parts equals attending the decoded history."""
    import oracle.attention as att
    import oracle.streaming as st
    rng = np.random.default_rng(44)
    B, Hq, Hkv, d, S, W, M = 2, 4, 2, 8, 2, 3, 4
    ks = np.array([[0.25, 2.0], [8.0, 0.5]], dtype=np.float32)
    vs = np.array([[0.5, 4.0], [1.0, 0.125]], dtype=np.float32)
    z = lambda n: np.zeros((B, n, Hkv, d), dtype=np.uint8)
    sk, sv, rk, rv, mk, mv = z(S), z(S), z(W), z(W), z(M), z(M)
    count = np.array([0, 0])
    hist = [[], []]
    for step in range(S + W + M + 2):
        kc = _fp8_codes(rng, (B, Hkv, d))
        vc = _fp8_codes(rng, (B, Hkv, d))
        kn = (orc8.decode(kc) * ks[:, :, None]).astype(np.float32)
        vn = (orc8.decode(vc) * vs[:, :, None]).astype(np.float32)
        before = count.copy()
        sk, sv, rk, rv, mk, mv, count, dropped = orc8.stream_append_fp8(
            sk, sv, rk, rv, mk, mv, kn, vn, ks, vs, count)
        full = before - S - W >= M
        assert dropped == int(full.sum()), "drops"
        for b in range(B):
            if full[b]:
                assert count[b] == before[b], "full main: no change"
            else:
                assert count[b] == before[b] + 1, "count advances"
                hist[b].append((kc[b], vc[b]))
        for b in range(B):
            t = int(count[b])
            ns, nw, nm = st.stream_lengths(t, S, W, M)
            for p in range(ns):
                assert np.array_equal(sk[b, p], hist[b][p][0]), "sink codes"
            for p in range(max(S, t - W), t):
                assert np.array_equal(rk[b, (p - S) % W], hist[b][p][0]) and \
                    np.array_equal(rv[b, (p - S) % W], hist[b][p][1]), "ring"
            for j in range(nm):
                assert np.array_equal(mk[b, j], hist[b][S + j][0]) and \
                    np.array_equal(mv[b, j], hist[b][S + j][1]), "main codes"
            q = rng.uniform(-1, 1, (1, Hq, d))
            dq = lambda c: orc8.dequantize_cache(c, ks[b:b + 1])
            dv = lambda c: orc8.dequantize_cache(c, vs[b:b + 1])
            parts = [(dq(sk[b:b + 1]), dv(sv[b:b + 1]), [ns]),
                     (dq(rk[b:b + 1]), dv(rv[b:b + 1]), [nw]),
                     (dq(mk[b:b + 1]), dv(mv[b:b + 1]), [nm])]
            got, _ = st.attend_branches(q, parts, 0.5)
            hk = np.stack([h[0] for h in hist[b]])[None]
            hv = np.stack([h[1] for h in hist[b]])[None]
            want, _ = att.attend(q, dq(hk), dv(hv), [t], 0.5)
            _close(got, want, 1e-14, f"fp8 stream t={t}")


FP8_PINS = [pin_fp8_format, pin_fp8_encode, pin_fp8_quantize,
            pin_fp8_attend, pin_fp8_append, pin_fp8_stream]
