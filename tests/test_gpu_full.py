"""The five workloads at full size, with the library's own split-K plan,
against the oracle on every (sequence, KV group) unit, plus properties that
hold at any size on every row (finite outputs, each output a convex
combination of value rows, 1 <= l <= n for the carry).  The ragged
workload's balanced launch also has its work queue checked."""

import numpy as np
import pytest
import torch

import oracle
from gpu_util import (check_carry, check_out, live_vmax, np64, oracle_rows,
                      say, to_dev)
from test_gpu_balanced import _check_queue
from gqa_kv_cache_decode_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _gqa():
    import gqa_kv_cache_decode_amd as g
    return g


def _run(w, d):
    g = _gqa()
    rows = w.batch * w.num_q_heads
    c = g.empty_carry(rows, w.dv)
    out = g.attend_decode(d["q"], d["k"], d["v"], d["lens"], w.scale,
                          carry_out=c)
    torch.cuda.synchronize()
    return out.cpu().numpy(), c


def _check_units(w, x, got, c, units, what):
    ref = oracle_rows(x, w, units)
    keys = sorted(ref)
    want = np.stack([ref[k][0] for k in keys])
    gotr = np.stack([got[b, h] for b, h in keys])
    vmax = live_vmax(x["v"], x["lens"])
    check_out(gotr, want, vmax, w.dtype, what)
    rows = [b * w.num_q_heads + h for b, h in keys]
    check_carry(c.m.cpu().numpy()[rows], c.l.cpu().numpy()[rows],
                np.array([ref[k][1] for k in keys]),
                np.array([ref[k][2] for k in keys]), w.dtype, what)
    return ref


def _properties(w, x, got, c, what):
    """Any size: outputs finite and inside the per-channel range of the
    group's live values (a softmax mix is convex); 1 <= l <= n."""
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    l = c.l.cpu().numpy().reshape(w.batch, w.num_q_heads)
    lens = np.minimum(np.maximum(x["lens"].numpy(), 0), w.max_len)
    slack = 1e-5 if w.dtype == "f32" else 4e-3
    for b in range(w.batch):
        n = int(lens[b])
        assert np.all(l[b] >= 1.0 - 1e-6) and np.all(l[b] <= n * (1 + 1e-5)), \
            f"{what}: partition out of [1, n] for b={b}"
        for g in range(w.num_kv_heads):
            vg = x["v"][b, :n, g].float()
            lo = vg.min(dim=0).values.numpy()
            hi = vg.max(dim=0).values.numpy()
            blk = got[b, g * w.hpk:(g + 1) * w.hpk]
            tol = slack * max(np.abs(lo).max(), np.abs(hi).max())
            assert np.all(blk >= lo - tol) and np.all(blk <= hi + tol), \
                f"{what}: output outside the value range (b={b}, g={g})"


def test_full_tiny_f32():
    w = wl.TINY_F32
    x = wl.make_inputs(w)
    got, c = _run(w, to_dev(x))
    units = [(b, g) for b in range(w.batch) for g in range(w.num_kv_heads)]
    _check_units(w, x, got, c, units, "tiny f32, every row")


def test_full_batched_bf16():
    w = wl.BATCHED_BF16
    say("[full] batched: drawing inputs")
    x = wl.make_inputs(w)
    got, c = _run(w, to_dev(x))
    units = [(b, g) for b in range(w.batch) for g in range(w.num_kv_heads)]
    _check_units(w, x, got, c, units, "batched bf16, every row")
    _properties(w, x, got, c, "batched bf16")


def test_full_ragged_bf16():
    """Every (sequence, KV group) unit of the ragged batch, through the
    partition / combine pair with the library's own (balanced) plan, whose
    device-built work queue is checked too."""
    g = _gqa()
    w = wl.RAGGED_BF16
    say("[full] ragged: drawing 8 GiB of K/V")
    x = wl.make_inputs(w)
    d = to_dev(x)
    plan = g.attend_plan(d["k"], d["v"], w.num_q_heads)
    ws = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device="cuda")
    g.attend_partition(d["q"], d["k"], d["v"], d["lens"], plan, ws, w.scale)
    c = g.empty_carry(w.batch * w.num_q_heads, w.dv)
    out = g.attend_combine(w.num_q_heads, d["k"], d["v"], d["lens"], plan, ws,
                           carry_out=c)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert plan.balanced_groups > 0, "balanced plan expected"
    _check_queue(ws, plan, x["lens"], w)
    del d, ws
    torch.cuda.empty_cache()
    units = [(b, g_) for b in range(w.batch) for g_ in range(w.num_kv_heads)]
    say(f"[full] ragged: oracle on all {len(units)} units")
    _check_units(w, x, got, c, units, "ragged bf16, every unit")
    _properties(w, x, got, c, "ragged bf16")


def test_full_long_context_with_window():
    """The long cache gives a carry; the 128-token window folds in with it;
    the oracle takes one pass over the concatenated keys."""
    g = _gqa()
    w = wl.LONG_WINDOW_BF16
    say("[full] long: drawing inputs")
    x = wl.make_inputs(w)
    d = to_dev(x)
    rows = w.batch * w.num_q_heads
    c = g.empty_carry(rows, w.dv)
    g.attend_decode(d["q"], d["k"], d["v"], d["lens"], carry_out=c, out=None)
    out = g.attend_decode(d["q"], d["wk"], d["wv"], d["wlens"], carry_in=c,
                          carry_out=c)
    torch.cuda.synchronize()
    kcat = torch.cat([x["k"], x["wk"]], dim=1)
    vcat = torch.cat([x["v"], x["wv"]], dim=1)
    ref, cref = oracle.attend(np64(x["q"]), np64(kcat), np64(vcat),
                              [w.max_len + w.window], w.scale)
    vmax = max(live_vmax(x["v"], x["lens"]), live_vmax(x["wv"], x["wlens"]))
    check_out(out.cpu().numpy(), ref, vmax, "bf16", "long + window, every row")
    check_carry(c.m.cpu().numpy(), c.l.cpu().numpy(), cref.m, cref.l, "bf16",
                "long + window carry")


def test_full_wide_spike():
    """Planted key at depth 1000 (cortiq-engine recovery trial at production
    shape): channel 0 of every head's output is exactly the planted key's
    softmax weight, since V[:, 0] is zero elsewhere."""
    w = wl.WIDE_SPIKE_BF16
    say("[full] spike: drawing inputs")
    x = wl.make_inputs(w)
    got, c = _run(w, to_dev(x))
    units = [(b, g) for b in range(w.batch) for g in range(w.num_kv_heads)]
    ref = _check_units(w, x, got, c, units, "spike bf16, every unit")
    _properties(w, x, got, c, "spike bf16")
    ratios = []
    for (b, h), (o, _, _, _) in ref.items():
        if h % w.hpk == 0:       # the head the spike was planted along
            ratios.append(got[b, h, 0] / o[0])
            assert o[0] > 1e-3, "planted key should carry visible weight"
    ratios = np.array(ratios)
    say(f"  recovery ratio got/want over planted heads: "
        f"{ratios.min():.6f} .. {ratios.max():.6f}")
    assert np.all(np.abs(ratios - 1.0) < 1e-3)
