"""decode_step at the benchmark's full sizes, in the launch configuration it
times: the new token appended at slot lens - 1 of every sequence (so the step
attends the whole cache, the new token included) by the step launch itself,
then split-K partials and the combine (the library's own plan).  Checked
against the oracle (needle-core push_kv then attend): the cache written bit
for bit, the lengths, and the output and carry on every (sequence, KV group)
unit.  The long-context
step is decode_step_branches over the main cache and the window, the new
token entering the window, against one oracle pass over the concatenated
keys."""

import numpy as np
import pytest
import torch

import oracle
import oracle.fp8 as of8
from gpu_util import (check_carry, check_out, live_vmax, np64, oracle_rows,
                      say, to_dev)
from gqa_kv_cache_decode_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _gqa():
    import gqa_kv_cache_decode_amd as g
    return g


def _new_rows(w, seed, dtype):
    gen = torch.Generator().manual_seed(seed)
    kn = torch.randn(w.batch, w.num_kv_heads, w.dk, generator=gen)
    vn = torch.randn(w.batch, w.num_kv_heads, w.dv, generator=gen)
    return kn.to(dtype), vn.to(dtype)


def _appended(x, kn, vn, slots, key="k", val="v"):
    """CPU copies of the caches with row `slots[b]` of every sequence
    replaced by the new rows (the oracle's push_kv on a free slot)."""
    k, v = x[key].clone(), x[val].clone()
    for b, p in enumerate(slots):
        k[b, p] = kn[b]
        v[b, p] = vn[b]
    return k, v


def _check_cache(dk_gpu, dv_gpu, k_want, v_want, what):
    assert torch.equal(dk_gpu.cpu().view(torch.uint8),
                       k_want.view(torch.uint8)), f"{what}: K cache bits"
    assert torch.equal(dv_gpu.cpu().view(torch.uint8),
                       v_want.view(torch.uint8)), f"{what}: V cache bits"


def _check_rows(w, x, got, cout, units, what):
    ref = oracle_rows(x, w, units)
    keys = sorted(ref)
    check_out(np.stack([got[b, h] for b, h in keys]),
              np.stack([ref[k][0] for k in keys]),
              live_vmax(x["v"], x["lens"]), w.dtype, what)
    rows = [b * w.num_q_heads + h for b, h in keys]
    check_carry(cout.m.cpu().numpy()[rows], cout.l.cpu().numpy()[rows],
                np.array([ref[k][1] for k in keys]),
                np.array([ref[k][2] for k in keys]), w.dtype, what + " carry")


def _step(w, x, kn, vn, bias=None):
    g = _gqa()
    d = to_dev(x)
    lens_in = (d["lens"] - 1).clamp_(min=0)
    lens_out = torch.full_like(lens_in, -1)
    dropped = torch.zeros(1, dtype=torch.int32, device="cuda")
    cout = g.empty_carry(w.batch * w.num_q_heads, w.dv)
    ws = g.step_workspace(d["k"], d["v"], w.num_q_heads)
    out = g.decode_step(d["q"], d["k"], d["v"], kn.cuda(), vn.cuda(), lens_in,
                        lens_out, w.scale, carry_out=cout, workspace=ws,
                        dropped=dropped,
                        bias=None if bias is None else bias.cuda())
    torch.cuda.synchronize()
    assert lens_out.cpu().tolist() == x["lens"].tolist(), "lens_out"
    assert int(dropped.item()) == 0, "no sequence is full"
    plan = g.attend_plan(d["k"], d["v"], w.num_q_heads)
    assert torch.all(ws[plan.workspace_bytes:] == 0), "counters back to zero"
    return d, out.cpu().numpy(), cout, lens_in.cpu().tolist()


@pytest.mark.parametrize("with_bias", [False, True])
def test_full_step_batched_bf16(with_bias):
    """bench.py's default step (and its --bias form): every unit."""
    w = wl.BATCHED_BF16
    say(f"[full step] batched bias={with_bias}: drawing inputs")
    x = wl.make_inputs(w)
    kn, vn = _new_rows(w, w.seed + 1000, torch.bfloat16)
    bias = None
    if with_bias:
        gen = torch.Generator().manual_seed(w.seed + 2000)
        bias = torch.randn(w.batch, w.max_len, generator=gen)
    d, got, cout, slots = _step(w, x, kn, vn, bias)
    x["k"], x["v"] = _appended(x, kn, vn, slots)
    _check_cache(d["k"], d["v"], x["k"], x["v"], "batched step")
    del d
    units = [(b, g) for b in range(w.batch) for g in range(w.num_kv_heads)]
    if bias is None:
        _check_rows(w, x, got, cout, units, "batched step, every row")
        return
    bias_np = bias.double().numpy()
    want, cw = oracle.attend(np64(x["q"]), np64(x["k"]), np64(x["v"]),
                             x["lens"].numpy(), w.scale, bias=bias_np)
    check_out(got, want, live_vmax(x["v"], x["lens"]), "bf16",
              "batched step + bias, every row")
    check_carry(cout.m.cpu().numpy(), cout.l.cpu().numpy(), cw.m, cw.l,
                "bf16", "batched step + bias carry")


def test_full_step_ragged():
    """bench.py's headline step: the ragged batch (64 sequences of 1..32768
    keys, NaN padding past each length), scheduled, the new token at slot
    lens - 1; the whole cache bit for bit and every unit."""
    w = wl.RAGGED_BF16
    say("[full step] ragged: drawing 8 GiB of K/V")
    x = wl.make_inputs(w)
    kn, vn = _new_rows(w, w.seed + 1000, torch.bfloat16)
    d, got, cout, slots = _step(w, x, kn, vn)
    assert slots == (x["lens"] - 1).tolist()
    x["k"], x["v"] = _appended(x, kn, vn, slots)
    _check_cache(d["k"], d["v"], x["k"], x["v"], "ragged step")
    del d
    torch.cuda.empty_cache()
    units = [(b, g) for b in range(w.batch) for g in range(w.num_kv_heads)]
    _check_rows(w, x, got, cout, units, "ragged step, every unit")


def test_full_step_wide_spike():
    """The spike shape (dk 192, 16 heads per KV group, 64K keys, every cache
    full but the new slot): every unit."""
    w = wl.WIDE_SPIKE_BF16
    say("[full step] spike: drawing inputs")
    x = wl.make_inputs(w)
    kn, vn = _new_rows(w, w.seed + 1000, torch.bfloat16)
    d, got, cout, slots = _step(w, x, kn, vn)
    assert slots == [w.max_len - 1] * w.batch
    # the new rows land in slot T - 1; every other row is unchanged
    kd = d["k"][:, slots[0]].cpu()
    vd = d["v"][:, slots[0]].cpu()
    assert torch.equal(kd.view(torch.int16), kn.view(torch.int16)), "K slot"
    assert torch.equal(vd.view(torch.int16), vn.view(torch.int16)), "V slot"
    assert torch.equal(d["k"][:, :slots[0]].cpu().view(torch.int16),
                       x["k"][:, :slots[0]].view(torch.int16)), "K untouched"
    del d
    x["k"], x["v"] = _appended(x, kn, vn, slots)
    units = [(b, g) for b in range(w.batch) for g in range(w.num_kv_heads)]
    _check_rows(w, x, got, cout, units, "spike step, every unit")


def test_full_step_fp8():
    """bench.py's fp8 step: the new bf16 rows quantised into the codes in
    the step launch, attended as decoded; every unit."""
    g = _gqa()
    w = wl.BATCHED_FP8
    say("[full step] fp8: drawing inputs")
    x = wl.make_fp8_inputs(w)
    kn, vn = _new_rows(w, w.seed + 1000, torch.bfloat16)
    kc = g.Fp8Cache(x["k"].cuda(), x["k_scale"].cuda())
    vc = g.Fp8Cache(x["v"].cuda(), x["v_scale"].cuda())
    lens_in = (x["lens"] - 1).clamp(min=0)
    li, lo = lens_in.cuda(), torch.full_like(lens_in, -1).cuda()
    cout = g.empty_carry(w.batch * w.num_q_heads, w.dv)
    ws = g.step_workspace(kc, vc, w.num_q_heads)
    out = g.decode_step(x["q"].cuda(), kc, vc, kn.cuda(), vn.cuda(), li, lo,
                        w.scale, carry_out=cout, workspace=ws)
    torch.cuda.synchronize()
    k2, v2, l2, nd = of8.kv_append_fp8(
        x["k"].numpy(), x["v"].numpy(), kn.float().numpy(),
        vn.float().numpy(), x["k_scale"].numpy(), x["v_scale"].numpy(),
        lens_in.numpy())
    assert lo.cpu().tolist() == l2.tolist() and nd == 0, "lens"
    assert np.array_equal(kc.codes.cpu().numpy(), k2), "K codes"
    assert np.array_equal(vc.codes.cpu().numpy(), v2), "V codes"
    got = out.cpu().numpy()
    m_got, l_got = cout.m.cpu().numpy(), cout.l.cpu().numpy()
    ks, vs = x["k_scale"].double().numpy(), x["v_scale"].double().numpy()
    q = np64(x["q"])
    hpk = w.hpk
    outs, wants, mg, lg, mw, lw, vmax = [], [], [], [], [], [], 0.0
    for b in range(w.batch):
        n = int(l2[b])
        for kg in range(w.num_kv_heads):
            hs = slice(kg * hpk, (kg + 1) * hpk)
            want, cw = of8.attend_fp8(
                q[b:b + 1, hs], k2[b:b + 1, :, kg:kg + 1],
                v2[b:b + 1, :, kg:kg + 1], ks[b:b + 1, kg:kg + 1],
                vs[b:b + 1, kg:kg + 1], [n], w.scale)
            wants.append(want[0])
            outs.append(got[b, hs])
            rows = [b * w.num_q_heads + kg * hpk + i for i in range(hpk)]
            mg.append(m_got[rows])
            lg.append(l_got[rows])
            mw.append(cw.m)
            lw.append(cw.l)
            vals = of8.dequantize_cache(v2[b:b + 1, :n, kg:kg + 1],
                                        vs[b:b + 1, kg:kg + 1])
            vmax = max(vmax, float(np.abs(vals).max()))
    check_out(np.stack(outs), np.stack(wants), vmax, "fp8",
              "fp8 step, every row")
    check_carry(np.concatenate(mg), np.concatenate(lg), np.concatenate(mw),
                np.concatenate(lw), "fp8", "fp8 step carry")


def test_full_step_long_context_branches():
    """bench.py's long-context step: decode_step_branches over the 256K-key
    main cache and the 128-slot window, the new token appended to the
    window in the same launch; the oracle attends the concatenation."""
    g = _gqa()
    w = wl.LONG_WINDOW_BF16
    say("[full step] long: drawing inputs")
    x = wl.make_inputs(w)
    d = to_dev(x)
    kn, vn = _new_rows(w, w.seed + 1000, torch.bfloat16)
    wl_in = (d["wlens"] - 1).clamp_(min=0)
    wl_out = torch.full_like(wl_in, -1)
    out = g.decode_step_branches(
        d["q"], [(d["k"], d["v"], d["lens"], None),
                 (d["wk"], d["wv"], wl_in, None)], 1,
        kn.cuda(), vn.cuda(), wl_out, w.scale)
    cout = g.empty_carry(w.batch * w.num_q_heads, w.dv)
    out2 = g.decode_step_branches(
        d["q"], [(d["k"], d["v"], d["lens"], None),
                 (d["wk"], d["wv"], wl_in, None)], 1,
        kn.cuda(), vn.cuda(), wl_out, w.scale, carry_out=cout)
    torch.cuda.synchronize()
    assert wl_out.cpu().tolist() == x["wlens"].tolist(), "window lens_out"
    assert torch.equal(out, out2), "repeating the step (same slot) differs"
    slots = wl_in.cpu().tolist()
    wk, wv = _appended(x, kn, vn, slots, key="wk", val="wv")
    _check_cache(d["wk"], d["wv"], wk, wv, "window after the step")
    del d
    kcat = torch.cat([x["k"], wk], dim=1)
    vcat = torch.cat([x["v"], wv], dim=1)
    ref, cref = oracle.attend(np64(x["q"]), np64(kcat), np64(vcat),
                              [w.max_len + w.window], w.scale)
    vmax = max(live_vmax(x["v"], x["lens"]), live_vmax(wv, x["wlens"]))
    check_out(out.cpu().numpy(), ref, vmax, "bf16", "long step, every row")
    check_carry(cout.m.cpu().numpy(), cout.l.cpu().numpy(), cref.m, cref.l,
                "bf16", "long step carry")
