"""HIP path vs the CPU oracle, element by element, at sizes the oracle finishes
in seconds: every workload shape shrunk to span several 32-token tiles and
split-K chunks with a ragged tail, plus the edge cases (empty and length-1
sequences, lengths past max_len, chunk boundaries, group sizes 1 and 16,
every compiled head width), the carry chain and merge, and the append."""

import numpy as np
import pytest
import torch

import oracle
from gpu_util import (check_carry, check_out, live_vmax, np64, oracle_rows,
                      say, to_dev)
from gqa_kv_cache_decode_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _gqa():
    import gqa_kv_cache_decode_amd as g
    return g


def _all_units(w):
    return [(b, g) for b in range(w.batch) for g in range(w.num_kv_heads)]


def _attend_vs_oracle(w, x, plan_chunk=None, what=""):
    g = _gqa()
    d = to_dev(x)
    rows = w.batch * w.num_q_heads
    cout = g.empty_carry(rows, w.dv)
    if plan_chunk is None:
        out = g.attend_decode(d["q"], d["k"], d["v"], d["lens"], w.scale,
                              carry_out=cout, out=torch.empty(
                                  w.batch, w.num_q_heads, w.dv, device="cuda"))
    else:
        plan = g.attend_plan(d["k"], d["v"], w.num_q_heads, plan_chunk)
        ws = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device="cuda")
        g.attend_partition(d["q"], d["k"], d["v"], d["lens"], plan, ws, w.scale)
        out = g.attend_combine(w.num_q_heads, d["k"], d["v"], d["lens"], plan,
                               ws, carry_out=cout, out=torch.empty(
                                   w.batch, w.num_q_heads, w.dv, device="cuda"))
    torch.cuda.synchronize()
    ref = oracle_rows(x, w, _all_units(w))
    got = out.cpu().numpy()
    want = np.stack([np.stack([ref[(b, h)][0] for h in range(w.num_q_heads)])
                     for b in range(w.batch)])
    vmax = live_vmax(x["v"], x["lens"])
    err = check_out(got, want, vmax, w.dtype, what or w.name)
    m_want = np.array([ref[(b, h)][1] for b in range(w.batch)
                       for h in range(w.num_q_heads)])
    l_want = np.array([ref[(b, h)][2] for b in range(w.batch)
                       for h in range(w.num_q_heads)])
    check_carry(cout.m.cpu().numpy(), cout.l.cpu().numpy(), m_want, l_want,
                w.dtype, what or w.name)
    acc_got = cout.acc.cpu().numpy()
    l_got = cout.l.cpu().numpy()
    live = l_got > 0
    ratio = np.zeros_like(acc_got)
    ratio[live] = acc_got[live] / l_got[live][:, None]
    check_out(ratio.reshape(got.shape), want, vmax, w.dtype,
              (what or w.name) + " carry acc/l")
    return got, err


SMALL = {
    "tiny_f32": wl.TINY_F32,
    "batched_bf16": wl.BATCHED_BF16.replace(batch=3, max_len=1000),
    "ragged_bf16": wl.RAGGED_BF16.replace(batch=6, max_len=3000),
    "long_bf16": wl.LONG_WINDOW_BF16.replace(max_len=5000, window=0),
    "spike_bf16": wl.WIDE_SPIKE_BF16.replace(batch=2, max_len=4000),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_attend_small(name):
    w = SMALL[name]
    say(f"[attend_small] {name} {w}")
    x = wl.make_inputs(w)
    _attend_vs_oracle(w, x, what=name)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("chunk", [64, 128, 256, 1024, 4096])
def test_split_independence(chunk, dtype):
    """Any chunking of the key axis gives the oracle's answer."""
    w = wl.RAGGED_BF16.replace(batch=5, max_len=2500, num_q_heads=32,
                               dtype=dtype)
    x = wl.make_inputs(w, lens_override=[2500, 1, 777, 1024, 1025])
    say(f"[split] chunk={chunk} {dtype}")
    _attend_vs_oracle(w, x, plan_chunk=chunk, what=f"chunk {chunk} {dtype}")


def test_padding_never_read():
    """NaN padding and zero padding give bit-identical results."""
    g = _gqa()
    w = wl.RAGGED_BF16.replace(batch=4, max_len=1500)
    outs = []
    for pad in (float("nan"), 0.0, 1e30):
        x = to_dev(wl.make_inputs(w, pad_value=pad))
        outs.append(g.attend_decode(x["q"], x["k"], x["v"], x["lens"]).cpu())
    torch.cuda.synchronize()
    assert torch.isfinite(outs[0]).all()
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])


EDGE = [
    ("mha_hpk1", wl.BATCHED_BF16.replace(batch=2, num_q_heads=8,
                                         num_kv_heads=8, max_len=700)),
    ("hpk16_d128", wl.BATCHED_BF16.replace(batch=2, num_q_heads=32,
                                           num_kv_heads=2, max_len=900)),
    ("hpk3_odd", wl.BATCHED_BF16.replace(batch=2, num_q_heads=12,
                                         num_kv_heads=4, max_len=333)),
    ("bf16_d64", wl.BATCHED_BF16.replace(batch=2, dk=64, dv=64, max_len=1100)),
    ("bf16_d256", wl.BATCHED_BF16.replace(batch=2, dk=256, dv=256,
                                          num_q_heads=8, num_kv_heads=2,
                                          max_len=600)),
    ("bf16_dk192_uniform", wl.WIDE_SPIKE_BF16.replace(batch=1, max_len=1500,
                                                      dist="uniform")),
    ("f32_hpk16", wl.TINY_F32.replace(num_q_heads=32, num_kv_heads=2,
                                      max_len=500, batch=2)),
    ("f32_d128", wl.TINY_F32.replace(dk=128, dv=128, num_q_heads=8,
                                     num_kv_heads=2, max_len=300)),
    ("f32_dk96_dv32", wl.TINY_F32.replace(dk=96, dv=32, max_len=130)),
    ("f32_mha", wl.TINY_F32.replace(num_q_heads=4, num_kv_heads=4,
                                    max_len=70)),
    ("f32_dk192_dv128", wl.TINY_F32.replace(dk=192, dv=128, num_q_heads=16,
                                            num_kv_heads=2, max_len=400)),
    ("f32_d256", wl.TINY_F32.replace(dk=256, dv=256, num_q_heads=8,
                                     num_kv_heads=4, max_len=300, batch=2)),
    ("f32_valu_dk48_dv80", wl.TINY_F32.replace(dk=48, dv=80, max_len=200,
                                               batch=2)),
]


@pytest.mark.parametrize("name,w", EDGE, ids=[e[0] for e in EDGE])
def test_edge_shapes(name, w):
    say(f"[edge] {name}")
    x = wl.make_inputs(w, lens_override=None if w.batch == 1 else
                       [w.max_len, max(1, w.max_len // 3)][:w.batch])
    _attend_vs_oracle(w, x, what=name)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_lengths_edge(dtype):
    """Empty, length 1, chunk boundaries, and lengths past max_len (clamped)."""
    base = wl.BATCHED_BF16 if dtype == "bf16" else wl.TINY_F32
    w = base.replace(batch=8, max_len=600, num_q_heads=8, num_kv_heads=4,
                     dk=64, dv=64)
    lens = [0, 1, 31, 32, 33, 256, 257, 10 ** 6]
    x = wl.make_inputs(w, lens_override=[min(n, 600) for n in lens])
    x["lens"] = torch.tensor(lens, dtype=torch.int32)
    got, _ = _attend_vs_oracle(w, x, what=f"lengths {dtype}")
    assert np.all(got[0] == 0.0), "empty sequence must give 0"


def test_negative_length_is_empty():
    g = _gqa()
    w = wl.BATCHED_BF16.replace(batch=2, max_len=100)
    x = to_dev(wl.make_inputs(w))
    x["lens"] = torch.tensor([-3, 50], dtype=torch.int32, device="cuda")
    c = g.empty_carry(w.batch * w.num_q_heads, w.dv)
    out = g.attend_decode(x["q"], x["k"], x["v"], x["lens"], carry_out=c,
                          out=torch.empty(2, 32, 128, device="cuda"))
    torch.cuda.synchronize()
    assert torch.all(out[0] == 0) and torch.all(c.l[:32] == 0)
    assert torch.all(torch.isneginf(c.m[:32]))


def _window_inputs(w):
    x = wl.make_inputs(w)
    # the window branch is a second cache holding the recent tokens
    return x


def test_carry_chain_and_merge():
    """Main cache -> carry -> recent window folded in, three ways, against the
    oracle's one pass over the concatenated keys."""
    g = _gqa()
    w = wl.LONG_WINDOW_BF16.replace(batch=2, max_len=3000, window=128)
    x = _window_inputs(w)
    d = to_dev(x)
    rows = w.batch * w.num_q_heads
    # one pass over main ++ window (the oracle's view)
    kcat = torch.cat([x["k"], x["wk"]], dim=1)
    vcat = torch.cat([x["v"], x["wv"]], dim=1)
    out_ref, c_ref = oracle.attend(np64(x["q"]), np64(kcat), np64(vcat),
                                   [w.max_len + w.window] * w.batch, w.scale)
    vmax = max(live_vmax(x["v"], x["lens"]), live_vmax(x["wv"], x["wlens"]))

    # (1) chained: carry_out of the main branch is carry_in of the window
    c1 = g.empty_carry(rows, w.dv)
    g.attend_decode(d["q"], d["k"], d["v"], d["lens"], carry_out=c1, out=None)
    out1 = g.attend_decode(d["q"], d["wk"], d["wv"], d["wlens"], carry_in=c1,
                           carry_out=c1)  # carry_out aliases carry_in
    # (2) two branches, then softmax_state_merge
    ca, cb = g.empty_carry(rows, w.dv), g.empty_carry(rows, w.dv)
    g.attend_decode(d["q"], d["k"], d["v"], d["lens"], carry_out=ca, out=None)
    g.attend_decode(d["q"], d["wk"], d["wv"], d["wlens"], carry_out=cb, out=None)
    out2 = torch.empty(rows, w.dv, device="cuda")
    cm = g.softmax_state_merge(ca, cb, out=out2)
    # (3) merge in place into b (dst aliases b), window first
    out3 = torch.empty(rows, w.dv, device="cuda")
    g.softmax_state_merge(cb, ca, dst=cb, out=out3)
    torch.cuda.synchronize()
    for what, o in (("chained", out1.cpu().numpy()),
                    ("merged", out2.cpu().numpy().reshape(out_ref.shape)),
                    ("merged in place", out3.cpu().numpy().reshape(out_ref.shape))):
        check_out(o, out_ref, vmax, "bf16", what)
    for what, c in (("chained", c1), ("merged", cm), ("merged in place", cb)):
        check_carry(c.m.cpu().numpy(), c.l.cpu().numpy(), c_ref.m, c_ref.l,
                    "bf16", what)


def test_merge_empty_rows():
    """Empty states (l == 0, any m, including the all-zero default) are the
    identity of the merge; two empties give (-inf, 0, 0) and output 0."""
    g = _gqa()
    rows, dv = 6, 16
    gen = torch.Generator().manual_seed(5)
    a = g.Carry(torch.randn(rows, generator=gen).cuda(),
                torch.rand(rows, generator=gen).cuda() + 0.5,
                torch.randn(rows, dv, generator=gen).cuda())
    b = g.Carry(torch.zeros(rows).cuda(), torch.zeros(rows).cuda(),
                torch.zeros(rows, dv).cuda())
    b.l[1] = 2.0
    b.m[1] = 0.25
    b.acc[1] = 1.0
    a.l[2] = 0.0
    a.m[2] = 123.0  # ignored: the row is empty
    out = torch.empty(rows, dv, device="cuda")
    d = g.softmax_state_merge(a, b, out=out)
    torch.cuda.synchronize()
    ref = oracle.merge(oracle.Carry(*(t.cpu().double().numpy() for t in
                                      (a.m, a.l, a.acc))),
                       oracle.Carry(*(t.cpu().double().numpy() for t in
                                      (b.m, b.l, b.acc))))
    assert np.allclose(d.l.cpu().numpy(), ref.l, rtol=1e-6)
    assert np.allclose(out.cpu().numpy(), oracle.finalize(ref), atol=1e-6)
    assert d.l[2].item() == 0.0 and np.isneginf(d.m[2].item())
    assert torch.all(out[2] == 0)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_append_bit_exact(dtype):
    """kv_append against the oracle's push_kv model: written rows are bit
    copies, other slots are untouched, lens and the drop count exact."""
    g = _gqa()
    B, T, Hkv, dk, dv = 6, 9, 4, 64, 32
    gen = torch.Generator().manual_seed(7)
    k = torch.randn(B, T, Hkv, dk, generator=gen).to(dtype)
    v = torch.randn(B, T, Hkv, dv, generator=gen).to(dtype)
    kn = torch.randn(B, Hkv, dk, generator=gen).to(dtype)
    vn = torch.randn(B, Hkv, dv, generator=gen).to(dtype)
    lens = torch.tensor([0, 3, 9, 8, -1, 5], dtype=torch.int32)
    view = torch.int16 if dtype == torch.bfloat16 else torch.int32
    k_want, v_want, l_want, dropped_want = oracle.kv_append(
        k.view(view).numpy(), v.view(view).numpy(), kn.view(view).numpy(),
        vn.view(view).numpy(), lens.numpy())
    kd, vd, ld = k.cuda(), v.cuda(), lens.cuda()
    dropped = torch.zeros(1, dtype=torch.int32, device="cuda")
    lens_out = torch.empty_like(ld)
    g.kv_append(kd, vd, kn.cuda(), vn.cuda(), ld, lens_out=lens_out,
                dropped=dropped)
    torch.cuda.synchronize()
    assert np.array_equal(kd.cpu().view(view).numpy(), k_want)
    assert np.array_equal(vd.cpu().view(view).numpy(), v_want)
    assert lens_out.cpu().numpy().tolist() == l_want.tolist()
    assert ld.cpu().tolist() == lens.tolist(), "lens_in untouched"
    assert int(dropped.item()) == dropped_want
    # in place (lens_out aliases lens_in), a second token
    kn2 = torch.randn(B, Hkv, dk, generator=gen).to(dtype)
    vn2 = torch.randn(B, Hkv, dv, generator=gen).to(dtype)
    k_want2, v_want2, l_want2, dropped_want2 = oracle.kv_append(
        k_want, v_want, kn2.view(view).numpy(), vn2.view(view).numpy(),
        l_want)
    g.kv_append(kd, vd, kn2.cuda(), vn2.cuda(), lens_out, dropped=dropped)
    torch.cuda.synchronize()
    assert np.array_equal(kd.cpu().view(view).numpy(), k_want2)
    assert np.array_equal(vd.cpu().view(view).numpy(), v_want2)
    assert lens_out.cpu().numpy().tolist() == l_want2.tolist()
    assert int(dropped.item()) == dropped_want + dropped_want2


def test_decode_step_append_then_attend():
    """needle-core decode order: push the new token, then attend over the
    cache including it (ctx_len = cache.len after push_kv)."""
    g = _gqa()
    w = wl.BATCHED_BF16.replace(batch=3, max_len=520)
    x = wl.make_inputs(w, lens_override=[519, 100, 1])
    gen = torch.Generator().manual_seed(9)
    kn = torch.randn(3, 8, 128, generator=gen).to(torch.bfloat16)
    vn = torch.randn(3, 8, 128, generator=gen).to(torch.bfloat16)
    d = to_dev(x)
    lens_after = torch.empty_like(d["lens"])
    g.kv_append(d["k"], d["v"], kn.cuda(), vn.cuda(), d["lens"],
                lens_out=lens_after)
    out = g.attend_decode(d["q"], d["k"], d["v"], lens_after)
    torch.cuda.synchronize()
    k2 = x["k"].clone()
    v2 = x["v"].clone()
    for b, n in enumerate([519, 100, 1]):
        k2[b, n] = kn[b]
        v2[b, n] = vn[b]
    ref, _ = oracle.attend(np64(x["q"]), np64(k2), np64(v2), [520, 101, 2],
                           w.scale)
    check_out(out.cpu().numpy(), ref, live_vmax(v2, [520, 101, 2]), "bf16",
              "append then attend")
