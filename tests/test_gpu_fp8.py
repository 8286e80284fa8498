"""fp8 (E4M3) KV caches on the GPU against the oracle: every code decoded
exactly (through V directly, through K via the logits), the quantising
append bit for bit (rounding, ties, saturation, signed zero, a full cache),
attention over every compiled head width and every kind of plan (split-K
with the combine kernel, a single chunk written directly, an explicit and a
scheduled plan), with a bias and a carry, the fused decode step (append
quantised in the same launch), and the multi-branch and index-gathered
launches over fp8 caches."""

import numpy as np
import pytest
import torch

import oracle
import oracle.fp8 as of8
import oracle.streaming as ost
from gpu_util import check_carry, check_out, np64, say
from gqa_kv_cache_decode_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _gqa():
    import gqa_kv_cache_decode_amd as g
    return g


def _caches(g, x, key="k", val="v"):
    return (g.Fp8Cache(x[key].cuda(), x["k_scale"].cuda()),
            g.Fp8Cache(x[val].cuda(), x["v_scale"].cuda()))


def _oracle(x, w, lens=None, carry_in=None, bias=None, k=None, v=None):
    return of8.attend_fp8(
        np64(x["q"]), (x["k"] if k is None else k).numpy(),
        (x["v"] if v is None else v).numpy(), x["k_scale"].double().numpy(),
        x["v_scale"].double().numpy(),
        (x["lens"] if lens is None else lens).numpy(), w.scale,
        carry_in=carry_in, bias=bias)


def _vmax(x, lens=None, v=None):
    vals = of8.dequantize_cache((x["v"] if v is None else v).numpy(),
                                x["v_scale"].double().numpy())
    lens = x["lens"] if lens is None else lens
    m = 0.0
    for b in range(vals.shape[0]):
        n = int(min(max(int(lens[b]), 0), vals.shape[1]))
        if n:
            m = max(m, float(np.abs(vals[b, :n]).max()))
    return m


def _carry(g, rows, dv, seed):
    gen = torch.Generator().manual_seed(seed)
    m = torch.randn(rows, generator=gen)
    l = torch.rand(rows, generator=gen) + 0.5
    l[::3] = 0.0
    acc = torch.randn(rows, dv, generator=gen)
    return (g.Carry(m.cuda(), l.cuda(), acc.cuda()),
            oracle.Carry(m.double().numpy(), l.double().numpy(),
                         acc.double().numpy()))


FINITE = [c for c in range(256) if c not in (0x7F, 0xFF)]


def test_e4m3_decode_every_code():
    """V: one live key per sequence, so out = decode(code) * v_scale for
    every finite code.  K: two keys, k0 = 0 and k1 with the code under test
    at dimension 0, q = e0, V = (0, 1): out = sigmoid(scale * k_scale *
    decode(code)) with k_scale chosen so that the logit is +-1 whatever the
    code's magnitude; a wrong decode of any code moves the logit."""
    g = _gqa()
    B, Hkv, d = 32, 8, 128          # 256 units, one per code (two repeat)
    codes = torch.tensor(FINITE + FINITE[:2], dtype=torch.uint8)
    vals = of8.decode(codes.numpy())
    # V path
    v = torch.full((B, 4, Hkv, d), 0x7F, dtype=torch.uint8)
    reps = B * Hkv * d // len(FINITE) + 1
    v[:, 0] = torch.tensor(FINITE * reps, dtype=torch.uint8)[
        :B * Hkv * d].view(B, Hkv, d)
    k = torch.zeros((B, 4, Hkv, d), dtype=torch.uint8)
    gen = torch.Generator().manual_seed(80)
    x = {"q": torch.randn(B, Hkv, d, generator=gen).to(torch.bfloat16),
         "k": k, "v": v,
         "lens": torch.ones(B, dtype=torch.int32),
         "k_scale": torch.rand(B, Hkv, generator=gen) + 0.5,
         "v_scale": torch.rand(B, Hkv, generator=gen) * 2 + 0.25}
    w = wl.BATCHED_FP8.replace(batch=B, num_q_heads=Hkv, num_kv_heads=Hkv,
                               max_len=4)
    kc, vc = _caches(g, x)
    say("[fp8] decode every code: V")
    out = g.attend_decode(x["q"].cuda(), kc, vc, x["lens"].cuda(), 0.0)
    torch.cuda.synchronize()
    want = of8.decode(v[:, 0].numpy()) * x["v_scale"].double().numpy()[:, :, None]
    got = out.cpu().numpy()
    rel = np.abs(got - want) / np.maximum(np.abs(want), 2.0 ** -20)
    assert np.all(rel <= 2.0 ** -22), f"V decode: rel err {rel.max():.3e}"
    # K path: unit (b, g) holds code codes[b * Hkv + g]
    k = torch.zeros((B, 2, Hkv, d), dtype=torch.uint8)
    k[:, 1, :, 0] = codes.view(B, Hkv)
    v = torch.zeros((B, 2, Hkv, d), dtype=torch.uint8)
    v[:, 1] = 0x38                                       # 1.0
    q = torch.zeros(B, Hkv, d)
    q[..., 0] = 1.0
    mag = np.maximum(np.abs(vals), 2.0 ** -9).reshape(B, Hkv)
    x = {"q": q.to(torch.bfloat16), "k": k, "v": v,
         "lens": torch.full((B,), 2, dtype=torch.int32),
         "k_scale": torch.from_numpy((1.0 / mag).astype(np.float32)),
         "v_scale": torch.ones(B, Hkv)}
    kc, vc = _caches(g, x)
    say("[fp8] decode every code: K")
    out = g.attend_decode(x["q"].cuda(), kc, vc, x["lens"].cuda(), 1.0)
    torch.cuda.synchronize()
    want, _ = _oracle(x, w.replace(max_len=2, scale=1.0))
    err = float(np.max(np.abs(out.cpu().numpy() - want)))
    assert err <= 2e-5, f"K decode through the logits: err {err:.3e}"


def _append_rows(B, Hkv, d, scales, seed):
    """bf16 rows exercising the quantiser: normal values at the scale's
    range, a tenth far past 448 * scale, a tenth tiny, exact midpoints
    between neighbouring codes (exact products where the scale is a power
    of two), +-0."""
    gen = torch.Generator().manual_seed(seed)
    s = scales[:, :, None].float()
    x = torch.randn(B, Hkv, d, generator=gen) * 100.0 * s
    pick = torch.rand(B, Hkv, d, generator=gen)
    x = torch.where(pick < 0.1, x * 100.0, x)
    x = torch.where((pick >= 0.1) & (pick < 0.2), x * 1e-5, x)
    c = torch.randint(0, 0x7D, (B, Hkv, d), generator=gen)
    lo = torch.from_numpy(of8.decode(c.to(torch.uint8).numpy()))
    hi = torch.from_numpy(of8.decode((c + 1).to(torch.uint8).numpy()))
    sign = torch.where(torch.rand(B, Hkv, d, generator=gen) < 0.5, -1.0, 1.0)
    mid = ((lo + hi) / 2 * sign).float() * s
    x = torch.where((pick >= 0.2) & (pick < 0.4), mid, x)
    x[..., 0] = 0.0
    x[..., 1] = -0.0
    return x.to(torch.bfloat16)


@pytest.mark.parametrize("dk,dv", [(128, 128), (192, 128), (64, 64)])
def test_kv_append_quantises_bit_exact(dk, dv):
    g = _gqa()
    B, T, Hkv = 6, 6, 4
    gen = torch.Generator().manual_seed(81)
    ks = torch.rand(B, Hkv, generator=gen) * 0.3 + 0.01
    vs = torch.rand(B, Hkv, generator=gen) * 0.3 + 0.01
    ks[::2] = 2.0 ** torch.randint(-6, 2, (3, Hkv), generator=gen).float()
    vs[1::2] = 2.0 ** torch.randint(-6, 2, (3, Hkv), generator=gen).float()
    k = wl.make_e4m3_codes(gen, (B, T, Hkv, dk))
    v = wl.make_e4m3_codes(gen, (B, T, Hkv, dv))
    kn = _append_rows(B, Hkv, dk, ks, 82)
    vn = _append_rows(B, Hkv, dv, vs, 83)
    lens = torch.tensor([0, 3, 5, 6, -1, 2], dtype=torch.int32)
    kd, vd = g.Fp8Cache(k.cuda(), ks.cuda()), g.Fp8Cache(v.cuda(), vs.cuda())
    ld = lens.cuda()
    lo = torch.empty_like(ld)
    dropped = torch.zeros(1, dtype=torch.int32, device="cuda")
    say(f"[fp8] kv_append dk={dk} dv={dv}")
    g.kv_append(kd, vd, kn.cuda(), vn.cuda(), ld, lo, dropped)
    torch.cuda.synchronize()
    k2, v2, l2, nd = of8.kv_append_fp8(k.numpy(), v.numpy(), kn.float().numpy(),
                                       vn.float().numpy(), ks.numpy(),
                                       vs.numpy(), lens.numpy())
    assert lo.cpu().numpy().tolist() == l2.tolist(), "lens"
    assert int(dropped.item()) == nd == 2, "dropped"
    gk, gv = kd.codes.cpu().numpy(), vd.codes.cpu().numpy()
    bad = np.argwhere(gk != k2)
    assert bad.size == 0, f"K codes differ at {bad[:5].tolist()}: " \
        f"{gk[tuple(bad[0])]:#04x} vs {k2[tuple(bad[0])]:#04x}"
    assert np.array_equal(gv, v2), "V codes"


# bf16 values x and scales s for which x * fl(1 / s) and x / s round to
# different E4M3 codes: the append must follow the reciprocal reading.
DECIDING = [(5.09375, 0.7546296715736389), (0.95703125, 0.8059210777282715),
            (7.0, 0.8235293626785278), (11.9375, 0.9549999237060547),
            (0.00775146484375, 0.4177631735801697),
            (0.73046875, 0.6151316165924072)]


def test_kv_append_reciprocal_reading():
    """Values whose code depends on quantising with the rounded reciprocal
    of the scale rather than the quotient: bit for bit as the oracle."""
    g = _gqa()
    B, T, Hkv, d = len(DECIDING), 2, 1, 64
    xs = np.array([x for x, _ in DECIDING], dtype=np.float32)
    ss = np.array([s for _, s in DECIDING], dtype=np.float32)
    quo = of8.encode((xs / ss).astype(np.float32))
    prod = of8.encode((xs * (np.float32(1) / ss).astype(np.float32)).astype(
        np.float32))
    assert np.all(quo != prod), "each case decides between the readings"
    kn = torch.from_numpy(xs)[:, None, None].expand(B, Hkv, d).to(
        torch.bfloat16).contiguous()
    assert np.array_equal(kn[:, 0, 0].float().numpy(), xs), "bf16-exact"
    sc = torch.from_numpy(ss)[:, None].contiguous()
    k = torch.zeros(B, T, Hkv, d, dtype=torch.uint8)
    kd = g.Fp8Cache(k.cuda(), sc.cuda())
    vd = g.Fp8Cache(k.clone().cuda(), sc.cuda())
    lens = torch.zeros(B, dtype=torch.int32).cuda()
    say("[fp8] kv_append reciprocal reading")
    g.kv_append(kd, vd, kn.cuda(), kn.cuda(), lens, torch.empty_like(lens))
    torch.cuda.synchronize()
    want, _, _, _ = of8.kv_append_fp8(k.numpy(), k.numpy(), kn.float().numpy(),
                                      kn.float().numpy(), sc.numpy(),
                                      sc.numpy(), np.zeros(B, np.int32))
    assert np.array_equal(kd.codes.cpu().numpy(), want)
    assert np.all(kd.codes.cpu().numpy()[:, 0, 0, 0] == prod)


CASES = {
    # name: (workload, lens rule, explicit plan chunk)
    "d128_split": (wl.BATCHED_FP8.replace(batch=4, max_len=1500), "ragged",
                   None),
    "d128_direct": (wl.BATCHED_FP8.replace(batch=8, max_len=200), "ragged",
                    None),
    "d128_explicit": (wl.BATCHED_FP8.replace(batch=4, max_len=1000), "ragged",
                      128),
    # (two KV heads: the group split does not apply, so 1024 items are a
    # scheduled launch)
    "d128_scheduled": (wl.BATCHED_FP8.replace(batch=64, num_q_heads=16,
                                              num_kv_heads=2, max_len=1000),
                       "ragged", 128),
    "dk192_hpk16": (wl.BATCHED_FP8.replace(batch=3, num_q_heads=64,
                                           num_kv_heads=4, dk=192, dv=128,
                                           max_len=2100), "ragged", None),
    "d64": (wl.BATCHED_FP8.replace(batch=3, num_q_heads=8, num_kv_heads=4,
                                   dk=64, dv=64, max_len=700), "ragged", None),
    "d256_mha": (wl.BATCHED_FP8.replace(batch=3, num_q_heads=2,
                                        num_kv_heads=2, dk=256, dv=256,
                                        max_len=600), "ragged", None),
    # group split (64-wide heads): eight KV groups per work-group, a
    # wavefront per group over the whole chunk
    "d64_groupsplit": (wl.BATCHED_FP8.replace(batch=16, dk=64, dv=64,
                                              max_len=1100), "ragged", None),
    "d64_groupsplit_4k": (wl.BATCHED_FP8.replace(batch=16, dk=64, dv=64),
                          "ragged", None),
}


def _assert_group_split(g, w, kc, vc):
    """The library's plan for w is one the group-split launch takes: a plain
    chunked plan whose items, in sets of eight, are one round of one
    work-group per CU."""
    plan = g.attend_plan(kc, vc, w.num_q_heads, 0)
    assert w.dk + w.dv <= 128 and w.num_kv_heads % 8 == 0
    assert plan.sched_entries == 0 and plan.balanced_groups == 0
    assert 256 <= w.batch * w.num_kv_heads * plan.num_chunks // 8 < 512


def _lens(w, seed, cap=None):
    gen = torch.Generator().manual_seed(seed)
    top = w.max_len if cap is None else cap
    lens = torch.randint(0, top + 1, (w.batch,), generator=gen)
    lens[0] = 0
    if w.batch > 1:
        lens[1] = top
    return lens.to(torch.int32)


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("extra", ["plain", "carry_bias"])
def test_attend_fp8(name, extra):
    g = _gqa()
    w, _, chunk = CASES[name]
    x = wl.make_fp8_inputs(w, lens_override=_lens(w, 91).tolist())
    kc, vc = _caches(g, x)
    q, ld = x["q"].cuda(), x["lens"].cuda()
    rows = w.batch * w.num_q_heads
    cin = cin_np = bias = bias_np = None
    if extra == "carry_bias":
        cin, cin_np = _carry(g, rows, w.dv, 92)
        gen = torch.Generator().manual_seed(93)
        bias = torch.randn(w.batch, w.max_len + 4, generator=gen) * 2.0
        bias[torch.rand(bias.shape, generator=gen) < 0.1] = -float("inf")
        bias_np = bias.double().numpy()
        bias = bias.cuda()
    cout = g.empty_carry(rows, w.dv)
    if "groupsplit" in name:
        _assert_group_split(g, w, kc, vc)
    say(f"[fp8] attend {name} {extra}")
    if chunk is None:
        out = g.attend_decode(q, kc, vc, ld, w.scale, carry_in=cin,
                              carry_out=cout, bias=bias)
    else:
        plan = g.attend_plan(kc, vc, w.num_q_heads, chunk)
        if name == "d128_scheduled":
            assert plan.sched_entries > 0, "a scheduled plan"
        ws = torch.empty(plan.workspace_bytes, dtype=torch.uint8,
                         device="cuda")
        g.attend_partition(q, kc, vc, ld, plan, ws, w.scale, bias=bias)
        out = g.attend_combine(w.num_q_heads, kc, vc, ld, plan, ws,
                               carry_in=cin, carry_out=cout)
    torch.cuda.synchronize()
    want, cw = _oracle(x, w, carry_in=cin_np, bias=bias_np)
    vmax = _vmax(x)
    if cin_np is not None:
        vmax = max(vmax, float(np.max(np.abs(oracle.finalize(cin_np)))))
    check_out(out.cpu().numpy(), want, vmax, "fp8", name)
    check_carry(cout.m.cpu().numpy(), cout.l.cpu().numpy(), cw.m, cw.l, "fp8",
                name + " carry")
    if extra == "plain":
        assert torch.all(out[0] == 0), "an empty sequence gives 0"


STEP_CASES = {
    "d128_split": wl.BATCHED_FP8.replace(batch=4, max_len=1500),
    "d128_direct": wl.BATCHED_FP8.replace(batch=8, max_len=200),
    "d128_fused": wl.BATCHED_FP8.replace(batch=3, num_q_heads=8,
                                         num_kv_heads=2, max_len=300),
    "d64_balanced": wl.BATCHED_FP8.replace(batch=64, num_q_heads=8,
                                            num_kv_heads=8, dk=64, dv=64,
                                            max_len=4100),
    "dk192_hpk16": wl.BATCHED_FP8.replace(batch=3, num_q_heads=64,
                                          num_kv_heads=4, dk=192, dv=128,
                                          max_len=2100),
    "d256_mha": wl.BATCHED_FP8.replace(batch=3, num_q_heads=2,
                                       num_kv_heads=2, dk=256, dv=256,
                                       max_len=600),
    "d64_groupsplit": wl.BATCHED_FP8.replace(batch=16, dk=64, dv=64,
                                             max_len=1100),
    "d64_groupsplit_4k": wl.BATCHED_FP8.replace(batch=16, dk=64, dv=64),
}


@pytest.mark.parametrize("name", list(STEP_CASES))
def test_decode_step_fp8(name):
    """The whole step in one launch: the new rows quantised into the cache
    (bit for bit as kv_append would) and attended as their decoded codes;
    an empty sequence, a full cache (dropped) and a bias on one case."""
    g = _gqa()
    w = STEP_CASES[name]
    lens_in = _lens(w, 101, cap=w.max_len - 1)
    if w.batch > 2:
        lens_in[2] = w.max_len          # full: the token is dropped
    x = wl.make_fp8_inputs(w, lens_override=lens_in.tolist())
    gen = torch.Generator().manual_seed(102)
    kn = (torch.randn(w.batch, w.num_kv_heads, w.dk, generator=gen) *
          4 * x["k_scale"][:, :, None]).to(torch.bfloat16)
    vn = (torch.randn(w.batch, w.num_kv_heads, w.dv, generator=gen) *
          4 * x["v_scale"][:, :, None]).to(torch.bfloat16)
    kc, vc = _caches(g, x)
    li = x["lens"].cuda()
    lo = torch.empty_like(li)
    dropped = torch.zeros(1, dtype=torch.int32, device="cuda")
    bias = bias_np = None
    if name in ("d128_split", "d64_groupsplit"):
        bias = torch.randn(w.batch, w.max_len, generator=gen)
        bias_np = bias.double().numpy()
        bias = bias.cuda()
    ws = g.step_workspace(kc, vc, w.num_q_heads)
    cout = g.empty_carry(w.batch * w.num_q_heads, w.dv)
    if "groupsplit" in name:
        _assert_group_split(g, w, kc, vc)
    say(f"[fp8] decode_step {name}")
    out = g.decode_step(x["q"].cuda(), kc, vc, kn.cuda(), vn.cuda(), li, lo,
                        w.scale, carry_out=cout, workspace=ws,
                        dropped=dropped, bias=bias)
    torch.cuda.synchronize()
    k2, v2, l2, nd = of8.kv_append_fp8(
        x["k"].numpy(), x["v"].numpy(), kn.float().numpy(),
        vn.float().numpy(), x["k_scale"].numpy(), x["v_scale"].numpy(),
        lens_in.numpy())
    assert lo.cpu().numpy().tolist() == l2.tolist(), "lens"
    assert int(dropped.item()) == nd, "dropped"
    assert np.array_equal(kc.codes.cpu().numpy(), k2), "K codes"
    assert np.array_equal(vc.codes.cpu().numpy(), v2), "V codes"
    k2t, v2t = torch.from_numpy(k2), torch.from_numpy(v2)
    want, cw = _oracle(x, w, lens=torch.from_numpy(l2), bias=bias_np,
                       k=k2t, v=v2t)
    check_out(out.cpu().numpy(), want,
              _vmax(x, lens=torch.from_numpy(l2), v=v2t), "fp8",
              name + " step")
    check_carry(cout.m.cpu().numpy(), cout.l.cpu().numpy(), cw.m, cw.l, "fp8",
                name + " step carry")


def test_branches_fp8():
    """attend_branches over two fp8 caches with their own scales, then
    decode_step_branches appending to the second: equal to the oracle over
    both caches' decoded keys."""
    g = _gqa()
    w1 = wl.BATCHED_FP8.replace(batch=3, max_len=3000)
    w2 = wl.BATCHED_FP8.replace(batch=3, max_len=64, seed_index=8)
    x1 = wl.make_fp8_inputs(w1, lens_override=[3000, 17, 0])
    x2 = wl.make_fp8_inputs(w2, lens_override=[64, 40, 5])
    k1, v1 = _caches(g, x1)
    k2, v2 = _caches(g, x2)
    l1, l2 = x1["lens"].cuda(), x2["lens"].cuda()
    q = x1["q"].cuda()

    def deq(x, key, sc, k=None):
        return of8.dequantize_cache((x[key] if k is None else k).numpy(),
                                    x[sc].double().numpy())

    say("[fp8] attend_branches")
    out = g.attend_branches(q, [(k1, v1, l1), (k2, v2, l2)], w1.scale)
    torch.cuda.synchronize()
    want, _ = ost.attend_branches(
        np64(x1["q"]), [(deq(x1, "k", "k_scale"), deq(x1, "v", "v_scale"),
                         x1["lens"].numpy()),
                        (deq(x2, "k", "k_scale"), deq(x2, "v", "v_scale"),
                         x2["lens"].numpy())], w1.scale)
    vmax = max(_vmax(x1), _vmax(x2))
    check_out(out.cpu().numpy(), want, vmax, "fp8", "branches")

    gen = torch.Generator().manual_seed(111)
    kn = torch.randn(3, w1.num_kv_heads, w1.dk, generator=gen).to(torch.bfloat16)
    vn = torch.randn(3, w1.num_kv_heads, w1.dv, generator=gen).to(torch.bfloat16)
    lo = torch.empty_like(l2)
    say("[fp8] decode_step_branches")
    out = g.decode_step_branches(q, [(k1, v1, l1), (k2, v2, l2)], 1,
                                 kn.cuda(), vn.cuda(), lo, w1.scale)
    torch.cuda.synchronize()
    kk, vv, ll, _ = of8.kv_append_fp8(
        x2["k"].numpy(), x2["v"].numpy(), kn.float().numpy(),
        vn.float().numpy(), x2["k_scale"].numpy(), x2["v_scale"].numpy(),
        x2["lens"].numpy())
    assert lo.cpu().numpy().tolist() == ll.tolist() == [64, 41, 6]
    assert np.array_equal(k2.codes.cpu().numpy(), kk), "appended K codes"
    want, _ = ost.attend_branches(
        np64(x1["q"]), [(deq(x1, "k", "k_scale"), deq(x1, "v", "v_scale"),
                         x1["lens"].numpy()),
                        (deq(x2, "k", "k_scale", torch.from_numpy(kk)),
                         deq(x2, "v", "v_scale", torch.from_numpy(vv)), ll)],
        w1.scale)
    vmax = max(_vmax(x1), _vmax(x2, lens=torch.from_numpy(ll),
                                v=torch.from_numpy(vv)))
    check_out(out.cpu().numpy(), want, vmax, "fp8", "step branches")


def test_gathered_fp8():
    """Index-gathered decode over an fp8 cache (pooled index rows with
    duplicates and INVALID entries, split over several chunks)."""
    g = _gqa()
    w = wl.BATCHED_FP8.replace(batch=4, max_len=9000)
    x = wl.make_fp8_inputs(w, lens_override=[9000, 8000, 0, 4000])
    kc, vc = _caches(g, x)
    idx = wl.make_index_rows(w, x["lens"], 5000, 64, 121)
    say("[fp8] attend_gathered")
    out = g.attend_gathered(x["q"].cuda(), kc, vc, x["lens"].cuda(),
                            idx.cuda(), w.scale)
    torch.cuda.synchronize()
    kd = of8.dequantize_cache(x["k"].numpy(), x["k_scale"].double().numpy())
    vd = of8.dequantize_cache(x["v"].numpy(), x["v_scale"].double().numpy())
    want, _ = ost.attend_gathered(np64(x["q"]), kd, vd, x["lens"].numpy(),
                                  idx.numpy(), w.scale)
    check_out(out.cpu().numpy(), want, _vmax(x), "fp8", "gathered")
