"""A seeded sweep over the supported space, against the oracle: cache dtype
(bf16, fp8, fp32 on the matrix-core and vector-ALU paths), head widths, KV
heads, query heads per KV head (including sizes that are not powers of
two), batch, cache length, lengths that are ragged, empty, full or past the
cache, an additive bias, a carry_in, and the plain attend or the fused
decode step (append into the cache, full caches dropped).  Each case is
small enough for the oracle to finish at once; together they cross the
plan kinds (one chunk, split-K with the combine, the fused fold of small
steps)."""

import numpy as np
import pytest
import torch

import oracle
import oracle.fp8 as of8
from gpu_util import check_carry, check_out, np64, say
from gqa_kv_cache_decode_amd import workloads as wl

pytestmark = pytest.mark.gpu

WIDTHS = {"bf16": [(64, 64), (128, 128), (192, 128), (256, 256)],
          "fp8": [(64, 64), (128, 128), (192, 128), (256, 256)],
          "f32": [(64, 64), (128, 128), (192, 128), (48, 80)]}


def _cases(n=120, seed=2027):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        dt = str(rng.choice(["bf16", "bf16", "fp8", "f32"]))
        dk, dv = WIDTHS[dt][rng.integers(len(WIDTHS[dt]))]
        hkv = int(rng.choice([1, 2, 4, 8]))
        hpk = int(rng.choice([1, 2, 3, 4, 5, 8, 16]))
        B = int(rng.integers(1, 7))
        T = int(rng.choice([1, 17, 64, 200, 777, 2100, 4100]))
        lens = rng.integers(0, T + 1, B)
        for b in range(B):          # empty, full, past the cache, negative
            r = rng.random()
            lens[b] = 0 if r < 0.1 else T if r < 0.25 else \
                T + 3 if r < 0.3 else -2 if r < 0.35 else lens[b]
        cases.append(dict(i=i, dt=dt, dk=dk, dv=dv, hkv=hkv, hq=hkv * hpk,
                          B=B, T=T, lens=lens.astype(np.int32).tolist(),
                          step=bool(rng.random() < 0.5),
                          bias=bool(rng.random() < 0.3),
                          carry=bool(rng.random() < 0.3)))
    return cases


CASES = _cases()


def _id(c):
    return (f"{c['i']}-{c['dt']}-d{c['dk']}x{c['dv']}-h{c['hq']}/{c['hkv']}"
            f"-b{c['B']}-t{c['T']}{'-step' if c['step'] else ''}"
            f"{'-bias' if c['bias'] else ''}{'-carry' if c['carry'] else ''}")


@pytest.mark.parametrize("c", CASES, ids=_id)
def test_sweep(c):
    import gqa_kv_cache_decode_amd as g
    say(f"[sweep] {_id(c)} lens={c['lens']}")
    w = wl.DecodeWorkload(f"sweep{c['i']}", batch=c["B"], num_q_heads=c["hq"],
                          num_kv_heads=c["hkv"], dk=c["dk"], dv=c["dv"],
                          max_len=c["T"], dtype=c["dt"],
                          seed_index=300 + c["i"])
    B, Hq, Hkv, T = w.batch, w.num_q_heads, w.num_kv_heads, w.max_len
    fp8 = w.dtype == "fp8"
    gen = torch.Generator().manual_seed(400 + c["i"])
    x = (wl.make_fp8_inputs(w, lens_override=c["lens"]) if fp8 else
         wl.make_inputs(w, lens_override=c["lens"]))
    io = torch.bfloat16 if fp8 else w.torch_dtype
    lens_in = x["lens"]
    bias = None
    if c["bias"]:   # rows padded to a multiple of 4 positions
        bias = torch.randn(B, (T + 3) // 4 * 4, generator=gen)
    cin = cin_np = None
    rows = B * Hq
    if c["carry"]:
        m = torch.randn(rows, generator=gen)
        l = torch.rand(rows, generator=gen) + 0.5
        l[::3] = 0.0
        acc = torch.randn(rows, w.dv, generator=gen)
        cin = g.Carry(m.cuda(), l.cuda(), acc.cuda())
        cin_np = oracle.Carry(m.double().numpy(), l.double().numpy(),
                              acc.double().numpy())
    cout = g.empty_carry(rows, w.dv)
    if fp8:
        kc = g.Fp8Cache(x["k"].cuda(), x["k_scale"].cuda())
        vc = g.Fp8Cache(x["v"].cuda(), x["v_scale"].cuda())
    else:
        kc, vc = x["k"].cuda(), x["v"].cuda()
    q = x["q"].cuda()
    bias_d = None if bias is None else bias.cuda()

    # what the oracle attends: the caches after the append for a step
    k_att, v_att, lens_att = x["k"], x["v"], lens_in.numpy()
    if c["step"]:
        ks = x["k_scale"][:, :, None] if fp8 else 1.0
        vs = x["v_scale"][:, :, None] if fp8 else 1.0
        kn = (torch.randn(B, Hkv, w.dk, generator=gen) * 4 * ks).to(io)
        vn = (torch.randn(B, Hkv, w.dv, generator=gen) * 4 * vs).to(io)
        li = lens_in.cuda()
        lo = torch.full_like(li, -77)
        dropped = torch.zeros(1, dtype=torch.int32, device="cuda")
        out = g.decode_step(q, kc, vc, kn.cuda(), vn.cuda(), li, lo, w.scale,
                            carry_in=cin, carry_out=cout,
                            workspace=g.step_workspace(kc, vc, Hq),
                            dropped=dropped, bias=bias_d)
        torch.cuda.synchronize()
        if fp8:
            k2, v2, lens_att, nd = of8.kv_append_fp8(
                x["k"].numpy(), x["v"].numpy(), kn.float().numpy(),
                vn.float().numpy(), x["k_scale"].numpy(),
                x["v_scale"].numpy(), lens_in.numpy())
            assert np.array_equal(kc.codes.cpu().numpy(), k2) and \
                np.array_equal(vc.codes.cpu().numpy(), v2), "appended codes"
            k_att, v_att = torch.from_numpy(k2), torch.from_numpy(v2)
        else:
            bits = torch.int16 if io == torch.bfloat16 else torch.int32
            k2, v2, lens_att, nd = oracle.kv_append(
                x["k"].view(bits).numpy(), x["v"].view(bits).numpy(),
                kn.view(bits).numpy(), vn.view(bits).numpy(), lens_in.numpy())
            assert np.array_equal(kc.cpu().view(bits).numpy(), k2) and \
                np.array_equal(vc.cpu().view(bits).numpy(), v2), \
                "appended rows"
            k_att = torch.from_numpy(k2).view(io)
            v_att = torch.from_numpy(v2).view(io)
        assert lo.cpu().numpy().tolist() == list(lens_att), "lens_out"
        assert int(dropped.item()) == nd, "dropped"
    else:
        out = g.attend_decode(q, kc, vc, lens_in.cuda(), w.scale,
                              carry_in=cin, carry_out=cout, bias=bias_d)
        torch.cuda.synchronize()

    bias_np = None if bias is None else bias[:, :T].double().numpy()
    if fp8:
        want, cw = of8.attend_fp8(np64(x["q"]), k_att.numpy(), v_att.numpy(),
                                  x["k_scale"].double().numpy(),
                                  x["v_scale"].double().numpy(), lens_att,
                                  w.scale, carry_in=cin_np, bias=bias_np)
        vals = of8.dequantize_cache(v_att.numpy(),
                                    x["v_scale"].double().numpy())
    else:
        vals = np64(v_att)
        want, cw = oracle.attend(np64(x["q"]), np64(k_att), vals, lens_att,
                                 w.scale, carry_in=cin_np, bias=bias_np)
    vmax = 0.0
    for b in range(B):
        n = int(min(max(int(lens_att[b]), 0), T))
        if n:
            vmax = max(vmax, float(np.abs(vals[b, :n]).max()))
    if cin_np is not None:
        vmax = max(vmax, float(np.max(np.abs(oracle.finalize(cin_np)))))
    check_out(out.cpu().numpy(), want, max(vmax, 1e-30), w.dtype, _id(c))
    check_carry(cout.m.cpu().numpy(), cout.l.cpu().numpy(), cw.m, cw.l,
                w.dtype, _id(c) + " carry")


MFMA_WIDTHS = {"bf16": WIDTHS["bf16"], "fp8": WIDTHS["fp8"],
               "f32": [(64, 64), (128, 128), (192, 128)]}


def _multi_cases(n, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        dt = str(rng.choice(["bf16", "bf16", "fp8", "f32"]))
        dk, dv = MFMA_WIDTHS[dt][rng.integers(len(MFMA_WIDTHS[dt]))]
        hkv = int(rng.choice([1, 2, 4]))
        hpk = int(rng.choice([1, 2, 3, 4, 8, 16]))
        B = int(rng.integers(1, 5))
        cases.append(dict(i=i, dt=dt, dk=dk, dv=dv, hkv=hkv, hq=hkv * hpk,
                          B=B, rng=int(rng.integers(1 << 30))))
    return cases


def _draw(c, T, lens, idx):
    w = wl.DecodeWorkload(f"sweep{idx}", batch=c["B"], num_q_heads=c["hq"],
                          num_kv_heads=c["hkv"], dk=c["dk"], dv=c["dv"],
                          max_len=T, dtype=c["dt"], seed_index=idx)
    return w, (wl.make_fp8_inputs(w, lens_override=lens) if c["dt"] == "fp8"
               else wl.make_inputs(w, lens_override=lens))


def _dev_cache(g, x, fp8):
    if fp8:
        return (g.Fp8Cache(x["k"].cuda(), x["k_scale"].cuda()),
                g.Fp8Cache(x["v"].cuda(), x["v_scale"].cuda()))
    return x["k"].cuda(), x["v"].cuda()


def _values(x, fp8):
    """The cache as the oracle attends it: fp64 values (fp8 decoded)."""
    if fp8:
        return (of8.dequantize_cache(x["k"].numpy(),
                                     x["k_scale"].double().numpy()),
                of8.dequantize_cache(x["v"].numpy(),
                                     x["v_scale"].double().numpy()))
    return np64(x["k"]), np64(x["v"])


def _live_vmax(v, lens):
    m = 0.0
    for b in range(v.shape[0]):
        n = int(min(max(int(lens[b]), 0), v.shape[1]))
        if n:
            m = max(m, float(np.abs(v[b, :n]).max()))
    return m


@pytest.mark.parametrize("c", _multi_cases(40, 2028),
                         ids=lambda c: f"{c['i']}-{c['dt']}-d{c['dk']}x{c['dv']}"
                                       f"-h{c['hq']}/{c['hkv']}-b{c['B']}")
def test_sweep_branches(c):
    """attend_branches over 1..4 caches of random lengths (one with a bias
    now and then) and a carry_in, against the oracle's fold of the branches."""
    import gqa_kv_cache_decode_amd as g
    import oracle.streaming as ost
    rng = np.random.default_rng(c["rng"])
    fp8 = c["dt"] == "fp8"
    nbr = int(rng.integers(1, 5))
    dev_br, np_br, vmax = [], [], 0.0
    for j in range(nbr):
        T = int(rng.choice([1, 40, 130, 700, 2500]))
        lens = [int(rng.integers(-1, T + 3)) for _ in range(c["B"])]
        w, x = _draw(c, T, lens, 500 + 10 * c["i"] + j)
        k, v = _dev_cache(g, x, fp8)
        kv, vv = _values(x, fp8)
        bias = None
        if rng.random() < 0.3:
            bias = torch.randn(c["B"], (T + 3) // 4 * 4,
                               generator=torch.Generator().manual_seed(j))
        dev_br.append((k, v, x["lens"].cuda(),
                       None if bias is None else bias.cuda()))
        np_br.append((kv, vv, x["lens"].numpy(),
                      None if bias is None else bias[:, :T].double().numpy()))
        vmax = max(vmax, _live_vmax(vv, x["lens"].numpy()))
        q = x["q"]          # every draw gives a q of the same shape; keep the last
    say(f"[sweep branches] {c['dt']} {nbr} branches "
        f"T={[b[0].shape[1] if not fp8 else b[0].codes.shape[1] for b in dev_br]}")
    rows = c["B"] * c["hq"]
    cin = cin_np = None
    if rng.random() < 0.5:
        gen = torch.Generator().manual_seed(c["i"])
        m = torch.randn(rows, generator=gen)
        l = torch.rand(rows, generator=gen) + 0.5
        l[::4] = 0.0
        acc = torch.randn(rows, c["dv"], generator=gen)
        cin = g.Carry(m.cuda(), l.cuda(), acc.cuda())
        cin_np = oracle.Carry(m.double().numpy(), l.double().numpy(),
                              acc.double().numpy())
        vmax = max(vmax, float(np.max(np.abs(oracle.finalize(cin_np)))))
    cout = g.empty_carry(rows, c["dv"])
    out = g.attend_branches(q.cuda(), dev_br, 0.0, carry_in=cin,
                            carry_out=cout)
    torch.cuda.synchronize()
    want, cw = ost.attend_branches(np64(q), np_br, 0.0, carry_in=cin_np)
    what = f"branches {c['i']}"
    check_out(out.cpu().numpy(), want, max(vmax, 1e-30), c["dt"], what)
    check_carry(cout.m.cpu().numpy(), cout.l.cpu().numpy(), cw.m, cw.l,
                c["dt"], what + " carry")


@pytest.mark.parametrize("c", _multi_cases(40, 2029),
                         ids=lambda c: f"{c['i']}-{c['dt']}-d{c['dk']}x{c['dv']}"
                                       f"-h{c['hq']}/{c['hkv']}-b{c['B']}")
def test_sweep_gathered(c):
    """attend_gathered with random index rows (duplicates, INVALID and
    out-of-range entries, empty rows) against the oracle's selection."""
    import gqa_kv_cache_decode_amd as g
    import oracle.streaming as ost
    rng = np.random.default_rng(c["rng"])
    fp8 = c["dt"] == "fp8"
    T = int(rng.choice([1, 50, 300, 3000]))
    lens = [int(rng.integers(-1, T + 3)) for _ in range(c["B"])]
    w, x = _draw(c, T, lens, 700 + c["i"])
    width = int(rng.choice([1, 7, 64, 500, 2100]))
    idx = rng.integers(-3, T + 5, (c["B"], width)).astype(np.int32)
    if width > 4:
        idx[:, 1] = idx[:, 0]                   # a duplicate in every row
    if c["B"] > 1 and rng.random() < 0.3:
        idx[1] = -1                             # a row selecting nothing
    k, v = _dev_cache(g, x, fp8)
    say(f"[sweep gathered] {c['dt']} T={T} width={width}")
    out = g.attend_gathered(x["q"].cuda(), k, v, x["lens"].cuda(),
                            torch.from_numpy(idx).cuda(), 0.0)
    torch.cuda.synchronize()
    kv, vv = _values(x, fp8)
    want, _ = ost.attend_gathered(np64(x["q"]), kv, vv, x["lens"].numpy(),
                                  idx, 0.0)
    check_out(out.cpu().numpy(), want,
              max(_live_vmax(vv, x["lens"].numpy()), 1e-30), c["dt"],
              f"gathered {c['i']}")
