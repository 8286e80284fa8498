"""Multi-branch attention and the streaming sink / ring / main layout on the
GPU against the oracle: stream_append bit for bit over runs of decode steps
(sink filling, ring wrap-around, eviction into main, a full main cache, an
invalid count, no sink, no main cache), attend_branches over the three parts
equal to attention over the whole history, and attend_branches over up to
four caches of different lengths with biases and an aliased carry."""

import numpy as np
import pytest
import torch

import oracle
import oracle.streaming as ost
from gpu_util import check_carry, check_out, live_vmax, np64, say
from gqa_kv_cache_decode_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _gqa():
    import gqa_kv_cache_decode_amd as g
    return g


def _bits(t):
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32)


LAYOUTS = {
    # name: (dtype, S, W, M, dk, dv, Hq, Hkv)
    "bf16_sink_ring_main": ("bf16", 4, 16, 40, 128, 128, 8, 2),
    "f32_sink_ring_main": ("f32", 4, 16, 24, 64, 64, 4, 2),
    "bf16_no_sink": ("bf16", 0, 8, 20, 64, 64, 4, 1),
    "bf16_sink_ring_only": ("bf16", 4, 8, 0, 192, 128, 16, 1),
}


@pytest.mark.parametrize("name", list(LAYOUTS))
def test_stream_steps(name):
    """A run of decode steps through stream_append, each checked bit for bit
    against the oracle's layout model; every few steps the three parts are
    attended with attend_branches and compared with the oracle's attention
    over the whole history of each sequence."""
    g = _gqa()
    dt, S, W, M, dk, dv, Hq, Hkv = LAYOUTS[name]
    tdt = wl.DTYPES[dt]
    B = 3
    gen = torch.Generator().manual_seed(61)
    z = lambda n, d: torch.zeros(B, n, Hkv, d, dtype=tdt)
    host = {"sk": z(S, dk) if S else None, "sv": z(S, dv) if S else None,
            "rk": z(W, dk), "rv": z(W, dv),
            "mk": z(M, dk) if M else None, "mv": z(M, dv) if M else None}
    dev = {k: (None if t is None else t.cuda()) for k, t in host.items()}
    count = torch.tensor([0, 5, -1], dtype=torch.int32)
    count_d = count.cuda()
    dropped = torch.zeros(1, dtype=torch.int32, device="cuda")
    drop_ref = 0
    hist_k = [[] for _ in range(B)]
    hist_v = [[] for _ in range(B)]
    # sequence 1 starts with 5 tokens already seen: placed by the oracle's
    # layout model (only sequence 1 is valid in these seeding appends)
    for i in range(5):
        kn = torch.randn(B, Hkv, dk, generator=gen).to(tdt)
        vn = torch.randn(B, Hkv, dv, generator=gen).to(tdt)
        res = ost.stream_append(*(None if host[k] is None else
                                  _bits(host[k]).numpy()
                                  for k in ("sk", "sv", "rk", "rv", "mk", "mv")),
                                _bits(kn).numpy(), _bits(vn).numpy(),
                                np.array([-1, i, -1]))
        for k, arr in zip(("sk", "sv", "rk", "rv", "mk", "mv"), res[:6]):
            if arr is not None:
                host[k] = torch.from_numpy(arr).view(tdt)
        hist_k[1].append(kn[1])
        hist_v[1].append(vn[1])
    dev = {k: (None if t is None else t.cuda()) for k, t in host.items()}
    steps = S + W + M + 4
    for step in range(steps):
        kn = torch.randn(B, Hkv, dk, generator=gen).to(tdt)
        vn = torch.randn(B, Hkv, dv, generator=gen).to(tdt)
        before = count.clone()
        cnt_out, ls, lr, lm = g.stream_append(
            dev["rk"], dev["rv"], kn.cuda(), vn.cuda(), count_d,
            sink=None if not S else (dev["sk"], dev["sv"]),
            main=None if not M else (dev["mk"], dev["mv"]), dropped=dropped)
        torch.cuda.synchronize()
        res = ost.stream_append(*(None if host[k] is None else
                                  _bits(host[k]).numpy()
                                  for k in ("sk", "sv", "rk", "rv", "mk", "mv")),
                                _bits(kn).numpy(), _bits(vn).numpy(),
                                before.numpy())
        for k, arr in zip(("sk", "sv", "rk", "rv", "mk", "mv"), res[:6]):
            if arr is None:
                continue
            host[k] = torch.from_numpy(arr).view(tdt)
            assert torch.equal(_bits(dev[k].cpu()), _bits(host[k])), \
                f"{name} step {step}: {k} differs"
        count = torch.from_numpy(res[6])
        drop_ref += res[7]
        assert cnt_out.cpu().tolist() == count.tolist(), "count"
        assert int(dropped.item()) == drop_ref, "dropped"
        for b in range(B):
            ns, nw, nm = ost.stream_lengths(int(count[b]), S, W, M)
            if S:
                assert int(ls[b]) == ns, "lens_sink"
            assert int(lr[b]) == nw, "lens_ring"
            if M:
                assert int(lm[b]) == nm, "lens_main"
            if b < 2 and int(count[b]) > int(before[b]):
                hist_k[b].append(kn[b])
                hist_v[b].append(vn[b])
        count_d = cnt_out
        if step % 5 == 4 or step == steps - 1:
            q = torch.randn(B, Hq, dk, generator=gen).to(tdt)
            branches = []
            if S:
                branches.append((dev["sk"], dev["sv"], ls))
            branches.append((dev["rk"], dev["rv"], lr))
            if M:
                branches.append((dev["mk"], dev["mv"], lm))
            out = g.attend_branches(q.cuda(), branches, 0.0)
            torch.cuda.synchronize()
            for b in range(2):
                t = int(count[b])
                keep = list(range(min(t, S))) + list(range(max(S, t - W), t))
                nm = ost.stream_lengths(t, S, W, M)[2]
                keep += list(range(S, S + nm))
                kc = torch.stack([hist_k[b][p] for p in keep])[None]
                vc = torch.stack([hist_v[b][p] for p in keep])[None]
                want, _ = oracle.attend(np64(q[b:b + 1]), np64(kc), np64(vc),
                                        [len(keep)], 0.0)
                check_out(out[b:b + 1].cpu().numpy(), want,
                          float(vc.float().abs().max()), dt,
                          f"{name} step {step} b={b} t={t}")
            assert torch.all(out[2] == 0), "invalid sequence attends nothing"


def _cache(B, T, Hkv, d, dt, seed):
    gen = torch.Generator().manual_seed(seed)
    return torch.randn(B, T, Hkv, d, generator=gen).to(wl.DTYPES[dt])


@pytest.mark.parametrize("dt,dk,dv,Hq,Hkv", [("bf16", 128, 128, 32, 4),
                                             ("bf16", 192, 128, 16, 1),
                                             ("f32", 64, 64, 8, 4)])
@pytest.mark.parametrize("nbr", [2, 4])
def test_attend_branches(dt, dk, dv, Hq, Hkv, nbr):
    """Up to four caches of different lengths (one split into many chunks,
    one empty for some sequences), a bias on some branches, carry_in with
    carry_out aliasing it: against the oracle's branch-by-branch carry."""
    g = _gqa()
    B = 3
    Ts = [5000, 128, 4, 700][:nbr]
    gen = torch.Generator().manual_seed(62)
    q = torch.randn(B, Hq, dk, generator=gen).to(wl.DTYPES[dt])
    branches_d, branches_h = [], []
    for i, T in enumerate(Ts):
        k = _cache(B, T, Hkv, dk, dt, 70 + i)
        v = _cache(B, T, Hkv, dv, dt, 80 + i)
        lens = torch.randint(0, T + 1, (B,), generator=gen).to(torch.int32)
        lens[0] = T
        if i == 1:
            lens[2] = 0
        bias = None
        if i % 2 == 1:
            bias = torch.randn(B, (T + 3) // 4 * 4, generator=gen)
        branches_h.append((np64(k), np64(v), lens.numpy()) +
                          (() if bias is None else (bias.double().numpy(),)))
        branches_d.append((k.cuda(), v.cuda(), lens.cuda()) +
                          (() if bias is None else (bias.cuda(),)))
    rows = B * Hq
    m = torch.randn(rows, generator=gen)
    l = torch.rand(rows, generator=gen) + 0.5
    l[::4] = 0.0
    acc = torch.randn(rows, dv, generator=gen)
    cin_np = oracle.Carry(m.double().numpy(), l.double().numpy(),
                          acc.double().numpy())
    carry = g.Carry(m.cuda(), l.cuda(), acc.cuda())
    say(f"[branches] {dt} {dk}/{dv} hpk {Hq // Hkv} x{nbr}")
    out = g.attend_branches(q.cuda(), branches_d, 0.0, carry_in=carry,
                            carry_out=carry)
    torch.cuda.synchronize()
    want, cw = ost.attend_branches(np64(q), branches_h, 0.0, carry_in=cin_np)
    vmax = max(max(float(np.max(np.abs(b[1]))) for b in branches_h),
               float(np.max(np.abs(oracle.finalize(cin_np)))))
    check_out(out.cpu().numpy(), want, vmax, dt, f"branches x{nbr}")
    check_carry(carry.m.cpu().numpy(), carry.l.cpu().numpy(), cw.m, cw.l, dt,
                f"branches x{nbr} carry")


@pytest.mark.parametrize("dt,dk,dv,Hq,Hkv", [("bf16", 128, 128, 32, 4),
                                             ("bf16", 192, 128, 16, 1),
                                             ("f32", 64, 64, 8, 4)])
def test_decode_step_branches(dt, dk, dv, Hq, Hkv):
    """A long cache attended as is plus a window taking the new token (with a
    bias on the window), one partition launch and one combine: the window
    after the append bit for bit, lens and drops exactly, out and carry
    against the oracle (append, then attend over both branches)."""
    g = _gqa()
    B = 4
    gen = torch.Generator().manual_seed(63)
    tdt = wl.DTYPES[dt]
    q = torch.randn(B, Hq, dk, generator=gen).to(tdt)
    mk, mv = _cache(B, 3000, Hkv, dk, dt, 91), _cache(B, 3000, Hkv, dv, dt, 92)
    wk, wv = _cache(B, 128, Hkv, dk, dt, 93), _cache(B, 128, Hkv, dv, dt, 94)
    mlens = torch.tensor([3000, 1, 0, 2047], dtype=torch.int32)
    wlens = torch.tensor([127, 0, 128, -1], dtype=torch.int32)  # 2 drops
    kn = torch.randn(B, Hkv, dk, generator=gen).to(tdt)
    vn = torch.randn(B, Hkv, dv, generator=gen).to(tdt)
    bias = torch.randn(B, 128, generator=gen)
    wkd, wvd = wk.cuda(), wv.cuda()
    lo = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    dropped = torch.zeros(1, dtype=torch.int32, device="cuda")
    cout = g.empty_carry(B * Hq, dv)
    out = g.decode_step_branches(
        q.cuda(), [(mk.cuda(), mv.cuda(), mlens.cuda()),
                   (wkd, wvd, wlens.cuda(), bias.cuda())], 1, kn.cuda(),
        vn.cuda(), lo, 0.0, carry_out=cout, dropped=dropped)
    torch.cuda.synchronize()
    k_ref, v_ref, l_ref, drop_ref = oracle.kv_append(
        _bits(wk).numpy(), _bits(wv).numpy(), _bits(kn).numpy(),
        _bits(vn).numpy(), wlens.numpy())
    assert np.array_equal(_bits(wkd.cpu()).numpy(), k_ref), "window K"
    assert np.array_equal(_bits(wvd.cpu()).numpy(), v_ref), "window V"
    assert lo.cpu().tolist() == l_ref.tolist(), "lens_out"
    assert int(dropped.item()) == drop_ref == 2, "dropped"
    wk2 = torch.from_numpy(k_ref).view(tdt)
    wv2 = torch.from_numpy(v_ref).view(tdt)
    want, cw = ost.attend_branches(
        np64(q), [(np64(mk), np64(mv), mlens.numpy()),
                  (np64(wk2), np64(wv2), l_ref, bias.double().numpy())], 0.0)
    vmax = max(float(mv.float().abs().max()), float(wv2.float().abs().max()))
    check_out(out.cpu().numpy(), want, vmax, dt, "decode_step_branches")
    check_carry(cout.m.cpu().numpy(), cout.l.cpu().numpy(), cw.m, cw.l, dt,
                "decode_step_branches carry")


@pytest.mark.parametrize("S,W,M", [(4, 16, 40), (0, 8, 20), (4, 8, 0)])
def test_stream_steps_fp8(S, W, M):
    """stream_append over fp8 caches whose three parts share the scales: the
    new bf16 rows quantised into sink / ring slots and the evicted ring rows
    moved to main as codes, bit for bit against the oracle over a run of
    steps (an invalid count, a full main cache); attend_branches over the
    three parts equals the oracle's attention over the decoded history."""
    import oracle.fp8 as of8
    g = _gqa()
    B, Hq, Hkv, d = 3, 8, 2, 128
    gen = torch.Generator().manual_seed(62)
    ks = (torch.rand(B, Hkv, generator=gen) * 0.45 + 0.05).float()
    vs = (torch.rand(B, Hkv, generator=gen) * 0.9 + 0.1).float()
    ksd, vsd = ks.cuda(), vs.cuda()
    z = lambda n: torch.zeros(B, n, Hkv, d, dtype=torch.uint8)
    host = {"sk": z(S) if S else None, "sv": z(S) if S else None,
            "rk": z(W), "rv": z(W),
            "mk": z(M) if M else None, "mv": z(M) if M else None}
    dev = {k: (None if t is None else t.cuda()) for k, t in host.items()}
    part = lambda kk, vv: (g.Fp8Cache(dev[kk], ksd), g.Fp8Cache(dev[vv], vsd))
    count = torch.tensor([0, 3, -1], dtype=torch.int32)
    count_d = count.cuda()
    # sequence 1 starts with 3 tokens already placed by the oracle
    hist = [[] for _ in range(B)]
    for i in range(3):
        kn = (torch.randn(B, Hkv, d, generator=gen) * 4 * ks[:, :, None]).to(
            torch.bfloat16)
        vn = (torch.randn(B, Hkv, d, generator=gen) * 4 * vs[:, :, None]).to(
            torch.bfloat16)
        res = of8.stream_append_fp8(
            *(None if host[k] is None else host[k].numpy()
              for k in ("sk", "sv", "rk", "rv", "mk", "mv")),
            kn.float().numpy(), vn.float().numpy(), ks.numpy(), vs.numpy(),
            np.array([-1, i, -1]))
        for k, arr in zip(("sk", "sv", "rk", "rv", "mk", "mv"), res[:6]):
            if arr is not None:
                host[k] = torch.from_numpy(arr)
        hist[1].append((of8.quantize(kn[1].float().numpy(),
                                     ks[1].numpy()[:, None]),
                        of8.quantize(vn[1].float().numpy(),
                                     vs[1].numpy()[:, None])))
    dev = {k: (None if t is None else t.cuda()) for k, t in host.items()}
    dropped = torch.zeros(1, dtype=torch.int32, device="cuda")
    drop_ref = 0
    steps = S + W + M + 4
    say(f"[stream fp8] S={S} W={W} M={M}: {steps} steps")
    for step in range(steps):
        kn = (torch.randn(B, Hkv, d, generator=gen) * 4 * ks[:, :, None]).to(
            torch.bfloat16)
        vn = (torch.randn(B, Hkv, d, generator=gen) * 4 * vs[:, :, None]).to(
            torch.bfloat16)
        before = count.clone()
        rk, rv = part("rk", "rv")
        cnt_out, ls, lr, lm = g.stream_append(
            rk, rv, kn.cuda(), vn.cuda(), count_d,
            sink=part("sk", "sv") if S else None,
            main=part("mk", "mv") if M else None, dropped=dropped)
        torch.cuda.synchronize()
        res = of8.stream_append_fp8(
            *(None if host[k] is None else host[k].numpy()
              for k in ("sk", "sv", "rk", "rv", "mk", "mv")),
            kn.float().numpy(), vn.float().numpy(), ks.numpy(), vs.numpy(),
            before.numpy())
        for k, arr in zip(("sk", "sv", "rk", "rv", "mk", "mv"), res[:6]):
            if arr is None:
                continue
            host[k] = torch.from_numpy(arr)
            assert torch.equal(dev[k].cpu(), host[k]), \
                f"S={S} W={W} M={M} step {step}: {k} codes differ"
        count = torch.from_numpy(res[6])
        drop_ref += res[7]
        assert cnt_out.cpu().tolist() == count.tolist(), "count"
        assert int(dropped.item()) == drop_ref, "dropped"
        for b in range(2):
            if int(count[b]) > int(before[b]):
                hist[b].append((of8.quantize(kn[b].float().numpy(),
                                             ks[b].numpy()[:, None]),
                                of8.quantize(vn[b].float().numpy(),
                                             vs[b].numpy()[:, None])))
        count_d = cnt_out
        if step % 6 == 5 or step == steps - 1:
            q = torch.randn(B, Hq, d, generator=gen).to(torch.bfloat16)
            branches = []
            if S:
                branches.append((*part("sk", "sv"), ls))
            branches.append((*part("rk", "rv"), lr))
            if M:
                branches.append((*part("mk", "mv"), lm))
            out = g.attend_branches(q.cuda(), branches, 0.0)
            torch.cuda.synchronize()
            for b in range(2):
                t = int(count[b])
                nm = ost.stream_lengths(t, S, W, M)[2]
                keep = list(range(min(t, S))) + \
                    list(range(max(S, t - W), t)) + list(range(S, S + nm))
                kc = np.stack([hist[b][p][0] for p in keep])[None]
                vc = np.stack([hist[b][p][1] for p in keep])[None]
                want, _ = of8.attend_fp8(
                    np64(q[b:b + 1]), kc, vc, ks[b:b + 1].double().numpy(),
                    vs[b:b + 1].double().numpy(), [len(keep)], 0.0)
                vmax = float(np.abs(of8.dequantize_cache(
                    vc, vs[b:b + 1].double().numpy())).max())
                check_out(out[b:b + 1].cpu().numpy(), want, vmax, "fp8",
                          f"fp8 S={S} W={W} M={M} step {step} b={b} t={t}")
            assert torch.all(out[2] == 0), "invalid sequence attends nothing"


def test_stream_fp8_needs_shared_scales():
    g = _gqa()
    B, Hkv, d = 2, 2, 128
    codes = lambda n: torch.zeros(B, n, Hkv, d, dtype=torch.uint8,
                                  device="cuda")
    s1 = torch.ones(B, Hkv, device="cuda")
    s2 = torch.ones(B, Hkv, device="cuda")
    ring = (g.Fp8Cache(codes(8), s1), g.Fp8Cache(codes(8), s1))
    main = (g.Fp8Cache(codes(8), s2), g.Fp8Cache(codes(8), s2))
    kn = torch.zeros(B, Hkv, d, dtype=torch.bfloat16, device="cuda")
    count = torch.zeros(B, dtype=torch.int32, device="cuda")
    with pytest.raises(g.GqaError, match="INVALID_ARGUMENT"):
        g.stream_append(*ring, kn, kn, count, main=main)
