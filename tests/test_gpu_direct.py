"""The single-chunk plan against the oracle: when a batch has enough
(sequence, KV group) units and its caches fit one chunk, the partition launch
folds carry_in and writes out and carry_out itself (no partials, no combine
launch).  Covered for every head width of both matrix-core families (bf16 with
four wavefronts for dk + dv <= 256, else two; fp32 with two), with ragged,
empty and over-long lengths, a carry_in from a window branch with carry_out
aliasing it, and through decode_step, eagerly and replayed from a HIP graph."""

import numpy as np
import pytest
import torch

import oracle
from gpu_util import check_carry, check_out, live_vmax, np64, say, to_dev
from gqa_kv_cache_decode_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _gqa():
    import gqa_kv_cache_decode_amd as g
    return g


def _lens(batch, max_len, seed):
    """Ragged lengths with the edge values planted: 0, 1, max_len and a
    length past max_len (read as max_len)."""
    gen = torch.Generator().manual_seed(seed)
    lens = torch.randint(0, max_len + 1, (batch,), generator=gen)
    lens[0], lens[1], lens[2], lens[3] = 0, 1, max_len, max_len + 5
    return lens.to(torch.int32)


# every shape has batch * num_kv_heads >= 256 and max_len <= 4096
DIRECT = {
    "bf16_d128_hpk4": wl.BATCHED_BF16.replace(batch=64, num_q_heads=16,
                                               num_kv_heads=4, max_len=700),
    "bf16_d64_hpk2": wl.BATCHED_BF16.replace(batch=128, num_q_heads=4,
                                              num_kv_heads=2, dk=64, dv=64,
                                              max_len=333),
    "bf16_dk192_hpk16": wl.WIDE_SPIKE_BF16.replace(batch=64, max_len=300),
    "bf16_d256_mha": wl.BATCHED_BF16.replace(batch=256, num_q_heads=1,
                                             num_kv_heads=1, dk=256, dv=256,
                                             max_len=130),
    "f32_d128_hpk2": wl.TINY_F32.replace(batch=64, num_q_heads=8,
                                         num_kv_heads=4, dk=128, dv=128,
                                         max_len=300),
    "f32_d64_hpk2": wl.TINY_F32.replace(batch=128, num_q_heads=4,
                                        num_kv_heads=2, max_len=257),
}


def _window_carry(g, w, d):
    """carry of a 128-token window branch over the same queries."""
    ww = w.replace(max_len=128, ragged=False,
                   seed_index=w.seed_index + 60)
    xw = wl.make_inputs(ww)
    carry = g.empty_carry(w.batch * w.num_q_heads, w.dv)
    g.attend_decode(d["q"], xw["k"].cuda(), xw["v"].cuda(),
                    xw["lens"].cuda(), w.scale, carry_out=carry, out=None)
    torch.cuda.synchronize()
    return carry


def _np_carry(c):
    return oracle.Carry(c.m.cpu().double().numpy(), c.l.cpu().double().numpy(),
                        c.acc.cpu().double().numpy())


@pytest.mark.parametrize("name", list(DIRECT))
@pytest.mark.parametrize("with_carry", [False, True])
def test_direct_attend(name, with_carry):
    g = _gqa()
    w = DIRECT[name]
    lens = _lens(w.batch, w.max_len, 5)
    x = wl.make_inputs(w, lens_override=lens.tolist())
    say(f"[direct] {name} carry={with_carry}")
    d = to_dev(x)
    plan = g.attend_plan(d["k"], d["v"], w.num_q_heads)
    assert plan.num_chunks == 1, "single-chunk plan expected"
    rows = w.batch * w.num_q_heads
    cin = _window_carry(g, w, d) if with_carry else None
    cin_np = _np_carry(cin) if with_carry else None
    cout = cin if with_carry else g.empty_carry(rows, w.dv)  # aliases carry_in
    out = g.attend_decode(d["q"], d["k"], d["v"], d["lens"], w.scale,
                          carry_in=cin, carry_out=cout)
    torch.cuda.synchronize()
    ref, cref = oracle.attend(np64(x["q"]), np64(x["k"]), np64(x["v"]),
                              x["lens"].numpy(), w.scale, carry_in=cin_np)
    vmax = live_vmax(x["v"], x["lens"])
    if with_carry:
        vmax = max(vmax, float(np.max(np.abs(oracle.finalize(cin_np)))))
    check_out(out.cpu().numpy(), ref, vmax, w.dtype, name)
    check_carry(cout.m.cpu().numpy(), cout.l.cpu().numpy(), cref.m, cref.l,
                w.dtype, name + " carry")
    if not with_carry:
        empty = x["lens"].numpy() <= 0
        o = out.cpu().numpy()
        assert np.all(o[empty] == 0.0), "empty sequence gives 0"
        m = cout.m.cpu().numpy().reshape(w.batch, -1)
        assert np.all(np.isneginf(m[empty])), "empty carry m = -inf"


def _new_rows(w, seed):
    gen = torch.Generator().manual_seed(seed)
    kn = torch.randn(w.batch, w.num_kv_heads, w.dk, generator=gen)
    vn = torch.randn(w.batch, w.num_kv_heads, w.dv, generator=gen)
    return kn.to(w.torch_dtype), vn.to(w.torch_dtype)


def _bits(t):
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32)


@pytest.mark.parametrize("name", ["bf16_d128_hpk4", "bf16_dk192_hpk16",
                                  "f32_d128_hpk2"])
def test_direct_decode_step(name):
    """append + attend in one launch with the single-chunk plan: the cache bit
    for bit, lens and drops exactly, out and carry (folding a window carry,
    carry_out aliasing it) within tolerance."""
    g = _gqa()
    w = DIRECT[name]
    lens_in = _lens(w.batch, w.max_len, 6)
    lens_in[4] = -3  # dropped, attended as empty
    x = wl.make_inputs(w, lens_override=lens_in.clamp(0, w.max_len).tolist(),
                       pad_value=0.0)
    d = to_dev(x)
    kn, vn = _new_rows(w, 21)
    cin = _window_carry(g, w, d)
    cin_np = _np_carry(cin)
    li = lens_in.cuda()
    lo = torch.full_like(li, -77)
    dropped = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = g.step_workspace(d["k"], d["v"], w.num_q_heads)
    out = g.decode_step(d["q"], d["k"], d["v"], kn.cuda(), vn.cuda(), li, lo,
                        w.scale, carry_in=cin, carry_out=cin, workspace=ws,
                        dropped=dropped)
    torch.cuda.synchronize()
    k_ref, v_ref, l_ref, drop_ref = oracle.kv_append(
        _bits(x["k"]).numpy(), _bits(x["v"]).numpy(), _bits(kn).numpy(),
        _bits(vn).numpy(), lens_in.numpy())
    assert np.array_equal(_bits(d["k"].cpu()).numpy(), k_ref), "K after append"
    assert np.array_equal(_bits(d["v"].cpu()).numpy(), v_ref), "V after append"
    assert lo.cpu().numpy().tolist() == l_ref.tolist(), "lens"
    assert int(dropped.item()) == drop_ref, "dropped"
    k64 = torch.from_numpy(k_ref).view(w.torch_dtype)
    v64 = torch.from_numpy(v_ref).view(w.torch_dtype)
    ref, cref = oracle.attend(np64(x["q"]), np64(k64), np64(v64), l_ref,
                              w.scale, carry_in=cin_np)
    vmax = max(live_vmax(v64, l_ref),
               float(np.max(np.abs(oracle.finalize(cin_np)))))
    check_out(out.cpu().numpy(), ref, vmax, w.dtype, name + " step")
    check_carry(cin.m.cpu().numpy(), cin.l.cpu().numpy(), cref.m, cref.l,
                w.dtype, name + " step carry")


def test_direct_step_graph_replays():
    """A captured single-chunk decode step replayed three times with eager
    work between replays; each replay matches the eager result bit for bit
    (the step rewrites the same slot from the same lengths)."""
    g = _gqa()
    w = DIRECT["bf16_d128_hpk4"]
    lens0 = _lens(w.batch, w.max_len, 7).clamp(0, w.max_len - 1)
    x = wl.make_inputs(w, lens_override=lens0.tolist(), pad_value=0.0)
    d = to_dev(x)
    kn, vn = _new_rows(w, 22)
    knd, vnd = kn.cuda(), vn.cuda()
    ws = g.step_workspace(d["k"], d["v"], w.num_q_heads)
    li = lens0.cuda()
    lo = torch.empty_like(li)
    out = torch.empty(w.batch, w.num_q_heads, w.dv, device="cuda")
    g.decode_step(d["q"], d["k"], d["v"], knd, vnd, li, lo, w.scale, out=out,
                  workspace=ws)
    torch.cuda.synchronize()
    eager = out.clone()
    lens_eager = lo.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        g.decode_step(d["q"], d["k"], d["v"], knd, vnd, li, lo, w.scale,
                      out=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        g.decode_step(d["q"], d["k"], d["v"], knd, vnd, li, lo, w.scale,
                      out=out, workspace=ws)
    for rep in range(3):
        out.fill_(float("nan"))
        lo.fill_(-1)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep}: out"
        assert torch.equal(lo, lens_eager), f"replay {rep}: lens"
        _ = (d["q"].float() * 2).sum().item()  # eager work in between
