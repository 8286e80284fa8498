"""decode_step (kv_append + attend in one launch) against the oracle: the
cache after the append bit for bit, lengths and drop count exactly, outputs and
carries within tolerance; on shapes whose partials are folded in the launch's
last work-group and on shapes that keep the separate combine; over consecutive
steps and HIP-graph replays (the arrival counters must return to zero)."""

import numpy as np
import pytest
import torch

import oracle
from gpu_util import check_carry, check_out, live_vmax, np64, say
from gqa_kv_cache_decode_amd import workloads as wl

pytestmark = pytest.mark.gpu

FUSE_BYTES = 64 * 1024


def _gqa():
    import gqa_kv_cache_decode_amd as g
    return g


def _fuses(g, d, w):
    plan = g.attend_plan(d["k"], d["v"], w.num_q_heads)
    return w.hpk * plan.num_chunks * (w.dv + 2) * 4 <= FUSE_BYTES, plan


def _new_rows(w, seed):
    gen = torch.Generator().manual_seed(seed)
    kn = torch.randn(w.batch, w.num_kv_heads, w.dk, generator=gen)
    vn = torch.randn(w.batch, w.num_kv_heads, w.dv, generator=gen)
    return kn.to(w.torch_dtype), vn.to(w.torch_dtype)


def _bits(t):
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32)


def _check_step(w, x, lens_in, kn, vn, d_after, lens_out, out, carry_in=None,
                carry_out=None, dropped=None, what=""):
    """Oracle: push_kv then attention over the cache including the new token."""
    k_ref, v_ref, l_ref, drop_ref = oracle.kv_append(
        _bits(x["k"]).numpy(), _bits(x["v"]).numpy(), _bits(kn).numpy(),
        _bits(vn).numpy(), np.asarray(lens_in))
    assert np.array_equal(_bits(d_after["k"].cpu()).numpy(), k_ref), \
        f"{what}: K cache after append"
    assert np.array_equal(_bits(d_after["v"].cpu()).numpy(), v_ref), \
        f"{what}: V cache after append"
    assert lens_out.cpu().numpy().tolist() == l_ref.tolist(), f"{what}: lens"
    if dropped is not None:
        assert int(dropped.item()) == drop_ref, f"{what}: dropped"
    k64 = torch.from_numpy(k_ref).view(w.torch_dtype)
    v64 = torch.from_numpy(v_ref).view(w.torch_dtype)
    ref, cref = oracle.attend(np64(x["q"]), np64(k64), np64(v64), l_ref,
                              w.scale, carry_in=carry_in)
    vmax = live_vmax(v64, l_ref)
    check_out(out.cpu().numpy(), ref, vmax, w.dtype, what)
    if carry_out is not None:
        check_carry(carry_out.m.cpu().numpy(), carry_out.l.cpu().numpy(),
                    cref.m, cref.l, w.dtype, what + " carry")
    return ref


STEP_SHAPES = {
    "batched_bf16": (wl.BATCHED_BF16.replace(batch=4, max_len=1200),
                     [1199, 500, 0, 1]),
    "ragged_full_and_negative": (wl.RAGGED_BF16.replace(batch=5, max_len=900),
                                 [900, 37, -2, 899, 450]),
    "spike_bf16_unfused": (wl.WIDE_SPIKE_BF16.replace(batch=2, max_len=4000),
                           [3999, 2500]),
    "long_bf16_unfused": (wl.LONG_WINDOW_BF16.replace(max_len=40000, window=0),
                          [39000]),
    "tiny_f32": (wl.TINY_F32, [255]),
    "f32_d128": (wl.TINY_F32.replace(dk=128, dv=128, num_q_heads=16,
                                     num_kv_heads=4, max_len=700, batch=3),
                 [699, 0, 350]),
    "f32_vector_alu_shape": (wl.TINY_F32.replace(dk=48, dv=80, max_len=300,
                                                 batch=2), [299, 10]),
}


@pytest.mark.parametrize("name", list(STEP_SHAPES))
def test_step_vs_oracle(name):
    g = _gqa()
    w, lens0 = STEP_SHAPES[name]
    x = wl.make_inputs(w, lens_override=[min(max(n, 0), w.max_len)
                                         for n in lens0], pad_value=0.0)
    kn, vn = _new_rows(w, 11)
    d = {k: (t.cuda() if isinstance(t, torch.Tensor) else t)
         for k, t in x.items()}
    fused, _ = _fuses(g, d, w)
    say(f"[step] {name}: fused fold = {fused}")
    lens_in = torch.tensor(lens0, dtype=torch.int32, device="cuda")
    lens_out = torch.full_like(lens_in, -77)
    dropped = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = g.step_workspace(d["k"], d["v"], w.num_q_heads)
    out = g.decode_step(d["q"], d["k"], d["v"], kn.cuda(), vn.cuda(), lens_in,
                        lens_out, w.scale, workspace=ws, dropped=dropped)
    torch.cuda.synchronize()
    _check_step(w, x, lens0, kn, vn, d, lens_out, out, dropped=dropped,
                what=name)
    plan = g.attend_plan(d["k"], d["v"], w.num_q_heads)
    assert torch.all(ws[plan.workspace_bytes:] == 0), "counters back to zero"
    assert lens_in.cpu().tolist() == lens0, "lens_in is not written"


@pytest.mark.parametrize("name", ["batched_bf16", "spike_bf16_unfused"])
def test_step_carry_in_out(name):
    """carry_in (a recent-window branch over the same queries) folds in;
    carry_out aliases carry_in."""
    g = _gqa()
    w, lens0 = STEP_SHAPES[name]
    x = wl.make_inputs(w, lens_override=[min(max(n, 0), w.max_len)
                                         for n in lens0], pad_value=0.0)
    kn, vn = _new_rows(w, 12)
    d = {k: (t.cuda() if isinstance(t, torch.Tensor) else t)
         for k, t in x.items()}
    # the window branch: its own small cache, attended first for the carry
    ww = w.replace(max_len=128)
    xw = wl.make_inputs(ww.replace(seed_index=ww.seed_index + 50))
    rows = w.batch * w.num_q_heads
    carry = g.empty_carry(rows, w.dv)
    g.attend_decode(d["q"], xw["k"].cuda(), xw["v"].cuda(), xw["lens"].cuda(),
                    w.scale, carry_out=carry, out=None)
    torch.cuda.synchronize()
    cin_np = oracle.Carry(carry.m.cpu().double().numpy(),
                          carry.l.cpu().double().numpy(),
                          carry.acc.cpu().double().numpy())
    lens_in = torch.tensor(lens0, dtype=torch.int32, device="cuda")
    lens_out = torch.empty_like(lens_in)
    out = g.decode_step(d["q"], d["k"], d["v"], kn.cuda(), vn.cuda(), lens_in,
                        lens_out, w.scale, carry_in=carry, carry_out=carry)
    torch.cuda.synchronize()
    _check_step(w, x, lens0, kn, vn, d, lens_out, out, carry_in=cin_np,
                carry_out=carry, what=name + " with carry")


@pytest.mark.parametrize("name", ["batched_bf16", "long_bf16_unfused",
                                  "tiny_f32"])
def test_consecutive_steps(name):
    """Four steps alternating two length arrays, each checked."""
    g = _gqa()
    w, lens0 = STEP_SHAPES[name]
    lens0 = [max(0, n - 3) for n in lens0]
    x = wl.make_inputs(w, lens_override=lens0, pad_value=0.0)
    d = {k: (t.cuda() if isinstance(t, torch.Tensor) else t)
         for k, t in x.items()}
    ws = g.step_workspace(d["k"], d["v"], w.num_q_heads)
    la = torch.tensor(lens0, dtype=torch.int32, device="cuda")
    lb = torch.empty_like(la)
    cur = {"k": x["k"].clone(), "v": x["v"].clone(), "q": x["q"]}
    lens = list(lens0)
    for step in range(4):
        kn, vn = _new_rows(w, 100 + step)
        out = g.decode_step(d["q"], d["k"], d["v"], kn.cuda(), vn.cuda(), la,
                            lb, w.scale, workspace=ws)
        torch.cuda.synchronize()
        ref = _check_step(w, {"q": cur["q"], "k": cur["k"], "v": cur["v"]},
                          lens, kn, vn, d, lb, out, what=f"{name} step {step}")
        cur["k"], cur["v"] = d["k"].cpu(), d["v"].cpu()
        lens = lb.cpu().tolist()
        la, lb = lb, la


def test_step_graph_replays():
    """One captured step replayed three times, with eager work and a
    synchronisation between replays; every replay equals the eager step."""
    g = _gqa()
    w, lens0 = STEP_SHAPES["batched_bf16"]
    x = wl.make_inputs(w, lens_override=lens0, pad_value=0.0)
    kn, vn = _new_rows(w, 13)
    d = {k: (t.cuda() if isinstance(t, torch.Tensor) else t)
         for k, t in x.items()}
    knd, vnd = kn.cuda(), vn.cuda()
    ws = g.step_workspace(d["k"], d["v"], w.num_q_heads)
    lens_in = torch.tensor(lens0, dtype=torch.int32, device="cuda")
    lens_out = torch.empty_like(lens_in)
    out = torch.empty(w.batch, w.num_q_heads, w.dv, device="cuda")
    g.decode_step(d["q"], d["k"], d["v"], knd, vnd, lens_in, lens_out,
                  w.scale, out=out, workspace=ws)
    torch.cuda.synchronize()
    eager = out.clone()
    _check_step(w, x, lens0, kn, vn, d, lens_out, out, what="eager")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        g.decode_step(d["q"], d["k"], d["v"], knd, vnd, lens_in, lens_out,
                      w.scale, out=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        g.decode_step(d["q"], d["k"], d["v"], knd, vnd, lens_in, lens_out,
                      w.scale, out=out, workspace=ws)
    plan = g.attend_plan(d["k"], d["v"], w.num_q_heads)
    for rep in range(3):
        out.fill_(float("nan"))
        lens_out.fill_(-1)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep} differs from eager"
        assert lens_out.cpu().tolist() == [n + 1 for n in lens0]
        assert torch.all(ws[plan.workspace_bytes:] == 0)
        _ = (torch.randn(1000, device="cuda") * 2).sum().item()  # eager work
