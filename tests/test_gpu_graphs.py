"""HIP graph capture of the launch forms not covered by the decode-step graph
test: a balanced plan (balance kernel, work-queue partition, piece
combine), the fp8 group-split decode step and the index-gathered attend.
Each is captured once and replayed three times with eager work and a
synchronisation between replays; every replay must equal the eager call bit
for bit (the work queue's counter, the arrival counters and the selection
counts are rebuilt inside every replay)."""

import ctypes

import numpy as np
import pytest
import torch

from gpu_util import say, to_dev
from gqa_kv_cache_decode_amd import binding as bd
from gqa_kv_cache_decode_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _gqa():
    import gqa_kv_cache_decode_amd as g
    return g


def _replays(call, outs, what):
    """call() once eagerly, capture it, replay 3 times; outs: the tensors it
    writes."""
    call()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()  # an eager call on the capture stream first
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan") if o.is_floating_point() else -7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert torch.equal(o, e), f"{what}: replay {rep} differs from eager"
        _ = (torch.randn(1000, device="cuda") * 2).sum().item()  # eager work
    return eager


def _ragged(w, seed):
    gen = torch.Generator().manual_seed(seed)
    lens = torch.randint(1, w.max_len + 1, (w.batch,), generator=gen)
    lens[0] = w.max_len
    return lens.to(torch.int32).tolist()


def test_balanced_plan_graph():
    g = _gqa()
    w = wl.RAGGED_BF16.replace(batch=8, num_q_heads=32, max_len=3000)
    x = wl.make_inputs(w, lens_override=_ragged(w, 5))
    d = to_dev(x)
    plan = g.attend_plan(d["k"], d["v"], w.num_q_heads, g.CHUNK_BALANCED)
    assert plan.balanced_groups > 0, "balanced plan expected"
    ws = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device="cuda")
    rows = w.batch * w.num_q_heads
    out = torch.empty(w.batch, w.num_q_heads, w.dv, device="cuda")
    cout = g.empty_carry(rows, w.dv)
    say("[graph] balanced partition + combine")

    def call():
        g.attend_partition(d["q"], d["k"], d["v"], d["lens"], plan, ws, w.scale)
        g.attend_combine(w.num_q_heads, d["k"], d["v"], d["lens"], plan, ws,
                         carry_out=cout, out=out)

    _replays(call, [out, cout.m, cout.l, cout.acc], "balanced")
    # and the eager result is the library's own attend
    ref = g.attend_decode(d["q"], d["k"], d["v"], d["lens"], w.scale)
    torch.cuda.synchronize()
    assert torch.allclose(out, ref, atol=1e-5, rtol=1e-5)


def test_fp8_group_split_step_graph():
    g = _gqa()
    w = wl.BATCHED_FP8.replace(batch=16, dk=64, dv=64, max_len=1100)
    lens0 = _ragged(w.replace(max_len=w.max_len - 1), 6)
    x = wl.make_fp8_inputs(w, lens_override=lens0)
    kc = g.Fp8Cache(x["k"].cuda(), x["k_scale"].cuda())
    vc = g.Fp8Cache(x["v"].cuda(), x["v_scale"].cuda())
    plan = g.attend_plan(kc, vc, w.num_q_heads, 0)
    assert plan.sched_entries == 0 and plan.balanced_groups == 0
    assert 256 <= w.batch * w.num_kv_heads * plan.num_chunks // 8 < 512
    gen = torch.Generator().manual_seed(7)
    kn = (torch.randn(w.batch, w.num_kv_heads, w.dk, generator=gen) *
          x["k_scale"][:, :, None]).to(torch.bfloat16).cuda()
    vn = (torch.randn(w.batch, w.num_kv_heads, w.dv, generator=gen) *
          x["v_scale"][:, :, None]).to(torch.bfloat16).cuda()
    q = x["q"].cuda()
    lens_in = torch.tensor(lens0, dtype=torch.int32, device="cuda")
    lens_out = torch.empty_like(lens_in)
    ws = g.step_workspace(kc, vc, w.num_q_heads)
    out = torch.empty(w.batch, w.num_q_heads, w.dv, device="cuda")
    say("[graph] fp8 group-split decode step")

    def call():
        g.decode_step(q, kc, vc, kn, vn, lens_in, lens_out, w.scale, out=out,
                      workspace=ws)

    _replays(call, [out, lens_out], "fp8 split step")
    assert lens_out.cpu().tolist() == [n + 1 for n in lens0]


def test_gathered_graph():
    g = _gqa()
    w = wl.RAGGED_BF16.replace(batch=4, num_q_heads=32, max_len=9000)
    lens = _ragged(w, 8)
    x = wl.make_inputs(w, lens_override=lens)
    d = to_dev(x)
    rng = np.random.default_rng(9)
    width = 2048
    idx = rng.integers(-1, w.max_len + 20, (w.batch, width)).astype(np.int32)
    idxd = torch.from_numpy(idx).cuda()
    c = bd._cache(d["k"], d["v"])
    need = bd.library().gqa_attend_gathered_workspace_bytes(
        ctypes.byref(c), w.num_q_heads, width)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    out = torch.empty(w.batch, w.num_q_heads, w.dv, device="cuda")
    say("[graph] gathered attend")

    def call():
        g.attend_gathered(d["q"], d["k"], d["v"], d["lens"], idxd, w.scale,
                          out=out, workspace=ws)

    _replays(call, [out], "gathered")
