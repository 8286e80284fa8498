"""Scheduled partition launches (many (sequence, KV group, chunk) items): the
block -> item table the library builds on the device holds every live item
exactly once and -1 elsewhere, gives the eight XCDs (block i runs on XCD
i % 8) item counts within one sequence's items of each other, and the
results match the oracle, for both matrix-core families, through the
partition/combine pair and through decode_step."""

import math

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
    gen = torch.Generator().manual_seed(seed)
    lens = torch.randint(0, max_len + 1, (batch,), generator=gen)
    lens[0], lens[1], lens[2], lens[3] = 0, 1, max_len, max_len + 9
    return lens.to(torch.int32)


def _check_table(ws, plan, lens, w):
    """Every live item once, -1 elsewhere, XCD loads balanced."""
    assert plan.sched_entries > 0, "scheduled plan expected"
    t = ws[plan.off_sched:plan.off_sched + 4 * plan.sched_entries]
    table = t.cpu().view(torch.int32).numpy()
    nc, chunk, H = plan.num_chunks, plan.chunk_tokens, w.num_kv_heads
    live = []
    for b, n in enumerate(lens.tolist()):
        n = min(max(n, 0), w.max_len)
        for g in range(H):
            live += [(b * H + g) * nc + c for c in range(math.ceil(n / chunk))]
    got = table[table >= 0]
    assert np.all((table >= 0) | (table == -1)), "entries are items or -1"
    assert sorted(got.tolist()) == sorted(live), "each live item exactly once"
    per_xcd = [int(np.sum(table[x::8] >= 0)) for x in range(8)]
    say(f"  items per XCD {per_xcd}")
    assert max(per_xcd) - min(per_xcd) <= H * nc, "XCD shares balanced"


def _oracle_check(x, w, out, cout, what):
    ref, cref = oracle.attend(np64(x["q"]), np64(x["k"]), np64(x["v"]),
                              x["lens"].numpy(), w.scale)
    vmax = live_vmax(x["v"], x["lens"])
    check_out(out.cpu().numpy(), ref, vmax, w.dtype, what)
    check_carry(cout.m.cpu().numpy(), cout.l.cpu().numpy(), cref.m, cref.l,
                w.dtype, what + " carry")


SCHED = {
    # (workload, explicit chunk): batch * num_kv_heads * num_chunks >= 1024
    "bf16_d128": (wl.RAGGED_BF16.replace(batch=64, num_q_heads=32,
                                         num_kv_heads=4, max_len=1000), 128),
    "bf16_dk192_hpk16": (wl.WIDE_SPIKE_BF16.replace(batch=32, max_len=700),
                         64),
    "f32_d64": (wl.TINY_F32.replace(batch=64, num_q_heads=8, num_kv_heads=4,
                                    max_len=600), 64),
}


@pytest.mark.parametrize("name", list(SCHED))
def test_scheduled_partition(name):
    g = _gqa()
    w, chunk = SCHED[name]
    lens = _lens(w.batch, w.max_len, 31)
    x = wl.make_inputs(w, lens_override=lens.tolist())
    say(f"[sched] {name}")
    d = to_dev(x)
    plan = g.attend_plan(d["k"], d["v"], w.num_q_heads, chunk)
    ws = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device="cuda")
    g.attend_partition(d["q"], d["k"], d["v"], d["lens"], plan, ws, w.scale)
    cout = g.empty_carry(w.batch * w.num_q_heads, w.dv)
    out = g.attend_combine(w.num_q_heads, d["k"], d["v"], d["lens"], plan, ws,
                           carry_out=cout)
    torch.cuda.synchronize()
    _check_table(ws, plan, lens, w)
    _oracle_check(x, w, out, cout, name)


def test_scheduled_decode_step():
    """decode_step with an automatic plan large enough to be scheduled (an
    fp32 cache: bf16 / fp8 ones get a balanced plan instead); the schedule
    counts the new token of each appended sequence and does the lengths and
    drops of every sequence."""
    g = _gqa()
    w = wl.TINY_F32.replace(batch=64, num_q_heads=16, num_kv_heads=8,
                            dk=64, dv=64, max_len=4100, scale=0.0)
    lens = _lens(w.batch, w.max_len, 32)
    lens[5] = w.max_len - 1   # the append fills the cache
    lens[6] = 4095            # the new token opens the second chunk
    lens[7] = -2              # negative: nothing appended, drop counted
    x = wl.make_inputs(w, lens_override=lens.clamp(0, w.max_len).tolist(),
                       pad_value=0.0)
    d = to_dev(x)
    plan = g.attend_plan(d["k"], d["v"], w.num_q_heads)
    assert plan.sched_entries > 0 and plan.balanced_groups == 0, \
        "scheduled plan expected"
    gen = torch.Generator().manual_seed(33)
    kn = torch.randn(w.batch, w.num_kv_heads, w.dk, generator=gen).to(
        w.torch_dtype)
    vn = torch.randn(w.batch, w.num_kv_heads, w.dv, generator=gen).to(
        w.torch_dtype)
    li = lens.cuda()
    lo = torch.empty_like(li)
    ws = g.step_workspace(d["k"], d["v"], w.num_q_heads)
    cout = g.empty_carry(w.batch * w.num_q_heads, w.dv)
    lo.fill_(12345)           # every entry must be written by the step
    dropped = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = g.decode_step(d["q"], d["k"], d["v"], kn.cuda(), vn.cuda(), li, lo,
                        w.scale, carry_out=cout, workspace=ws,
                        dropped=dropped)
    torch.cuda.synchronize()
    bits = lambda t: t.view(torch.int16)
    k_ref, v_ref, l_ref, n_drop = oracle.kv_append(
        bits(x["k"]).numpy(), bits(x["v"]).numpy(), bits(kn).numpy(),
        bits(vn).numpy(), lens.numpy())
    assert np.array_equal(bits(d["k"].cpu()).numpy(), k_ref), "K after append"
    assert np.array_equal(bits(d["v"].cpu()).numpy(), v_ref), "V after append"
    assert lo.cpu().numpy().tolist() == l_ref.tolist(), "lens"
    assert int(dropped.item()) == n_drop == 3, "drops: full, past, negative"
    _check_table(ws, plan, torch.from_numpy(l_ref.astype(np.int32)), w)
    xa = {"q": x["q"], "k": torch.from_numpy(k_ref).view(w.torch_dtype),
          "v": torch.from_numpy(v_ref).view(w.torch_dtype),
          "lens": torch.from_numpy(l_ref.astype(np.int32))}
    _oracle_check(xa, w, out, cout, "scheduled decode_step")
