"""Balanced launches: a bf16 / fp8 cache whose chunked launch would take
several rounds of work-groups gets the library's balanced plan (a work
queue of runs of 32-token tiles, shrinking towards its end, taken by 512
persistent work-groups).  Checked against the oracle through every entry
point that takes such a plan: attend_decode, the attend_partition /
attend_combine pair, and decode_step (the append in the same launch, the
lengths and drops written by the balance kernel).  Shapes cover empty,
negative, full and past-the-cache lengths, one long sequence among tiny
ones, fewer items than work-groups, every compiled head shape, the additive
bias, carry_in and fp8 caches.  The queue the balance kernel builds is
checked word for word."""

import math

import numpy as np
import pytest
import torch

import oracle
import oracle.fp8 as of8
from gpu_util import check_carry, check_out, live_vmax, np64, say, to_dev
from gqa_kv_cache_decode_amd import workloads as wl

pytestmark = pytest.mark.gpu

TILE = 32


def _gqa():
    import gqa_kv_cache_decode_amd as g
    return g


def _phase_runs(nt):
    """The three phases of a sequence of nt tiles: runs of 128 tiles over
    the whole runs of its first 3/4, of 32 up to 23/25, of 8 over the rest."""
    e0 = nt * 3 // 4 // 128 * 128
    e1 = e0 + max(nt * 23 // 25 - e0, 0) // 32 * 32
    return [(0, e0, 128), (e0, e1, 32), (e1, nt, 8)]


def _seq_runs(nt, k):
    """Runs (first, end tile) of phase k of a sequence of nt tiles."""
    s, e, L = _phase_runs(nt)[k]
    return [(s + j * L, min(s + (j + 1) * L, e)) for j in range(-(-(e - s) // L))]


def _check_queue(ws, plan, lens, w, launched=True):
    """The work queue, word for word: the runs phase by phase and sequence
    by sequence, each sequence's first run per phase, the item count; after
    the partition launch the counter has passed every item once and each of
    the 512 work-groups' final fetch."""
    assert plan.balanced_groups == 512, "balanced plan expected"
    t = ws[plan.off_sched:plan.off_sched + 4 * plan.sched_entries]
    q = t.cpu().view(torch.int32).numpy().astype(np.int64)
    B = w.batch
    n = np.clip(np.asarray(lens, dtype=np.int64), 0, w.max_len)
    nt = (n + TILE - 1) // TILE
    runs, base, pre = [], [], []
    for k in range(3):
        base.append(len(runs))
        pk = []
        for b in range(B):
            pk.append(len(runs) - base[k])
            runs += [(b, t0, t1) for t0, t1 in _seq_runs(int(nt[b]), k)]
        pk.append(len(runs) - base[k])
        pre.append(pk)
    base.append(len(runs))
    items = len(runs) * w.num_kv_heads
    assert q[1] == items, "item count"
    assert q[2:6].tolist() == base, "phase starts"
    off = 6 + 3 * (B + 1)
    assert q[6:off].reshape(3, B + 1).tolist() == pre, "runs per sequence"
    got = q[off:off + 3 * len(runs)].reshape(-1, 3)
    assert got.tolist() == [list(r) for r in runs], "runs"
    if launched:
        assert q[0] == items + 512, "every item taken once"
    return items


def _random_carry(rows, dv, seed):
    """A carry with live rows, empty rows (l = 0, m arbitrary) and rows
    that dominate."""
    rng = np.random.default_rng(seed)
    m = rng.normal(0.0, 2.0, rows)
    l = rng.uniform(0.5, 3.0, rows)
    acc = rng.normal(0.0, 1.0, (rows, dv)) * l[:, None]
    l[rng.random(rows) < 0.2] = 0.0
    m[l == 0.0] = 5.0     # ignored: the row is empty
    m[rng.random(rows) < 0.05] += 30.0   # carry far above the keys
    return oracle.Carry(m, l, acc)


def _dev_carry(c):
    g = _gqa()
    rows, dv = c.acc.shape
    d = g.empty_carry(rows, dv)
    d.m.copy_(torch.from_numpy(c.m).float())
    d.l.copy_(torch.from_numpy(c.l).float())
    d.acc.copy_(torch.from_numpy(c.acc).float())
    return d


def _oracle_check(x, w, out, cout, what, carry_in=None, bias=None):
    ref, cref = oracle.attend(np64(x["q"]), np64(x["k"]), np64(x["v"]),
                              x["lens"].numpy(), w.scale, carry_in=carry_in,
                              bias=bias)
    vmax = live_vmax(x["v"], x["lens"])
    if carry_in is not None:
        vmax = max(vmax, float(np.max(np.abs(finalize_rows(carry_in)))))
    check_out(out.cpu().numpy(), ref, vmax, w.dtype, what)
    if cout is not None:
        check_carry(cout.m.cpu().numpy(), cout.l.cpu().numpy(), cref.m,
                    cref.l, w.dtype, what + " carry")


def finalize_rows(c):
    live = c.l > 0
    out = np.zeros_like(c.acc)
    out[live] = c.acc[live] / c.l[live][:, None]
    return out


# Shapes the library balances by itself (a chunked launch would take
# several rounds of work-groups): name -> (workload, lens recipe)
SHAPES = {
    "d128_ragged": (wl.RAGGED_BF16.replace(batch=32, num_q_heads=32,
                                           num_kv_heads=8, max_len=16400),
                    "ragged"),
    "d128_skewed": (wl.RAGGED_BF16.replace(batch=128, num_q_heads=32,
                                           num_kv_heads=8, max_len=8192),
                    "skewed"),
    "d128_sparse": (wl.RAGGED_BF16.replace(batch=64, num_q_heads=64,
                                           num_kv_heads=8, max_len=8200),
                    "sparse"),
    "dk192_hpk16": (wl.WIDE_SPIKE_BF16.replace(batch=64, max_len=16400,
                                               dist="normal", ragged=True),
                    "ragged"),
}

# Small shapes with a balanced plan asked for explicitly (units then span
# many ranges each): every compiled head shape, odd group sizes.
SMALL = {
    "d64_hpk2": wl.RAGGED_BF16.replace(batch=16, num_q_heads=16,
                                       num_kv_heads=8, dk=64, dv=64,
                                       max_len=1500),
    "d128_hpk4": wl.RAGGED_BF16.replace(batch=8, num_q_heads=32,
                                        num_kv_heads=8, max_len=900),
    "d128_hpk5": wl.RAGGED_BF16.replace(batch=5, num_q_heads=10,
                                        num_kv_heads=2, max_len=3000),
    "dk192_hpk16": wl.WIDE_SPIKE_BF16.replace(batch=4, max_len=700,
                                              dist="normal", ragged=True),
    "d256_hpk3": wl.RAGGED_BF16.replace(batch=6, num_q_heads=12,
                                        num_kv_heads=4, dk=256, dv=256,
                                        max_len=1300),
}


def _lens(w, recipe, seed):
    gen = torch.Generator().manual_seed(seed)
    B, T = w.batch, w.max_len
    if recipe == "skewed":    # one long unit among tiny ones
        lens = torch.randint(1, 41, (B,), generator=gen)
        lens[3] = T
        lens[77] = T - 5
    elif recipe == "sparse":  # fewer tiles than work-groups
        lens = torch.zeros(B, dtype=torch.int64)
        lens[::5] = torch.randint(1, 60, (len(lens[::5]),), generator=gen)
    else:
        lens = torch.randint(0, T + 1, (B,), generator=gen)
        lens[0], lens[1], lens[2], lens[3] = 0, 1, T, T + 9
    return lens.to(torch.int32)


def _plan_ws(g, d, w):
    plan = g.attend_plan(d["k"], d["v"], w.num_q_heads)
    assert plan.balanced_groups == 512, "balanced plan expected"
    ws = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device="cuda")
    return plan, ws


@pytest.mark.parametrize("name", list(SHAPES))
def test_balanced_attend_decode(name):
    """attend_decode with carry_in and carry_out (aliased), against the
    oracle's merge of carry_in with one pass over the keys."""
    g = _gqa()
    w, recipe = SHAPES[name]
    lens = _lens(w, recipe, 41)
    x = wl.make_inputs(w, lens_override=lens.tolist())
    say(f"[balanced] attend_decode {name}")
    d = to_dev(x)
    plan, ws = _plan_ws(g, d, w)
    cin = _random_carry(w.batch * w.num_q_heads, w.dv, 42)
    c = _dev_carry(cin)
    out = g.attend_decode(d["q"], d["k"], d["v"], d["lens"], w.scale,
                          carry_in=c, carry_out=c, workspace=ws)
    torch.cuda.synchronize()
    items = _check_queue(ws, plan, lens, w)
    say(f"  {items} queue items over {plan.balanced_groups} work-groups")
    _oracle_check(x, w, out, c, f"balanced attend_decode {name}",
                  carry_in=cin)


@pytest.mark.parametrize("name", ["small_" + n for n in SMALL] +
                         ["d128_skewed"])
def test_balanced_partition_combine(name):
    """The explicit pair: whole units leave their state per query row, cut
    ones their pieces; attend_combine folds both with carry_in.  The small
    shapes ask for the balanced plan (GQA_CHUNK_BALANCED)."""
    g = _gqa()
    if name.startswith("small_"):
        w, recipe = SMALL[name[len("small_"):]], "ragged"
    else:
        w, recipe = SHAPES[name]
    lens = _lens(w, recipe, 43)
    x = wl.make_inputs(w, lens_override=lens.tolist())
    say(f"[balanced] partition/combine {name}")
    d = to_dev(x)
    plan = g.attend_plan(d["k"], d["v"], w.num_q_heads, g.CHUNK_BALANCED)
    assert plan.balanced_groups == 512
    ws = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device="cuda")
    g.attend_partition(d["q"], d["k"], d["v"], d["lens"], plan, ws, w.scale)
    cin = _random_carry(w.batch * w.num_q_heads, w.dv, 44)
    cout = g.empty_carry(w.batch * w.num_q_heads, w.dv)
    out = g.attend_combine(w.num_q_heads, d["k"], d["v"], d["lens"], plan, ws,
                           carry_in=_dev_carry(cin), carry_out=cout)
    torch.cuda.synchronize()
    _check_queue(ws, plan, lens, w)
    _oracle_check(x, w, out, cout, f"balanced partition/combine {name}",
                  carry_in=cin)


@pytest.mark.parametrize("name", ["d128_ragged", "d128_skewed",
                                  "dk192_hpk16"])
@pytest.mark.parametrize("with_bias", [False, True])
def test_balanced_decode_step(name, with_bias):
    """decode_step on a balanced plan: the append and the lengths / drops
    (full, past-the-cache and negative lengths), the new token attended, the
    additive bias over every position including the new one."""
    g = _gqa()
    w, recipe = SHAPES[name]
    lens = _lens(w, recipe, 45)
    if recipe != "skewed":
        lens[4] = w.max_len - 1   # the append fills the cache
        lens[5] = -2              # negative: nothing appended, drop counted
    x = wl.make_inputs(w, lens_override=lens.clamp(0, w.max_len).tolist(),
                       pad_value=0.0)
    say(f"[balanced] decode_step {name} bias={with_bias}")
    d = to_dev(x)
    gen = torch.Generator().manual_seed(46)
    kn = torch.randn(w.batch, w.num_kv_heads, w.dk, generator=gen).to(
        w.torch_dtype)
    vn = torch.randn(w.batch, w.num_kv_heads, w.dv, generator=gen).to(
        w.torch_dtype)
    bias = None
    if with_bias:
        stride = (w.max_len + 3) // 4 * 4
        bias = torch.randn(w.batch, stride, generator=gen)
        bias[0, 5:9] = -math.inf    # removed keys
    li = lens.cuda()
    lo = torch.full_like(li, 12345)
    dropped = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = g.step_workspace(d["k"], d["v"], w.num_q_heads)
    plan = g.attend_plan(d["k"], d["v"], w.num_q_heads)
    assert plan.balanced_groups == 512
    cout = g.empty_carry(w.batch * w.num_q_heads, w.dv)
    out = g.decode_step(d["q"], d["k"], d["v"], kn.cuda(), vn.cuda(), li, lo,
                        w.scale, carry_out=cout, workspace=ws,
                        dropped=dropped,
                        bias=None if bias is None else bias.cuda())
    torch.cuda.synchronize()
    bits = lambda t: t.view(torch.int16)
    k_ref, v_ref, l_ref, n_drop = oracle.kv_append(
        bits(x["k"]).numpy(), bits(x["v"]).numpy(), bits(kn).numpy(),
        bits(vn).numpy(), lens.numpy())
    assert np.array_equal(bits(d["k"].cpu()).numpy(), k_ref), "K after append"
    assert np.array_equal(bits(d["v"].cpu()).numpy(), v_ref), "V after append"
    assert lo.cpu().numpy().tolist() == l_ref.tolist(), "lens"
    assert int(dropped.item()) == n_drop, "drops"
    _check_queue(ws, plan, l_ref, w)
    xa = {"q": x["q"], "k": torch.from_numpy(k_ref).view(w.torch_dtype),
          "v": torch.from_numpy(v_ref).view(w.torch_dtype),
          "lens": torch.from_numpy(l_ref.astype(np.int32))}
    _oracle_check(xa, w, out, cout, f"balanced decode_step {name}",
                  bias=None if bias is None else bias.double().numpy())


def test_balanced_decode_step_fp8():
    """fp8 caches: the new bf16 rows quantised into the slot in the step
    launch; attention over the decoded codes, against the fp8 oracle."""
    g = _gqa()
    w = wl.BATCHED_FP8.replace(batch=32, max_len=16400, ragged=True)
    lens = _lens(w, "ragged", 47)
    lens[4] = w.max_len - 1
    x = wl.make_fp8_inputs(w, lens_override=lens.clamp(0, w.max_len).tolist())
    say("[balanced] decode_step fp8")
    kc = g.Fp8Cache(x["k"].cuda(), x["k_scale"].cuda())
    vc = g.Fp8Cache(x["v"].cuda(), x["v_scale"].cuda())
    plan = g.attend_plan(kc, vc, w.num_q_heads)
    assert plan.balanced_groups == 512
    gen = torch.Generator().manual_seed(48)
    kn = torch.randn(w.batch, w.num_kv_heads, w.dk, generator=gen).to(
        torch.bfloat16)
    vn = torch.randn(w.batch, w.num_kv_heads, w.dv, generator=gen).to(
        torch.bfloat16)
    li = lens.cuda()
    lo = torch.full_like(li, -7)
    ws = g.step_workspace(kc, vc, w.num_q_heads)
    cout = g.empty_carry(w.batch * w.num_q_heads, w.dv)
    out = g.decode_step(x["q"].cuda(), kc, vc, kn.cuda(), vn.cuda(), li, lo,
                        w.scale, carry_out=cout, workspace=ws)
    torch.cuda.synchronize()
    k2, v2, l2, nd = of8.kv_append_fp8(
        x["k"].numpy(), x["v"].numpy(), kn.float().numpy(),
        vn.float().numpy(), x["k_scale"].numpy(), x["v_scale"].numpy(),
        lens.numpy())
    assert lo.cpu().tolist() == l2.tolist(), "lens"
    assert np.array_equal(kc.codes.cpu().numpy(), k2), "K codes"
    assert np.array_equal(vc.codes.cpu().numpy(), v2), "V codes"
    _check_queue(ws, plan, l2, w)
    ref, cref = of8.attend_fp8(np64(x["q"]), k2, v2,
                               x["k_scale"].double().numpy(),
                               x["v_scale"].double().numpy(), l2, w.scale)
    vals = of8.dequantize_cache(v2, x["v_scale"].double().numpy())
    vmax = max(float(np.nanmax(np.abs(vals[b, :max(int(l2[b]), 0)])))
               if l2[b] > 0 else 0.0 for b in range(w.batch))
    check_out(out.cpu().numpy(), ref, vmax, "fp8", "balanced fp8 step")
    check_carry(cout.m.cpu().numpy(), cout.l.cpu().numpy(), cref.m, cref.l,
                "fp8", "balanced fp8 step carry")


def test_balanced_many_pieces():
    """Rows with hundreds of pieces: one 800K-token sequence (533 runs, more
    than the combine folds per batch) beside a 140K-token one (97 runs), so
    the combine's register, loop and multi-batch paths all fold pieces."""
    g = _gqa()
    w = wl.RAGGED_BF16.replace(batch=2, num_q_heads=2, num_kv_heads=1, dk=64,
                               dv=64, max_len=800000, dist="normal")
    lens = torch.tensor([800000, 140000], dtype=torch.int32)
    runs = [sum(len(_seq_runs(-(-n // TILE), k)) for k in range(3))
            for n in lens.tolist()]
    assert runs[0] > 512 and 32 < runs[1] < 512, runs
    x = wl.make_inputs(w, lens_override=lens.tolist())
    say(f"[balanced] many pieces: runs per row {runs}")
    d = to_dev(x)
    plan = g.attend_plan(d["k"], d["v"], w.num_q_heads, g.CHUNK_BALANCED)
    assert plan.balanced_groups == 512
    ws = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device="cuda")
    g.attend_partition(d["q"], d["k"], d["v"], d["lens"], plan, ws, w.scale)
    cin = _random_carry(w.batch * w.num_q_heads, w.dv, 49)
    cout = g.empty_carry(w.batch * w.num_q_heads, w.dv)
    out = g.attend_combine(w.num_q_heads, d["k"], d["v"], d["lens"], plan, ws,
                           carry_in=_dev_carry(cin), carry_out=cout)
    torch.cuda.synchronize()
    _check_queue(ws, plan, lens, w)
    _oracle_check(x, w, out, cout, "balanced many pieces", carry_in=cin)
