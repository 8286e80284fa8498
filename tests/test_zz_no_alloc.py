"""attend_decode_noalloc (the allocation-free attend_decode, on the library's
own device scratch array) against attend_decode with a workspace of the
caller's: two calls in a row through the C ABI, the second with a smaller
input, each identical bit for bit to attend_decode on the same inputs and
within the oracle's tolerance.  The first is a balanced plan (ragged batch,
carry in and out), the second a small chunked one with a bias."""

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


def _carry_in(rows, dv, seed):
    rng = np.random.default_rng(seed)
    m = rng.normal(0.0, 2.0, rows)
    l = rng.uniform(0.5, 3.0, rows)
    acc = rng.normal(0.0, 1.0, (rows, dv)) * l[:, None]
    l[rng.random(rows) < 0.2] = 0.0
    return oracle.Carry(m, l, acc)


def _dev(g, c):
    d = g.empty_carry(*c.acc.shape)
    d.m.copy_(torch.from_numpy(c.m).float())
    d.l.copy_(torch.from_numpy(c.l).float())
    d.acc.copy_(torch.from_numpy(c.acc).float())
    return d


def _case(g, w, lens, seed, with_carry, with_bias, balanced):
    x = wl.make_inputs(w, lens_override=lens)
    d = to_dev(x)
    plan = g.attend_plan(d["k"], d["v"], w.num_q_heads)
    assert (plan.balanced_groups > 0) == balanced, "plan kind"
    rows = w.batch * w.num_q_heads
    cin = _carry_in(rows, w.dv, seed) if with_carry else None
    bias = None
    if with_bias:
        gen = torch.Generator().manual_seed(seed)
        bias = torch.randn(w.batch, (w.max_len + 3) // 4 * 4, generator=gen)
    runs = []
    for noalloc in (True, False):
        cout = g.empty_carry(rows, w.dv)
        out = torch.full((w.batch, w.num_q_heads, w.dv), float("nan"),
                         device="cuda")
        kw = dict(carry_in=None if cin is None else _dev(g, cin),
                  carry_out=cout, out=out,
                  bias=None if bias is None else bias.cuda())
        if noalloc:
            g.attend_decode_noalloc(d["q"], d["k"], d["v"], d["lens"],
                                    w.scale, **kw)
        else:
            g.attend_decode(d["q"], d["k"], d["v"], d["lens"], w.scale, **kw)
        torch.cuda.synchronize()
        runs.append((out.cpu(), cout.m.cpu(), cout.l.cpu(), cout.acc.cpu()))
    for a, b in zip(*runs):
        assert torch.equal(a, b), "noalloc differs from attend_decode"
    ref, cref = oracle.attend(np64(x["q"]), np64(x["k"]), np64(x["v"]),
                              x["lens"].numpy(), w.scale, carry_in=cin,
                              bias=None if bias is None else
                              bias.double().numpy())
    vmax = live_vmax(x["v"], x["lens"])
    if cin is not None:
        vmax = max(vmax, float(np.max(np.abs(oracle.finalize(cin)))))
    check_out(runs[0][0].numpy(), ref, vmax, w.dtype, f"noalloc {w.name}")
    check_carry(runs[0][1].numpy(), runs[0][2].numpy(), cref.m, cref.l,
                w.dtype, f"noalloc {w.name} carry")


def test_noalloc_matches_attend_decode():
    g = _gqa()
    # first call: a balanced plan (a multi-round ragged batch)
    w1 = wl.RAGGED_BF16.replace(batch=32, num_q_heads=32, num_kv_heads=8,
                                max_len=16400)
    gen = torch.Generator().manual_seed(61)
    lens1 = torch.randint(0, w1.max_len + 1, (w1.batch,), generator=gen)
    lens1[0], lens1[1] = 0, w1.max_len
    say("[noalloc] call 1: balanced ragged batch, carry in and out")
    _case(g, w1, lens1.tolist(), 62, True, False, balanced=True)
    # second call, smaller: a chunked plan with a bias
    w2 = wl.BATCHED_BF16.replace(batch=2, max_len=777)
    say("[noalloc] call 2: small batch, bias")
    _case(g, w2, [777, 300], 63, False, True, balanced=False)
