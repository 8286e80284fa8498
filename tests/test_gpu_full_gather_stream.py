"""The index-gathered and streaming workloads at full size, in the calls the
benchmark times, against the oracle on every (sequence, KV group) unit.

Gathered: 16 sequences of a 32K-slot bf16 cache (8 KV heads, 32 query heads,
128-wide heads), each attending the 2048 slots its index row names (pools of
64 consecutive slots, with duplicate and invalid entries), the benchmark's
first index set (DSA-style selection: metrale's topk_to_mask and
expand_selection; usearch's attend over the selected rows).

Streaming: the long-context shape kept as 4 sink keys, a 128-key ring and a
main cache 1024 slots short of full (cortiq-engine's sink + window layout);
one stream_append, which moves the ring's oldest key into main and writes the
new key into its ring slot, then attend_branches over the three parts.  The
layout is compared bit for bit with the oracle's model of it, the attention
with the oracle's attention over the union of the parts."""

import numpy as np
import pytest
import torch

from oracle import streaming as ost
from gpu_util import check_carry, check_out, live_vmax, np64, say, to_dev
from gqa_kv_cache_decode_amd import workloads as wl

pytestmark = pytest.mark.gpu

SINK = 4      # the streaming workload's sink keys
ROOM = 1024   # main slots left free, so each step grows main


def _gqa():
    import gqa_kv_cache_decode_amd as g
    return g


def _bits(t: torch.Tensor) -> np.ndarray:
    """A host bf16 tensor's stored bits (bit-exact comparisons)."""
    return t.view(torch.int16).numpy()


def _bf16_bits_f64(a: np.ndarray) -> np.ndarray:
    """bf16 values from their stored bits, as float64 (exact)."""
    return (a.view(np.uint16).astype(np.uint32) << 16).view(
        np.float32).astype(np.float64)


def test_full_gathered_bf16():
    g = _gqa()
    w = wl.GATHER_BF16
    say("[full] gathered: drawing inputs")
    x = wl.make_inputs(w)
    idx = wl.make_index_rows(w, x["lens"], wl.GATHER_WIDTH, wl.GATHER_POOL,
                             w.seed + 3000)
    d = to_dev(x)
    rows = w.batch * w.num_q_heads
    cout = g.empty_carry(rows, w.dv)
    out = g.attend_gathered(d["q"], d["k"], d["v"], d["lens"], idx.cuda(),
                            w.scale, carry_out=cout)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    m_got, l_got = cout.m.cpu().numpy(), cout.l.cpu().numpy()
    del d
    say("[full] gathered: oracle, one sequence at a time")
    want = np.empty_like(got, dtype=np.float64)
    m_want = np.empty(rows)
    l_want = np.empty(rows)
    for b in range(w.batch):
        o, c = ost.attend_gathered(np64(x["q"][b:b + 1]),
                                   np64(x["k"][b:b + 1]),
                                   np64(x["v"][b:b + 1]),
                                   x["lens"][b:b + 1].numpy(),
                                   idx[b:b + 1].numpy(), w.scale)
        want[b] = o[0]
        r = slice(b * w.num_q_heads, (b + 1) * w.num_q_heads)
        m_want[r], l_want[r] = c.m, c.l
    # every row selects at least one pool here, so every row is live
    assert np.all(l_want > 0)
    vmax = live_vmax(x["v"], x["lens"])
    check_out(got, want, vmax, w.dtype, "gathered bf16, every row")
    check_carry(m_got, l_got, m_want, l_want, w.dtype,
                "gathered bf16 carry, every row")


def test_full_stream_step():
    g = _gqa()
    w = wl.LONG_WINDOW_BF16
    S, W = SINK, w.window
    n_main = w.max_len - S - W - ROOM
    say("[full] stream: drawing inputs")
    x = wl.make_inputs(w)
    gen = torch.Generator().manual_seed(w.seed + 1000)
    kn = torch.randn(w.batch, w.num_kv_heads, w.dk, generator=gen).to(
        w.torch_dtype)
    vn = torch.randn(w.batch, w.num_kv_heads, w.dv, generator=gen).to(
        w.torch_dtype)
    # the parts as the benchmark lays them out: main is the long cache, the
    # sink a copy of its first keys, the ring the window cache
    mk_h, mv_h = x["k"], x["v"]
    sk_h, sv_h = mk_h[:, :S].clone(), mv_h[:, :S].clone()
    rk_h, rv_h = x["wk"], x["wv"]
    mk, mv = mk_h.cuda(), mv_h.cuda()
    sk, sv = sk_h.cuda(), sv_h.cuda()
    rk, rv = rk_h.cuda(), rv_h.cuda()
    count0 = np.full(w.batch, S + W + n_main, dtype=np.int32)
    count = torch.from_numpy(count0.copy()).cuda()
    dropped = torch.zeros(1, dtype=torch.int32, device="cuda")
    say("[full] stream: stream_append + attend_branches")
    cnt, ls, lr, lm = g.stream_append(rk, rv, kn.cuda(), vn.cuda(), count,
                                      count_out=count, sink=(sk, sv),
                                      main=(mk, mv), dropped=dropped)
    rows = w.batch * w.num_q_heads
    cout = g.empty_carry(rows, w.dv)
    out = g.attend_branches(x["q"].cuda(),
                            [(sk, sv, ls), (rk, rv, lr), (mk, mv, lm)],
                            w.scale, carry_out=cout)
    torch.cuda.synchronize()

    # layout: every part bit for bit against the oracle's model
    e = ost.stream_append(_bits(sk_h), _bits(sv_h), _bits(rk_h), _bits(rv_h),
                          _bits(mk_h), _bits(mv_h), _bits(kn), _bits(vn),
                          count0)
    names = ["sink k", "sink v", "ring k", "ring v", "main k", "main v"]
    for name, got_t, want_a in zip(names, (sk, sv, rk, rv, mk, mv), e[:6]):
        assert np.array_equal(_bits(got_t.cpu()), want_a), \
            f"stream layout: {name} differs from the oracle's"
    assert cnt.cpu().numpy().tolist() == e[6].tolist(), "count"
    assert int(dropped.item()) == e[7] == 0, "dropped"
    n_s, n_r, n_m = ost.stream_lengths(int(e[6][0]), S, W, w.max_len)
    assert (n_s, n_r, n_m) == (S, W, n_main + 1)
    for t, n in ((ls, n_s), (lr, n_r), (lm, n_m)):
        assert t.cpu().tolist() == [n] * w.batch, "part lengths"

    # attention over the three parts (the state carried from part to part)
    say("[full] stream: oracle")
    lens_of = lambda n: np.full(w.batch, n, dtype=np.int64)
    f64 = _bf16_bits_f64
    want, cw = ost.attend_branches(
        np64(x["q"]),
        [(f64(e[0]), f64(e[1]), lens_of(n_s)),
         (f64(e[2]), f64(e[3]), lens_of(n_r)),
         (f64(e[4]), f64(e[5]), lens_of(n_m))],
        w.scale)
    vmax = max(float(np.max(np.abs(f64(e[1])))),
               float(np.max(np.abs(f64(e[3])))),
               float(np.max(np.abs(f64(e[5][:, :n_m])))))
    check_out(out.cpu().numpy(), want, vmax, w.dtype,
              "stream step, every row")
    check_carry(cout.m.cpu().numpy(), cout.l.cpu().numpy(), cw.m, cw.l,
                w.dtype, "stream step carry, every row")
