"""Index-gathered decode on the GPU against the oracle: index rows of
consecutive-token pools and single tokens, with duplicates, INVALID (-1)
padding, slots past the live length and rows that select nothing; every
compiled head width of both families; a selection that fits one chunk
(written directly) and one split over many chunks; live lengths longer than
one window of the launch's selection bitmap; a carry_in with carry_out
aliasing it."""

import numpy as np
import pytest
import torch

import oracle
import oracle.streaming as ost
from gpu_util import check_carry, check_out, np64, say, to_dev
from gqa_kv_cache_decode_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _gqa():
    import gqa_kv_cache_decode_amd as g
    return g


def _index_rows(B, T, lens, width, pool, seed):
    """Per sequence: pools of `pool` consecutive slots plus single slots,
    then ~5% duplicates, ~5% INVALID, a few slots past the live length, in
    shuffled order; sequence 1 selects nothing."""
    rng = np.random.default_rng(seed)
    idx = np.full((B, width), -1, dtype=np.int32)
    for b in range(B):
        n = int(min(max(lens[b], 0), T))
        if b == 1 or n == 0:
            continue
        picks = []
        npools = max(1, (width // 2) // pool)
        for s in rng.integers(0, max(n - pool, 1), npools):
            picks += list(range(int(s), min(int(s) + pool, n)))
        picks += list(rng.integers(0, n, width - len(picks) if width > len(picks) else 0))
        row = np.array(picks[:width], dtype=np.int64)
        k = max(1, width // 20)
        row[rng.integers(0, width, k)] = row[rng.integers(0, width, k)]  # dups
        row[rng.integers(0, width, k)] = -1
        row[rng.integers(0, width, 2)] = n + rng.integers(0, 50, 2)      # past
        rng.shuffle(row)
        idx[b] = row
    return idx


CASES = {
    # name: (workload, width, pool)
    "bf16_d128_split": (wl.RAGGED_BF16.replace(batch=4, max_len=9000), 5000,
                        64),
    "bf16_d128_direct": (wl.BATCHED_BF16.replace(batch=4, max_len=3000), 200,
                         16),
    "bf16_dk192_hpk16": (wl.WIDE_SPIKE_BF16.replace(batch=3, max_len=4000),
                         1500, 32),
    "bf16_d64": (wl.BATCHED_BF16.replace(batch=3, num_q_heads=8,
                                         num_kv_heads=4, dk=64, dv=64,
                                         max_len=2000), 700, 8),
    "bf16_d256_mha": (wl.BATCHED_BF16.replace(batch=3, num_q_heads=2,
                                              num_kv_heads=2, dk=256, dv=256,
                                              max_len=1200), 500, 16),
    "f32_d64": (wl.TINY_F32.replace(batch=3, max_len=1000), 400, 16),
    "f32_d128": (wl.TINY_F32.replace(batch=3, num_q_heads=8, num_kv_heads=4,
                                     dk=128, dv=128, max_len=900), 300, 8),
    # live lengths past one LDS window of the in-launch selection (65536
    # slots for bf16 64-wide heads, 131072 for fp32 64-wide heads): ranks
    # carried across several windows
    "bf16_d64_windows": (wl.BATCHED_BF16.replace(batch=3, num_q_heads=2,
                                                 num_kv_heads=1, dk=64, dv=64,
                                                 max_len=400000), 3000, 64),
    "f32_d64_windows": (wl.TINY_F32.replace(batch=2, num_q_heads=2,
                                            num_kv_heads=1, max_len=600000),
                        2000, 16),
}


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("with_carry", [False, True])
def test_gathered(name, with_carry):
    g = _gqa()
    w, width, pool = CASES[name]
    gen = torch.Generator().manual_seed(71)
    lens = torch.randint(w.max_len // 2, w.max_len + 1, (w.batch,),
                         generator=gen).to(torch.int32)
    lens[0] = w.max_len
    x = wl.make_inputs(w, lens_override=lens.tolist())
    d = to_dev(x)
    idx = _index_rows(w.batch, w.max_len, lens.tolist(), width, pool, 72)
    rows = w.batch * w.num_q_heads
    cin = cin_np = None
    if with_carry:
        m = torch.randn(rows, generator=gen)
        l = torch.rand(rows, generator=gen) + 0.5
        l[::3] = 0.0
        acc = torch.randn(rows, w.dv, generator=gen)
        cin = g.Carry(m.cuda(), l.cuda(), acc.cuda())
        cin_np = oracle.Carry(m.double().numpy(), l.double().numpy(),
                              acc.double().numpy())
    cout = cin if with_carry else g.empty_carry(rows, w.dv)
    say(f"[gather] {name} carry={with_carry}")
    out = g.attend_gathered(d["q"], d["k"], d["v"], d["lens"],
                            torch.from_numpy(idx).cuda(), w.scale,
                            carry_in=cin, carry_out=cout)
    torch.cuda.synchronize()
    want, cw = ost.attend_gathered(np64(x["q"]), np64(x["k"]), np64(x["v"]),
                                   x["lens"].numpy(), idx, w.scale,
                                   carry_in=cin_np)
    vmax = float(x["v"].float().nan_to_num().abs().max())
    if with_carry:
        vmax = max(vmax, float(np.max(np.abs(oracle.finalize(cin_np)))))
    check_out(out.cpu().numpy(), want, vmax, w.dtype, name)
    check_carry(cout.m.cpu().numpy(), cout.l.cpu().numpy(), cw.m, cw.l,
                w.dtype, name + " carry")
    if not with_carry:
        assert torch.all(out[1] == 0), "a row selecting nothing gives 0"
