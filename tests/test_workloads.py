"""The seeded input generators: determinism, shapes, padding, planted spike."""

import math

import torch

from gqa_kv_cache_decode_amd import workloads as wl


def test_deterministic_and_shapes():
    w = wl.BATCHED_BF16.replace(batch=2, max_len=64)
    a, b = wl.make_inputs(w), wl.make_inputs(w)
    for key in ("q", "k", "v", "lens"):
        assert torch.equal(a[key].view(torch.int16) if a[key].is_floating_point()
                           else a[key],
                           b[key].view(torch.int16) if b[key].is_floating_point()
                           else b[key])
    assert a["q"].shape == (2, 32, 128) and a["q"].dtype == torch.bfloat16
    assert a["k"].shape == (2, 64, 8, 128) and a["v"].shape == (2, 64, 8, 128)
    assert a["lens"].tolist() == [64, 64]


def test_ragged_padding_is_poisoned():
    w = wl.RAGGED_BF16.replace(batch=6, max_len=50)
    x = wl.make_inputs(w)
    lens = x["lens"].tolist()
    assert all(1 <= n <= 50 for n in lens)
    for b, n in enumerate(lens):
        assert torch.isfinite(x["k"][b, :n].float()).all()
        assert torch.isnan(x["k"][b, n:].float()).all()
        assert torch.isnan(x["v"][b, n:].float()).all()


def test_spike_is_planted():
    w = wl.WIDE_SPIKE_BF16.replace(batch=2, max_len=1500)
    x = wl.make_inputs(w)
    p = x["spike_pos"]
    assert p == 500
    v = x["v"].float()
    assert torch.all(v[:, p, :, 0] == 1.0)
    mask = torch.ones(1500, dtype=torch.bool)
    mask[p] = False
    assert torch.all(v[:, mask, :, 0] == 0.0)
    k = x["k"].float()
    for b in range(2):
        for g in range(4):
            h0 = g * w.hpk
            qh = x["q_hat"][b, h0]
            gain = float(k[b, p, g] @ qh) - float(k[b, p - 1, g] @ qh)
            assert gain > 8.0 - 6.0      # +8 along q_hat over a N(0,1) background
    assert abs(float(x["q"][0, 0].float().norm()) - math.sqrt(192)) < 0.1


def test_window_branch():
    w = wl.LONG_WINDOW_BF16.replace(max_len=300)
    x = wl.make_inputs(w)
    assert x["wk"].shape == (1, 128, 4, 128) and x["wlens"].tolist() == [128]
