"""The additive logit bias (needle-core self_attn_incremental, attn_bias) on
the GPU against the oracle: random biases and -inf masks (single keys, whole
chunks, every key of a sequence), on every compiled head width of both
families, through each kind of plan (split-K with the combine kernel, a
single chunk written directly, a scheduled launch, the fused decode step),
with padded bias rows and a carry_in."""

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
    lens[0] = 0
    if batch > 1:
        lens[1] = max_len
    return lens.to(torch.int32)


def _bias(batch, max_len, stride, seed, chunk=None):
    """fp32 [batch, stride]: N(0, 2) terms, ~10% of keys removed (-inf), the
    whole first chunk of sequence 1 removed, every key of sequence 2
    removed; the padding columns past max_len hold NaN (never read)."""
    gen = torch.Generator().manual_seed(seed)
    bias = torch.randn(batch, stride, generator=gen) * 2.0
    drop = torch.rand(batch, stride, generator=gen) < 0.1
    bias[drop] = -float("inf")
    if batch > 1 and chunk:
        bias[1, :chunk] = -float("inf")
    if batch > 2:
        bias[2, :] = -float("inf")
    bias[:, max_len:] = float("nan")
    return bias


def _run_and_check(w, chunk_hint, plan_chunk=None, with_carry=False,
                   stride_pad=8, what=""):
    g = _gqa()
    lens = _lens(w.batch, w.max_len, 41)
    x = wl.make_inputs(w, lens_override=lens.tolist())
    d = to_dev(x)
    bias = _bias(w.batch, w.max_len, w.max_len + stride_pad, 42, chunk_hint)
    bd = bias.cuda()
    rows = w.batch * w.num_q_heads
    cin = cin_np = None
    if with_carry:
        gen = torch.Generator().manual_seed(43)
        m = torch.randn(rows, generator=gen)
        l = torch.rand(rows, generator=gen) + 0.5
        l[::3] = 0.0  # some empty carry rows
        acc = torch.randn(rows, w.dv, generator=gen)
        cin = g.Carry(m.cuda(), l.cuda(), acc.cuda())
        cin_np = oracle.Carry(m.double().numpy(), l.double().numpy(),
                              acc.double().numpy())
    cout = g.empty_carry(rows, w.dv)
    if plan_chunk is None:
        out = g.attend_decode(d["q"], d["k"], d["v"], d["lens"], w.scale,
                              carry_in=cin, carry_out=cout, bias=bd)
    else:
        plan = g.attend_plan(d["k"], d["v"], w.num_q_heads, plan_chunk)
        ws = torch.empty(plan.workspace_bytes, dtype=torch.uint8,
                         device="cuda")
        g.attend_partition(d["q"], d["k"], d["v"], d["lens"], plan, ws,
                           w.scale, bias=bd)
        out = g.attend_combine(w.num_q_heads, d["k"], d["v"], d["lens"], plan,
                               ws, carry_in=cin, carry_out=cout)
    torch.cuda.synchronize()
    ref, cref = oracle.attend(np64(x["q"]), np64(x["k"]), np64(x["v"]),
                              x["lens"].numpy(), w.scale, carry_in=cin_np,
                              bias=bias.double().numpy())
    vmax = live_vmax(x["v"], x["lens"])
    if with_carry:
        vmax = max(vmax, float(np.max(np.abs(oracle.finalize(cin_np)))))
    check_out(out.cpu().numpy(), ref, vmax, w.dtype, what)
    check_carry(cout.m.cpu().numpy(), cout.l.cpu().numpy(), cref.m, cref.l,
                w.dtype, what + " carry")
    if not with_carry and w.batch > 2:
        o = out.cpu().numpy()
        assert np.all(o[0] == 0.0) and np.all(o[2] == 0.0), \
            "no keys / every key removed: out 0"


CASES = {
    # name: (workload, chunk of the first-chunk mask, explicit plan chunk)
    "bf16_d128_split": (wl.BATCHED_BF16.replace(batch=4, max_len=1500),
                        512, None),
    "bf16_d128_explicit_split": (wl.BATCHED_BF16.replace(batch=4,
                                                         max_len=1000),
                                 128, 128),
    "bf16_dk192_hpk16": (wl.WIDE_SPIKE_BF16.replace(batch=3, max_len=2100),
                         256, None),
    "bf16_d64": (wl.BATCHED_BF16.replace(batch=3, num_q_heads=8,
                                         num_kv_heads=4, dk=64, dv=64,
                                         max_len=700), 128, None),
    "bf16_d256_mha": (wl.BATCHED_BF16.replace(batch=3, num_q_heads=2,
                                              num_kv_heads=2, dk=256, dv=256,
                                              max_len=600), 128, None),
    "bf16_single_chunk": (wl.BATCHED_BF16.replace(batch=64, num_q_heads=16,
                                                  num_kv_heads=4,
                                                  max_len=300), 64, None),
    "bf16_scheduled": (wl.RAGGED_BF16.replace(batch=64, num_q_heads=32,
                                              num_kv_heads=4, max_len=1000),
                       128, 128),
    "f32_mfma_d64": (wl.TINY_F32.replace(batch=3, max_len=700), 64, None),
    "f32_mfma_d128_scheduled": (wl.TINY_F32.replace(
        batch=64, num_q_heads=8, num_kv_heads=4, dk=128, dv=128,
        max_len=300), 64, 64),
    "f32_vector_alu": (wl.TINY_F32.replace(batch=3, dk=48, dv=80,
                                           max_len=400), 128, None),
    # small launches: decode_step folds the partials in its last work-group
    "f32_tiny_fused": (wl.TINY_F32.replace(batch=3), 64, None),
    "bf16_small_fused": (wl.BATCHED_BF16.replace(batch=3, num_q_heads=8,
                                                 num_kv_heads=2,
                                                 max_len=300), 64, None),
}


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("with_carry", [False, True])
def test_bias_attend(name, with_carry):
    w, chunk_hint, plan_chunk = CASES[name]
    say(f"[bias] {name} carry={with_carry}")
    _run_and_check(w, chunk_hint, plan_chunk, with_carry,
                   what=f"{name} carry={with_carry}")


@pytest.mark.parametrize("name", ["bf16_d128_split", "bf16_single_chunk",
                                  "f32_mfma_d64", "f32_vector_alu",
                                  "f32_tiny_fused", "bf16_small_fused"])
def test_bias_decode_step(name):
    """decode_step with a bias: the row covers the new token's position."""
    g = _gqa()
    w, chunk_hint, _ = CASES[name]
    lens_in = _lens(w.batch, w.max_len, 44).clamp(max=w.max_len - 1)
    x = wl.make_inputs(w, lens_override=lens_in.tolist(), pad_value=0.0)
    d = to_dev(x)
    gen = torch.Generator().manual_seed(45)
    kn = torch.randn(w.batch, w.num_kv_heads, w.dk, generator=gen).to(
        w.torch_dtype)
    vn = torch.randn(w.batch, w.num_kv_heads, w.dv, generator=gen).to(
        w.torch_dtype)
    bias = _bias(w.batch, w.max_len, w.max_len + 4, 46, chunk_hint)
    li = lens_in.cuda()
    lo = torch.empty_like(li)
    ws = g.step_workspace(d["k"], d["v"], w.num_q_heads)
    cout = g.empty_carry(w.batch * w.num_q_heads, w.dv)
    out = g.decode_step(d["q"], d["k"], d["v"], kn.cuda(), vn.cuda(), li, lo,
                        w.scale, carry_out=cout, workspace=ws,
                        bias=bias.cuda())
    torch.cuda.synchronize()
    bits = (lambda t: t.view(torch.int16)) if w.dtype == "bf16" else \
        (lambda t: t.view(torch.int32))
    k_ref, v_ref, l_ref, _ = oracle.kv_append(
        bits(x["k"]).numpy(), bits(x["v"]).numpy(), bits(kn).numpy(),
        bits(vn).numpy(), lens_in.numpy())
    assert lo.cpu().numpy().tolist() == l_ref.tolist(), "lens"
    k64 = torch.from_numpy(k_ref).view(w.torch_dtype)
    v64 = torch.from_numpy(v_ref).view(w.torch_dtype)
    ref, cref = oracle.attend(np64(x["q"]), np64(k64), np64(v64), l_ref,
                              w.scale, bias=bias.double().numpy())
    check_out(out.cpu().numpy(), ref, live_vmax(v64, l_ref), w.dtype,
              name + " step")
    check_carry(cout.m.cpu().numpy(), cout.l.cpu().numpy(), cref.m, cref.l,
                w.dtype, name + " step carry")
