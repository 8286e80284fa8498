"""Shared pieces of the GPU parity tests: device transfer, oracle calls on the
same seeded inputs, and the tolerance checks."""

from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from gqa_kv_cache_decode_amd import workloads as wl

# max |out_gpu - out_oracle| <= TOL * max|V| over the attended values
# (fp32 accumulation in both families).
# fp8 caches are attended on their decoded values, which are exact bf16
# values: the same arithmetic, and the same bound, as bf16 caches.
TOL = {"f32": 1e-5, "bf16": 4e-3, "fp8": 4e-3}
# Carry checks (a reading; the tolerance above pins only the output):
# m within M_TOL * max(1, |m|); the log-sum-exp m + ln l within LSE_TOL.
M_TOL = {"f32": 1e-5, "bf16": 1e-3, "fp8": 1e-3}
LSE_TOL = {"f32": 1e-4, "bf16": 1e-3, "fp8": 1e-3}


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def np64(t: torch.Tensor) -> np.ndarray:
    """Stored values as float64 (bf16 and fp32 convert exactly)."""
    return t.float().numpy().astype(np.float64) if t.dtype == torch.bfloat16 \
        else t.numpy().astype(np.float64)


def live_vmax(v: torch.Tensor, lens) -> float:
    m = 0.0
    for b in range(v.shape[0]):
        n = int(min(max(int(lens[b]), 0), v.shape[1]))
        if n:
            m = max(m, float(v[b, :n].float().abs().max()))
    return m


def to_dev(x: dict) -> dict:
    return {k: (t.cuda() if isinstance(t, torch.Tensor) else t)
            for k, t in x.items()}


def oracle_rows(x: dict, w: wl.DecodeWorkload, rows_bg, carry_in=None,
                cache=("k", "v", "lens")):
    """Oracle over selected (b, g) units: returns {(b, h): (out, m, l)}."""
    res = {}
    kk, vv, ll = cache
    hpk = w.hpk
    for b, g in rows_bg:
        n = int(min(max(int(x[ll][b]), 0), x[kk].shape[1]))
        q = np64(x["q"][b:b + 1, g * hpk:(g + 1) * hpk])
        k = np64(x[kk][b:b + 1, :n, g:g + 1])
        v = np64(x[vv][b:b + 1, :n, g:g + 1])
        cin = None
        if carry_in is not None:
            rows = [b * w.num_q_heads + g * hpk + i for i in range(hpk)]
            cin = oracle.Carry(carry_in.m[rows], carry_in.l[rows],
                               carry_in.acc[rows])
        out, c = oracle.attend(q, k, v, [n], w.scale, carry_in=cin)
        for i in range(hpk):
            res[(b, g * hpk + i)] = (out[0, i], c.m[i], c.l[i], c.acc[i])
    return res


def rel_l2(got: np.ndarray, want: np.ndarray) -> float:
    """Relative L2 error ||got - want|| / ||want|| over all the rows given
    (the cortiq-engine recovery example's background-error diagnostic); 0
    when both are zero."""
    num = float(np.linalg.norm(np.asarray(got, np.float64) - want))
    den = float(np.linalg.norm(want))
    return num / den if den > 0 else num


def check_out(got: np.ndarray, want: np.ndarray, vmax: float, dtype: str,
              what: str) -> float:
    assert np.all(np.isfinite(got)), f"{what}: non-finite GPU output"
    err = float(np.max(np.abs(got - want))) if got.size else 0.0
    bound = TOL[dtype] * max(vmax, 1e-30)
    say(f"  {what}: max|err| = {err:.3e}  (bound {bound:.3e}, "
        f"{err / max(vmax, 1e-30):.2e} * max|V|), rel L2 "
        f"{rel_l2(got, want):.2e}")
    assert err <= bound, f"{what}: max|err| {err:.3e} > {bound:.3e}"
    return err


def check_carry(m_got, l_got, m_want, l_want, dtype: str, what: str) -> None:
    m_got, l_got = np.asarray(m_got, np.float64), np.asarray(l_got, np.float64)
    m_want, l_want = np.asarray(m_want), np.asarray(l_want)
    empty = l_want == 0
    assert np.array_equal(l_got[empty], l_want[empty]), f"{what}: empty l"
    assert np.all(np.isneginf(m_got[empty])), f"{what}: empty m is -inf"
    live = ~empty
    dm = np.abs(m_got[live] - m_want[live])
    assert np.all(dm <= M_TOL[dtype] * np.maximum(1.0, np.abs(m_want[live]))), \
        f"{what}: m err {dm.max():.3e}"
    lse = np.abs((m_got[live] + np.log(l_got[live])) -
                 (m_want[live] + np.log(l_want[live])))
    assert np.all(lse <= LSE_TOL[dtype]), f"{what}: lse err {lse.max():.3e}"
