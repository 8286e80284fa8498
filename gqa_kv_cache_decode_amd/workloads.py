"""Seeded synthetic decode workloads.

This module only draws inputs: queries, K/V caches, per-sequence lengths and
the recent-window branch.  It holds none of the attention arithmetic, so both
the HIP path and the CPU oracle can be fed from it without sharing any of the
method.

Shapes follow the pages' workloads:

* needle-core ``attn.rs`` (module doc): 8 query heads over 4 KV heads; the
  cache is ``[max_len, num_kv_heads, head_dim]`` per sequence (struct KvCache).
  A leading batch dimension is added here: ``[batch, max_len, Hkv, d]``.
* usearch "linear-algebra", section Attention: 128-wide bf16 rows with 8 query
  heads sharing one KV head; a carry folds a recent window into the main branch.
* cortiq-engine ``NystromState``, ``new``: exact window width 128; example
  ``o1_recovery.rs`` ``trial()``: unit-vector query scaled by sqrt(d), keys
  uniform times 1.732, values uniform with channel 0 zeroed, one planted key
  ``K[p] += amp * q_hat`` with ``V[p, 0] = 1`` at ``p = t - depth``.

Every draw comes from a ``torch.Generator('cpu')`` seeded per workload, in fp32,
and is then rounded to the storage dtype with round-to-nearest-even (torch's
``.to(torch.bfloat16)``).  Draw order: q, lens, K, V, window K, window V.
For ragged workloads only the live slots ``[0, lens[b])`` are drawn; the
padding slots are filled with ``pad_value`` (NaN by default, so that any read
of a padding slot poisons the result).
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch

BASE_SEED = 20261203

DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.uint8}


@dataclasses.dataclass(frozen=True)
class DecodeWorkload:
    """One decode attention problem, described by what it is and its sizes."""

    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    dk: int
    dv: int
    max_len: int
    dtype: str = "bf16"            # storage of K and V: "f32" | "bf16" | "fp8"
                                   # (fp8: E4M3 codes + scales, q in bf16)
    dist: str = "normal"           # "normal" | "uniform" | "spike"
    ragged: bool = False           # lens ~ U{1..max_len} instead of all max_len
    scale: float = 0.0             # 0 means 1/sqrt(dk)
    window: int = 0                # tokens in a second, recent-window branch
    spike_depth: int = 1000        # planted key position p = T - depth ("spike")
    spike_amp: float = 8.0         # planted amplitude along q_hat ("spike")
    seed_index: int = 0            # seed = BASE_SEED + seed_index

    @property
    def hpk(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def seed(self) -> int:
        return BASE_SEED + self.seed_index

    @property
    def torch_dtype(self) -> torch.dtype:
        return DTYPES[self.dtype]

    @property
    def esz(self) -> int:
        """Bytes per stored K/V element."""
        return {"f32": 4, "bf16": 2, "fp8": 1}[self.dtype]

    @property
    def q_esz(self) -> int:
        """Bytes per query element (bf16 queries go with fp8 caches)."""
        return 4 if self.dtype == "f32" else 2

    def resolved_scale(self) -> float:
        return self.scale if self.scale != 0.0 else 1.0 / math.sqrt(self.dk)

    def replace(self, **kw) -> "DecodeWorkload":
        return dataclasses.replace(self, **kw)


# The five workloads, numbered as listed: tiny fp32, batched bf16, ragged batch,
# long context with a recent window, wide group with a planted spike.
TINY_F32 = DecodeWorkload(
    "tiny_f32_b1_hq8_hkv4_d64_t256", batch=1, num_q_heads=8, num_kv_heads=4,
    dk=64, dv=64, max_len=256, dtype="f32", dist="uniform", scale=0.125,
    seed_index=1)
BATCHED_BF16 = DecodeWorkload(
    "batched_bf16_b16_hq32_hkv8_d128_t4096", batch=16, num_q_heads=32,
    num_kv_heads=8, dk=128, dv=128, max_len=4096, dtype="bf16",
    dist="normal", seed_index=2)
RAGGED_BF16 = DecodeWorkload(
    "ragged_bf16_b64_hq64_hkv8_d128_max32768", batch=64, num_q_heads=64,
    num_kv_heads=8, dk=128, dv=128, max_len=32768, dtype="bf16",
    dist="normal", ragged=True, seed_index=3)
LONG_WINDOW_BF16 = DecodeWorkload(
    "long_bf16_b1_hq32_hkv4_d128_t262144_w128", batch=1, num_q_heads=32,
    num_kv_heads=4, dk=128, dv=128, max_len=262144, dtype="bf16",
    dist="normal", window=128, seed_index=4)
WIDE_SPIKE_BF16 = DecodeWorkload(
    "spike_bf16_b8_hq64_hkv4_dk192_dv128_t65536", batch=8, num_q_heads=64,
    num_kv_heads=4, dk=192, dv=128, max_len=65536, dtype="bf16",
    dist="spike", seed_index=5)

WORKLOADS = [TINY_F32, BATCHED_BF16, RAGGED_BF16, LONG_WINDOW_BF16,
             WIDE_SPIKE_BF16]

# Index-gathered decode (a "next" shape, not one of the five above): a
# DSA-style selection of GATHER_WIDTH slots per sequence out of a 32K cache,
# GATHER_POOL consecutive slots per selected pool (metrale DSA expand_selection
# turns selected pools of index_kpool tokens into raw token indices).
GATHER_BF16 = DecodeWorkload(
    "gather_bf16_b16_hq32_hkv8_d128_t32768_sel2048", batch=16,
    num_q_heads=32, num_kv_heads=8, dk=128, dv=128, max_len=32768,
    dtype="bf16", dist="normal", seed_index=6)
GATHER_WIDTH = 2048
GATHER_POOL = 64

# fp8 KV storage (a "next" shape): the batched shape with K and V held as
# one-byte E4M3 codes plus one fp32 scale per (sequence, KV head) each.
BATCHED_FP8 = DecodeWorkload(
    "batched_fp8_b16_hq32_hkv8_d128_t4096", batch=16, num_q_heads=32,
    num_kv_heads=8, dk=128, dv=128, max_len=4096, dtype="fp8",
    dist="normal", seed_index=7)

E4M3_NAN = 0x7F


def make_e4m3_codes(g: torch.Generator, shape, exp_lo: int = 4,
                    exp_hi: int = 9) -> torch.Tensor:
    """Random E4M3 bit patterns (uint8): uniform sign bit, exponent field
    uniform over [exp_lo, exp_hi], uniform 3-bit mantissa.  Bit patterns
    only (a log-uniform spread of magnitudes); exp_hi < 15 keeps the NaN
    pattern out."""
    sign = torch.randint(0, 2, shape, generator=g, dtype=torch.int32)
    e = torch.randint(exp_lo, exp_hi + 1, shape, generator=g, dtype=torch.int32)
    m = torch.randint(0, 8, shape, generator=g, dtype=torch.int32)
    return ((sign << 7) | (e << 3) | m).to(torch.uint8)


def make_fp8_inputs(w: DecodeWorkload, pad_code: int = E4M3_NAN,
                    lens_override: Optional[list] = None) -> dict:
    """Draw an fp8-cache workload on the CPU: q [B, Hq, dk] bf16 (normal),
    lens [B] (as ``make_inputs``), K/V codes [B, max_len, Hkv, d] uint8
    (``make_e4m3_codes`` over the live slots, ``pad_code`` — the NaN code by
    default — past them) and fp32 scales k_scale [B, Hkv] ~ U(0.05, 0.5),
    v_scale [B, Hkv] ~ U(0.1, 1.0).  Draw order: q, lens, K, V, scales."""
    assert w.dtype == "fp8"
    g = torch.Generator().manual_seed(w.seed)
    B, Hq, Hkv, dk, dv, T = (w.batch, w.num_q_heads, w.num_kv_heads, w.dk,
                             w.dv, w.max_len)
    res = {"q": _normal(g, (B, Hq, dk)).to(torch.bfloat16)}
    if lens_override is not None:
        lens = torch.tensor(lens_override, dtype=torch.int32)
        assert lens.numel() == B
    elif w.ragged:
        lens = torch.randint(1, T + 1, (B,), generator=g,
                             dtype=torch.int64).to(torch.int32)
    else:
        lens = torch.full((B,), T, dtype=torch.int32)
    res["lens"] = lens
    k = torch.full((B, T, Hkv, dk), pad_code, dtype=torch.uint8)
    v = torch.full((B, T, Hkv, dv), pad_code, dtype=torch.uint8)
    for b in range(B):
        n = int(min(max(int(lens[b]), 0), T))
        k[b, :n] = make_e4m3_codes(g, (n, Hkv, dk))
        v[b, :n] = make_e4m3_codes(g, (n, Hkv, dv))
    res["k"], res["v"] = k, v
    res["k_scale"] = _uniform(g, (B, Hkv), 0.05, 0.5)
    res["v_scale"] = _uniform(g, (B, Hkv), 0.1, 1.0)
    return res


def make_index_rows(w: DecodeWorkload, lens, width: int, pool: int,
                    seed: int, invalid_frac: float = 0.02,
                    dup_frac: float = 0.02) -> torch.Tensor:
    """Index rows [B, width] int32 in the shape of a pooled top-k
    selection: width // pool distinct pools of `pool` consecutive slots each
    (pool starts drawn without replacement among the live pools), then a
    fraction of entries replaced by duplicates of other entries and by -1
    (INVALID), in a shuffled order.  Holds no attention arithmetic."""
    g = torch.Generator().manual_seed(seed)
    rows = torch.full((w.batch, width), -1, dtype=torch.int32)
    for b in range(w.batch):
        n = int(min(max(int(lens[b]), 0), w.max_len))
        npool = max(n // pool, 1)
        k = min(width // pool, npool)
        starts = torch.randperm(npool, generator=g)[:k] * pool
        row = (starts[:, None] + torch.arange(pool)[None, :]).reshape(-1)
        row = row[row < n][:width]
        full = torch.full((width,), -1, dtype=torch.int64)
        full[:row.numel()] = row
        m = int(width * dup_frac)
        if m and row.numel():
            src = torch.randint(0, row.numel(), (m,), generator=g)
            dst = torch.randint(0, width, (m,), generator=g)
            full[dst] = full[src]
        m = int(width * invalid_frac)
        if m:
            full[torch.randint(0, width, (m,), generator=g)] = -1
        rows[b] = full[torch.randperm(width, generator=g)].to(torch.int32)
    return rows


def _uniform(g: torch.Generator, shape, lo: float, hi: float) -> torch.Tensor:
    return torch.empty(shape, dtype=torch.float32).uniform_(lo, hi, generator=g)


def _normal(g: torch.Generator, shape) -> torch.Tensor:
    return torch.empty(shape, dtype=torch.float32).normal_(generator=g)


def _draw(g, shape, dist):
    if dist == "normal":
        return _normal(g, shape)
    return _uniform(g, shape, -1.0, 1.0)


def make_inputs(w: DecodeWorkload, pad_value: float = float("nan"),
                lens_override: Optional[list] = None) -> dict:
    """Draw one workload on the CPU.

    Returns a dict of CPU tensors in storage dtype:
      q      [B, Hq, dk]
      k      [B, max_len, Hkv, dk]
      v      [B, max_len, Hkv, dv]
      lens   [B] int32 (live tokens per sequence)
    and, when ``w.window`` > 0, ``wk``/``wv`` ``[B, window, Hkv, d]`` and
    ``wlens`` ``[B]``.  For the "spike" distribution it also returns
    ``spike_pos`` (the planted slot) and ``q_hat`` (fp32 unit queries).
    """
    assert w.dtype != "fp8", "fp8 caches: make_fp8_inputs"
    g = torch.Generator().manual_seed(w.seed)
    B, Hq, Hkv, dk, dv, T = (w.batch, w.num_q_heads, w.num_kv_heads, w.dk,
                             w.dv, w.max_len)
    dt = w.torch_dtype
    res = {}

    # q
    if w.dist == "spike":
        u = _uniform(g, (B, Hq, dk), -1.0, 1.0)
        q_hat = u / u.norm(dim=-1, keepdim=True)
        q32 = q_hat * math.sqrt(dk)
        res["q_hat"] = q_hat
    else:
        q32 = _draw(g, (B, Hq, dk), w.dist)
    res["q"] = q32.to(dt)

    # lens
    if lens_override is not None:
        lens = torch.tensor(lens_override, dtype=torch.int32)
        assert lens.numel() == B
    elif w.ragged:
        lens = torch.randint(1, T + 1, (B,), generator=g, dtype=torch.int64)
        lens = lens.to(torch.int32)
    else:
        lens = torch.full((B,), T, dtype=torch.int32)
    res["lens"] = lens

    # K, V: drawn per sequence over the live slots only
    k = torch.empty((B, T, Hkv, dk), dtype=dt)
    v = torch.empty((B, T, Hkv, dv), dtype=dt)
    spike_pos = None
    if w.dist == "spike":
        spike_pos = max(T - w.spike_depth, 0)
    for b in range(B):
        n = int(min(max(int(lens[b]), 0), T))
        if w.dist == "spike":
            kb = _uniform(g, (n, Hkv, dk), -1.0, 1.0) * 1.732
            vb = _uniform(g, (n, Hkv, dv), -1.0, 1.0)
            vb[..., 0] = 0.0
            if spike_pos < n:
                for grp in range(Hkv):
                    h0 = grp * w.hpk
                    kb[spike_pos, grp] += w.spike_amp * res["q_hat"][b, h0]
                    vb[spike_pos, grp, 0] = 1.0
        else:
            kb = _draw(g, (n, Hkv, dk), w.dist)
            vb = _draw(g, (n, Hkv, dv), w.dist)
        k[b, :n] = kb.to(dt)
        v[b, :n] = vb.to(dt)
        if n < T:
            k[b, n:] = pad_value
            v[b, n:] = pad_value
    res["k"], res["v"] = k, v
    if spike_pos is not None:
        res["spike_pos"] = spike_pos

    if w.window > 0:
        res["wk"] = _draw(g, (B, w.window, Hkv, dk), w.dist).to(dt)
        res["wv"] = _draw(g, (B, w.window, Hkv, dv), w.dist).to(dt)
        res["wlens"] = torch.full((B,), w.window, dtype=torch.int32)
    return res


def algorithmic_bytes(w: DecodeWorkload, lens) -> int:
    """HBM bytes one attend pass must move at minimum.

    K and V of every live token once per KV group, q once, the fp32 output
    once, and for fp8 caches the two fp32 scales of each (sequence, KV
    head).  Split-K partials are not counted (they are overhead).
    """
    n_tot = sum(int(min(max(int(x), 0), w.max_len)) for x in lens)
    kv = n_tot * w.num_kv_heads * (w.dk + w.dv) * w.esz
    q = w.batch * w.num_q_heads * w.dk * w.q_esz
    out = w.batch * w.num_q_heads * w.dv * 4
    scales = w.batch * w.num_kv_heads * 2 * 4 if w.dtype == "fp8" else 0
    return kv + q + out + scales
