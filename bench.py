#!/usr/bin/env python3
"""Decode-step benchmark of exact GQA decode attention on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--replays R]
                    [--workload all|tiny|batched|ragged|long|spike|
                                stream|gather|fp8]

A step is the whole hot path on one batch: the new token's K/V rows appended
to every sequence's cache (needle-core push_kv) and attention over the cache
including it, as one decode_step call (split-K partition launch with the
append folded in, then the log-sum-exp combine where the plan needs one).
The long-context workload attends its main cache and its recent window in
one decode_step_branches call, the new token entering the window.

By default the five workloads run in one process: tiny fp32, batched bf16,
ragged bf16, long context + window, wide group with a planted spike.  The
headline (`value`, `ms_per_step`, `config`, `roofline`) is the ragged batch,
the largest workload on one GPU; every workload has its own entry under
`configs`.  One JSON line goes to stdout; diagnostics go to stderr.

Host phase (before the GPU is touched): every workload's inputs are drawn,
and the CPU oracle is run on the step's exact inputs over the (sequence, KV
group) units by a pool of forked worker processes, one per host core, for a
bounded time per workload; this is the CPU baseline and also the reference
the GPU outputs are checked against afterwards (max error and relative L2
per workload).

GPU phase, per workload: W eager warm-up steps; a HIP graph of K steps is
captured, replayed five times untimed, then replayed R times, each replay
timed on its own with a synchronisation on both sides (median, p10, p90 of
the per-step time over the R replays).  Successive steps rotate over copies
of the cache (>= 1 GiB in all where it fits) so each step streams from HBM
rather than from the 256 MB last-level cache.  The dominant kernel (the
partition launch that streams the cache, in its decode-step form) is then
timed on its own: K eager steps, each with the library's profiling request,
which brackets exactly that kernel with a pair of HIP events on its stream.
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import multiprocessing as mp
import os
import re
import sys
import time
from pathlib import Path

import numpy as np

ROOT = Path(__file__).resolve().parent
if str(ROOT) not in sys.path:
    sys.path.insert(0, str(ROOT))

METRIC = ("KV-cache GB/s streamed (and % HBM peak) in GQA decode; "
          "µs per decode step")
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, AMD published figure
ROTATE_TARGET_BYTES = 1 << 30
CSRC = ROOT / "gqa_kv_cache_decode_amd" / "csrc"
# Sources of the dominant (partition) kernel: recorded counter readings are
# only reported while these are unchanged.
_MFMA16 = ["partition_mfma16.h", "fp8_common.h", "device_common.h", "launch.h",
           "step_common.h", "gather_common.h"]
PARTITION_SOURCES = {"bf16": ["partition_bf16.hip"] + _MFMA16,
                     "fp8": ["partition_fp8.hip"] + _MFMA16,
                     "f32": ["partition_f32.hip", "device_common.h", "launch.h",
                             "step_common.h", "gather_common.h"]}
COPY_BYTES = 256 << 20      # calibration copy for the byte counters
WARM_REPLAYS = 5            # untimed replays of the step graph before timing
DEFAULT_SET = ["tiny", "batched", "ragged", "long", "spike"]
HEADLINE = "ragged"         # the largest workload that fits one GPU
ONE_THREAD_SET = ["tiny", "batched"]   # also timed on one host core
MAX_HOST_WORKERS = 16       # host processes at most (one GPU's share of a node)
# max |out - out_oracle| <= TOL * max|V| over the attended values
TOL = {"f32": 1e-5, "bf16": 4e-3, "fp8": 4e-3}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse_args(argv=None):
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--replays", type=int, default=7,
                   help="timed replays of the K-step graph per workload")
    p.add_argument("--workload", default="all",
                   choices=["all"] + DEFAULT_SET + ["stream", "gather", "fp8"],
                   help="all: the five workloads, headline ragged.  "
                        "stream: the long-context shapes kept as 4 sink "
                        "keys + a 128-key window ring + a main cache; each "
                        "step appends (evicting the ring's oldest key into "
                        "main) and attends the three parts in one launch.  "
                        "gather: index-gathered decode of 2048 selected "
                        "slots (pools of 64) per sequence of a 32K cache.  "
                        "fp8: the batched shape over fp8 (E4M3) caches with "
                        "per-(sequence, KV head) scales")
    p.add_argument("--rotate", type=int, default=0,
                   help="cache copies to rotate over (0 = enough for 1 GiB)")
    p.add_argument("--cpu-seconds", type=float, default=4.0,
                   help="wall-clock budget of the oracle per workload")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-ceiling", action="store_true")
    p.add_argument("--bias", action="store_true",
                   help="attend with an additive logit bias (fp32 per "
                        "sequence and position, N(0, 1))")
    p.add_argument("--set", action="append", default=[], metavar="FIELD=N",
                   help="replace an integer field of the workload's shape "
                        "(batch, num_q_heads, num_kv_heads, dk, dv, max_len; "
                        "repeatable), for sweeps and counter runs of one "
                        "workload; its traffic record then does not apply")
    p.add_argument("--profile-pass", action="store_true",
                   help="no timing: a few eager steps of one workload and "
                        f"three {COPY_BYTES >> 20} MiB calibration copies, "
                        "for hardware-counter runs")
    return p.parse_args(argv)


def workload_by_name(name):
    from gqa_kv_cache_decode_amd import workloads as wl
    return {"tiny": wl.TINY_F32, "batched": wl.BATCHED_BF16,
            "ragged": wl.RAGGED_BF16, "long": wl.LONG_WINDOW_BF16,
            "spike": wl.WIDE_SPIKE_BF16, "stream": wl.LONG_WINDOW_BF16,
            "gather": wl.GATHER_BF16, "fp8": wl.BATCHED_FP8}[name]


SHAPE_FIELDS = ("batch", "num_q_heads", "num_kv_heads", "dk", "dv", "max_len")


def shaped_workload(name, overrides):
    """The named workload with `overrides` ("field=N" strings) applied; the
    name records them."""
    w = workload_by_name(name)
    if not overrides:
        return w
    kv = {}
    for item in overrides:
        field, _, val = item.partition("=")
        if field not in SHAPE_FIELDS or not val.lstrip("-").isdigit():
            raise SystemExit(f"--set {item}: expected one of "
                             f"{', '.join(SHAPE_FIELDS)} = an integer")
        kv[field] = int(val)
    tag = "_".join(f"{k}{v}" for k, v in kv.items())
    return w.replace(name=f"{w.name}+{tag}", **kv)


def kv_bytes(w, lens_total, hkv=None):
    return lens_total * (hkv or w.num_kv_heads) * (w.dk + w.dv) * w.esz


def library_plan(w):
    """The library's own plan for the workload's cache (a host-only call)."""
    from gqa_kv_cache_decode_amd import binding as bd
    dt = {"f32": 0, "bf16": 1, "fp8": 2}[w.dtype]
    sc = 0x30000 if w.dtype == "fp8" else None
    c = bd._Cache(0x10000, 0x20000, w.batch, w.max_len, w.num_kv_heads, w.dk,
                  w.dv, dt, sc, sc)
    p = bd.Plan()
    st = bd.library().gqa_attend_plan(ctypes.byref(c), w.num_q_heads, 0,
                                      ctypes.byref(p))
    assert st == 0, "no plan for the workload"
    return p


def kernel_name(w, bias, gather, step=True, balanced=None):
    """The partition kernel's name as the profiler prints it (template
    arguments: head widths, wavefronts, decode step, bias, gathered, and fp8
    for the bf16 / fp8 family; a balanced plan's kernel has no gathered
    form).  `balanced`: whether the library's plan is balanced (asked from
    the library when None)."""
    tf = lambda b: "true" if b else "false"
    if w.dtype == "f32":
        flags = f"{tf(step)}, {tf(bias)}, {tf(gather)}"
        return f"partition_f32_mfma_kernel<{w.dk}, {w.dv}, 4, {flags}>"
    if w.dtype == "fp8":
        waves = 8 if w.dk + w.dv <= 128 else 4
    else:
        waves = 2
    if balanced is None:
        balanced = not gather and library_plan(w).balanced_groups > 0
    fp8 = tf(w.dtype == "fp8")
    if balanced:
        return (f"partition_balanced_kernel<{w.dk}, {w.dv}, {waves}, "
                f"{tf(step)}, {tf(bias)}, {fp8}>")
    if (w.dtype == "fp8" and not gather and w.dk + w.dv <= 128 and
            w.num_kv_heads % waves == 0):
        # the group-split launch (64-wide fp8 heads): a plain chunked plan
        # whose items, in sets of `waves` KV groups, are one round of one
        # work-group per CU
        p = library_plan(w)
        if (p.sched_entries == 0 and p.num_chunks > 1 and
                256 <= w.batch * w.num_kv_heads * p.num_chunks // waves < 512):
            return (f"partition_split_kernel<{w.dk}, {w.dv}, {waves}, "
                    f"{tf(step)}, {tf(bias)}, {fp8}>")
    return (f"partition_bf16_kernel<{w.dk}, {w.dv}, {waves}, {tf(step)}, "
            f"{tf(bias)}, {tf(gather)}, {fp8}>")


# ---------------------------------------------------------------------------
# Stored values as float64 (host side, numpy only: the forked oracle workers
# never call into torch)

def _f64(a):
    """bf16 bit patterns (uint16 / int16 arrays) or fp32 values as fp64."""
    if a.dtype in (np.uint16, np.int16):
        return (a.view(np.uint16).astype(np.uint32) << 16).view(
            np.float32).astype(np.float64)
    return a.astype(np.float64)


def _np_view(t):
    """Zero-copy numpy view of a CPU tensor (bf16 as its uint16 bits)."""
    import torch
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


# ---------------------------------------------------------------------------
# Workload cases: host inputs, the oracle per (sequence, KV group) unit of
# the step's exact inputs, and the GPU step

class Case:
    """One workload: inputs drawn on the host, the step's oracle units, the
    GPU step and its byte accounting."""

    has_oracle = True

    def __init__(self, name, args):
        from gqa_kv_cache_decode_amd import workloads as wl
        self.name = name
        self.w = shaped_workload(name, args.set)
        self.args = args
        self.bias = bool(args.bias)
        w = self.w
        t = time.time()
        self.x = self.draw(wl)
        log(f"[bench] {name}: inputs drawn in {time.time() - t:.1f}s")
        import torch
        gen = torch.Generator().manual_seed(w.seed + 1000)
        io = torch.bfloat16 if w.dtype == "fp8" else w.torch_dtype
        self.k_new = torch.randn(w.batch, w.num_kv_heads, w.dk,
                                 generator=gen).to(io)
        self.v_new = torch.randn(w.batch, w.num_kv_heads, w.dv,
                                 generator=gen).to(io)
        self.bias_t = None
        if self.bias:
            gb = torch.Generator().manual_seed(w.seed + 2000)
            pad = (w.max_len + 3) // 4 * 4
            self.bias_t = torch.randn(w.batch, pad, generator=gb)
        self.units = [(b, g) for b in range(w.batch)
                      for g in range(w.num_kv_heads)]
        self.q_np = _np_view(self.x["q"])
        self.kn_np = _np_view(self.k_new)
        self.vn_np = _np_view(self.v_new)

    def draw(self, wl):
        return wl.make_inputs(self.w)

    # -- host side ---------------------------------------------------------
    def unit_bytes(self, n):
        w = self.w
        return (n * (w.dk + w.dv) * w.esz +
                w.hpk * (w.dk * w.q_esz + w.dv * 4))

    def q_unit(self, b, g):
        h = self.w.hpk
        return _f64(self.q_np[b, g * h:(g + 1) * h])[None]

    # -- byte accounting (algorithmic; split-K partials excluded) ------------
    def new_row_bytes(self):
        """The new token's rows read (in the query dtype) and written to the
        cache (in the cache dtype)."""
        w = self.w
        return w.batch * w.num_kv_heads * (w.dk + w.dv) * (w.q_esz + w.esz)

    def fixed_bytes(self):
        """q, the lengths read and written, fp8 scales."""
        w = self.w
        q = w.batch * w.num_q_heads * w.dk * w.q_esz
        scales = 2 * w.batch * w.num_kv_heads * 4 if w.dtype == "fp8" else 0
        return q + 2 * w.batch * 4 + scales

    def out_bytes(self):
        w = self.w
        return w.batch * w.num_q_heads * w.dv * 4


class SingleCase(Case):
    """decode_step on one cache: the new token goes to slot lens - 1 (every
    workload length is >= 1) and the query attends over [0, lens)."""

    def __init__(self, name, args):
        super().__init__(name, args)
        x = self.x
        self.lens = x["lens"].numpy().astype(np.int64)
        self.k_np = _np_view(x["k"])
        self.v_np = _np_view(x["v"])
        self.bias_np = None if self.bias_t is None else self.bias_t.numpy()

    def oracle_unit(self, key):
        """Oracle output rows of unit (b, g) on the step's inputs: the cache
        up to the slot, then the new token."""
        import oracle
        b, g = key
        n = int(self.lens[b])
        k = np.concatenate([_f64(self.k_np[b, :n - 1, g]),
                            _f64(self.kn_np[b, g])[None]])
        v = np.concatenate([_f64(self.v_np[b, :n - 1, g]),
                            _f64(self.vn_np[b, g])[None]])
        bias = None if self.bias_np is None else self.bias_np[b:b + 1, :n]
        out, _ = oracle.attend(self.q_unit(b, g), k[None, :, None],
                               v[None, :, None], [n], self.w.scale, bias=bias)
        return out[0], float(np.abs(v).max()), self.unit_bytes(n)

    def attended_tokens(self):
        return int(np.minimum(self.lens, self.w.max_len).sum())

    def step_bytes(self):
        w = self.w
        n_tot = self.attended_tokens()
        b = (kv_bytes(w, n_tot - w.batch) + self.new_row_bytes() +
             self.fixed_bytes() + self.out_bytes())
        return b + (4 * n_tot if self.bias else 0)

    def kernel(self):
        return kernel_name(self.w, self.bias, False)

    def gpu(self, copies):
        return SingleGpu(self, copies)


class Fp8Case(SingleCase):
    """The batched shape over fp8 (E4M3) caches: the new bf16 rows are
    quantised into the slot with the sequence's scales."""

    def draw(self, wl):
        return wl.make_fp8_inputs(self.w)

    def __init__(self, name, args):
        super().__init__(name, args)
        self.ks = self.x["k_scale"].numpy()
        self.vs = self.x["v_scale"].numpy()

    def oracle_unit(self, key):
        import oracle.fp8 as ofp8
        b, g = key
        n = int(self.lens[b])
        kq = ofp8.quantize(_f64(self.kn_np[b, g]), self.ks[b, g])
        vq = ofp8.quantize(_f64(self.vn_np[b, g]), self.vs[b, g])
        k = np.concatenate([self.k_np[b, :n - 1, g], kq[None]])
        v = np.concatenate([self.v_np[b, :n - 1, g], vq[None]])
        out, _ = ofp8.attend_fp8(self.q_unit(b, g), k[None, :, None],
                                 v[None, :, None], self.ks[b:b + 1, g:g + 1],
                                 self.vs[b:b + 1, g:g + 1], [n], self.w.scale)
        vmax = float(np.abs(ofp8.decode(v)).max() * self.vs[b, g])
        return out[0], vmax, self.unit_bytes(n)


class LongCase(Case):
    """decode_step_branches over the long main cache (attended as is) and the
    recent window, which takes the new token at slot window - 1."""

    def __init__(self, name, args):
        super().__init__(name, args)
        x = self.x
        self.k_np, self.v_np = _np_view(x["k"]), _np_view(x["v"])
        self.wk_np, self.wv_np = _np_view(x["wk"]), _np_view(x["wv"])
        self.bias = False   # the branches here carry no bias

    def oracle_unit(self, key):
        """One pass over main, the window up to the slot and the new token:
        the concatenation the carry algebra makes the branches equal to."""
        import oracle
        b, g = key
        w = self.w
        W = w.window
        k = np.concatenate([_f64(self.k_np[b, :, g]),
                            _f64(self.wk_np[b, :W - 1, g]),
                            _f64(self.kn_np[b, g])[None]])
        v = np.concatenate([_f64(self.v_np[b, :, g]),
                            _f64(self.wv_np[b, :W - 1, g]),
                            _f64(self.vn_np[b, g])[None]])
        n = k.shape[0]
        out, _ = oracle.attend(self.q_unit(b, g), k[None, :, None],
                               v[None, :, None], [n], w.scale)
        return out[0], float(np.abs(v).max()), self.unit_bytes(n)

    def attended_tokens(self):
        return self.w.batch * (self.w.max_len + self.w.window)

    def step_bytes(self):
        w = self.w
        return (kv_bytes(w, self.attended_tokens() - w.batch) +
                self.new_row_bytes() + self.fixed_bytes() + self.out_bytes())

    def kernel(self):
        # the branches' launch is never balanced
        return kernel_name(self.w, False, False, balanced=False)

    def gpu(self, copies):
        return LongGpu(self, copies)


class StreamCase(Case):
    """The long-context history kept as sink / window ring / main cache: each
    step appends (the ring's oldest key moving to main), then attends the
    three parts in one partition launch and one combine."""

    has_oracle = False
    SINK = 4            # permanent sink keys (cortiq-engine default)
    ROOM = 1024         # free main slots, so the steps grow main

    def __init__(self, name, args):
        super().__init__(name, args)
        w = self.w
        self.bias = False
        self.n_main = w.max_len - self.SINK - w.window - self.ROOM

    def step_bytes(self):
        w = self.w
        # sink + ring + main keys, q once; the new row written, the evicted
        # row read and written; counts and the three lengths
        return (kv_bytes(w, w.batch * (self.SINK + w.window + self.n_main)) +
                w.batch * w.num_q_heads * w.dk * w.q_esz +
                3 * w.batch * w.num_kv_heads * (w.dk + w.dv) * w.esz +
                5 * w.batch * 4 + self.out_bytes())

    def kernel(self):
        return kernel_name(self.w, False, False, step=False, balanced=False)

    def gpu(self, copies):
        return StreamGpu(self, copies)


class GatherCase(Case):
    """Index-gathered decode: the steps rotate over index sets that select
    enough distinct rows (>= 1 GiB in all) that no step hits the MALL."""

    has_oracle = False

    def __init__(self, name, args):
        super().__init__(name, args)
        self.bias = False

    def kernel(self):
        return kernel_name(self.w, False, True, step=False, balanced=False)

    def gpu(self, copies):
        return GatherGpu(self, copies)


CASES = {"tiny": SingleCase, "batched": SingleCase, "ragged": SingleCase,
         "spike": SingleCase, "fp8": Fp8Case, "long": LongCase,
         "stream": StreamCase, "gather": GatherCase}


# ---------------------------------------------------------------------------
# GPU side of each case

def _copies(args, one_copy_bytes):
    if args.rotate:
        return args.rotate
    return max(1, min(8, math.ceil(ROTATE_TARGET_BYTES / one_copy_bytes)))


def clone_cache(c):
    """A copy of a K or V cache (an fp8 cache keeps sharing its scales)."""
    from gqa_kv_cache_decode_amd import Fp8Cache
    if isinstance(c, Fp8Cache):
        return Fp8Cache(c.codes.clone(), c.scale)
    return c.clone()


class SingleGpu:
    def __init__(self, case, copies):
        import torch
        import gqa_kv_cache_decode_amd as g
        w, x, dev = case.w, case.x, torch.device("cuda")
        self.case, self.copies = case, copies
        self.q = x["q"].to(dev)
        self.kn, self.vn = case.k_new.to(dev), case.v_new.to(dev)
        self.out = torch.empty(w.batch, w.num_q_heads, w.dv,
                               dtype=torch.float32, device=dev)
        kc, vc = x["k"].to(dev), x["v"].to(dev)
        if w.dtype == "fp8":
            kc = g.Fp8Cache(kc, x["k_scale"].to(dev))
            vc = g.Fp8Cache(vc, x["v_scale"].to(dev))
        self.k = [kc] + [clone_cache(kc) for _ in range(copies - 1)]
        self.v = [vc] + [clone_cache(vc) for _ in range(copies - 1)]
        lens = x["lens"].to(dev)
        self.lens_before = (lens - 1).clamp_(min=0)
        self.lens_cur = [lens.clone() for _ in range(copies)]
        self.bias = None if case.bias_t is None else case.bias_t.to(dev)
        # zero-filled once: its tail holds the arrival counters
        self.ws = g.step_workspace(self.k[0], self.v[0], w.num_q_heads)

    def step(self, r):
        import gqa_kv_cache_decode_amd as g
        c = self.case
        g.decode_step(self.q, self.k[r], self.v[r], self.kn, self.vn,
                      self.lens_before, self.lens_cur[r], c.w.scale,
                      out=self.out, workspace=self.ws, bias=self.bias)


class LongGpu:
    def __init__(self, case, copies):
        import torch
        import gqa_kv_cache_decode_amd as g
        from gqa_kv_cache_decode_amd import binding
        w, x, dev = case.w, case.x, torch.device("cuda")
        self.case, self.copies = case, copies
        self.q = x["q"].to(dev)
        self.kn, self.vn = case.k_new.to(dev), case.v_new.to(dev)
        self.out = torch.empty(w.batch, w.num_q_heads, w.dv,
                               dtype=torch.float32, device=dev)
        mk, mv = x["k"].to(dev), x["v"].to(dev)
        self.mk = [mk] + [mk.clone() for _ in range(copies - 1)]
        self.mv = [mv] + [mv.clone() for _ in range(copies - 1)]
        self.mlens = x["lens"].to(dev)
        wk, wv = x["wk"].to(dev), x["wv"].to(dev)
        self.wk = [wk] + [wk.clone() for _ in range(copies - 1)]
        self.wv = [wv] + [wv.clone() for _ in range(copies - 1)]
        wl_ = x["wlens"].to(dev)
        self.wlens_before = (wl_ - 1).clamp_(min=0)
        self.wlens_cur = [wl_.clone() for _ in range(copies)]
        self.ws = torch.empty(g.library().gqa_attend_branches_workspace_bytes(
            binding._branches([(mk, mv, self.mlens),
                               (wk, wv, self.wlens_before)], None), 2,
            w.num_q_heads), dtype=torch.uint8, device=dev)

    def step(self, r):
        import gqa_kv_cache_decode_amd as g
        g.decode_step_branches(
            self.q, [(self.mk[r], self.mv[r], self.mlens, None),
                     (self.wk[r], self.wv[r], self.wlens_before, None)], 1,
            self.kn, self.vn, self.wlens_cur[r], self.case.w.scale,
            out=self.out, workspace=self.ws)


class StreamGpu:
    def __init__(self, case, copies):
        import torch
        import gqa_kv_cache_decode_amd as g
        from gqa_kv_cache_decode_amd import binding
        w, x, dev = case.w, case.x, torch.device("cuda")
        S, W, mn = case.SINK, w.window, case.n_main
        self.case, self.copies = case, copies
        self.q = x["q"].to(dev)
        self.kn, self.vn = case.k_new.to(dev), case.v_new.to(dev)
        self.out = torch.empty(w.batch, w.num_q_heads, w.dv,
                               dtype=torch.float32, device=dev)
        mk, mv = x["k"].to(dev), x["v"].to(dev)
        self.main = [(mk, mv)] + [(mk.clone(), mv.clone())
                                  for _ in range(copies - 1)]
        self.sink = [(m[0][:, :S].clone(), m[1][:, :S].clone())
                     for m in self.main]
        rk, rv = x["wk"].to(dev), x["wv"].to(dev)
        self.ring = [(rk.clone(), rv.clone()) for _ in range(copies)]
        i32 = lambda v: torch.full((w.batch,), v, dtype=torch.int32,
                                   device=dev)
        self.count = [i32(S + W + mn) for _ in range(copies)]
        self.lens = [(i32(S), i32(W), i32(mn)) for _ in range(copies)]
        self.ws = torch.empty(g.library().gqa_attend_branches_workspace_bytes(
            binding._branches(self.branches(0), None), 3, w.num_q_heads),
            dtype=torch.uint8, device=dev)

    def branches(self, r):
        ls, lr, lm = self.lens[r]
        return [(*self.sink[r], ls), (*self.ring[r], lr),
                (*self.main[r], lm)]

    def step(self, r):
        import gqa_kv_cache_decode_amd as g
        g.stream_append(self.ring[r][0], self.ring[r][1], self.kn, self.vn,
                        self.count[r], count_out=self.count[r],
                        sink=self.sink[r], main=self.main[r],
                        lens=self.lens[r])
        g.attend_branches(self.q, self.branches(r), self.case.w.scale,
                          out=self.out, workspace=self.ws)


class GatherGpu:
    def __init__(self, case, copies):
        import torch
        import gqa_kv_cache_decode_amd as g
        from gqa_kv_cache_decode_amd import binding
        from gqa_kv_cache_decode_amd import workloads as wl
        w, x, dev = case.w, case.x, torch.device("cuda")
        self.case = case
        self.q = x["q"].to(dev)
        self.out = torch.empty(w.batch, w.num_q_heads, w.dv,
                               dtype=torch.float32, device=dev)
        self.k, self.v, self.lens = (x["k"].to(dev), x["v"].to(dev),
                                     x["lens"].to(dev))
        sel_bytes = w.batch * wl.GATHER_WIDTH * w.num_kv_heads * \
            (w.dk + w.dv) * w.esz
        self.copies = copies = case.args.rotate or max(
            1, min(16, math.ceil(ROTATE_TARGET_BYTES / sel_bytes)))
        self.idx, sel = [], []
        for r in range(copies):
            rows = wl.make_index_rows(w, x["lens"], wl.GATHER_WIDTH,
                                      wl.GATHER_POOL, w.seed + 3000 + r)
            self.idx.append(rows.to(dev))
            sel.append(sum(len(set(rr.tolist()) - {-1}) for rr in rows))
        self.n_sel = sum(sel) // len(sel)
        self.ws = torch.empty(
            g.library().gqa_attend_gathered_workspace_bytes(
                ctypes.byref(binding._cache(self.k, self.v)), w.num_q_heads,
                wl.GATHER_WIDTH), dtype=torch.uint8, device=dev)

    def step(self, r):
        import gqa_kv_cache_decode_amd as g
        g.attend_gathered(self.q, self.k, self.v, self.lens, self.idx[r],
                          self.case.w.scale, out=self.out, workspace=self.ws)


def gather_bytes(case, gpu):
    from gqa_kv_cache_decode_amd import workloads as wl
    w = case.w
    # the distinct selected rows (mean over the index sets), q, the index
    # rows (read by the partition launch, which selects), the output
    return (kv_bytes(w, gpu.n_sel) + w.batch * w.num_q_heads * w.dk * w.q_esz +
            w.batch * wl.GATHER_WIDTH * 4 + case.out_bytes())


# ---------------------------------------------------------------------------
# CPU baseline: the oracle over the step's (sequence, KV group) units

_HOST_CASE = None   # the case the forked workers evaluate


def _oracle_worker(job):
    """Worker i of n: its share of the units, cyclically, until the budget
    is spent (it finishes the unit in hand).  Returns the bytes and unit
    count done, its elapsed time and the outputs of the units it did."""
    i, n, budget = job
    from threadpoolctl import threadpool_limits
    case = _HOST_CASE
    units = case.units
    mine = units[i::n] if i < len(units) else [units[i % len(units)]]
    done, nbytes, outs = 0, 0, {}
    t0 = time.perf_counter()
    with threadpool_limits(limits=1):
        while True:
            for key in mine:
                out, vmax, nb = case.oracle_unit(key)
                nbytes += nb
                done += 1
                outs.setdefault(key, (out, vmax))
                if time.perf_counter() - t0 >= budget:
                    return nbytes, done, time.perf_counter() - t0, outs
    # (never reached)


def host_workers():
    return max(1, min(len(os.sched_getaffinity(0)), MAX_HOST_WORKERS))


def cpu_model():
    try:
        for line in Path("/proc/cpuinfo").read_text().splitlines():
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def run_oracle(case, workers, budget):
    """Evaluates the oracle on `workers` forked processes (the GPU is not
    initialised yet, and the workers only use numpy)."""
    global _HOST_CASE
    _HOST_CASE = case
    ctx = mp.get_context("fork")
    with ctx.Pool(workers) as pool:
        res = pool.map(_oracle_worker,
                       [(i, workers, budget) for i in range(workers)],
                       chunksize=1)
    _HOST_CASE = None
    nbytes = sum(r[0] for r in res)
    done = sum(r[1] for r in res)
    wall = max(r[2] for r in res)
    outs = {}
    for r in res:
        for k, v in r[3].items():
            outs.setdefault(k, v)
    return {"gbs": nbytes / wall / 1e9, "evaluations": done, "wall_s": wall,
            "workers": workers, "outs": outs}


def cpu_phase(cases, args):
    workers = host_workers()
    per = {}
    for name, case in cases.items():
        if not case.has_oracle:
            continue
        r = run_oracle(case, workers, args.cpu_seconds)
        log(f"[bench] {name}: oracle {r['gbs']:.3f} GB/s on {workers} "
            f"processes ({r['evaluations']} unit evaluations, "
            f"{len(r['outs'])}/{len(case.units)} units)")
        if name in ONE_THREAD_SET:
            one = run_oracle(case, 1, min(args.cpu_seconds, 3.0))
            r["one_thread_gbs"] = one["gbs"]
            log(f"[bench] {name}: oracle {one['gbs']:.3f} GB/s on 1 process")
        per[name] = r
    return per


# ---------------------------------------------------------------------------
# GPU timing

_BENCH_LIB = None


def bench_lib():
    """The measurement helpers of libgqa_bench.so (read stream, copy, spin,
    timing events)."""
    global _BENCH_LIB
    if _BENCH_LIB is None:
        from gqa_kv_cache_decode_amd.build import BENCH_LIB
        lib = ctypes.CDLL(str(BENCH_LIB))
        lib.gqa_bench_read_stream.argtypes = [ctypes.c_void_p, ctypes.c_size_t,
                                              ctypes.c_void_p, ctypes.c_int,
                                              ctypes.c_void_p]
        lib.gqa_bench_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_size_t, ctypes.c_int,
                                       ctypes.c_void_p]
        lib.gqa_bench_spin.argtypes = [ctypes.c_int, ctypes.c_void_p]
        lib.gqa_bench_events_create.argtypes = [ctypes.c_int, ctypes.c_void_p]
        lib.gqa_bench_events_destroy.argtypes = [ctypes.c_int, ctypes.c_void_p]
        lib.gqa_bench_events_elapsed.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(ctypes.c_float)]
        _BENCH_LIB = lib
    return _BENCH_LIB


def _stream_handle(torch):
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def time_dominant_kernel(torch, gpu, K):
    """K eager steps queued behind a bounded spin kernel, each asking the
    library to bracket its partition launch with a HIP event pair on the
    launch's stream: the per-launch device times of exactly that kernel."""
    import gqa_kv_cache_decode_amd as g
    lib = bench_lib()
    ev = (ctypes.c_void_p * (2 * K))()
    assert lib.gqa_bench_events_create(2 * K, ev) == 0
    try:
        torch.cuda.synchronize()
        lib.gqa_bench_spin(min(1000000, 20000 + 200 * K), _stream_handle(torch))
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(K):
            g.profile_next_launch(ev[2 * i], ev[2 * i + 1])
            gpu.step(i % gpu.copies)
        e1.record()
        torch.cuda.synchronize()
        ms = []
        for i in range(K):
            t = ctypes.c_float()
            assert lib.gqa_bench_events_elapsed(ev[2 * i], ev[2 * i + 1],
                                                ctypes.byref(t)) == 0
            ms.append(t.value)
        eager_ms = e0.elapsed_time(e1) / K
    finally:
        g.profile_next_launch(0, 0)
        lib.gqa_bench_events_destroy(2 * K, ev)
    return ms, eager_ms


def time_steps(torch, gpu, K, W, R):
    """ms per step of R timed replays of a graph of K steps."""
    for i in range(W):
        gpu.step(i % gpu.copies)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        gpu.step(0)  # one eager call on the capture stream first
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        for i in range(K):
            gpu.step(i % gpu.copies)
    torch.cuda.synchronize()
    # untimed replays of the whole graph: a timed replay right after a single
    # warm one ran ~8% slower (clocks still ramping on a fresh box)
    for _ in range(WARM_REPLAYS):
        gr.replay()
    torch.cuda.synchronize()
    per = []
    for _ in range(R):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        gr.replay()
        e1.record()
        torch.cuda.synchronize()
        per.append(e0.elapsed_time(e1) / K)
    del gr
    return per


def read_ceiling(torch, nbytes=4 << 30, reps=5):
    """A plain nontemporal 16-byte-vector read of 4 GiB: the HBM read rate
    reachable on this GPU (best of `reps`)."""
    lib = bench_lib()
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    blocks = 65536  # measured best for this kernel on MI355X
    sink = torch.zeros(blocks, dtype=torch.int32, device="cuda")
    best = 0.0
    for _ in range(reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        rc = lib.gqa_bench_read_stream(buf.data_ptr(), nbytes, sink.data_ptr(),
                                       blocks, _stream_handle(torch))
        e1.record()
        torch.cuda.synchronize()
        assert rc == 0
        best = max(best, nbytes / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    del buf
    return best


def code_text(src):
    """C++ source with its comments removed and whitespace collapsed: what
    the compiler sees, so that editing a comment keeps counter readings."""
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    return " ".join(src.split())


def partition_source_hash(dtype):
    h = hashlib.sha256()
    for name in PARTITION_SOURCES[dtype]:
        h.update(code_text((CSRC / name).read_text()).encode())
    return h.hexdigest()[:16]


def profile_name(name, bias):
    """Name of a workload's counter readings under profiles/."""
    return name + ("_bias" if bias else "")


def measured_traffic(workload, dtype, kernel=None):
    """HBM bytes per dominant-kernel launch from committed counter readings,
    if they were taken on the current kernel sources (and on `kernel`)."""
    path = ROOT / "profiles" / f"traffic_{workload}.json"
    if not path.exists():
        return None
    rec = json.loads(path.read_text())
    if rec.get("partition_source_sha256_16") != partition_source_hash(dtype):
        return None
    if kernel is not None and rec.get("kernel") != kernel:
        return None
    return rec.get("traffic_bytes_per_launch")


def _pct(a, p):
    return float(np.percentile(np.asarray(a), p))


def check_outputs(case, out, outs):
    """GPU output rows against the oracle's, over the units it evaluated:
    max error in units of max|V| (the tolerance's scale) and the relative L2
    error ||o - o_ref|| / ||o_ref|| (cortiq-engine background_error)."""
    if not outs:
        return None
    w = case.w
    h = w.hpk
    got, want, vmax = [], [], 0.0
    for (b, g), (o, vm) in outs.items():
        got.append(out[b, g * h:(g + 1) * h].astype(np.float64))
        want.append(o)
        vmax = max(vmax, vm)
    got, want = np.stack(got), np.stack(want)
    err = float(np.max(np.abs(got - want)))
    rel = float(np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-300))
    tol = TOL[w.dtype]
    return {"units_checked": len(outs), "units": len(case.units),
            "max_err_over_vmax": err / max(vmax, 1e-300),
            "tolerance_over_vmax": tol, "rel_l2": rel,
            "within_tolerance": bool(err <= tol * vmax and
                                     np.all(np.isfinite(got)))}


def gpu_phase(torch, case, args, oracle_res):
    w = case.w
    if isinstance(case, GatherCase):
        copies = 0
    elif isinstance(case, LongCase):
        copies = _copies(args, (case.x["k"].numel() + case.x["v"].numel()) *
                         w.esz)
    else:
        copies = _copies(args, (case.x["k"].numel() + case.x["v"].numel()) *
                         w.esz)
    gpu = case.gpu(copies)
    torch.cuda.synchronize()
    K, R = args.steps, args.replays
    per = time_steps(torch, gpu, K, args.warmup, R)
    kms, eager_ms = time_dominant_kernel(torch, gpu, K)
    out = gpu.out.cpu().numpy()
    if isinstance(case, GatherCase):
        step_bytes = gather_bytes(case, gpu)
        dom_bytes = step_bytes - case.out_bytes()
    else:
        step_bytes = case.step_bytes()
        # the dominant kernel: everything the step reads and the cache rows
        # it writes; the outputs are counted with whichever kernel writes them
        dom_bytes = step_bytes - case.out_bytes()
    med = _pct(per, 50)
    kavg = float(np.mean(kms))
    gbs = step_bytes / (med * 1e-3) / 1e9
    kgbs = dom_bytes / (kavg * 1e-3) / 1e9
    kernel = case.kernel()
    res = {
        "workload": w.name, "kv_dtype": "fp8_e4m3" if w.dtype == "fp8"
        else w.dtype,
        "batch": w.batch, "num_q_heads": w.num_q_heads,
        "num_kv_heads": w.num_kv_heads, "dk": w.dk, "dv": w.dv,
        "seq_len": w.max_len, "window": w.window,
        "attended_tokens": (None if isinstance(case, (GatherCase, StreamCase))
                            else case.attended_tokens()),
        "rotating_cache_copies": gpu.copies,
        "us_per_step": round(med * 1e3, 2),
        "us_per_step_p10": round(_pct(per, 10) * 1e3, 2),
        "us_per_step_p90": round(_pct(per, 90) * 1e3, 2),
        "timed_replays": R, "steps_per_replay": K,
        "step_bytes": step_bytes,
        "gbs_per_step": round(gbs, 1),
        "hbm_frac_per_step": round(gbs / HBM_PEAK_GBS, 4),
        "eager_us_per_step": round(eager_ms * 1e3, 2),
        "kernel": kernel,
        "kernel_avg_us": round(kavg * 1e3, 3),
        "kernel_p10_us": round(_pct(kms, 10) * 1e3, 3),
        "kernel_p90_us": round(_pct(kms, 90) * 1e3, 3),
        "kernel_bytes": dom_bytes,
        "kernel_gbs": round(kgbs, 1),
        "kernel_hbm_frac": round(kgbs / HBM_PEAK_GBS, 4),
        "kernel_traffic": None if case.args.set else measured_traffic(
            profile_name(case.name, case.bias), w.dtype, kernel),
        "parity": (check_outputs(case, out, oracle_res["outs"])
                   if oracle_res else None),
    }
    log(f"[bench] {case.name}: step {res['us_per_step']} us "
        f"(p10 {res['us_per_step_p10']}, p90 {res['us_per_step_p90']}), "
        f"{gbs:.1f} GB/s = {gbs / HBM_PEAK_GBS:.3f} of peak; kernel "
        f"{res['kernel_avg_us']} us, {kgbs:.1f} GB/s; parity "
        f"{res['parity']}")
    del gpu
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def profile_pass(torch, case, args):
    """Eager launches for counter collection: 2 warm-up steps, 6 more steps
    (the dispatches to read), then 3 plain copies of COPY_BYTES."""
    copies = _copies(args, (case.x["k"].numel() + case.x["v"].numel()) *
                     case.w.esz)
    gpu = case.gpu(copies)
    for r in range(2):
        gpu.step(r % gpu.copies)
    torch.cuda.synchronize()
    for i in range(6):
        gpu.step(i % gpu.copies)
    torch.cuda.synchronize()
    lib = bench_lib()
    src = torch.ones(COPY_BYTES, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        assert lib.gqa_bench_copy(dst.data_ptr(), src.data_ptr(), COPY_BYTES,
                                  256 * 16, _stream_handle(torch)) == 0
    torch.cuda.synchronize()
    step_bytes = gather_bytes(case, gpu) if isinstance(case, GatherCase) \
        else case.step_bytes()
    print(json.dumps({"profile_pass": case.w.name, "kernel": case.kernel(),
                      "kernel_algorithmic_bytes":
                          step_bytes - case.out_bytes(),
                      "copy_bytes": COPY_BYTES,
                      "source_sha256_16": partition_source_hash(case.w.dtype)}),
          flush=True)


def main(argv=None):
    args = parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not "
              "supported (the decode path needs no collectives).",
              file=sys.stderr)
        sys.exit(2)
    names = DEFAULT_SET if args.workload == "all" else [args.workload]
    if args.profile_pass and len(names) != 1:
        print("--profile-pass needs one --workload", file=sys.stderr)
        sys.exit(2)

    import torch
    # host phase: nothing here touches the GPU, so the oracle workers can be
    # forked from this process
    cases = {n: CASES[n](n, args) for n in names}
    oracle_res = {}
    if not args.no_cpu_baseline and not args.profile_pass:
        oracle_res = cpu_phase(cases, args)

    import gqa_kv_cache_decode_amd as g
    g.library()
    if args.profile_pass:
        profile_pass(torch, cases[names[0]], args)
        return

    per_workload = {}
    for n in names:
        per_workload[n] = gpu_phase(torch, cases[n], args, oracle_res.get(n))
        cases[n].x = None   # host copies are no longer needed

    ceiling = None
    if not args.no_ceiling:
        ceiling = read_ceiling(torch)
        log(f"[bench] pure-read stream ceiling: {ceiling:.1f} GB/s")
        for r in per_workload.values():
            r["step_frac_of_read_ceiling"] = round(r["gbs_per_step"] / ceiling,
                                                   4)
            r["kernel_frac_of_read_ceiling"] = round(r["kernel_gbs"] / ceiling,
                                                     4)

    head_name = HEADLINE if HEADLINE in per_workload else names[0]
    head = per_workload[head_name]
    hw = cases[head_name].w
    cpu = None
    if oracle_res:
        hr = oracle_res.get(head_name)
        per_cfg = {n: {"gbs": round(r["gbs"], 4), "cores": r["workers"],
                       "unit_evaluations": r["evaluations"],
                       "units_covered": len(r["outs"]),
                       "units": len(cases[n].units),
                       "wall_s": round(r["wall_s"], 2),
                       **({"one_thread_gbs": round(r["one_thread_gbs"], 4)}
                          if "one_thread_gbs" in r else {})}
                   for n, r in oracle_res.items()}
        if hr is not None:
            cpu = {"value": round(hr["gbs"], 4), "unit": "GB/s",
                   "cores": hr["workers"], "kind": "oracle",
                   "sample": (f"{hr['evaluations']} (sequence, KV group) unit "
                              f"evaluations of {hw.name} on the decode step's "
                              f"inputs ({len(hr['outs'])} of "
                              f"{len(cases[head_name].units)} units), fp64 "
                              f"numpy oracle, {hr['workers']} forked "
                              f"processes, {hr['wall_s']:.1f} s wall"),
                   "cpu_model": cpu_model(),
                   "per_config": per_cfg}
    value = head["gbs_per_step"]
    line = {
        "metric": METRIC, "value": value, "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(head["us_per_step"] / 1e3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        # fp8 codes are decoded to bf16 for the matrix cores
        "dtype": "bf16" if hw.dtype == "fp8" else hw.dtype,
        "data": "synthetic (seeded; shapes and distributions of the workload)",
        "config": {"workload": head["workload"], "batch": hw.batch,
                   "num_q_heads": hw.num_q_heads,
                   "num_kv_heads": hw.num_kv_heads, "dk": hw.dk, "dv": hw.dv,
                   "seq_len": hw.max_len, "window": hw.window,
                   "kv_dtype": head["kv_dtype"],
                   "additive_bias": bool(args.bias),
                   "timing": (f"median of {args.replays} timed replays of a "
                              f"HIP graph of K steps"),
                   "warm_graph_replays": WARM_REPLAYS},
        "us_per_step": head["us_per_step"],
        "us_per_step_p10": head["us_per_step_p10"],
        "us_per_step_p90": head["us_per_step_p90"],
        "hbm_frac_per_step": head["hbm_frac_per_step"],
        "read_ceiling_gbs": None if ceiling is None else round(ceiling, 1),
        "roofline": {"bound": "hbm", "achieved": head["kernel_gbs"],
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": head["kernel_hbm_frac"],
                     "traffic": head["kernel_traffic"],
                     "kernel": head["kernel"],
                     "algorithmic_bytes_per_launch": head["kernel_bytes"],
                     "avg_launch_us": head["kernel_avg_us"]},
        "cpu_baseline": cpu,
        "configs": per_workload,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
