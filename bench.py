#!/usr/bin/env python3
"""Decode-step benchmark of exact GQA decode attention on one MI355X.

One step is the whole hot path on one batch: kv_append of the new token, then
attend_decode (split-K partition + log-sum-exp combine) over the cache
including it; the long-context workload also folds its recent window in
through the carry.  Prints ONE JSON line on stdout; diagnostics go to stderr.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

The timed region replays a HIP graph of K steps with all inputs resident in
HBM.  Successive steps rotate over R copies of the cache (R * cache >= 1 GiB
where memory allows) so that each step streams from HBM rather than from the
256 MB last-level cache.
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import re
import sys
import time
import types
from pathlib import Path

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
           "step_common.h"]
PARTITION_SOURCES = {"bf16": ["partition_bf16.hip"] + _MFMA16,
                     "fp8": ["partition_fp8.hip"] + _MFMA16,
                     "f32": ["partition_f32.hip", "device_common.h", "launch.h",
                             "step_common.h"]}
COPY_BYTES = 256 << 20      # calibration copy for the byte counters
WARM_REPLAYS = 5            # untimed replays of the step graph before timing


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse_args():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=60)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="batched",
                   choices=["tiny", "batched", "ragged", "long", "spike",
                            "stream", "gather", "fp8"],
                   help="stream: the long-context shapes kept as 4 sink "
                        "keys + a 128-key window ring + a main cache; each "
                        "step appends (evicting the ring's oldest key into "
                        "main) and attends the three parts in one launch.  "
                        "gather: index-gathered decode of 2048 selected "
                        "slots (pools of 64) per sequence of a 32K cache.  "
                        "fp8: the batched shape over fp8 (E4M3) caches with "
                        "per-(sequence, KV head) scales")
    p.add_argument("--rotate", type=int, default=0,
                   help="cache copies to rotate over (0 = enough for 1 GiB)")
    p.add_argument("--cpu-seconds", type=float, default=15.0,
                   help="budget of the oracle's CPU-baseline timing")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-ceiling", action="store_true")
    p.add_argument("--bias", action="store_true",
                   help="attend with an additive logit bias (fp32 per "
                        "sequence and position, N(0, 1))")
    p.add_argument("--profile-pass", action="store_true",
                   help="no timing: a few eager partition launches and three "
                        f"{COPY_BYTES >> 20} MiB calibration copies, for "
                        "hardware-counter runs")
    return p.parse_args()


def workload_by_name(name):
    from gqa_kv_cache_decode_amd import workloads as wl
    return {"tiny": wl.TINY_F32, "batched": wl.BATCHED_BF16,
            "ragged": wl.RAGGED_BF16, "long": wl.LONG_WINDOW_BF16,
            "spike": wl.WIDE_SPIKE_BF16, "stream": wl.LONG_WINDOW_BF16,
            "gather": wl.GATHER_BF16, "fp8": wl.BATCHED_FP8}[name]


STREAM_SINK = 4            # permanent sink keys (cortiq-engine default)
STREAM_ROOM = 256          # free main slots, so the first steps grow main


class StreamState:
    """The long-context history kept as sink / window ring / main cache, R
    copies.  Main holds max_len - STREAM_SINK - window - STREAM_ROOM keys."""

    def __init__(self, g, torch, w, x, copies, dev):
        S, W, T = STREAM_SINK, w.window, w.max_len
        mn = T - S - W - STREAM_ROOM
        self.count0 = S + W + mn
        mk, mv = x["k"].to(dev), x["v"].to(dev)
        self.main = [(mk, mv)] + [(mk.clone(), mv.clone())
                                  for _ in range(copies - 1)]
        self.sink = [(m[0][:, :S].clone(), m[1][:, :S].clone())
                     for m in self.main]
        rk, rv = x["wk"].to(dev), x["wv"].to(dev)
        self.ring = [(rk.clone(), rv.clone()) for _ in range(copies)]
        B = w.batch
        i32 = lambda v: torch.full((B,), v, dtype=torch.int32, device=dev)
        self.count = [i32(self.count0) for _ in range(copies)]
        self.lens = [(i32(S), i32(W), i32(mn)) for _ in range(copies)]
        self.ws = torch.empty(g.library().gqa_attend_branches_workspace_bytes(
            self.branch_array(g, 0), 3, w.num_q_heads), dtype=torch.uint8,
            device=dev)
        self.plan = g.attend_plan(mk, mv, w.num_q_heads)
        self.pws = torch.empty(self.plan.workspace_bytes, dtype=torch.uint8,
                               device=dev)
        self.n_main = mn

    def branches(self, r):
        ls, lr, lm = self.lens[r]
        return [(*self.sink[r], ls), (*self.ring[r], lr), (*self.main[r], lm)]

    def branch_array(self, g, r):
        from gqa_kv_cache_decode_amd import binding as bd
        return bd._branches(self.branches(r), None)


def kv_bytes(w, lens_total, hkv=None):
    return lens_total * (hkv or w.num_kv_heads) * (w.dk + w.dv) * w.esz


def clone_cache(c):
    """A copy of a K or V cache (an fp8 cache keeps sharing its scales)."""
    from gqa_kv_cache_decode_amd import Fp8Cache
    if isinstance(c, Fp8Cache):
        return Fp8Cache(c.codes.clone(), c.scale)
    return c.clone()


class Branch:
    """One attend branch: R cache copies, lens before/after the append."""

    def __init__(self, g, torch, w, k, v, lens_after, copies, append,
                 bias=False, seed=0):
        self.w = w
        # optional additive bias, one fp32 term per (sequence, position)
        self.bias = None
        if bias:
            gen = torch.Generator().manual_seed(seed)
            pad = (k.shape[1] + 3) // 4 * 4
            self.bias = torch.randn(k.shape[0], pad, generator=gen).to(
                k.device)
        self.k = [k] + [clone_cache(k) for _ in range(copies - 1)]
        self.v = [v] + [clone_cache(v) for _ in range(copies - 1)]
        self.append = append
        self.lens_after = lens_after
        self.lens_before = (lens_after - 1).clamp_(min=0) if append else None
        self.lens_cur = [lens_after.clone() for _ in range(copies)]
        self.plan = g.attend_plan(self.k[0], self.v[0], w.num_q_heads)
        # decode_step's workspace (zero-filled once) also serves the plain
        # partition/combine calls: its head is the split-K partial area
        self.ws = g.step_workspace(self.k[0], self.v[0], w.num_q_heads)
        self.n_tot = int(lens_after.clamp(0, k.shape[1]).sum().item())


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not "
              "supported (the decode path needs no collectives).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import gqa_kv_cache_decode_amd as g
    from gqa_kv_cache_decode_amd import binding
    from gqa_kv_cache_decode_amd import workloads as wl

    w = workload_by_name(args.workload)
    fp8 = w.dtype == "fp8"
    t_gen = time.time()
    x = wl.make_fp8_inputs(w) if fp8 else wl.make_inputs(w)
    log(f"[bench] workload {w.name}: inputs drawn in {time.time() - t_gen:.1f}s")
    dev = torch.device("cuda")
    B, Hq, Hkv = w.batch, w.num_q_heads, w.num_kv_heads

    main_bytes = (x["k"].numel() + x["v"].numel()) * w.esz
    copies = args.rotate or max(1, min(8, math.ceil(ROTATE_TARGET_BYTES /
                                                    main_bytes)))
    q = x["q"].to(dev)
    gen = torch.Generator().manual_seed(w.seed + 1000)
    io_dt = torch.bfloat16 if fp8 else w.torch_dtype   # q and new rows
    k_new = torch.randn(B, Hkv, w.dk, generator=gen).to(io_dt).to(dev)
    v_new = torch.randn(B, Hkv, w.dv, generator=gen).to(io_dt).to(dev)
    out = torch.empty(B, Hq, w.dv, dtype=torch.float32, device=dev)

    stream = args.workload == "stream"
    gather = args.workload == "gather"
    branches = []
    if gather:
        # one cache; the steps rotate over index sets that select disjoint
        # enough rows (>= 1 GiB in all) that no step hits the 256 MB MALL
        gk, gv, glens = x["k"].to(dev), x["v"].to(dev), x["lens"].to(dev)
        sel_bytes = (w.batch * wl.GATHER_WIDTH * Hkv * (w.dk + w.dv) * w.esz)
        copies = args.rotate or max(1, min(16, math.ceil(ROTATE_TARGET_BYTES /
                                                         sel_bytes)))
        gidx, gsel = [], []
        for r in range(copies):
            rows = wl.make_index_rows(w, x["lens"], wl.GATHER_WIDTH,
                                      wl.GATHER_POOL, w.seed + 3000 + r)
            gidx.append(rows.to(dev))
            gsel.append(sum(len(set(rr.tolist()) - {-1}) for rr in rows))
        gws = torch.empty(binding.library().gqa_attend_gathered_workspace_bytes(
            ctypes.byref(binding._cache(gk, gv)), Hq, wl.GATHER_WIDTH),
            dtype=torch.uint8, device=dev)
        carry = None
    elif stream:
        st = StreamState(g, torch, w, x, copies, dev)
        carry = None
    elif w.window:
        # the long cache is attended as is; the new token enters the window
        branches.append(Branch(g, torch, w, x["k"].to(dev), x["v"].to(dev),
                               x["lens"].to(dev), copies, append=False,
                               bias=args.bias, seed=w.seed + 2000))
        branches.append(Branch(g, torch, w, x["wk"].to(dev), x["wv"].to(dev),
                               x["wlens"].to(dev), copies, append=True,
                               bias=args.bias, seed=w.seed + 2001))
        carry = g.empty_carry(B * Hq, w.dv)
    else:
        kc, vc = x["k"].to(dev), x["v"].to(dev)
        if fp8:
            kc = g.Fp8Cache(kc, x["k_scale"].to(dev))
            vc = g.Fp8Cache(vc, x["v_scale"].to(dev))
        branches.append(Branch(g, torch, w, kc, vc, x["lens"].to(dev), copies,
                               append=True, bias=args.bias,
                               seed=w.seed + 2000))
        carry = None
    del x
    torch.cuda.synchronize()
    if gather:
        log(f"[bench] {copies} rotating index sets over one cache of "
            f"{main_bytes / 2**30:.2f} GiB")
    else:
        log(f"[bench] {copies} rotating cache copies, "
            f"{main_bytes * copies / 2**30:.2f} GiB of K/V resident")

    def stream_step(r):
        """One streaming decode step: the new token enters the ring (its
        oldest key moving to main), then the three parts are attended in one
        partition launch and one combine."""
        g.stream_append(st.ring[r][0], st.ring[r][1], k_new, v_new,
                        st.count[r], count_out=st.count[r], sink=st.sink[r],
                        main=st.main[r], lens=st.lens[r])
        g.attend_branches(q, st.branches(r), w.scale, out=out,
                          workspace=st.ws)

    if w.window and not stream:
        # the long cache and the window taking the new token: one partition
        # launch over both branches, one combine folding their partials
        mb, wb = branches
        bws = torch.empty(g.library().gqa_attend_branches_workspace_bytes(
            binding._branches([(mb.k[0], mb.v[0], mb.lens_cur[0]),
                               (wb.k[0], wb.v[0], wb.lens_before)], None),
            2, Hq), dtype=torch.uint8, device=dev)

    def step(r):
        """One decode step: the branch holding the new token runs decode_step
        (append + attend, one launch where the partials fold in-kernel); with
        a long cache beside the window, both branches run in one
        decode_step_branches (two launches)."""
        if w.window:
            mb, wb = branches
            g.decode_step_branches(
                q, [(mb.k[r], mb.v[r], mb.lens_cur[r], mb.bias),
                    (wb.k[r], wb.v[r], wb.lens_before, wb.bias)], 1,
                k_new, v_new, wb.lens_cur[r], w.scale, out=out,
                workspace=bws)
            return
        for i, br in enumerate(branches):
            last = i == len(branches) - 1
            cin = carry if i > 0 else None
            cout = None if last else carry
            o = out if last else None
            if br.append:
                g.decode_step(q, br.k[r], br.v[r], k_new, v_new,
                              br.lens_before, br.lens_cur[r], w.scale,
                              carry_in=cin, carry_out=cout, out=o,
                              workspace=br.ws, bias=br.bias)
            else:
                g.attend_partition(q, br.k[r], br.v[r], br.lens_cur[r],
                                   br.plan, br.ws, w.scale, bias=br.bias)
                g.attend_combine(Hq, br.k[r], br.v[r], br.lens_cur[r],
                                 br.plan, br.ws, carry_in=cin,
                                 carry_out=cout, out=o)

    if gather:
        def gather_step(r):
            g.attend_gathered(q, gk, gv, glens, gidx[r], w.scale, out=out,
                              workspace=gws)
        step = gather_step
        # the whole call (selection, gathered partition, combine) is timed
        # as the dominant launch: there is no separate partition entry
        partition_only = gather_step
        dom = types.SimpleNamespace(n_tot=sum(gsel) // len(gsel), bias=None)
    elif stream:
        step = stream_step
        dom = types.SimpleNamespace(n_tot=B * st.n_main, bias=None)

        def partition_only(r):
            g.attend_partition(q, *st.main[r], st.lens[r][2], st.plan, st.pws,
                               w.scale)
    else:
        dom = branches[0]

        def partition_only(r):
            g.attend_partition(q, dom.k[r], dom.v[r], dom.lens_cur[r],
                               dom.plan, dom.ws, w.scale, bias=dom.bias)

    if args.profile_pass:
        profile_pass(torch, step, partition_only, copies, w, dom)
        return

    # warm up eagerly (also fixes lens_cur to the post-append lengths)
    for i in range(args.warmup):
        step(i % copies)
    torch.cuda.synchronize()

    def graph_of(fn, n):
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            fn(0)  # one eager call on the capture stream first
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            for i in range(n):
                fn(i % copies)
        torch.cuda.synchronize()
        return gr

    def time_graph(gr, n):
        """ms per step of one replay of a graph of n steps."""
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        gr.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    K = args.steps
    g_step = graph_of(step, K)
    # untimed replays of the whole graph: the first timed replay after a
    # single warm one ran ~8% slower (clocks still ramping on a fresh box)
    for _ in range(WARM_REPLAYS):
        g_step.replay()
    torch.cuda.synchronize()
    # the timed region: exactly K steps (one replay), synchronised on both sides
    ms_step = time_graph(g_step, K)

    # the dominant kernel alone: K eager launches queued back to back behind a
    # bounded spin kernel (so host launch latency never shows), one HIP event
    # pair on their stream around the whole batch; the average per launch
    # includes the dispatch gap between consecutive launches.
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    bench_lib().gqa_bench_spin(
        min(1000000, 20000 + 200 * K),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    e0.record()
    for i in range(K):
        partition_only(i % copies)
    e1.record()
    torch.cuda.synchronize()
    ms_part = e0.elapsed_time(e1) / K

    # eager reference timing of one step (diagnostic)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        step(i % copies)
    torch.cuda.synchronize()
    ms_eager = (time.perf_counter() - t0) * 1e3 / K

    # bytes
    q_bytes = B * Hq * w.dk * w.q_esz
    # fp8: the K and V scale of every (sequence, KV head), read per launch
    scale_bytes = 2 * B * Hkv * 4 if fp8 else 0
    out_bytes = B * Hq * w.dv * 4
    step_bytes = 0
    # a bias term counts once per attended (sequence, position)
    bias_bytes = (lambda br: 4 * br.n_tot if br.bias is not None else 0)
    for i, br in enumerate(branches):
        # q counts once per step (one launch reads it for every branch)
        step_bytes += kv_bytes(w, br.n_tot) + bias_bytes(br) + \
            (q_bytes if i == 0 else 0)
        if br.append:
            # the new rows read (bf16 for fp8 caches) and written, the lengths
            step_bytes += (B * Hkv * (w.dk + w.dv) * (w.q_esz + w.esz) +
                           2 * B * 4)
    if stream:
        # sink + ring + main keys, q once; the new row written, the evicted
        # row read and written; counts and the three lengths
        step_bytes += (kv_bytes(w, B * (STREAM_SINK + w.window + st.n_main)) +
                       q_bytes + 3 * B * Hkv * (w.dk + w.dv) * w.esz +
                       5 * B * 4)
    if gather:
        # the distinct selected rows (mean over the index sets), q, and the
        # index rows read by the selection kernel
        step_bytes += (kv_bytes(w, dom.n_tot) + q_bytes +
                       B * wl.GATHER_WIDTH * 4)
    step_bytes += out_bytes + scale_bytes
    part_bytes = kv_bytes(w, dom.n_tot) + q_bytes + bias_bytes(dom) + \
        scale_bytes
    value = step_bytes / (ms_step * 1e-3) / 1e9
    achieved = part_bytes / (ms_part * 1e-3) / 1e9
    log(f"[bench] step {ms_step * 1e3:.2f} us (graph), eager {ms_eager * 1e3:.1f}"
        f" us; partition {ms_part * 1e3:.2f} us; step bytes {step_bytes}; "
        f"{value:.1f} GB/s per step, partition {achieved:.1f} GB/s")

    ceiling = None
    if not args.no_ceiling:
        ceiling = read_ceiling(torch)
        log(f"[bench] pure-read stream ceiling: {ceiling:.1f} GB/s")

    traffic = measured_traffic(profile_name(args), w.dtype)
    kernel = kernel_name(w, args.bias, gather)
    if gather:
        kernel = f"attend_gathered call: select_kernel + {kernel} + combine"
    roofline = {"bound": "hbm", "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": traffic,
                "kernel": kernel,
                "algorithmic_bytes_per_launch": part_bytes,
                "avg_launch_us": round(ms_part * 1e3, 3)}

    cpu = None
    if not args.no_cpu_baseline:
        del branches, dom, g_step
        torch.cuda.empty_cache()
        cpu = cpu_baseline(w, args.cpu_seconds)

    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s",
        "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        # fp8 codes are decoded to bf16 for the matrix cores
        "dtype": "bf16" if fp8 else w.dtype,
        "data": "synthetic (seeded; shapes and distributions of the workload)",
        "config": {"workload": (f"stream_sink{STREAM_SINK}_ring{w.window}_"
                                f"main_of_{w.name}" if stream else w.name),
                   "selected_per_sequence": (wl.GATHER_WIDTH if gather
                                             else None),
                   "batch": B, "num_q_heads": Hq,
                   "num_kv_heads": Hkv, "dk": w.dk, "dv": w.dv,
                   "seq_len": w.max_len, "window": w.window,
                   "kv_dtype": "fp8_e4m3" if fp8 else w.dtype,
                   "rotating_cache_copies": copies,
                   "additive_bias": bool(args.bias),
                   "timing": "HIP graph of K steps",
                   "warm_graph_replays": WARM_REPLAYS},
        "us_per_step": round(ms_step * 1e3, 2),
        "hbm_frac_per_step": round(value / HBM_PEAK_GBS, 4),
        "eager_us_per_step": round(ms_eager * 1e3, 2),
        "read_ceiling_gbs": None if ceiling is None else round(ceiling, 1),
        # the same figures against the pure-read stream measured in this run
        "step_frac_of_read_ceiling": (None if ceiling is None
                                      else round(value / ceiling, 4)),
        "partition_frac_of_read_ceiling": (None if ceiling is None
                                           else round(achieved / ceiling, 4)),
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def kernel_name(w, bias, gather):
    """The dominant partition kernel's name as the profiler prints it
    (template arguments: head widths, wavefronts, decode step, bias,
    gathered, and fp8 for the bf16 / fp8 family)."""
    tf = lambda b: "true" if b else "false"
    flags = f"false, {tf(bias)}, {tf(gather)}"
    if w.dtype == "f32":
        return f"partition_f32_mfma_kernel<{w.dk}, {w.dv}, 4, {flags}>"
    if w.dtype == "fp8":
        waves = 8 if w.dk + w.dv <= 128 else 4
    else:
        waves = 2
    return (f"partition_bf16_kernel<{w.dk}, {w.dv}, {waves}, {flags}, "
            f"{tf(w.dtype == 'fp8')}>")


_BENCH_LIB = None


def bench_lib():
    """The measurement helpers (read stream, copy, spin) of libgqa_bench.so."""
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
        _BENCH_LIB = lib
    return _BENCH_LIB


def read_ceiling(torch, nbytes=4 << 30, reps=5):
    """A plain nontemporal 16-byte-vector read of 4 GiB: the HBM read rate
    reachable on this GPU (best of `reps`)."""
    lib = bench_lib()
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    blocks = 65536  # measured best for this kernel on MI355X
    sink = torch.zeros(blocks, dtype=torch.int32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    best = 0.0
    for _ in range(reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        rc = lib.gqa_bench_read_stream(buf.data_ptr(), nbytes, sink.data_ptr(),
                                       blocks, stream)
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


def profile_name(args):
    """Name of the workload's counter readings under profiles/."""
    return args.workload + ("_bias" if args.bias else "")


def measured_traffic(workload, dtype):
    """HBM bytes per partition launch from committed counter readings, if they
    were taken on the current kernel sources (else None)."""
    path = ROOT / "profiles" / f"traffic_{workload}.json"
    if not path.exists():
        return None
    rec = json.loads(path.read_text())
    if rec.get("partition_source_sha256_16") != partition_source_hash(dtype):
        return None
    return rec.get("traffic_bytes_per_launch")


def profile_pass(torch, step, partition_only, copies, w, dom):
    """Eager launches for counter collection: 2 warm-up steps, 6 partition
    launches (the dispatches to read), then 3 plain copies of COPY_BYTES."""
    for r in range(2):
        step(r % copies)
    torch.cuda.synchronize()
    for i in range(6):
        partition_only(i % copies)
    torch.cuda.synchronize()
    lib = bench_lib()
    src = torch.ones(COPY_BYTES, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for _ in range(3):
        assert lib.gqa_bench_copy(dst.data_ptr(), src.data_ptr(), COPY_BYTES,
                                  256 * 16, stream) == 0
    torch.cuda.synchronize()
    q_bytes = w.batch * w.num_q_heads * w.dk * w.q_esz
    b_bytes = 4 * dom.n_tot if dom.bias is not None else 0
    s_bytes = 2 * w.batch * w.num_kv_heads * 4 if w.dtype == "fp8" else 0
    print(json.dumps({"profile_pass": w.name,
                      "partition_algorithmic_bytes": kv_bytes(w, dom.n_tot) +
                      q_bytes + b_bytes + s_bytes, "copy_bytes": COPY_BYTES,
                      "source_sha256_16": partition_source_hash(w.dtype)}),
          flush=True)


def cpu_baseline(w, budget_s):
    """The oracle as it stands, on the host, one BLAS thread, over the (b, g)
    units of the same workload in a fixed shuffled order, repeated until the
    time budget is spent (a small workload is evaluated several times over)."""
    import numpy as np
    import oracle
    import oracle.fp8 as ofp8
    from gqa_kv_cache_decode_amd import workloads as wl
    from threadpoolctl import threadpool_limits
    fp8 = w.dtype == "fp8"
    x = wl.make_fp8_inputs(w) if fp8 else wl.make_inputs(w)
    hpk = w.hpk
    units = [(b, gg) for b in range(w.batch) for gg in range(w.num_kv_heads)]
    order = np.random.default_rng(0).permutation(len(units))
    done_bytes = 0
    done = 0
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        while time.perf_counter() - t0 <= budget_s:
            idx = order[done % len(units)]
            b, gg = units[idx]
            n = int(min(max(int(x["lens"][b]), 0), w.max_len))
            q = x["q"][b:b + 1, gg * hpk:(gg + 1) * hpk].float().numpy()
            if fp8:
                ofp8.attend_fp8(q, x["k"][b:b + 1, :n, gg:gg + 1].numpy(),
                                x["v"][b:b + 1, :n, gg:gg + 1].numpy(),
                                x["k_scale"][b:b + 1, gg:gg + 1].numpy(),
                                x["v_scale"][b:b + 1, gg:gg + 1].numpy(),
                                [n], w.scale)
            else:
                k = x["k"][b:b + 1, :n, gg:gg + 1].float().numpy()
                v = x["v"][b:b + 1, :n, gg:gg + 1].float().numpy()
                oracle.attend(q, k, v, [n], w.scale)
            done_bytes += (n * (w.dk + w.dv) * w.esz +
                           hpk * (w.dk * w.q_esz + w.dv * 4))
            done += 1
        el = time.perf_counter() - t0
    return {"value": round(done_bytes / el / 1e9, 4), "unit": "GB/s",
            "cores": 1, "kind": "oracle",
            "sample": f"{done} (sequence, KV group) unit evaluations "
                      f"({done / len(units):.2f} passes over the "
                      f"{len(units)} units) of {w.name}, fp64 numpy oracle"
                      f"{' (codes decoded in fp64)' if fp8 else ''}, "
                      f"1 thread, {el:.1f} s wall"}


if __name__ == "__main__":
    main()
