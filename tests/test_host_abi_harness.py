"""The C ABI's host code (csrc/abi.cpp) under the address and undefined-
behaviour sanitizers, without a GPU: tests/host/abi_harness.cpp builds it
with stand-ins for the kernel launchers that check every launch against the
caller's buffers (inputs, outputs, workspace) at the extents its kernel
reads and writes, and calls every entry point on random shapes, from one
token to 2M-token caches and 9000-sequence batches.  The stand-ins answer
"is this head shape compiled" from the built library itself, and the
harness's plans are compared field by field with the built library's."""

import ctypes
import re
import shutil
import subprocess
from pathlib import Path

import pytest

from gqa_kv_cache_decode_amd import binding as bd

ROOT = Path(__file__).resolve().parents[1]
CSRC = ROOT / "gqa_kv_cache_decode_amd" / "csrc"
DIMS = [4, 8, 16, 32, 48, 60, 64, 96, 128, 192, 256, 260, 320, 512]


def _cache(dtype, B, T, hkv, dk, dv):
    sc = 0xB0000 if dtype == bd.FP8_E4M3 else None
    return bd._Cache(0x10000, 0x20000, B, T, hkv, dk, dv, dtype, sc, sc)


@pytest.fixture(scope="module")
def harness(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("no host C++ compiler")
    d = tmp_path_factory.mktemp("abi_harness")
    exe = d / "abi_harness"
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__",
           "-I/opt/rocm/include", f"-I{ROOT / 'include'}", f"-I{CSRC}",
           str(ROOT / "tests" / "host" / "abi_harness.cpp"),
           str(CSRC / "abi.cpp"), "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-4000:]
    # the head shapes the built library compiles, as its plan call reports
    lib = bd.library()
    rows = []
    for dt in (0, 1, bd.FP8_E4M3):  # fp32, bf16, fp8 (gqa_dtype)
        for dk in DIMS:
            for dv in DIMS:
                for hpk in range(1, 18):
                    c = _cache(dt, 1, 64, 1, dk, dv)
                    p = bd.Plan()
                    if lib.gqa_attend_plan(ctypes.byref(c), hpk, 0,
                                           ctypes.byref(p)) == 0:
                        rows.append(f"{dt} {dk} {dv} {hpk}")
    table = d / "support.txt"
    table.write_text("\n".join(rows) + "\n")
    return exe, table


def _run(harness, *args):
    exe, table = harness
    with open(table) as f:
        return subprocess.run([str(exe), *map(str, args)], stdin=f,
                              capture_output=True, text=True, timeout=600)


@pytest.mark.parametrize("seed", [7, 8])
def test_every_launch_stays_in_the_callers_buffers(harness, seed):
    r = _run(harness, "sweep", seed, 20000)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert "runtime error" not in r.stderr and "ERROR: AddressSanitizer" \
        not in r.stderr
    tail = r.stdout.strip().splitlines()
    m = re.fullmatch(r"calls (\d+) launches (\d+) refused (\d+) violations (\d+)",
                     tail[-1])
    assert m and int(m.group(3)) == 0 and int(m.group(4)) == 0, tail
    assert int(m.group(1)) > 100000 and int(m.group(2)) > 100000
    kinds = dict(zip(tail[-2].split()[1::2], map(int, tail[-2].split()[2::2])))
    # every launch form was exercised
    for k in ("balanced", "scheduled", "gathered", "branches", "steps",
              "fused", "direct"):
        assert kinds[k] > 0, (k, kinds)


def test_harness_plans_are_the_librarys(harness):
    """The harness's build of the planner (with stand-in support functions)
    plans exactly as the built library does."""
    r = _run(harness, "plans", 3, 4000)
    assert r.returncode == 0, r.stderr[-2000:]
    lib = bd.library()
    n = 0
    for line in r.stdout.splitlines():
        lhs, rhs = line.split(" -> ")
        dt, dk, dv, hpk, hkv, B, T, chunk = map(int, lhs.split())
        c = _cache(dt, B, T, hkv, dk, dv)
        p = bd.Plan()
        st = lib.gqa_attend_plan(ctypes.byref(c), hpk * hkv, chunk,
                                 ctypes.byref(p))
        got = [st]
        if st == 0:
            got += [p.chunk_tokens, p.num_chunks, p.off_l, p.off_acc,
                    p.off_sched, p.sched_entries, p.workspace_bytes,
                    p.balanced_groups]
        want = list(map(int, rhs.split()))
        if st != 0:
            want = want[:1]
        assert got == want, line
        n += 1
    assert n == 4000
