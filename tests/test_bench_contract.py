"""bench.py's host-side contract, without a GPU: more than one GPU is refused
with a message, the byte counts behind `value` and `roofline.achieved` are
the algorithmic ones, the recorded HBM traffic is only reported for the
kernel sources it was measured on, and the kernel it names as dominant is
the one the committed counter readings were taken on."""

import json
import re
import subprocess
import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
sys.path.insert(0, str(ROOT))

import bench  # noqa: E402
from gqa_kv_cache_decode_amd import workloads as wl  # noqa: E402


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_is_refused(n):
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus",
                        str(n)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == "", "no JSON line for a refused run"


@pytest.mark.parametrize("w", wl.WORKLOADS + [wl.BATCHED_FP8],
                         ids=lambda w: w.name)
def test_byte_accounting(w):
    """K and V once per live token and KV group, at the stored width; the
    workload module's minimum adds q, the fp32 output and fp8 scales."""
    lens = [w.max_len] * w.batch
    n_tot = w.batch * w.max_len
    esz = {"f32": 4, "bf16": 2, "fp8": 1}[w.dtype]
    assert bench.kv_bytes(w, n_tot) == \
        n_tot * w.num_kv_heads * (w.dk + w.dv) * esz
    q = w.batch * w.num_q_heads * w.dk * (4 if w.dtype == "f32" else 2)
    out = w.batch * w.num_q_heads * w.dv * 4
    scales = 8 * w.batch * w.num_kv_heads if w.dtype == "fp8" else 0
    assert wl.algorithmic_bytes(w, lens) == \
        bench.kv_bytes(w, n_tot) + q + out + scales
    # lengths outside [0, max_len] count as clamped
    odd = [-5, w.max_len + 7] + [1] * (w.batch - 2) if w.batch > 2 else \
        [w.max_len + 7] * w.batch
    n_odd = sum(min(max(x, 0), w.max_len) for x in odd)
    assert wl.algorithmic_bytes(w, odd) == \
        bench.kv_bytes(w, n_odd) + q + out + scales


def test_traffic_only_for_the_measured_sources(tmp_path, monkeypatch):
    rec = {"partition_source_sha256_16": bench.partition_source_hash("bf16"),
           "traffic_bytes_per_launch": 12345}
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / "traffic_x.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", tmp_path)
    assert bench.measured_traffic("x", "bf16") == 12345
    # the same record read against another kernel family's sources
    assert bench.measured_traffic("x", "f32") is None
    rec["partition_source_sha256_16"] = "0" * 16
    (tmp_path / "profiles" / "traffic_x.json").write_text(json.dumps(rec))
    assert bench.measured_traffic("x", "bf16") is None
    assert bench.measured_traffic("missing", "bf16") is None


def test_source_hash_covers_the_kernel_sources():
    for dtype, names in bench.PARTITION_SOURCES.items():
        for n in names:
            assert (bench.CSRC / n).is_file(), f"{dtype}: {n}"
        assert re.fullmatch(r"[0-9a-f]{16}", bench.partition_source_hash(dtype))


@pytest.mark.parametrize("profile", sorted(
    p.stem[len("traffic_"):] for p in (ROOT / "profiles").glob("traffic_*.json")))
def test_dominant_kernel_name(profile):
    """The kernel bench.py labels as dominant is the one the committed
    counter readings of that workload were taken on."""
    rec = json.loads((ROOT / "profiles" / f"traffic_{profile}.json").read_text())
    bias = profile.endswith("_bias")
    w = bench.workload_by_name(profile[:-len("_bias")] if bias else profile)
    assert bench.kernel_name(w, bias, False) == rec["kernel"]


def test_source_hash_ignores_comments_only():
    a = "int f() { return 1; } // one\n/* a block\n   comment */\n"
    b = "int f()  {\n  return 1;\n}"
    assert bench.code_text(a) == bench.code_text(b)
    assert bench.code_text("int f() { return 2; }") != bench.code_text(b)
