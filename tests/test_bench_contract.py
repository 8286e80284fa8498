"""bench.py's host-side contract, without a GPU: more than one GPU is refused
with a message, the default run covers the five workloads with the ragged
batch as the headline, the byte counts behind `value` and
`roofline.achieved` are the algorithmic ones, the recorded HBM traffic is
only reported for the kernel sources (and the kernel) it was measured on,
and the host phase's oracle units are the decode step's exact inputs."""

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
    name = profile[:-len("_bias")] if bias else profile
    case = bench.CASES[name].__new__(bench.CASES[name])
    case.w, case.bias = bench.workload_by_name(name), bias
    assert case.kernel() == rec["kernel"]


def test_default_run_is_the_five_workloads():
    args = bench.parse_args([])
    assert args.workload == "all"
    assert bench.DEFAULT_SET == ["tiny", "batched", "ragged", "long", "spike"]
    assert bench.HEADLINE == "ragged"
    names = [bench.workload_by_name(n).name for n in bench.DEFAULT_SET]
    assert names == [w.name for w in wl.WORKLOADS]


def _post_append(x, kn, vn):
    """The cache the decode step attends: the new token at slot lens - 1."""
    k, v = x["k"].clone(), x["v"].clone()
    for b, n in enumerate(x["lens"].tolist()):
        k[b, n - 1] = kn[b]
        v[b, n - 1] = vn[b]
    return k, v


@pytest.mark.parametrize("name", ["tiny", "batched"])
def test_host_oracle_units_are_the_step(name, monkeypatch):
    """The forked oracle workers evaluate every (sequence, KV group) unit of
    the step's inputs (the cache with the new token at its slot), and the
    output check scores a perfect answer as zero error."""
    import numpy as np
    import oracle
    args = bench.parse_args(["--workload", name])
    case = bench.CASES[name](name, args)
    if name == "batched":   # keep the test small: two sequences
        w = case.w.replace(batch=2, max_len=300)
        monkeypatch.setattr(bench, "workload_by_name", lambda n: w)
        case = bench.CASES[name](name, args)
    res = bench.run_oracle(case, 2, 0.5)
    assert len(res["outs"]) == len(case.units)
    k, v = _post_append(case.x, case.k_new, case.v_new)
    f64 = lambda t: t.float().numpy().astype(np.float64)
    ref, _ = oracle.attend(f64(case.x["q"]), f64(k), f64(v),
                           case.x["lens"].numpy(), case.w.scale)
    for (b, g), (o, vmax) in res["outs"].items():
        h = case.w.hpk
        assert np.array_equal(o, ref[b, g * h:(g + 1) * h])
    chk = bench.check_outputs(case, ref.astype(np.float32), res["outs"])
    assert chk["units_checked"] == len(case.units)
    assert chk["within_tolerance"] and chk["rel_l2"] < 1e-6
    bad = ref.astype(np.float32).copy()
    bad[0, 0, 0] += 1.0
    assert not bench.check_outputs(case, bad, res["outs"])["within_tolerance"]


def test_step_byte_accounting():
    """A step moves the attended K/V once per KV group (the cached part from
    the cache, the new token's rows read and written once each), q, the
    lengths and the fp32 output."""
    args = bench.parse_args(["--workload", "batched"])
    case = bench.SingleCase.__new__(bench.SingleCase)
    case.w, case.bias = wl.BATCHED_BF16, False
    import numpy as np
    case.lens = np.full(16, 4096)
    w = case.w
    kv = 16 * 4095 * 8 * 256 * 2
    new = 16 * 8 * 256 * (2 + 2)
    q = 16 * 32 * 128 * 2
    out = 16 * 32 * 128 * 4
    assert case.step_bytes() == kv + new + q + 2 * 16 * 4 + out


def test_source_hash_ignores_comments_only():
    a = "int f() { return 1; } // one\n/* a block\n   comment */\n"
    b = "int f()  {\n  return 1;\n}"
    assert bench.code_text(a) == bench.code_text(b)
    assert bench.code_text("int f() { return 2; }") != bench.code_text(b)


def test_kernel_names_follow_the_plan():
    """The ragged batch runs the balanced (work-queue) kernel, the other
    bf16 workloads the chunked one."""
    names = {n: bench.workload_by_name(n) for n in bench.DEFAULT_SET}
    assert bench.kernel_name(names["ragged"], False, False).startswith(
        "partition_balanced_kernel<128, 128, 2, true, false, false>")
    for n in ("batched", "spike"):
        assert bench.kernel_name(names[n], False, False).startswith(
            "partition_bf16_kernel<")
    assert bench.kernel_name(names["tiny"], False, False).startswith(
        "partition_f32_mfma_kernel<64, 64, 4, true")
    # the fp8 batched step: the shared-group launch at 128-wide heads, the
    # group split (eight KV groups per work-group) at 64-wide ones
    fp8 = bench.workload_by_name("fp8")
    assert bench.kernel_name(fp8, False, False) == (
        "partition_bf16_kernel<128, 128, 4, true, false, false, true>")
    assert bench.kernel_name(fp8.replace(dk=64, dv=64), False, False) == (
        "partition_split_kernel<64, 64, 8, true, false, true>")


def test_shape_overrides():
    """--set replaces integer shape fields, names the result after them, and
    rejects anything else."""
    args = bench.parse_args(["--workload", "tiny", "--set", "max_len=1024",
                             "--set", "batch=2"])
    w = bench.shaped_workload("tiny", args.set)
    base = bench.workload_by_name("tiny")
    assert (w.max_len, w.batch) == (1024, 2)
    assert w.name == base.name + "+max_len1024_batch2"
    assert w.replace(name=base.name, max_len=base.max_len, batch=base.batch) == base
    assert bench.shaped_workload("tiny", []) is base
    for bad in (["dtype=1"], ["dk=x"], ["scale=2"]):
        with pytest.raises(SystemExit):
            bench.shaped_workload("tiny", bad)
