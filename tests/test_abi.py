"""The C ABI on the CPU: the library loads, exports every entry point the
header declares, and rejects bad arguments before any HIP call (every call
here fails validation, so nothing is launched)."""

import ctypes
import re
from pathlib import Path

import pytest

from gqa_kv_cache_decode_amd import binding as bd

ROOT = Path(__file__).resolve().parents[1]
HEADER = ROOT / "include" / "gqa_decode.h"

OK, INVALID, SHAPE, UNSUPPORTED, WORKSPACE, DEVICE = range(6)


@pytest.fixture(scope="module")
def lib():
    if not bd.LIB_PATH.exists():
        pytest.fail("libgqa_decode.so is not built (run the build first)")
    return bd.library()


def _declared():
    text = HEADER.read_text()
    return re.findall(r"GQA_API\s+[\w\s\*]+?\b(gqa_\w+)\s*\(", text)


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert len(names) == 19, names
    for n in names:
        assert hasattr(lib, n), f"missing export {n}"
    assert set(names) == set(bd._SIGNATURES), "binding covers the header"


def test_version_and_status_strings(lib):
    assert lib.gqa_abi_version() == 5
    names = [lib.gqa_status_string(i).decode() for i in range(7)]
    assert names == ["GQA_OK", "GQA_ERR_INVALID_ARGUMENT",
                     "GQA_ERR_SHAPE_MISMATCH", "GQA_ERR_UNSUPPORTED",
                     "GQA_ERR_WORKSPACE_TOO_SMALL", "GQA_ERR_DEVICE",
                     "GQA_ERR_UNKNOWN"]


def _cache(B=16, T=4096, H=8, dk=128, dv=128, dtype=1, k=0x10000, v=0x20000,
           ks=None, vs=None):
    return bd._Cache(k, v, B, T, H, dk, dv, dtype, ks, vs)


def _plan(lib, c, hq, chunk=0):
    p = bd.Plan()
    st = lib.gqa_attend_plan(ctypes.byref(c), hq, chunk, ctypes.byref(p))
    return st, p


def test_plan_layout(lib):
    c = _cache()
    st, p = _plan(lib, c, 32)
    assert st == OK
    assert p.chunk_tokens % 64 == 0 and p.chunk_tokens > 0
    assert p.num_chunks == -(-4096 // p.chunk_tokens)
    rows = 16 * 32
    ml = rows * p.num_chunks * 4
    up = lambda x: (x + 255) // 256 * 256
    assert p.off_l == up(ml) and p.off_acc == 2 * up(ml)
    assert p.workspace_bytes == 2 * up(ml) + up(ml * 128)
    assert lib.gqa_attend_workspace_bytes(ctypes.byref(c), 32) == \
        p.workspace_bytes
    st, p = _plan(lib, c, 32, chunk=320)
    assert st == OK and p.chunk_tokens == 320 and p.num_chunks == 13


@pytest.mark.parametrize("kw,hq,chunk,want", [
    (dict(), 30, 0, SHAPE),                 # Hq not a multiple of Hkv
    (dict(), 0, 0, INVALID),
    (dict(), 32, 100, INVALID),             # chunk not a multiple of 64
    (dict(), 32, -64, INVALID),
    (dict(B=0), 32, 0, INVALID),
    (dict(dtype=7), 32, 0, INVALID),
    (dict(dk=96, dv=96), 32, 0, UNSUPPORTED),  # no bf16 kernel for 96
    (dict(), 8 * 17, 0, UNSUPPORTED),       # 17 heads per KV head
    (dict(dtype=0, dk=512, dv=64), 32, 0, UNSUPPORTED),  # dk > 256
    (dict(dtype=0, dk=256, dv=256), 32, 0, OK),
    (dict(dtype=0, dk=96, dv=32), 32, 0, OK),
    (dict(dk=192, dv=128, H=4), 64, 0, OK),
    (dict(H=64, dk=256, dv=256, T=1 << 20), 64, 1 << 16, UNSUPPORTED),  # span
])
def test_plan_validation(lib, kw, hq, chunk, want):
    st, _ = _plan(lib, _cache(**kw), hq, chunk)
    assert st == want


def test_attend_rejects_before_launch(lib):
    c = _cache()
    hq = 32
    _, p = _plan(lib, c, hq)
    q, lens, ws, out = (ctypes.c_void_p(x) for x in
                        (0x30000, 0x40000, 0x50000, 0x60000))
    nbytes = p.workspace_bytes
    carry = bd._Carry(0x70000, 0x80000, 0x90000)

    def f(q_, hq_, c_, lens_, scale, cin, cout, out_, ws_, nbytes_, bias=None,
          stride=0):
        return lib.gqa_attend_decode(q_, hq_, ctypes.byref(c_), lens_, scale,
                                     bias, stride, cin, cout, out_, ws_,
                                     nbytes_, None)

    # null q, null lens
    assert f(None, hq, c, lens, 0.0, None, None, out, ws, nbytes) == INVALID
    assert f(q, hq, c, None, 0.0, None, None, out, ws, nbytes) == INVALID
    # neither out nor carry_out
    assert f(q, hq, c, lens, 0.0, None, None, None, ws, nbytes) == INVALID
    # non-finite scale
    for s in (float("nan"), float("inf")):
        assert f(q, hq, c, lens, s, None, None, out, ws, nbytes) == INVALID
    # misaligned q
    assert f(ctypes.c_void_p(0x30002), hq, c, lens, 0.0, None, None, out, ws,
             nbytes) == INVALID
    # workspace too small
    assert f(q, hq, c, lens, 0.0, None, None, out, ws, nbytes - 1) == WORKSPACE
    # a carry with a null member
    bad = bd._Carry(0x70000, None, 0x90000)
    assert f(q, hq, c, lens, 0.0, ctypes.byref(bad), None, out, ws,
             nbytes) == INVALID
    assert f(q, 30, c, lens, 0.0, ctypes.byref(carry), None, out, ws,
             nbytes) == SHAPE
    # the additive bias: short rows, a row stride not a multiple of 4, a
    # misaligned pointer; a well-formed one passes the checks (it is the
    # workspace size that is then wrong here)
    bias = ctypes.c_void_p(0xA0000)
    for ptr, stride in ((bias, c.max_len - 4), (bias, c.max_len + 2),
                        (ctypes.c_void_p(0xA0004), c.max_len)):
        assert f(q, hq, c, lens, 0.0, None, None, out, ws, nbytes, ptr,
                 stride) == INVALID
    assert f(q, hq, c, lens, 0.0, None, None, out, ws, nbytes - 1, bias,
             c.max_len) == WORKSPACE
    # null cache data
    c0 = _cache(k=0)
    assert f(q, hq, c0, lens, 0.0, None, None, out, ws, nbytes) == INVALID


def test_partition_combine_plan_checks(lib):
    c = _cache()
    _, p = _plan(lib, c, 32)
    q, lens, ws = (ctypes.c_void_p(x) for x in (0x30000, 0x40000, 0x50000))
    bad = bd.Plan(chunk_tokens=p.chunk_tokens, num_chunks=p.num_chunks + 1,
                  off_l=p.off_l, off_acc=p.off_acc, off_sched=p.off_sched,
                  sched_entries=p.sched_entries,
                  workspace_bytes=p.workspace_bytes)
    assert lib.gqa_attend_partition(q, 32, ctypes.byref(c), lens, 0.0, None,
                                    0, ctypes.byref(bad), ws,
                                    p.workspace_bytes, None) == SHAPE
    assert lib.gqa_attend_partition(q, 32, ctypes.byref(c), lens, 0.0, None,
                                    0, None, ws, p.workspace_bytes,
                                    None) == INVALID
    assert lib.gqa_attend_combine(32, ctypes.byref(c), lens, ctypes.byref(p),
                                  ws, p.workspace_bytes, None, None, None,
                                  None) == INVALID
    assert lib.gqa_attend_combine(32, ctypes.byref(c), lens, ctypes.byref(p),
                                  None, p.workspace_bytes, None, None,
                                  ctypes.c_void_p(0x60000), None) == INVALID


def test_append_and_merge_reject(lib):
    c = _cache()
    p = ctypes.c_void_p(0x30000)
    assert lib.gqa_kv_append(ctypes.byref(c), None, p, p, p, None, None) == \
        INVALID
    assert lib.gqa_kv_append(None, p, p, p, p, None, None) == INVALID
    assert lib.gqa_kv_append(ctypes.byref(_cache(T=0)), p, p, p, p, None,
                             None) == INVALID
    a = bd._Carry(0x10000, 0x20000, 0x30000)
    assert lib.gqa_softmax_state_merge(ctypes.byref(a), None, ctypes.byref(a),
                                       4, 8, None, None) == INVALID
    assert lib.gqa_softmax_state_merge(ctypes.byref(a), ctypes.byref(a),
                                       ctypes.byref(a), 0, 8, None, None) == \
        INVALID
    assert lib.gqa_softmax_state_merge(ctypes.byref(a), ctypes.byref(a),
                                       ctypes.byref(a), 4, 0, None, None) == \
        INVALID


def _branch(c, lens=0x40000, bias=None, stride=0):
    return bd._Branch(c, lens, bias, stride)


def test_branches_layout_and_checks(lib):
    """Multi-branch attend: per-branch chunking, one partial row over all
    branches' chunks, and the argument checks (before any launch)."""
    main = _cache(B=1, T=262144, H=4)
    win = _cache(B=1, T=128, H=4, k=0x30000, v=0x38000)
    arr = (bd._Branch * 2)(_branch(main), _branch(win, lens=0x48000))
    nbytes = lib.gqa_attend_branches_workspace_bytes(arr, 2, 32)
    # each branch chunked by its own plan; one partial row of 32 query rows
    # over both branches' chunks
    _, pm = _plan(lib, main, 32)
    _, pw = _plan(lib, win, 32)
    assert pm.num_chunks > 1 and pw.num_chunks == 1
    ml = 32 * (pm.num_chunks + pw.num_chunks) * 4
    al = lambda x: (x + 255) // 256 * 256
    assert nbytes == 2 * al(ml) + al(ml * 128)
    q, out, ws = (ctypes.c_void_p(x) for x in (0x50000, 0x60000, 0x70000))
    f = lib.gqa_attend_branches
    assert f(q, 32, arr, 2, 0.0, None, None, out, ws, nbytes - 1,
             None) == WORKSPACE
    # branch count outside 1..4
    assert f(q, 32, arr, 0, 0.0, None, None, out, ws, nbytes, None) == INVALID
    arr5 = (bd._Branch * 5)(*[_branch(main)] * 5)
    assert f(q, 32, arr5, 5, 0.0, None, None, out, ws, nbytes,
             None) == INVALID
    # branches must agree on batch, heads, widths and dtype
    for bad in (_cache(B=2, T=128, H=4), _cache(B=1, T=128, H=8),
                _cache(B=1, T=128, H=4, dv=64), _cache(B=1, T=128, H=4,
                                                       dtype=0)):
        arr_bad = (bd._Branch * 2)(_branch(main), _branch(bad))
        assert f(q, 32, arr_bad, 2, 0.0, None, None, out, ws, nbytes,
                 None) == SHAPE
    # the vector-ALU head widths are not supported here
    odd = _cache(B=1, T=128, H=4, dk=48, dv=80, dtype=0)
    arr_odd = (bd._Branch * 1)(_branch(odd))
    assert f(q, 32, arr_odd, 1, 0.0, None, None, out, ws, nbytes,
             None) == UNSUPPORTED
    # a branch with a null lens, a bad bias
    arr_nl = (bd._Branch * 2)(_branch(main), _branch(win, lens=None))
    assert f(q, 32, arr_nl, 2, 0.0, None, None, out, ws, nbytes,
             None) == INVALID
    arr_bb = (bd._Branch * 2)(_branch(main),
                              _branch(win, bias=0xA0000, stride=64))
    assert f(q, 32, arr_bb, 2, 0.0, None, None, out, ws, nbytes,
             None) == INVALID



def test_stream_append_checks(lib):
    """stream_append rejects bad layouts before any launch."""
    ring = _cache(B=4, T=128, H=2)
    sink = _cache(B=4, T=4, H=2, k=0x30000, v=0x38000)
    main = _cache(B=4, T=4096, H=2, k=0x40000, v=0x48000)
    p = [ctypes.c_void_p(0x50000 + 0x1000 * i) for i in range(8)]
    f = lib.gqa_stream_append

    def call(s_, r_, m_, ls=p[4], lm=p[6], kn=p[0]):
        return f(None if s_ is None else ctypes.byref(s_),
                 None if r_ is None else ctypes.byref(r_),
                 None if m_ is None else ctypes.byref(m_), kn, p[1], p[2],
                 p[3], ls, p[5], lm, None, None)

    assert call(sink, None, main) == INVALID              # no ring
    assert call(sink, ring, main, ls=None) == INVALID     # sink without lens
    assert call(sink, ring, main, lm=None) == INVALID     # main without lens
    assert call(sink, ring, main, kn=None) == INVALID
    assert call(sink, ring, main, kn=ctypes.c_void_p(0x50002)) == INVALID
    for bad in (_cache(B=5, T=4, H=2), _cache(B=4, T=4, H=1),
                _cache(B=4, T=4, H=2, dv=64), _cache(B=4, T=4, H=2, dtype=0)):
        assert call(bad, ring, main) == SHAPE
        assert call(None, ring, bad) == SHAPE
    odd = _cache(B=4, T=16, H=1, dk=3, dv=3)   # 6-byte rows
    assert call(None, odd, None) == UNSUPPORTED


def test_decode_step_branches_checks(lib):
    main = _cache(B=1, T=262144, H=4)
    win = _cache(B=1, T=128, H=4, k=0x30000, v=0x38000)
    arr = (bd._Branch * 2)(_branch(main), _branch(win, lens=0x48000))
    nbytes = lib.gqa_attend_branches_workspace_bytes(arr, 2, 32)
    q, kn, vn, lo, out, ws = (ctypes.c_void_p(x) for x in
                              (0x50000, 0x51000, 0x52000, 0x53000, 0x60000,
                               0x70000))
    f = lib.gqa_decode_step_branches

    def call(ab, lo_=lo, kn_=kn, n=nbytes):
        return f(q, 32, arr, 2, ab, kn_, vn, lo_, None, 0.0, None, None, out,
                 ws, n, None)

    assert call(2) == INVALID                       # no such branch
    assert call(-1) == INVALID
    assert call(1, lo_=ctypes.c_void_p(0x48000)) == INVALID  # lens_out = lens
    assert call(1, lo_=None) == INVALID
    assert call(1, kn_=ctypes.c_void_p(0x51004)) == INVALID  # misaligned
    assert call(1, n=nbytes - 1) == WORKSPACE


def test_gathered_checks(lib):
    c = _cache(B=4, T=8192, H=8)
    nbytes = lib.gqa_attend_gathered_workspace_bytes(ctypes.byref(c), 32, 2048)
    assert nbytes > 0
    assert lib.gqa_attend_gathered_workspace_bytes(ctypes.byref(c), 32, 0) == 0
    odd = _cache(B=4, T=8192, H=8, dk=48, dv=80, dtype=0)
    assert lib.gqa_attend_gathered_workspace_bytes(ctypes.byref(odd), 32,
                                                   64) == 0
    huge = _cache(B=1, T=(1 << 20) + 64, H=1)
    assert lib.gqa_attend_gathered_workspace_bytes(ctypes.byref(huge), 8,
                                                   64) == 0
    q, lens, idx, out, ws = (ctypes.c_void_p(x) for x in
                             (0x30000, 0x40000, 0x41000, 0x60000, 0x70000))
    f = lib.gqa_attend_gathered

    def call(c_, idx_=idx, width=2048, n=nbytes):
        return f(q, 32, ctypes.byref(c_), lens, idx_, width, 0.0, None, None,
                 out, ws, n, None)

    assert call(c, idx_=None) == INVALID
    assert call(c, width=0) == INVALID
    assert call(odd) == UNSUPPORTED
    assert call(huge) in (UNSUPPORTED, SHAPE)   # 8 q heads over 1 KV head ok
    assert call(c, n=nbytes - 1) == WORKSPACE


def test_fp8_checks(lib):
    """fp8 caches: the bf16 family's plan and shapes; scales required and
    4-byte aligned; no kernel for other head widths; stream_append needs
    the parts to share the scales, aligned bf16 rows and widths of 16;
    unknown dtypes rejected."""
    f8 = dict(dtype=bd.FP8_E4M3, ks=0xB0000, vs=0xB1000)
    c8 = _cache(**f8)
    _, p8 = _plan(lib, c8, 32)
    st, pb = _plan(lib, _cache(), 32)
    assert st == 0 and p8.chunk_tokens == pb.chunk_tokens and \
        p8.num_chunks == pb.num_chunks and \
        p8.workspace_bytes == pb.workspace_bytes, "same plan as bf16"
    q, lens, ws, out = (ctypes.c_void_p(x) for x in
                        (0x30000, 0x40000, 0x50000, 0x60000))

    def attend(c, nbytes=p8.workspace_bytes):
        return lib.gqa_attend_decode(q, 32, ctypes.byref(c), lens, 0.0, None,
                                     0, None, None, out, ws, nbytes, None)

    assert attend(c8, p8.workspace_bytes - 1) == WORKSPACE  # checks pass
    for bad in (_cache(dtype=bd.FP8_E4M3, ks=None, vs=0xB1000),
                _cache(dtype=bd.FP8_E4M3, ks=0xB0000, vs=None),
                _cache(dtype=bd.FP8_E4M3, ks=0xB0002, vs=0xB1000)):
        assert attend(bad) == INVALID
    assert attend(_cache(dtype=3)) == INVALID
    assert _plan(lib, _cache(dk=96, dv=96, **f8), 32)[0] == UNSUPPORTED
    assert _plan(lib, _cache(dk=128, dv=64, **f8), 32)[0] == UNSUPPORTED
    # kv_append: bf16 rows of an fp8 cache are read in 16-byte pieces
    pp = ctypes.c_void_p(0x30000)
    assert lib.gqa_kv_append(ctypes.byref(c8), ctypes.c_void_p(0x30008), pp,
                             pp, pp, None, None) == INVALID
    assert lib.gqa_kv_append(ctypes.byref(_cache(dtype=bd.FP8_E4M3)), pp, pp,
                             pp, pp, None, None) == INVALID   # no scales
    # stream_append over fp8 parts: the parts share the scales, the bf16 rows
    # are 16-byte aligned, the widths are multiples of 16
    ring = _cache(B=4, T=128, H=2, **f8)
    p = [ctypes.c_void_p(0x50000 + 0x1000 * i) for i in range(8)]
    sa = lib.gqa_stream_append
    other = _cache(B=4, T=64, H=2, k=0x60000, v=0x70000, dtype=bd.FP8_E4M3,
                   ks=0xC0000, vs=f8["vs"])
    assert sa(None, ctypes.byref(ring), ctypes.byref(other), p[0], p[1], p[2],
              p[3], None, p[5], p[6], None, None) == INVALID
    assert sa(ctypes.byref(other), ctypes.byref(ring), None, p[0], p[1], p[2],
              p[3], p[4], p[5], None, None, None) == INVALID
    assert sa(None, ctypes.byref(ring), None, ctypes.c_void_p(0x50008), p[1],
              p[2], p[3], None, p[5], None, None, None) == INVALID
    narrow = _cache(B=4, T=128, H=2, dk=72, dv=72, **f8)
    assert sa(None, ctypes.byref(narrow), None, p[0], p[1], p[2], p[3], None,
              p[5], None, None, None) == UNSUPPORTED
    # a branch of another dtype
    arr = (bd._Branch * 2)(_branch(c8), _branch(_cache()))
    assert lib.gqa_attend_branches_workspace_bytes(arr, 2, 32) == 0


def test_fp8_group_split_plan(lib):
    """fp8 chunking for the group split (64-wide heads: a work-group holds
    eight KV groups, a wavefront a whole chunk of its group): the chunk gives
    the split launch one round of one work-group per CU (256 to 511), with no
    schedule; other shapes keep the bf16 rule."""
    f8 = dict(dtype=bd.FP8_E4M3, ks=0xB0000, vs=0xB1000)
    d64 = dict(dk=64, dv=64)
    cases = [
        # (cache fields, hq, chunk, chunks): the batched fp8 shape with
        # 64-wide heads: eight wavefronts, eight groups per work-group
        (dict(B=16, T=4096, H=8, **d64), 32, 256, 16),
        # a test size that takes the split
        (dict(B=16, T=1100, H=8, **d64), 32, 64, 18),
    ]
    for kw, hq, chunk, n in cases:
        st, p = _plan(lib, _cache(**kw, **f8), hq)
        assert st == 0 and (p.chunk_tokens, p.num_chunks) == (chunk, n), kw
        assert p.sched_entries == 0 and p.balanced_groups == 0, kw
        assert 256 <= kw["B"] * kw["H"] * n // 8 < 512, kw
    # wider heads, too few work-groups, or KV heads that do not divide into
    # sets of eight: the bf16 rule
    for kw, hq in [(dict(B=16, T=4096, H=8), 32), (dict(B=8, T=2000, H=8), 32),
                   (dict(B=4, T=1500, H=8, **d64), 32),
                   (dict(B=16, T=4096, H=4, **d64), 16),
                   (dict(B=8, T=600, H=8, **d64), 32)]:
        _, p = _plan(lib, _cache(**kw, **f8), hq)
        _, pb = _plan(lib, _cache(**kw), hq)
        assert (p.chunk_tokens, p.num_chunks) == (pb.chunk_tokens,
                                                  pb.num_chunks), kw


def test_profile_request_validation(lib):
    """One event without the other is rejected; setting and cancelling a
    request makes no HIP call."""
    P = ctypes.c_void_p
    assert lib.gqa_profile_next_launch(P(0x1000), None) == INVALID
    assert lib.gqa_profile_next_launch(None, P(0x1000)) == INVALID
    assert lib.gqa_profile_next_launch(P(0x1000), P(0x2000)) == OK
    assert lib.gqa_profile_next_launch(None, None) == OK


def test_balanced_plan_layout(lib):
    """A bf16 / fp8 cache whose chunked launch would take several rounds of
    work-groups gets a balanced plan from the library (never from an
    explicit chunk length, never for fp32): 512 persistent work-groups, one
    piece slot of hpk rows per queue item (at most tiles * 0.0212 + 12 runs
    per sequence, times the KV heads), then the queue; every area 256-byte
    aligned and disjoint."""
    up = lambda x: (x + 255) // 256 * 256
    for dtype in (1, 2):
        ks = 0x30000 if dtype == 2 else None
        c = _cache(B=64, T=32768, H=8, dtype=dtype, ks=ks, vs=ks)
        st, p = _plan(lib, c, 64)
        assert st == OK and p.balanced_groups == 512
        runs = 64 * (1024 * 212 // 10000 + 12)
        items = runs * 8
        assert p.chunk_tokens == 32 and p.num_chunks == items
        hpk = 8
        ml = items * hpk * 4
        assert p.off_l == up(ml) and p.off_acc == 2 * up(ml)
        assert p.off_sched == p.off_acc + up(ml * 128)
        words = 6 + 3 * 65 + 3 * runs
        assert p.sched_entries == words
        assert p.workspace_bytes == p.off_sched + up(words * 4)
        assert lib.gqa_attend_workspace_bytes(ctypes.byref(c), 64) == \
            p.workspace_bytes
        # an explicit chunk length keeps the chunked (scheduled) plan
        st, q = _plan(lib, c, 64, chunk=2048)
        assert st == OK and q.balanced_groups == 0 and q.sched_entries > 0
    st, p = _plan(lib, _cache(B=64, T=32768, H=8, dtype=0), 64)
    assert st == OK and p.balanced_groups == 0 and p.sched_entries > 0
    # asked for explicitly: any bf16 / fp8 shape, never fp32
    st, p = _plan(lib, _cache(B=2, T=300, H=2), 4, chunk=-1)
    assert st == OK and p.balanced_groups == 512
    assert p.sched_entries == 6 + 3 * 3 + 3 * 2 * (10 * 212 // 10000 + 12)
    st, _ = _plan(lib, _cache(B=2, T=300, H=2, dtype=0), 4, chunk=-1)
    assert st == UNSUPPORTED
    st, _ = _plan(lib, _cache(B=2, T=300, H=2), 4, chunk=-2)
    assert st == INVALID
    # one round of work-groups: chunked, no schedule
    st, p = _plan(lib, _cache(), 32)
    assert st == OK and p.balanced_groups == 0 and p.sched_entries == 0


def test_balanced_plan_tampering_is_rejected(lib):
    """A balanced plan handed back with any field changed is refused before
    anything is enqueued."""
    c = _cache(B=64, T=32768, H=8)
    st, p = _plan(lib, c, 64)
    assert st == OK and p.balanced_groups
    P = ctypes.c_void_p
    for field, delta in (("balanced_groups", 8), ("off_sched", 256),
                         ("num_chunks", 2), ("chunk_tokens", 32)):
        bad = bd.Plan.from_buffer_copy(p)
        setattr(bad, field, getattr(bad, field) + delta)
        st = lib.gqa_attend_partition(P(0x40000), 64, ctypes.byref(c),
                                      P(0x50000), 0.0, None, 0,
                                      ctypes.byref(bad), P(0x60000),
                                      p.workspace_bytes, None)
        assert st == SHAPE, field


def test_noalloc_rejects_before_any_hip_call(lib):
    """The allocation-free attend_decode checks its arguments, and that its
    plan fits the library's 32 MiB scratch array, before any HIP call (so
    these run on a machine without a GPU)."""
    P = ctypes.c_void_p
    big = _cache(B=64, T=1 << 20, H=8, dtype=0)   # fp32 chunked: > 32 MiB
    assert lib.gqa_attend_workspace_bytes(ctypes.byref(big), 64) > 32 << 20
    out = P(0x70000)
    st = lib.gqa_attend_decode_noalloc(P(0x40000), 64, ctypes.byref(big),
                                       P(0x50000), 0.0, None, 0, None, None,
                                       out, None)
    assert st == WORKSPACE
    c = _cache()
    assert lib.gqa_attend_decode_noalloc(None, 32, ctypes.byref(c),
                                         P(0x50000), 0.0, None, 0, None, None,
                                         out, None) == INVALID
    assert lib.gqa_attend_decode_noalloc(P(0x40000), 30, ctypes.byref(c),
                                         P(0x50000), 0.0, None, 0, None, None,
                                         out, None) == SHAPE
    assert lib.gqa_attend_decode_noalloc(P(0x40000), 32, ctypes.byref(c),
                                         P(0x50000), float("nan"), None, 0,
                                         None, None, out, None) == INVALID
