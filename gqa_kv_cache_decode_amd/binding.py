"""ctypes binding of libgqa_decode.so (include/gqa_decode.h).

Argument marshalling only: torch tensors become device pointers and sizes, and
every call is enqueued on torch's current HIP stream.  All compute happens in
the library's HIP kernels.  A missing library raises ``GqaError`` at the first
call; there is no other path.
"""

from __future__ import annotations

import ctypes
import dataclasses
import math
from pathlib import Path
from typing import Optional

import torch

LIB_PATH = Path(__file__).resolve().with_name("libgqa_decode.so")

DTYPE_CODES = {torch.float32: 0, torch.bfloat16: 1}
FP8_E4M3 = 2                       # gqa_dtype of an Fp8Cache
CHUNK_BALANCED = -1                # GQA_CHUNK_BALANCED: attend_plan asks for
                                   # a balanced plan
FP8_STORAGE = (torch.uint8, torch.float8_e4m3fn)


class GqaError(RuntimeError):
    """A failed library call (the status name is in the message)."""


class _Cache(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("batch", ctypes.c_int32), ("max_len", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("dk", ctypes.c_int32),
                ("dv", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p)]


class _Carry(ctypes.Structure):
    _fields_ = [("m", ctypes.c_void_p), ("l", ctypes.c_void_p),
                ("acc", ctypes.c_void_p)]


class _Branch(ctypes.Structure):
    _fields_ = [("cache", _Cache), ("lens", ctypes.c_void_p),
                ("bias", ctypes.c_void_p), ("bias_stride", ctypes.c_int64)]


class Plan(ctypes.Structure):
    """gqa_plan: split-K chunking and workspace layout of one attend call."""

    _fields_ = [("chunk_tokens", ctypes.c_int32), ("num_chunks", ctypes.c_int32),
                ("off_l", ctypes.c_size_t), ("off_acc", ctypes.c_size_t),
                ("off_sched", ctypes.c_size_t), ("sched_entries", ctypes.c_int32),
                ("workspace_bytes", ctypes.c_size_t),
                ("balanced_groups", ctypes.c_int32)]


_lib = None
_AUTO = object()   # default of ``out``: allocate one (None means "no output")
_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_CACHE_P = ctypes.POINTER(_Cache)
_CARRY_P = ctypes.POINTER(_Carry)
_PLAN_P = ctypes.POINTER(Plan)

_BRANCH_P = ctypes.POINTER(_Branch)

_SIGNATURES = {
    "gqa_attend_gathered_workspace_bytes": (ctypes.c_size_t,
                                            [_CACHE_P, _I32, _I32]),
    "gqa_attend_gathered": (_I32, [_P, _I32, _CACHE_P, _P, _P, _I32,
                                   ctypes.c_float, _CARRY_P, _CARRY_P, _P, _P,
                                   ctypes.c_size_t, _P]),
    "gqa_decode_step_branches": (_I32, [_P, _I32, _BRANCH_P, _I32, _I32, _P,
                                        _P, _P, _P, ctypes.c_float, _CARRY_P,
                                        _CARRY_P, _P, _P, ctypes.c_size_t,
                                        _P]),
    "gqa_stream_append": (_I32, [_CACHE_P, _CACHE_P, _CACHE_P, _P, _P, _P, _P,
                                 _P, _P, _P, _P, _P]),
    "gqa_attend_branches_workspace_bytes": (ctypes.c_size_t,
                                            [_BRANCH_P, _I32, _I32]),
    "gqa_attend_branches": (_I32, [_P, _I32, _BRANCH_P, _I32, ctypes.c_float,
                                   _CARRY_P, _CARRY_P, _P, _P,
                                   ctypes.c_size_t, _P]),
    "gqa_abi_version": (_I32, []),
    "gqa_profile_next_launch": (_I32, [_P, _P]),
    "gqa_status_string": (ctypes.c_char_p, [_I32]),
    "gqa_kv_append": (_I32, [_CACHE_P, _P, _P, _P, _P, _P, _P]),
    "gqa_attend_plan": (_I32, [_CACHE_P, _I32, _I32, _PLAN_P]),
    "gqa_attend_workspace_bytes": (ctypes.c_size_t, [_CACHE_P, _I32]),
    "gqa_attend_decode": (_I32, [_P, _I32, _CACHE_P, _P, ctypes.c_float,
                                 _P, ctypes.c_int64, _CARRY_P, _CARRY_P, _P,
                                 _P, ctypes.c_size_t, _P]),
    "gqa_attend_decode_noalloc": (_I32, [_P, _I32, _CACHE_P, _P,
                                         ctypes.c_float, _P, ctypes.c_int64,
                                         _CARRY_P, _CARRY_P, _P, _P]),
    "gqa_attend_partition": (_I32, [_P, _I32, _CACHE_P, _P, ctypes.c_float,
                                    _P, ctypes.c_int64, _PLAN_P, _P,
                                    ctypes.c_size_t, _P]),
    "gqa_attend_combine": (_I32, [_I32, _CACHE_P, _P, _PLAN_P, _P,
                                  ctypes.c_size_t, _CARRY_P, _CARRY_P, _P, _P]),
    "gqa_softmax_state_merge": (_I32, [_CARRY_P, _CARRY_P, _CARRY_P,
                                       ctypes.c_int64, _I32, _P, _P]),
    "gqa_decode_step_workspace_bytes": (ctypes.c_size_t, [_CACHE_P, _I32]),
    "gqa_decode_step": (_I32, [_P, _I32, _CACHE_P, _P, _P, _P, _P, _P,
                               ctypes.c_float, _P, ctypes.c_int64, _CARRY_P,
                               _CARRY_P, _P, _P, ctypes.c_size_t, _P]),
}


def library() -> ctypes.CDLL:
    """Load libgqa_decode.so (once) and declare its signatures."""
    global _lib
    if _lib is None:
        if not LIB_PATH.exists():
            raise GqaError(
                f"{LIB_PATH} is not built: run "
                "`python -m gqa_kv_cache_decode_amd.build` (needs hipcc)")
        lib = ctypes.CDLL(str(LIB_PATH))
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _check(status: int, what: str) -> None:
    if status != 0:
        name = library().gqa_status_string(status).decode()
        raise GqaError(f"{what}: {name}")


def _stream(t: torch.Tensor) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t: torch.Tensor, name: str, dtype=None, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise GqaError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise GqaError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise GqaError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise GqaError(f"{name} must have shape {tuple(shape)}, got "
                       f"{tuple(t.shape)}")


@dataclasses.dataclass
class Fp8Cache:
    """An fp8 K or V cache: ``codes`` [B, max_len, Hkv, d] (torch.uint8 or
    torch.float8_e4m3fn holding OCP E4M3 codes) and fp32 ``scale`` [B, Hkv]
    on the GPU; code c of KV head g of sequence b stands for
    decode(c) * scale[b, g].  Goes wherever a k_cache / v_cache tensor goes;
    queries and new K/V rows are then bf16."""

    codes: torch.Tensor
    scale: torch.Tensor

    @property
    def device(self):
        return self.codes.device

    @property
    def shape(self):
        return self.codes.shape


def _io_dtype(cache) -> torch.dtype:
    """dtype of the queries and new rows that go with a cache."""
    return torch.bfloat16 if isinstance(cache, Fp8Cache) else cache.dtype


def _fp8_cache(k: Fp8Cache, v: Fp8Cache) -> _Cache:
    if not (isinstance(k, Fp8Cache) and isinstance(v, Fp8Cache)):
        raise GqaError("K and V caches must both be Fp8Cache, or neither")
    for t, name in ((k.codes, "k_cache.codes"), (v.codes, "v_cache.codes")):
        _need(t, name)
        if t.dtype not in FP8_STORAGE:
            raise GqaError(f"{name} must be uint8 or float8_e4m3fn codes")
    kc, vc = k.codes, v.codes
    if kc.dim() != 4 or vc.dim() != 4 or kc.shape[:3] != vc.shape[:3]:
        raise GqaError("caches must be [batch, max_len, num_kv_heads, d] with "
                       "matching batch, max_len and heads")
    B, T, H, dk = kc.shape
    _need(k.scale, "k_cache.scale", torch.float32, (B, H))
    _need(v.scale, "v_cache.scale", torch.float32, (B, H))
    return _Cache(kc.data_ptr(), vc.data_ptr(), B, T, H, dk, vc.shape[3],
                  FP8_E4M3, k.scale.data_ptr(), v.scale.data_ptr())


def _cache(k, v) -> _Cache:
    if isinstance(k, Fp8Cache) or isinstance(v, Fp8Cache):
        return _fp8_cache(k, v)
    _need(k, "k_cache")
    _need(v, "v_cache", dtype=k.dtype)
    if k.dtype not in DTYPE_CODES:
        raise GqaError(f"cache dtype {k.dtype} is not supported")
    if k.dim() != 4 or v.dim() != 4 or k.shape[:3] != v.shape[:3]:
        raise GqaError("caches must be [batch, max_len, num_kv_heads, d] with "
                       "matching batch, max_len and heads")
    B, T, H, dk = k.shape
    return _Cache(k.data_ptr(), v.data_ptr(), B, T, H, dk, v.shape[3],
                  DTYPE_CODES[k.dtype], None, None)


@dataclasses.dataclass
class Carry:
    """Online-softmax carry: m [rows], l [rows], acc [rows, dv] (fp32)."""

    m: torch.Tensor
    l: torch.Tensor
    acc: torch.Tensor

    def _struct(self, rows: int, dv: int, name: str) -> _Carry:
        _need(self.m, name + ".m", torch.float32, (rows,))
        _need(self.l, name + ".l", torch.float32, (rows,))
        _need(self.acc, name + ".acc", torch.float32, (rows, dv))
        return _Carry(self.m.data_ptr(), self.l.data_ptr(), self.acc.data_ptr())


def empty_carry(rows: int, dv: int, device="cuda") -> Carry:
    return Carry(torch.full((rows,), -math.inf, device=device),
                 torch.zeros(rows, device=device),
                 torch.zeros(rows, dv, device=device))


def kv_append(k_cache, v_cache, k_new, v_new, lens, lens_out=None,
              dropped=None):
    """Append one token per sequence (needle-core KvCache::push_kv).

    k_new [B, Hkv, dk], v_new [B, Hkv, dv] in the cache dtype (bf16 for an
    Fp8Cache, quantised on the way in); lens [B] int32.  Writes lens_out
    (default: lens itself, updated in place); a full cache is left untouched
    and counted in ``dropped`` (int32 [1]) if given."""
    c = _cache(k_cache, v_cache)
    io = _io_dtype(k_cache)
    _need(k_new, "k_new", io, (c.batch, c.num_kv_heads, c.dk))
    _need(v_new, "v_new", io, (c.batch, c.num_kv_heads, c.dv))
    _need(lens, "lens", torch.int32, (c.batch,))
    if lens_out is None:
        lens_out = lens
    _need(lens_out, "lens_out", torch.int32, (c.batch,))
    if dropped is not None:
        _need(dropped, "dropped", torch.int32, (1,))
    _check(library().gqa_kv_append(ctypes.byref(c), _ptr(k_new), _ptr(v_new),
                                   _ptr(lens), _ptr(lens_out), _ptr(dropped),
                                   _stream(k_cache)), "kv_append")
    return lens_out


def attend_plan(k_cache, v_cache, num_q_heads: int, chunk_tokens: int = 0) -> Plan:
    c = _cache(k_cache, v_cache)
    p = Plan()
    _check(library().gqa_attend_plan(ctypes.byref(c), num_q_heads, chunk_tokens,
                                     ctypes.byref(p)), "attend_plan")
    return p


def workspace_bytes(k_cache, v_cache, num_q_heads: int) -> int:
    c = _cache(k_cache, v_cache)
    return int(library().gqa_attend_workspace_bytes(ctypes.byref(c),
                                                    num_q_heads))


def _workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 16), dtype=torch.uint8, device=device)


def _attend_args(q, k_cache, v_cache, lens):
    c = _cache(k_cache, v_cache)
    _need(q, "q", _io_dtype(k_cache))
    if q.dim() != 3 or q.shape[0] != c.batch or q.shape[2] != c.dk:
        raise GqaError(f"q must be [batch={c.batch}, num_q_heads, dk={c.dk}]")
    _need(lens, "lens", torch.int32, (c.batch,))
    return c, q.shape[1]


def _bias(c, bias):
    """(pointer, row stride) of an optional additive logit bias: fp32
    [batch, >= max_len] on the GPU with unit column stride (its row stride is
    passed as is: a multiple of 4, 16-byte aligned rows)."""
    if bias is None:
        return None, 0
    if not isinstance(bias, torch.Tensor) or not bias.is_cuda:
        raise GqaError("bias must be a GPU tensor")
    if bias.dtype != torch.float32 or bias.dim() != 2:
        raise GqaError("bias must be fp32 [batch, positions]")
    if bias.shape[0] != c.batch or bias.shape[1] < c.max_len or \
            bias.stride(1) != 1:
        raise GqaError(f"bias must be [batch={c.batch}, >= max_len="
                       f"{c.max_len}] with unit column stride")
    return ctypes.c_void_p(bias.data_ptr()), int(bias.stride(0))


def _carries(c, hq, carry_in, carry_out, out):
    rows = c.batch * hq
    cin = None if carry_in is None else carry_in._struct(rows, c.dv, "carry_in")
    cout = None if carry_out is None else carry_out._struct(rows, c.dv,
                                                            "carry_out")
    if out is not None:
        _need(out, "out", torch.float32, (c.batch, hq, c.dv))
    return (None if cin is None else ctypes.byref(cin),
            None if cout is None else ctypes.byref(cout))


def attend_decode(q, k_cache, v_cache, lens, scale: float = 0.0,
                  carry_in: Optional[Carry] = None,
                  carry_out: Optional[Carry] = None,
                  out=_AUTO,
                  workspace: Optional[torch.Tensor] = None, bias=None):
    """Exact GQA decode attention: q [B, Hq, dk] over the caches.

    Returns ``out`` [B, Hq, dv] fp32: allocated unless given; pass
    ``out=None`` together with ``carry_out`` to get the carry only.
    ``bias``: optional fp32 [B, >= max_len] additive logit terms."""
    c, hq = _attend_args(q, k_cache, v_cache, lens)
    bp, bs = _bias(c, bias)
    if out is _AUTO:
        out = torch.empty(c.batch, hq, c.dv, dtype=torch.float32,
                          device=q.device)
    cin, cout = _carries(c, hq, carry_in, carry_out, out)
    need = library().gqa_attend_workspace_bytes(ctypes.byref(c), hq)
    if workspace is None:
        workspace = _workspace(need, q.device)
    _need(workspace, "workspace")
    _check(library().gqa_attend_decode(
        _ptr(q), hq, ctypes.byref(c), _ptr(lens), float(scale), bp, bs, cin,
        cout,
        _ptr(out), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(q)), "attend_decode")
    return out


def attend_decode_noalloc(q, k_cache, v_cache, lens, scale: float = 0.0,
                          carry_in: Optional[Carry] = None,
                          carry_out: Optional[Carry] = None, out=_AUTO,
                          bias=None):
    """attend_decode on the library's own device scratch array (no
    workspace argument): for callers that cannot allocate.  ``out`` as in
    attend_decode (pass an existing tensor to allocate nothing here)."""
    c, hq = _attend_args(q, k_cache, v_cache, lens)
    bp, bs = _bias(c, bias)
    if out is _AUTO:
        out = torch.empty(c.batch, hq, c.dv, dtype=torch.float32,
                          device=q.device)
    cin, cout = _carries(c, hq, carry_in, carry_out, out)
    _check(library().gqa_attend_decode_noalloc(
        _ptr(q), hq, ctypes.byref(c), _ptr(lens), float(scale), bp, bs, cin,
        cout, _ptr(out), _stream(q)), "attend_decode_noalloc")
    return out


def attend_partition(q, k_cache, v_cache, lens, plan: Plan,
                     workspace: torch.Tensor, scale: float = 0.0,
                     bias=None) -> None:
    """Split-K partials of every live (query row, chunk) into ``workspace``."""
    c, hq = _attend_args(q, k_cache, v_cache, lens)
    bp, bs = _bias(c, bias)
    _need(workspace, "workspace")
    _check(library().gqa_attend_partition(
        _ptr(q), hq, ctypes.byref(c), _ptr(lens), float(scale), bp, bs,
        ctypes.byref(plan), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(q)),
        "attend_partition")


def attend_combine(num_q_heads: int, k_cache, v_cache, lens, plan: Plan,
                   workspace: torch.Tensor, carry_in: Optional[Carry] = None,
                   carry_out: Optional[Carry] = None,
                   out=_AUTO):
    """Fold the partials (and carry_in) into ``out`` and/or ``carry_out``;
    ``out`` is allocated unless given (None: carry only)."""
    c = _cache(k_cache, v_cache)
    _need(lens, "lens", torch.int32, (c.batch,))
    _need(workspace, "workspace")
    if out is _AUTO:
        out = torch.empty(c.batch, num_q_heads, c.dv, dtype=torch.float32,
                          device=lens.device)
    cin, cout = _carries(c, num_q_heads, carry_in, carry_out, out)
    _check(library().gqa_attend_combine(
        num_q_heads, ctypes.byref(c), _ptr(lens), ctypes.byref(plan),
        _ptr(workspace), workspace.numel() * workspace.element_size(), cin,
        cout, _ptr(out), _stream(lens)), "attend_combine")
    return out


def step_workspace(k_cache, v_cache, num_q_heads: int) -> torch.Tensor:
    """A zero-filled workspace for decode_step (reusable across steps)."""
    c = _cache(k_cache, v_cache)
    n = library().gqa_decode_step_workspace_bytes(ctypes.byref(c), num_q_heads)
    if n == 0:
        raise GqaError("decode_step: unsupported shape")
    return torch.zeros(n, dtype=torch.uint8, device=k_cache.device)


def decode_step(q, k_cache, v_cache, k_new, v_new, lens_in, lens_out,
                scale: float = 0.0, carry_in: Optional[Carry] = None,
                carry_out: Optional[Carry] = None, out=_AUTO,
                workspace: Optional[torch.Tensor] = None, dropped=None,
                bias=None):
    """kv_append of (k_new, v_new) then attend_decode, as one step.

    lens_out must be a different tensor from lens_in.  ``workspace`` must come
    from :func:`step_workspace` (zero-filled once, then reused)."""
    c, hq = _attend_args(q, k_cache, v_cache, lens_in)
    bp, bs = _bias(c, bias)
    io = _io_dtype(k_cache)
    _need(k_new, "k_new", io, (c.batch, c.num_kv_heads, c.dk))
    _need(v_new, "v_new", io, (c.batch, c.num_kv_heads, c.dv))
    _need(lens_out, "lens_out", torch.int32, (c.batch,))
    if dropped is not None:
        _need(dropped, "dropped", torch.int32, (1,))
    if out is _AUTO:
        out = torch.empty(c.batch, hq, c.dv, dtype=torch.float32,
                          device=q.device)
    cin, cout = _carries(c, hq, carry_in, carry_out, out)
    if workspace is None:
        workspace = step_workspace(k_cache, v_cache, hq)
    _need(workspace, "workspace")
    _check(library().gqa_decode_step(
        _ptr(q), hq, ctypes.byref(c), _ptr(k_new), _ptr(v_new), _ptr(lens_in),
        _ptr(lens_out), _ptr(dropped), float(scale), bp, bs, cin, cout,
        _ptr(out),
        _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(q)), "decode_step")
    return out


def softmax_state_merge(a: Carry, b: Carry, dst: Optional[Carry] = None,
                        out: Optional[torch.Tensor] = None) -> Carry:
    """dst = merge(a, b) row by row; ``out`` (optional) gets acc / l."""
    rows, dv = a.acc.shape
    if dst is None:
        dst = Carry(torch.empty_like(a.m), torch.empty_like(a.l),
                    torch.empty_like(a.acc))
    sa, sb, sd = (x._struct(rows, dv, n) for x, n in
                  ((a, "a"), (b, "b"), (dst, "dst")))
    if out is not None:
        _need(out, "out", torch.float32)
        if out.numel() != rows * dv:
            raise GqaError("out must hold rows * dv elements")
    _check(library().gqa_softmax_state_merge(
        ctypes.byref(sa), ctypes.byref(sb), ctypes.byref(sd), rows, dv,
        _ptr(out), _stream(a.m)), "softmax_state_merge")
    return dst


def _branches(branches, q):
    """ctypes array of gqa_branch from (k, v, lens[, bias]) tuples (a bias
    of None means none)."""
    if not 1 <= len(branches) <= 4:
        raise GqaError("attend_branches takes 1 to 4 branches")
    arr = (_Branch * len(branches))()
    for i, br in enumerate(branches):
        k, v, lens = br[:3]
        bias = br[3] if len(br) > 3 else None
        c = _cache(k, v)
        _need(lens, f"branch {i} lens", torch.int32, (c.batch,))
        bp, bs = _bias(c, bias)
        arr[i] = _Branch(c, lens.data_ptr(), bp, bs)
    return arr


def attend_branches(q, branches, scale: float = 0.0,
                    carry_in: Optional[Carry] = None,
                    carry_out: Optional[Carry] = None, out=_AUTO,
                    workspace: Optional[torch.Tensor] = None):
    """Attention of q over the union of several caches' live keys, one
    partition launch and one combine.  ``branches``: a list of
    (k_cache, v_cache, lens) or (k_cache, v_cache, lens, bias) tuples with the
    same batch, KV heads, head widths and dtype."""
    arr = _branches(branches, q)
    k0 = branches[0][0]
    c0, hq = _attend_args(q, k0, branches[0][1], branches[0][2])
    if out is _AUTO:
        out = torch.empty(c0.batch, hq, c0.dv, dtype=torch.float32,
                          device=q.device)
    cin, cout = _carries(c0, hq, carry_in, carry_out, out)
    need = library().gqa_attend_branches_workspace_bytes(arr, len(arr), hq)
    if need == 0:
        raise GqaError("attend_branches: invalid or unsupported branches")
    if workspace is None:
        workspace = _workspace(need, q.device)
    _need(workspace, "workspace")
    _check(library().gqa_attend_branches(
        _ptr(q), hq, arr, len(arr), float(scale), cin, cout, _ptr(out),
        _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(q)), "attend_branches")
    return out


def stream_append(ring_k, ring_v, k_new, v_new, count_in, count_out=None,
                  sink=None, main=None, dropped=None, lens=None):
    """One token per sequence into the sink / ring / main layout.

    ``sink`` and ``main`` are optional (k, v) cache pairs.  fp8 parts are
    :class:`Fp8Cache` pairs sharing the ring's scale tensors (k_new / v_new
    then bf16, quantised into the new slot).  Returns
    (count_out, lens_sink, lens_ring, lens_main): device int32 [batch]
    tensors (lens_sink / lens_main None without that part), the lengths
    :func:`attend_branches` takes; ``lens`` may give those three tensors to
    fill (e.g. under graph capture)."""
    rc = _cache(ring_k, ring_v)
    sc = None if sink is None else _cache(*sink)
    mc = None if main is None else _cache(*main)
    io = _io_dtype(ring_k)
    _need(k_new, "k_new", io, (rc.batch, rc.num_kv_heads, rc.dk))
    _need(v_new, "v_new", io, (rc.batch, rc.num_kv_heads, rc.dv))
    _need(count_in, "count_in", torch.int32, (rc.batch,))
    dev = ring_k.device
    new = lambda: torch.empty(rc.batch, dtype=torch.int32, device=dev)
    if count_out is None:
        count_out = new()
    _need(count_out, "count_out", torch.int32, (rc.batch,))
    if lens is not None:
        ls, lr, lm = lens
        for t, nm in ((ls, "lens_sink"), (lr, "lens_ring"), (lm, "lens_main")):
            if t is not None:
                _need(t, nm, torch.int32, (rc.batch,))
    else:
        ls = None if sc is None else new()
        lr = new()
        lm = None if mc is None else new()
    if dropped is not None:
        _need(dropped, "dropped", torch.int32, (1,))
    _check(library().gqa_stream_append(
        None if sc is None else ctypes.byref(sc), ctypes.byref(rc),
        None if mc is None else ctypes.byref(mc), _ptr(k_new), _ptr(v_new),
        _ptr(count_in), _ptr(count_out), _ptr(ls), _ptr(lr), _ptr(lm),
        _ptr(dropped), _stream(ring_k)), "stream_append")
    return count_out, ls, lr, lm


def decode_step_branches(q, branches, append_branch: int, k_new, v_new,
                         lens_out, scale: float = 0.0,
                         carry_in: Optional[Carry] = None,
                         carry_out: Optional[Carry] = None, out=_AUTO,
                         workspace: Optional[torch.Tensor] = None,
                         dropped=None):
    """decode_step over several caches: (k_new, v_new) is appended to branch
    ``append_branch`` (whose lens is the step's lens_in; ``lens_out`` gets
    the new lengths) and q attends every branch, two launches in all."""
    arr = _branches(branches, q)
    c0, hq = _attend_args(q, branches[0][0], branches[0][1], branches[0][2])
    ab = branches[append_branch]
    ca = _cache(ab[0], ab[1])
    io = _io_dtype(ab[0])
    _need(k_new, "k_new", io, (ca.batch, ca.num_kv_heads, ca.dk))
    _need(v_new, "v_new", io, (ca.batch, ca.num_kv_heads, ca.dv))
    _need(lens_out, "lens_out", torch.int32, (ca.batch,))
    if dropped is not None:
        _need(dropped, "dropped", torch.int32, (1,))
    if out is _AUTO:
        out = torch.empty(c0.batch, hq, c0.dv, dtype=torch.float32,
                          device=q.device)
    cin, cout = _carries(c0, hq, carry_in, carry_out, out)
    need = library().gqa_attend_branches_workspace_bytes(arr, len(arr), hq)
    if need == 0:
        raise GqaError("decode_step_branches: invalid or unsupported branches")
    if workspace is None:
        workspace = _workspace(need, q.device)
    _need(workspace, "workspace")
    _check(library().gqa_decode_step_branches(
        _ptr(q), hq, arr, len(arr), int(append_branch), _ptr(k_new),
        _ptr(v_new), _ptr(lens_out), _ptr(dropped), float(scale), cin, cout,
        _ptr(out), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(q)), "decode_step_branches")
    return out


def attend_gathered(q, k_cache, v_cache, lens, idx, scale: float = 0.0,
                    carry_in: Optional[Carry] = None,
                    carry_out: Optional[Carry] = None, out=_AUTO,
                    workspace: Optional[torch.Tensor] = None):
    """Index-gathered decode: each sequence attends only the cache slots its
    row of ``idx`` [B, width] (device int32) names; duplicates collapse,
    negative and out-of-range entries drop."""
    c, hq = _attend_args(q, k_cache, v_cache, lens)
    _need(idx, "idx", torch.int32)
    if idx.dim() != 2 or idx.shape[0] != c.batch:
        raise GqaError(f"idx must be [batch={c.batch}, width]")
    width = int(idx.shape[1])
    if out is _AUTO:
        out = torch.empty(c.batch, hq, c.dv, dtype=torch.float32,
                          device=q.device)
    cin, cout = _carries(c, hq, carry_in, carry_out, out)
    need = library().gqa_attend_gathered_workspace_bytes(ctypes.byref(c), hq,
                                                         width)
    if need == 0:
        raise GqaError("attend_gathered: unsupported shape")
    if workspace is None:
        workspace = _workspace(need, q.device)
    _need(workspace, "workspace")
    _check(library().gqa_attend_gathered(
        _ptr(q), hq, ctypes.byref(c), _ptr(lens), _ptr(idx), width,
        float(scale), cin, cout, _ptr(out), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(q)),
        "attend_gathered")
    return out


def profile_next_launch(start: int, stop: int) -> None:
    """gqa_profile_next_launch: the next partition kernel this thread
    enqueues is bracketed by the two hipEvent_t handles (raw ints; 0, 0
    cancels)."""
    _check(library().gqa_profile_next_launch(_P(start or None),
                                             _P(stop or None)),
           "profile_next_launch")
