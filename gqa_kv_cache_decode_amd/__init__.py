"""Exact grouped-query decode attention over a KV cache, HIP on MI355X (gfx950).

The compute lives in ``libgqa_decode.so`` (hand-written HIP kernels behind a
C ABI, declared in ``include/gqa_decode.h``).  The functions here are thin
ctypes bindings of the C entry points of the same names (without the
``gqa_`` prefix): they marshal torch tensors and the current HIP stream into
the C calls.  The library is loaded on first use and a missing build raises
at once.
"""

__all__ = ["kv_append", "attend_decode", "softmax_state_merge",
           "decode_step", "step_workspace", "attend_branches",
           "stream_append", "decode_step_branches", "attend_gathered",
           "attend_partition", "attend_combine", "attend_plan",
           "workspace_bytes", "Carry", "Fp8Cache", "empty_carry", "GqaError",
           "library", "profile_next_launch", "CHUNK_BALANCED",
           "attend_decode_noalloc"]


def __getattr__(name):
    if name in __all__:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
