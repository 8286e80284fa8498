"""CPU oracle for exact GQA decode attention (test infrastructure only).

Only ``tests/``, the smoke check in ``__graft_entry__`` and the CPU-baseline leg
of ``bench.py`` may import this package.  It shares no code with the HIP path.
"""

from .attention import (Carry, attend, empty_carry, finalize, group_logits,
                        kv_append, kv_head_of, live_length, merge,
                        resolve_scale, softmax_state)
from .streaming import (attend_branches, attend_gathered, selection_mask,
                        stream_append, stream_lengths)

__all__ = ["Carry", "attend", "empty_carry", "finalize", "group_logits",
           "kv_append", "kv_head_of", "live_length", "merge", "resolve_scale",
           "softmax_state", "attend_branches", "attend_gathered",
           "selection_mask", "stream_append", "stream_lengths"]
