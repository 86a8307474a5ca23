"""fp64 CPU oracle (test infrastructure only; see `oracle/attention.py`).

Only the tests, `__graft_entry__.smoke()` and the `cpu_baseline` leg of
`bench.py` use this package. The GPU library never imports it.
"""
from .attention import (NEG_INF, attend, attend_multi, fanout, finalize, kv_append, merge, scores,
                        token_offsets, triplet, widen)

__all__ = ["NEG_INF", "attend", "attend_multi", "fanout", "finalize", "kv_append", "merge", "scores",
           "token_offsets", "triplet", "widen"]
