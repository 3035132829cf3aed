"""CPU oracle for exact attention — test infrastructure, not part of the library.

Imported only by ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg
of ``bench.py``.  See ``oracle/attention.py`` for the definitions and sources.
"""
from .attention import (  # noqa: F401
    compare,
    default_scale,
    kv_head,
    masked_softmax,
    merge_partials,
    online_softmax_stats,
    ref_bwd,
    ref_decode,
    ref_decode_chunk,
    ref_decode_paged,
    e4m3_value,
    ref_fwd_fp8,
    gather_pages,
    ref_fwd,
    ref_fwd_rows,
    ref_probs,
    scores,
    tiled_fwd,
    valid_mask,
)
