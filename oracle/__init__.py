"""CPU oracle for exact softmax attention (test infrastructure only).

This package is the correctness reference for the GPU library, and nothing
else. Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg
of ``bench.py`` may import it; the library itself never does, and it shares no
code with the GPU path (no kernels, helpers, tables or constants).

Everything is plain numpy in float64:

* :mod:`oracle.attention` -- the definition: the full score matrix is formed,
  masked, softmaxed and applied to V, one (batch, head) at a time; and the
  analytic backward obtained from that definition by the chain rule; the
  merge of partial results over key ranges; variable-length batches.
* :mod:`oracle.online_fold` -- a separate implementation of the online-softmax
  recurrence (running max, running normaliser, rescaled running output), key
  block by key block. It does not import :mod:`oracle.attention`.

Pins: every function here is checked against facts the pages and mathematics
fix (closed forms, invariants, brute force on tiny inputs, finite differences,
hand-derived worked examples); see ``tests/test_oracle.py``. No function is
"parity unpinned".
"""

from .attention import (  # noqa: F401
    attn_fwd_head,
    attn_fwd_materialised,
    attn_probs,
    attn_bwd_group,
    attn_bwd_analytic,
    kv_head,
    merge_partials,
    attn_fwd_varlen,
    attn_bwd_varlen,
)
from .online_fold import attn_fwd_online_fold, fold_head  # noqa: F401
