"""Plain CPU fp64 oracle for exact softmax attention, forward and backward.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke check
of ``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may import
this package.  It shares no code with the HIP path and imports nothing from
it; both sides receive the same seeded input arrays from the input generator.

What it computes is the definition of attention the pages start from
(flash-attn-triton docs, "The argument": S = QK^T/sqrt(d), softmax, then PV),
written out with the score matrix materialised, plus the analytic gradient of
that definition.  The tiled method on the pages is exact algebra on the same
quantity (flash-attn-triton docs, "Tiling softmax is exact algebra"), so the
definition is the oracle; the tile recurrence of Fig. 3 and the merge of two
partial softmax results are written here too, but only so the tests can pin
the identity they rely on.

Modules:
  attention  -- forward (O, L), backward (dQ, dK, dV, D), row/column samplers,
                grouped-query, windowed and packed variable-length forms
  softmax    -- safe softmax, the Fig. 3 per-tile recurrence, merge of partials
"""

from .attention import (  # noqa: F401
    attention_forward,
    attention_backward,
    attention_forward_gqa,
    attention_backward_gqa,
    attention_backward_varlen,
    delta_rowsum,
    forward_rows,
    dq_rows,
    dkdv_cols,
)
from .softmax import (  # noqa: F401
    safe_softmax,
    online_softmax_tiles,
    merge_partials,
    partial_softmax_state,
)
