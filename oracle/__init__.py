"""CPU oracle for scaled dot-product attention — test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path never does.
"""

from .sdpa_oracle import (  # noqa: F401
    apply_mask,
    attention,
    attention_head,
    attention_rows,
    default_scale,
    row_softmax,
    scores,
    visible_keys,
    weighted_values,
)
