"""Float64 CPU oracle for fused linear cross-entropy.

TEST INFRASTRUCTURE ONLY.  Nothing in the product package may import, call or
execute anything here; only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
path: it is written from the formulas on the pages, in plain numpy float64,
with no blocking, fusion or reordering beyond what those formulas state (the
row chunking below only bounds memory; every row is computed independently,
exactly as the per-token formulas say).

Pinned by ``tests/test_oracle_*.py`` against closed forms, invariants, a
textbook routine (``torch.nn.functional.cross_entropy`` in float64), central
finite differences and a pure-Python brute force.  The pages print no loss or
gradient values for any input, so beyond those pins exact values are "parity
unpinned"; the budget arithmetic (``liger_chunk_plan``) is pinned to the chunk
table printed on the first page.
"""

from .lce import (  # noqa: F401
    IGNORE_INDEX,
    TargetRangeError,
    lce_oracle,
    lce_oracle_filtered,
    vocab_sort_order,
    lce_rows_oracle,
    ce_oracle,
    lse_rows,
    lse_all,
    grad_input_rows,
    grad_weight_rows,
    grad_bias_entries,
    filtered_grad_input_tile,
    filtered_grad_weight_tile,
    liger_chunk_plan,
)
