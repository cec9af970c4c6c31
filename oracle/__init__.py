"""fp64 CPU oracle for SAS gated block-sparse attention.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check in
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may import this
package.  The product library never does, and the two share no code.

The arithmetic lives in ``sas_oracle.c`` (plain C, fp64, OpenMP over
independent rows); this module is ctypes marshalling only.
"""

from .oracle import (  # noqa: F401
    OracleShape,
    build,
    gate_scores,
    attn_fwd,
    attn_bwd,
    topk_blocks,
    topk_budget,
    budget_ratio,
    threshold_blocks,
    sparse_fwd,
    num_threads,
)
