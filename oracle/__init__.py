"""Plain CPU oracle of In-context Sparse Attention (ISA) -- TEST INFRASTRUCTURE.

This package is the slow, obviously-correct fp64 definition that the HIP path
is checked against.  It is NOT part of the product: only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  It shares no code with ``sparse_attention_context_block_amd`` and
imports nothing from it.

Pages cited (by title and section):

  [notes]    "Lightning Unified Video Editing via In-Context Sparse Attention",
             papernotes.org ICML 2026 reading notes.  Sections used:
             "overall framework" (the four forward steps and the merge),
             "key design 1" (Context Pre-Selection), "key design 2" (block-wise
             0-th order Taylor sparse attention), "key design 3" (grouped
             computation by query sharpness), "training strategy" (defaults).
  [summary]  "LIVEditor-14B: Lightning Unified Video Editing via In-Context
             Sparse Attention", paperlayer.ai summary of arXiv 2605.04569v2.
             Sections used: 2 Preliminary (standard attention, block sparse
             attention, pooling attention), 3 In-Context Sparse Attention
             (pre-selection, Taylor sparse attention, grouped computation).

The decoupled rotary embedding ([notes] "training strategy") is in
``isa_oracle_rope`` with its readings R22-R24.

Every reading of a point the pages leave open is listed in ``isa_oracle``'s
module docstring.
"""

from .isa_oracle import (  # noqa: F401
    block_grid,
    pool_blocks,
    coarse_probs,
    context_scores,
    select_count,
    flat_count,
    top_k_context,
    sharpness,
    route_queries,
    gather_concat,
    exact_attention,
    taylor_attention,
    ns_count,
    top_ns_blocks,
    mixed_attention,
    decisions_ref,
    isa_ref,
    isa_ref_fixed,
    dense_ref,
)
from .isa_oracle_bwd import isa_ref_bwd, dense_ref_bwd  # noqa: F401
from .isa_oracle_rope import (  # noqa: F401
    round_to_bf16,
    round_to_dtype,
    rope_positions,
    rope_inv_freq,
    rotate_pairs,
    decoupled_rope,
    isa_ref_rope,
    isa_ref_bwd_rope,
)
