"""CPU oracle for the DSA layer (float64 NumPy).

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
benchmark's CPU-baseline leg, never by the product path. It shares no code
with the HIP library or its binding.
"""
from .dsa_oracle import (  # noqa: F401
    attend_selected,
    dsa_rows,
    full_causal_attention,
    index_scores,
    pack_mask,
    padded_indices,
    round_scores_fp32,
    select_topk,
)
from .front_end import indexer_front_end  # noqa: F401,E402
from .fp8_indexer import e4m3_round, index_scores_fp8, quantize_rows_fp8  # noqa: F401,E402
