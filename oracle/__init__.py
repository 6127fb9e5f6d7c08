"""fp64 CPU oracle -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path never does.
Every function here is pinned by ``tests/test_oracle_pins.py``.
"""

from .attention import (  # noqa: F401
    SCORE_MODS,
    DATA_SCORE_MODS,
    MASKS,
    raw_scores,
    alibi_slope,
    apply_score_mod,
    allowed_matrix,
    softmax_two_pass,
    attention,
    attention_backward,
    paged_decode_attention,
    diff_attention,
    diff_lambda_init,
    diff_lambda,
    diff_head,
    sigmoid,
    evoformer_projections,
    evoformer_row_gated_attention,
    evoformer_col_gated_attention,
)
