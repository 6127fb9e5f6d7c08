"""Seeded synthetic inputs shared by the oracle side and the HIP side.

This package holds no attention arithmetic: it draws normal variates, rounds
them to bfloat16 bit patterns, and builds document-id rows.  Both the fp64
oracle (``oracle/``) and the GPU path (``attention_variants_amd``) consume
what it produces; neither imports the other.
"""

from .inputs import (  # noqa: F401
    SEEDS,
    bf16_bits_from_f32,
    bf16_bits_to_f64,
    bf16_bits_to_f32,
    normal_bf16,
    doc_lengths,
    doc_ids,
    attention_inputs,
    diff_inputs,
    evoformer_inputs,
)
