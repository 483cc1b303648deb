"""CPU fp64 oracle (test infrastructure only; never imported by the product path)."""
from .attention import (  # noqa: F401
    allowed_mask,
    attention_bwd_ref,
    attention_ref,
    combine_ref,
    decode_ref,
    gqa_decode_ref,
    merge_partials,
    paged_decode_ref,
    probabilities_ref,
    split_bounds,
    split_partials_ref,
    tiled_model,
)
