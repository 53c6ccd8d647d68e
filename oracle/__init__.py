"""CPU float64 oracle for absorbed paged MLA decode -- test infrastructure only.

Only the tests, the smoke entry and the bench's CPU-baseline leg use it; the
product library never does.  ``mla_oracle`` holds the decode and the cache append,
``fp8_cache`` the E4M3 format and the per-token quantization of the FP8 latent cache.
"""
from .mla_oracle import (  # noqa: F401
    absorb_reference,
    absorbed_scores,
    append_rows,
    append_to_pool,
    default_scale,
    latent_row_bytes,
    latent_row_elements,
    mha_row_bytes,
    mla_decode,
    mqa_row_elements,
    naive_scores,
    new_token_positions,
    page_bytes,
    reconstruct_kv,
    rope_angles,
    rope_rotate,
    softmax_rows,
    staged_tile_bytes,
    up_v_reference,
)
