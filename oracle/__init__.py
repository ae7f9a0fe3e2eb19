"""CPU oracle for the StagQ batch-one GEMV (test infrastructure only).

Only tests, the smoke check and the benchmark's CPU-baseline leg import this
package.  It shares no code with the HIP library.
"""
from .stagq_oracle import (  # noqa: F401
    Fields, encode, quantize_value, codes, w_main, w_hat, gemv, half_step, affine_pair, budget,
    scale_x, gemv_scaled, initial_pair, uniform_codebooks, codebook_table, pair_loss,
)
from .stagq_encoder_full import (  # noqa: F401
    encode_full, lloyd_1d, place_codebook, pick_pairs, two_bit_error, clip_candidate, entry_bits, post_bits,
)
