"""CPU oracle for the LiteAttention step (test infrastructure only).

Only tests, the package smoke check and the benchmark's CPU-baseline leg may import this
package. It shares no code with the HIP path and imports nothing from it.
"""
from .lite_attn_oracle import (  # noqa: F401
    StepResult,
    bits_to_mask,
    empty_mask,
    lite_attn_step_ref,
    mask_geometry,
    mask_to_bits,
    run_chain_ref,
)
