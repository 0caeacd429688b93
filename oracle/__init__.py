"""CPU oracle (test infrastructure only).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package. The product library never does, and the oracle imports
nothing from the product package.
"""
from .rtq_oracle import (  # noqa: F401
    CLIP_GRID, F8_NAN, GROUP, RECIPE_ALL_F8, RECIPE_ALL_Q8, RECIPE_MIXED,
    decode_f8, dequant, dequant_f8, dequant_q4, dequant_q8, gemm_ref, pack_q4, project, project_f8,
    project_bf16, project_bias, project_q4, project_q8, quantize, quantize_f8, quantize_q4, quantize_q8, rel_fro,
    round_bf16, unpack_q4,
)
