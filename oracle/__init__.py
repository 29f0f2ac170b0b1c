"""CPU oracle (fp64, numpy) for the block-scaled GEMM -- test infrastructure only.

Imported by the tests, the smoke check and the benchmark's CPU-baseline leg; never
by the library.  It shares no code with the HIP path.
"""
from .oracle import (MX_BLOCK, NV_BLOCK, bits_to_f64, contract, decode_e2m1, decode_e4m3, decode_e8m0,
                     dequant, dequant_mxfp8, dequant_nvfp4, epilogue, reference, round_output,
                     round_to_bf16_bits, round_to_f16_bits, unpack_e2m1)
from .tolerance import accumulation_bound, compare, silu_kappa, silu_slope, silu_slope_max
