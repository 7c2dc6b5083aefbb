"""CPU oracle for the NF4 path.  Test infrastructure only: imported by tests,
the smoke check and the benchmark's CPU-baseline leg, never by the library."""

from .nf4_oracle import *  # noqa: F401,F403
from .nf4_oracle import (  # noqa: F401
    BLOCKSIZE, BLOCKSIZE2, DELTA, codebook, levels_f64, level_probabilities,
    inv_phi_bisect, inv_phi_stdlib, block_absmax, nearest_code, normalize, pack,
    unpack, quantize, int8_absmax_quantize, exact_mean_f32, double_quant,
    dequant_scales, f32_to_bf16_bits, bf16_bits_to_f32, dequantize, matmul_ref,
    rel_frobenius, storage_bytes, bits_per_param, f64_to_bf16_bits, f64_to_f16_bits,
    lora_merge, backward_ref, E4M3_MAX, e4m3_value, e4m3_encode, e4m3_ratio_table,
    f8_absmax_quantize, double_quant_f8, FP4_ZERO, FP4_PRODUCED, e2m1_value, fp4_codebook,
)
