"""Plain CPU oracle for block-scaled FP4 quantization and the probe-matched FP4 GEMM.

TEST INFRASTRUCTURE. Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline
leg may import or call anything here; the product library (fp4_block_scaled_tensor_amd)
never does, and the two share no code, tables or helpers. The only module both sides use
is ``synth`` (seeded input generators, no method arithmetic).

Written from the pages (cited per module) in NumPy: codebooks are enumerated from bit
fields, encoders compare against exact midpoints, float32 steps use NumPy float32
arithmetic (IEEE round-to-nearest-even, no fused multiply-add), exact steps use float64
or Fractions.

Pins (tests/test_oracle_*.py) and their strength:
- formats: UE5M3 maximum 61,440 and the 137x / 30x headroom figures from the pages; E4M3
  against torch's float8_e4m3fn cast; E2M1 codebook by definition (parity pinned by the
  OCP definition, not by the pages).
- quantizer: nearest-ness by brute force over the codebook, zero-scale rule, headroom
  saturation edge, E8M0 exponent rule; tensor-scale arithmetic itself is a reading
  (parity unpinned beyond self-consistency).
- Philox: the generic round structure against NumPy's Philox-4x64 bit generator, plus the
  published Philox-4x32-10 known-answer vectors; SR unbiasedness within 3 sigma.
- Hadamard: SciPy's Sylvester matrix, H H^T = n I.
- GEMM model: an exact-rational element-wise restatement (oracle.exact), RTZ addition
  against x86 SSE arithmetic under FE_TOWARDZERO, the K=64 B=32 textbook case, integer
  cases, and the float64 reference within the stated tolerance.
- fake quantization: decode against exact rationals, E8M0 fake-quant values against a
  brute-force nearest search over the block's scaled codebook, bfloat16 rounding against
  torch's cast, policy order-dependence and D=1 == per-request amax.
- MXFP4 -> FP8: E4M3 codes against torch's float8_e4m3fn cast, exact round trip of the
  values for blocks within 14 binades of their chunk's largest, the chunk scale rule and
  the 384 ceiling, hand-worked examples.
- tile-local scales: one stripe equals global current scaling, a power-of-two rescale of
  one stripe changes only that stripe's g, each stripe's largest block lands on T, and the
  stripe-alpha GEMM against the float64 product within the model tolerance.
"""
from . import formats, philox, hadamard, quantize, gemm, exact, fakequant, fp8convert, local
from .formats import UE5M3, E4M3, E8M0
from .quantize import (AmaxCache, QuantResult, block_health, quantize_1d, quantize_2d, quantize_col, tensor_amax,
                       tensor_scales, pack_codes, unpack_codes, transposed_view)
from .gemm import gemm_model, gemm_fp64, rtz_add_f32, operand_from_quant, output_scale, expand_2d_scales
from .fakequant import dequantize, fake_quant, f32_to_bf16_bits, FakeQuantPolicy
from .fp8convert import mxfp4_to_fp8, fp8_values
from .local import LocalQuant, quantize_1d_local, stripe_alpha

__all__ = [
    "formats", "philox", "hadamard", "quantize", "gemm", "exact", "fakequant", "fp8convert", "local",
    "UE5M3", "E4M3", "E8M0", "AmaxCache", "QuantResult", "quantize_1d", "quantize_2d", "quantize_col",
    "tensor_amax", "tensor_scales", "pack_codes", "unpack_codes", "transposed_view",
    "gemm_model", "gemm_fp64", "rtz_add_f32", "operand_from_quant", "output_scale", "expand_2d_scales",
    "dequantize", "fake_quant", "f32_to_bf16_bits", "FakeQuantPolicy", "mxfp4_to_fp8", "fp8_values",
    "LocalQuant", "quantize_1d_local", "stripe_alpha",
]
