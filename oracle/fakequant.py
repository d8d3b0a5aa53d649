"""Inference fake quantization and activation-scale policies (oracle; test infrastructure
only).

Source: "UE5M3 FP4 Block Scaling for Stable Language Model Pretraining".
- Approach section (접근 방법), training and inference setup: at inference the
  activation scale follows one of three policies: delayed (D = 50, the recipe's own),
  current (D = 1, the Transformer Engine setting) or calibrated-frozen (an amax fixed
  from calibration sequences). The delayed policy is order-dependent, so evaluation uses
  a fixed request order.
- Results section: held-out likelihoods are measured with FP4 fake quantization.
- Limits section: delayed scaling at inference is stateful and depends on request order.

Fake quantization is quantize-then-decode: the value an FP4 operand stands for,
    x_hat = E2M1(q) * S * g          (g = 1 for E8M0 scales),
returned as float32. E2M1(q) * S is exact (at most 6 significant bits, inside the float32
normal range for UE5M3 / E4M3, and a power-of-two shift for E8M0), so x_hat is that exact
product times g rounded once to float32 (nearest-even). A bfloat16 output is that float32
rounded to bfloat16, nearest-even (readings listed in the design notes).

A policy maps each request, in order, to the amax its quantization uses:
- delayed / current: a sample-and-hold cache with period D (D = 1 is current scaling):
  the request's own amax is sampled when the cache is empty or request % D == 0;
- frozen: a fixed amax, never sampled.
"""
from __future__ import annotations

import numpy as np

from . import formats as F
from .gemm import expand_2d_scales
from .quantize import AmaxCache, QuantResult, quantize_1d, tensor_amax


def scale_matrix(qr: QuantResult, view: str = "1d") -> np.ndarray:
    """Per-element block-scale values [rows, K] (float64, exact) of a quantized operand.
    view: '1d' (B consecutive elements along K), '2d' (forward weight view, 16x16 tiles) or
    '2dT' (the transposed weight view of the same tiles)."""
    sv = F.SCALE_VALUES[qr.fmt][qr.scales.astype(np.int64)]
    if view == "1d":
        return np.repeat(sv, qr.block, axis=1)
    if view in ("2d", "2dT"):
        return np.repeat(expand_2d_scales(sv, view == "2dT"), 16, axis=1)
    raise ValueError(view)


def dequantize(qr: QuantResult, view: str = "1d") -> np.ndarray:
    """float32 values x_hat = E2M1(q) * S * g of a quantized operand (codes [rows, K] as
    stored for that view)."""
    v = F.decode_e2m1(qr.codes) * scale_matrix(qr, view)       # exact in float64
    v32 = v.astype(np.float32)
    if not np.array_equal(v32.astype(np.float64), v):
        raise AssertionError("E2M1 * S is not exact in float32")
    if qr.fmt == F.E8M0:
        return v32
    return (v32 * np.float32(qr.g)).astype(np.float32)          # one float32 multiply, RNE


def f32_to_bf16_bits(y: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns of float32 values, nearest-even: of the two bfloat16 values
    bracketing y (truncation and truncation + 1 ulp), take the nearer; on an exact tie the
    one with an even last bit. Past the largest finite bfloat16 the upper neighbour is
    infinity, weighed as 2^128 (IEEE overflow rounding). Finite inputs only."""
    y = np.atleast_1d(np.asarray(y, dtype=np.float32))
    if not np.all(np.isfinite(y)):
        raise ValueError("finite inputs only")
    bits = y.view(np.uint32).astype(np.uint64)
    lo = bits >> 16                                   # truncation toward zero (sign kept)
    hi = lo + 1                                       # next bfloat16 away from zero

    def val(b):
        mag = np.where((b & 0x7FFF) == 0x7F80, 2.0 ** 128,
                       np.abs((b << 16).astype(np.uint32).view(np.float32).astype(np.float64)))
        return np.where(b & 0x8000, -mag, mag)

    d_lo = np.abs(y.astype(np.float64) - val(lo))
    d_hi = np.abs(val(hi) - y.astype(np.float64))
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (lo % 2 == 1))
    return np.where(pick_hi, hi, lo).astype(np.uint16)


def fake_quant(x: np.ndarray, fmt: int, block: int, amax=None, T: float = 448.0, out: str = "f32") -> np.ndarray:
    """Quantize x [rows, K] with 1D blocks along K (nearest-even), then decode. out='f32'
    gives float32 values, out='bf16' the bfloat16 bit patterns (uint16)."""
    y = dequantize(quantize_1d(x, fmt, block, amax=amax, T=T))
    if out == "f32":
        return y
    if out == "bf16":
        return f32_to_bf16_bits(y)
    raise ValueError(out)


class FakeQuantPolicy:
    """Activation-scale policy for fake-quantized inference requests, taken in order."""

    def __init__(self, kind: str, D: int | None = None, amax=None):
        if kind == "delayed":
            self.cache = AmaxCache(50 if D is None else D)
        elif kind == "current":
            self.cache = AmaxCache(1)
        elif kind == "frozen":
            if amax is None:
                raise ValueError("a frozen policy needs its calibration amax")
            self.cache = None
            self.amax = np.float32(amax)
        else:
            raise ValueError(kind)
        self.kind = kind

    def amax_for(self, request: int, x: np.ndarray) -> np.float32:
        if self.cache is None:
            return self.amax
        if self.cache.needs_sample(request):
            return self.cache.update(request, tensor_amax(x))
        return self.cache.amax

    def __call__(self, request: int, x: np.ndarray, fmt: int, block: int, T: float = 448.0,
                 out: str = "f32") -> np.ndarray:
        return fake_quant(x, fmt, block, amax=self.amax_for(request, x), T=T, out=out)
