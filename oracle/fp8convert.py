"""MXFP4 -> FP8 (E4M3) conversion with hierarchical scale alignment (oracle; test
infrastructure only).

Source: "Practical FP4 Training for Large-Scale MoE Models on Hopper GPUs", methodology
(방법론), hybrid-precision bullets: activations cached in MXFP4 (E2M1, block 32) are turned
directly into FP8 (E4M3, block 128) without a BF16 intermediate; a hierarchical scale
alignment bridges the block-size mismatch; the kernel works with bit shifts and integer
mappings and fuses the transpose with the conversion.

Reading (the page gives no formula; listed in the design notes):
- a 128-element chunk of a row holds four MXFP4 blocks with E8M0 codes e_0..e_3; its FP8
  scale is the E8M0 code c = e_max - min(6, e_max), e_max = max e_b, i.e. the largest
  block's power of two lowered by 2^6 so that its values (|E2M1| <= 6) land at most at
  6 * 2^6 = 384 inside E4M3's range (max 448);
- element x = E2M1(q) * 2^(e_b - 127) becomes y = E4M3(E2M1(q) * 2^(e_b - c)), nearest-even
  with subnormals, the sign kept; then y * 2^(c - 127) == x exactly whenever
  e_max - e_b <= 14 (the E2M1 grid step 0.5 * 2^(e_b - c) stays >= E4M3's 2^-9); smaller
  blocks round on E4M3's subnormal grid;
- outputs: FP8 codes in the operand's layout [rows x K] or transposed [K x rows], and the
  chunk scale codes [rows x K/128].
"""
from __future__ import annotations

import numpy as np

from . import formats as F

CHUNK = 128
HEADROOM_SHIFT = 6


def chunk_scale_codes(scales: np.ndarray) -> np.ndarray:
    """FP8 chunk scale codes [rows, K/128] from MXFP4 block codes [rows, K/32]."""
    e = np.asarray(scales, dtype=np.int64)
    R, nb = e.shape
    if nb % 4:
        raise ValueError("K must be a multiple of 128")
    emax = e.reshape(R, nb // 4, 4).max(axis=2)
    return (emax - np.minimum(HEADROOM_SHIFT, emax)).astype(np.uint8)


def encode_e4m3_signed(v: np.ndarray) -> np.ndarray:
    """E4M3 code of float64 values: magnitude nearest-even over the finite codebook
    (saturating at 448), sign bit 7 kept (also for values that round to zero)."""
    v = np.asarray(v, dtype=np.float64)
    mag = F.encode_nearest_even(np.abs(v), F.E4M3_VALUES)
    return (mag | (np.signbit(v).astype(np.int64) << 7)).astype(np.uint8)


def decode_e4m3_signed(codes: np.ndarray) -> np.ndarray:
    c = np.asarray(codes, dtype=np.int64)
    mag = F.E4M3_VALUES[c & 0x7F]
    return np.where(c & 0x80, -mag, mag)


def mxfp4_to_fp8(codes: np.ndarray, scales: np.ndarray, transpose: bool = False):
    """codes [rows, K] E2M1 (unpacked, sign in bit 3), scales [rows, K/32] E8M0 codes.
    Returns (FP8 codes [rows, K] or [K, rows], chunk scale codes [rows, K/128])."""
    codes = np.asarray(codes, dtype=np.uint8)
    e = np.asarray(scales, dtype=np.int64)
    R, K = codes.shape
    if K % CHUNK:
        raise ValueError("K must be a multiple of 128")
    c8 = chunk_scale_codes(e).astype(np.int64)
    shift = np.repeat(e, 32, axis=1) - np.repeat(c8, CHUNK, axis=1)        # e_b - c, <= 6
    v = F.decode_e2m1(codes) * np.ldexp(1.0, shift)                        # exact in float64
    y = encode_e4m3_signed(v)
    return (np.ascontiguousarray(y.T) if transpose else y), c8.astype(np.uint8)


def fp8_values(y: np.ndarray, c8: np.ndarray, transpose: bool = False) -> np.ndarray:
    """Real values (float64) of the FP8 output: E4M3(y) * 2^(c - 127)."""
    y = np.asarray(y)
    if transpose:
        y = y.T
    return decode_e4m3_signed(y) * np.ldexp(1.0, np.repeat(np.asarray(c8, dtype=np.int64), CHUNK, axis=1) - 127)
