"""Codebooks and round-to-nearest-even, saturating encoders (oracle; test infrastructure only).

Every codebook is enumerated from its bit fields, and every encoder picks the nearest
codebook entry by comparing against the exact midpoint of the two neighbours, breaking
exact ties toward the code whose least-significant bit is 0. No bit tricks.

Sources:
- "UE5M3 FP4 Block Scaling for Stable Language Model Pretraining", approach section
  (접근 방법), format bullet: the payload is E2M1 (sign, 2 exponent bits, 1 fraction
  bit); block scales are unsigned E5M3 with a wider positive codebook whose maximum is
  61,440; ties go to even for forward activations, weights and block scales.
- Same page, problem section (해결하려는 문제): the baseline scales are E4M3 (NVFP4) or
  the MX power-of-two scale (MXFP4).
- "Format-Aware Fusion for Fast FP4 Pretraining", related-papers list entry on FP8
  formats: E4M3 has no infinities and a single NaN mantissa pattern.
- "Practical FP4 Training for Large-Scale MoE Models on Hopper GPUs", methodology
  (방법론): MXFP4 is E2M1 with block size 32.

Readings where the pages are silent (listed in the design notes):
- E2M1 exponent bias 1, one subnormal (0.5), maximum 6, no Inf/NaN (the OCP MX
  definition of FP4 that "MXFP4" names).
- UE5M3 exponent bias 15, subnormals, exponent field 31 reserved and never produced;
  this gives exactly the stated maximum 2^15 * 1.875 = 61,440.
- E4M3 bias 7, 0x7F the only NaN; maximum 448.
- E8M0 value 2^(code-127), code 255 reserved.
"""
from __future__ import annotations

import numpy as np

UE5M3, E4M3, E8M0 = 0, 1, 2
FMT_NAMES = {UE5M3: "ue5m3", E4M3: "e4m3", E8M0: "e8m0"}


def _e2m1(code: int) -> float:
    s, e, m = (code >> 3) & 1, (code >> 1) & 3, code & 1
    mag = m * 0.5 if e == 0 else 2.0 ** (e - 1) * (1.0 + m / 2.0)
    return -mag if s else mag


def _ue5m3(code: int) -> float:
    e, m = code >> 3, code & 7
    if e == 31:
        return float("nan")
    if e == 0:
        return (m / 8.0) * 2.0 ** -14
    return 2.0 ** (e - 15) * (1.0 + m / 8.0)


def _e4m3(code: int) -> float:
    # positive half only (block scales are non-negative); 0x7F is NaN
    e, m = (code >> 3) & 15, code & 7
    if code == 0x7F:
        return float("nan")
    if e == 0:
        return (m / 8.0) * 2.0 ** -6
    return 2.0 ** (e - 7) * (1.0 + m / 8.0)


def _e8m0(code: int) -> float:
    return float("nan") if code == 255 else 2.0 ** (code - 127)


E2M1_VALUES = np.array([_e2m1(c) for c in range(16)], dtype=np.float64)
E2M1_MAGS = E2M1_VALUES[:8].copy()                     # codes 0..7, increasing
UE5M3_VALUES = np.array([_ue5m3(c) for c in range(248)], dtype=np.float64)   # finite codes
E4M3_VALUES = np.array([_e4m3(c) for c in range(127)], dtype=np.float64)     # finite, non-negative
E8M0_VALUES = np.array([_e8m0(c) for c in range(255)], dtype=np.float64)

SCALE_VALUES = {UE5M3: UE5M3_VALUES, E4M3: E4M3_VALUES, E8M0: E8M0_VALUES}
SCALE_MAX = {UE5M3: float(UE5M3_VALUES[-1]), E4M3: float(E4M3_VALUES[-1])}
SCALE_ONE_CODE = {UE5M3: int(np.where(UE5M3_VALUES == 1.0)[0][0]),
                  E4M3: int(np.where(E4M3_VALUES == 1.0)[0][0]),
                  E8M0: 127}


def encode_nearest_even(v: np.ndarray, values: np.ndarray) -> np.ndarray:
    """Nearest entry of the increasing codebook ``values`` (code c has value values[c]) for
    non-negative ``v``; exact ties go to the even code; v above the maximum saturates.
    Midpoints of neighbouring entries are exact in float64 (the entries have <= 4
    significant bits), so every comparison is exact for float32 or float64 inputs."""
    v = np.asarray(v, dtype=np.float64)
    if np.any(np.isnan(v)) or np.any(v < 0):
        raise ValueError("encoder input must be non-negative and not NaN")
    n = len(values)
    vs = np.minimum(v, values[-1])
    lo = np.clip(np.searchsorted(values, vs, side="right") - 1, 0, n - 1)
    hi = np.minimum(lo + 1, n - 1)
    mid = (values[lo] + values[hi]) / 2.0
    code = np.where(vs < mid, lo, np.where(vs > mid, hi, np.where(lo % 2 == 0, lo, hi)))
    code = np.where(lo == n - 1, n - 1, code)
    return code.astype(np.int64)


def encode_e2m1(r: np.ndarray) -> np.ndarray:
    """E2M1 code (sign in bit 3) of float32 values r: magnitude by nearest-even with
    saturation at 6; the sign bit of the input is kept, also for values that round to 0."""
    r = np.asarray(r, dtype=np.float32)
    sign = np.signbit(r).astype(np.int64)
    mag = encode_nearest_even(np.abs(r.astype(np.float64)), E2M1_MAGS)
    return (mag | (sign << 3)).astype(np.uint8)


def decode_e2m1(codes: np.ndarray) -> np.ndarray:
    return E2M1_VALUES[np.asarray(codes, dtype=np.int64) & 15]


def encode_scale(v: np.ndarray, fmt: int) -> np.ndarray:
    """Nearest-even, saturating encode of non-negative block-scale values (UE5M3 or E4M3)."""
    return encode_nearest_even(v, SCALE_VALUES[fmt]).astype(np.uint8)


def decode_scale(codes: np.ndarray, fmt: int) -> np.ndarray:
    return SCALE_VALUES[fmt][np.asarray(codes, dtype=np.int64)]
