"""Block-scaled FP4 quantizer (oracle; test infrastructure only).

Follows "UE5M3 FP4 Block Scaling for Stable Language Model Pretraining":
- approach section (접근 방법): E2M1 payload, UE5M3 block scales at block size 16
  (32 as a control); per-operand amax caches refreshed by sample-and-hold every D=50
  steps; the delay slides the codebook's real-value window through the scale target T
  (448 by default, 2048 for the wgrad dY operand of sensitive layers); ties-to-even for
  activations, weights and block scales; stochastic rounding only for the upstream
  gradient dY payload in both backward GEMMs; a block scale that rounds to zero is
  replaced by one; 2D weight scaling so the forward and backward GEMM views agree.
- key-contributions section (핵심 기여): T=448 leaves about 137x growth headroom for a
  stale amax and T=2048 keeps about 30x (61,440 / T).

Scale arithmetic (the pages give no formula; the reading under which headroom equals
61,440 / T, all in float32 with IEEE round-to-nearest-even):
    s_enc = (6 * T) / A      tensor encode scale, A = cached amax
    s_blk = T / A            maps the cached amax to block-scale value T
    g     = 1 / s_enc        tensor decode scale, applied by the GEMM epilogue
    S     = enc(amax_b * s_blk), nearest-even, saturating; S = 1 if it encodes to 0
    r     = x * (s_enc / S)  one division per block, one multiply per element
    q     = E2M1(r)          nearest-even (or stochastic, dY only)
If A is zero or not finite, or 6T/A overflows, s_enc = s_blk = g = 1.

MXFP4 (E8M0 scales, block 32; "Practical FP4 Training for Large-Scale MoE Models on
Hopper GPUs", methodology (방법론)): no tensor scale (g = 1); the block exponent is
floor(log2 amax_b) - 2 (2 = E2M1's largest exponent), clamped to [-127, 127]; a zero
block takes exponent 0; r = x * 2^-E, exact.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import formats as F
from .hadamard import fwht_tokens
from .philox import sr_uniform16


def tensor_scales(amax, T) -> tuple[np.float32, np.float32, np.float32]:
    """(s_enc, s_blk, g) from the cached amax A and the scale target T, float32 arithmetic."""
    A = np.float32(amax)
    T = np.float32(T)
    one = np.float32(1.0)
    if not (np.isfinite(A) and A > 0):
        return one, one, one
    with np.errstate(over="ignore", under="ignore"):
        s_enc = np.float32(np.float32(np.float32(6.0) * T) / A)
        if not np.isfinite(s_enc):
            return one, one, one
        s_blk = np.float32(T / A)
        g = np.float32(one / s_enc)
    return s_enc, s_blk, g


def e8m0_block(amax_b: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """(scale codes, payload multipliers 2^-E as float32) for MXFP4 block maxima."""
    amax_b = np.asarray(amax_b, dtype=np.float32)
    _, ex = np.frexp(amax_b.astype(np.float64))      # amax = f * 2^ex, f in [0.5, 1)
    E = np.clip(ex.astype(np.int64) - 1 - 2, -127, 127)
    E = np.where(amax_b == 0, 0, E)
    mult = np.ldexp(np.float64(1.0), -E).astype(np.float32)   # exact: 2^-127 .. 2^127
    return (E + 127).astype(np.uint8), mult


def block_health(x: np.ndarray, fmt: int, block: int = 16, amax=None, T: float = 448.0, view: str = "row",
                 hadamard_n: int = 0) -> tuple[int, int, int]:
    """Health counts of a quantization (saturated, zero-scale, non-finite blocks), from the
    block maxima alone, so that inputs holding Inf or NaN (outside the payload's contract)
    can be counted too.

    view: 'row' (blocks along the columns of x), 'col' (the weight-gradient view: blocks along
    the tokens of the optionally rotated x), '2d' (16x16 tiles). A block maximum is the float
    maximum of |x| over the block, NaN if the block holds a NaN.
    - saturated: the unrounded scale float32(amax_b * s_blk) exceeds the format maximum (so the
      scale clips; the key-contributions headroom of 61440/T is the growth that stays below
      it). E8M0 has no tensor scale and counts none.
    - zero-scale: the scale encodes to zero and the zero rule replaces it by one (E8M0: an
      all-zero block).
    - non-finite: the block maximum is Inf or NaN."""
    x = np.asarray(x, dtype=np.float32)
    if view == "col":
        x = transposed_view(x, hadamard_n)
    if view == "2d":
        R, K = x.shape
        amax_b = np.max(np.abs(x.reshape(R // 16, 16, K // 16, 16)), axis=(1, 3))
    else:
        R, K = x.shape
        amax_b = np.max(np.abs(x.reshape(R, K // block, block)), axis=2)
    n_nonfin = int(np.sum(~np.isfinite(amax_b)))
    if fmt == F.E8M0:
        return 0, int(np.sum(amax_b == 0)), n_nonfin
    _, s_blk, _ = tensor_scales(amax, T)
    with np.errstate(over="ignore", invalid="ignore"):
        v = (amax_b * s_blk).astype(np.float32)
    fin = np.isfinite(v)
    n_sat = int(np.sum(v[fin].astype(np.float64) > F.SCALE_MAX[fmt]) + np.sum(np.isposinf(v)))
    n_zero = int(np.sum(F.decode_scale(F.encode_scale(v[fin], fmt), fmt) == 0.0))
    return n_sat, n_zero, n_nonfin


@dataclass
class QuantResult:
    codes: np.ndarray        # uint8 E2M1 codes, [rows, K] (unpacked), sign in bit 3
    scales: np.ndarray       # uint8 scale codes, [rows, K/B] (1D) or [rows/16, K/16] (2D)
    g: np.float32            # tensor decode scale (1 for MXFP4)
    fmt: int
    block: int
    n_sat: int = 0           # blocks whose unrounded scale exceeded the format maximum
    n_zero: int = 0          # blocks whose scale rounded to zero and was replaced by one
                             # (E8M0: all-zero blocks, which take exponent 0)

    @property
    def packed(self) -> np.ndarray:
        return pack_codes(self.codes)

    def scale_values(self) -> np.ndarray:
        return F.SCALE_VALUES[self.fmt][self.scales.astype(np.int64)]


def pack_codes(codes: np.ndarray) -> np.ndarray:
    """Two E2M1 codes per byte: element 2j in the low nibble, 2j+1 in the high nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] & 15) | ((c[..., 1::2] & 15) << 4)


def unpack_codes(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 15
    out[..., 1::2] = p >> 4
    return out


def sr_e2m1(r: np.ndarray, u16: np.ndarray) -> np.ndarray:
    """Stochastic E2M1 rounding: |r| >= 6 gives 6; otherwise with lo <= |r| < hi the two
    neighbouring codebook values, round up iff u16 / 2^16 < (|r| - lo) / (hi - lo).
    (|r| - lo) is exact (Sterbenz) and hi - lo is a power of two, so the comparison is
    exact. The sign bit of r is kept."""
    r = np.asarray(r, dtype=np.float32)
    a = np.abs(r).astype(np.float64)
    mags = F.E2M1_MAGS
    lo = np.clip(np.searchsorted(mags, a, side="right") - 1, 0, 7)
    hi = np.minimum(lo + 1, 7)
    frac = np.where(lo < 7, (a - mags[lo]) / np.where(lo < 7, mags[hi] - mags[lo], 1.0), 0.0)
    up = (np.asarray(u16, dtype=np.float64) / 65536.0) < frac
    mag = np.where(a >= 6.0, 7, lo + up.astype(np.int64))
    return (mag | (np.signbit(r).astype(np.int64) << 3)).astype(np.uint8)


def _payload(xb: np.ndarray, mult: np.ndarray, rounding: str, seed: int, offset: int, K: int,
             row0: int = 0) -> np.ndarray:
    """Quantize block-shaped values xb [R, nb, B] with per-block multipliers [R, nb].
    ``row0``: logical row of xb[0] in the full operand (stochastic-rounding index base)."""
    r = (xb * mult[..., None]).astype(np.float32)     # float32 multiply, RNE
    R, nb, B = xb.shape
    if rounding == "rne":
        return F.encode_e2m1(r).reshape(R, nb * B)
    if rounding == "sr":
        idx = np.arange(R * K, dtype=np.uint64) + np.uint64(row0 * K)
        u = sr_uniform16(seed, offset, idx).reshape(R, nb, B)
        return sr_e2m1(r, u).reshape(R, nb * B)
    raise ValueError(rounding)


def quantize_1d(x: np.ndarray, fmt: int, block: int, amax=None, T: float = 448.0,
                rounding: str = "rne", seed: int = 0, offset: int = 0, row0: int = 0) -> QuantResult:
    """Quantize x [rows, K] with 1D blocks of ``block`` consecutive elements along K.
    ``row0`` is the logical row of x[0] when x is a row slice of a larger operand."""
    x = np.asarray(x, dtype=np.float32)
    R, K = x.shape
    if K % block:
        raise ValueError("K must be a multiple of the block size")
    if fmt == F.E8M0 and block != 32:
        raise ValueError("E8M0 scales use block 32")
    xb = x.reshape(R, K // block, block)
    amax_b = np.max(np.abs(xb), axis=2)
    if fmt == F.E8M0:
        codes, mult = e8m0_block(amax_b)
        q = _payload(xb, mult, rounding, seed, offset, K, row0)
        return QuantResult(q, codes, np.float32(1.0), fmt, block, 0, int(np.sum(amax_b == 0)))
    s_enc, s_blk, g = tensor_scales(amax, T)
    codes, mult, n_sat, n_zero = _block_scales(amax_b, s_enc, s_blk, fmt)
    q = _payload(xb, mult, rounding, seed, offset, K, row0)
    return QuantResult(q, codes, g, fmt, block, n_sat, n_zero)


def _block_scales(amax_b, s_enc, s_blk, fmt):
    v = (amax_b * s_blk).astype(np.float32)          # float32 multiply, RNE
    codes = F.encode_scale(v, fmt)
    n_sat = int(np.sum(v.astype(np.float64) > F.SCALE_MAX[fmt]))
    zero = F.decode_scale(codes, fmt) == 0.0
    n_zero = int(np.sum(zero))
    codes = np.where(zero, F.SCALE_ONE_CODE[fmt], codes).astype(np.uint8)
    sval = F.decode_scale(codes, fmt).astype(np.float32)   # exact
    mult = (s_enc / sval).astype(np.float32)               # float32 division, RNE
    return codes, mult, n_sat, n_zero


def quantize_2d(w: np.ndarray, fmt: int, amax=None, T: float = 448.0) -> QuantResult:
    """Weight quantization with one scale per 16x16 tile (rows x K). The same codes serve
    the forward view (rows, K-contiguous) and, transposed, the data-gradient view."""
    if fmt == F.E8M0:
        raise ValueError("2D tiles use UE5M3 or E4M3 scales")
    w = np.asarray(w, dtype=np.float32)
    N, K = w.shape
    if N % 16 or K % 16:
        raise ValueError("2D tiles need both dimensions to be multiples of 16")
    t = w.reshape(N // 16, 16, K // 16, 16)
    amax_t = np.max(np.abs(t), axis=(1, 3))
    s_enc, s_blk, g = tensor_scales(amax, T)
    codes, mult, n_sat, n_zero = _block_scales(amax_t, s_enc, s_blk, fmt)
    r = (t * mult[:, None, :, None]).astype(np.float32)
    q = F.encode_e2m1(r).reshape(N, K)
    return QuantResult(q, codes, g, fmt, 16, n_sat, n_zero)


def transposed_view(x: np.ndarray, hadamard_n: int = 0) -> np.ndarray:
    """The weight-gradient operand view of x [tokens, features]: optional blockwise FWHT
    along tokens, then transposed to [features, tokens] so blocks run along tokens."""
    x = np.asarray(x, dtype=np.float32)
    if hadamard_n:
        x = fwht_tokens(x, hadamard_n)
    return np.ascontiguousarray(x.T)


def quantize_col(x: np.ndarray, fmt: int, block: int, amax=None, T: float = 448.0,
                 rounding: str = "rne", seed: int = 0, offset: int = 0, hadamard_n: int = 0) -> QuantResult:
    """Quantize the transposed (weight-gradient) view of x [tokens, features]."""
    return quantize_1d(transposed_view(x, hadamard_n), fmt, block, amax, T, rounding, seed, offset)


def tensor_amax(x: np.ndarray, hadamard_n: int = 0) -> np.float32:
    """max |x| over the tensor as it is quantized (after the FWHT for Hadamard views)."""
    x = np.asarray(x, dtype=np.float32)
    if hadamard_n:
        x = fwht_tokens(x, hadamard_n)
    return np.float32(np.max(np.abs(x))) if x.size else np.float32(0.0)


class AmaxCache:
    """Per-operand sample-and-hold amax cache.

    Sample (replace the cached amax with the amax observed at this step) when the cache is
    empty or step % D == 0, otherwise hold. The cache is not checkpointed, so a resumed run
    starts empty and samples on first use. D=1 is current scaling.
    """

    def __init__(self, D: int = 50):
        if D < 1:
            raise ValueError("D must be >= 1")
        self.D = D
        self.valid = False
        self.amax = np.float32(0.0)

    def needs_sample(self, step: int) -> bool:
        return (not self.valid) or step % self.D == 0

    def update(self, step: int, amax_obs) -> np.float32:
        if self.needs_sample(step):
            self.amax = np.float32(amax_obs)
            self.valid = True
        return self.amax

    def reset(self) -> None:
        self.valid = False
