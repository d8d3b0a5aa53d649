"""Probe-matched block-scaled FP4 GEMM model and its float64 reference (oracle; test infrastructure only).

"UE5M3 FP4 Block Scaling for Stable Language Model Pretraining", approach section
(접근 방법), software GEMM model bullet, and key contributions (핵심 기여): the length-K dot
product is split into 64-product groups; each group becomes a float32 partial rounded to
nearest-even; groups are added in physical (K) order and an inexact cross-group addition
rounds toward zero; optionally the result is canonicalised onto the 1/1024 product
lattice with ties to even (torch.round(1024*c)/1024).

Readings (the design notes list them):
- A block of B products shares one scale pair, so its partial sum
  T_b = S_a * S_b * sum(q_a * q_b) is exact; inside a 64-group the block partials are
  added in K order with float32 round-to-nearest-even ('sequential'). For B=32 a group
  has two blocks and this equals one rounding of the exact group sum. The alternative
  reading, one rounding of the exact 64-product sum, is available as reading='single'.
- An exact zero block partial is +0. The first group initialises the accumulator
  (equivalently: the accumulator starts at +0 and every group is added toward zero, since
  +0 + G = G exactly and x + (-x) = +0 under round-toward-zero); canonicalisation, when enabled, acts on
  the accumulator before the output scale; the output scale is
  alpha = float32(g_a * g_b) [times 1/n for Hadamard-rotated weight-gradient operands],
  and y = float32(acc * alpha).

Operands are given as decoded payload values q [rows, K] (multiples of 0.5) and one scale
value per (row, block) [rows, K/B]; ``expand_2d_scales`` maps 16x16 tile scales to that.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

GROUP = 64


def expand_2d_scales(s2d: np.ndarray, transposed: bool) -> np.ndarray:
    """Per-(row, 16-block) scale values of a 2D-tiled weight.

    Forward view (rows = output features, K = input features): S[r, b] = s2d[r//16, b].
    Data-gradient view (the transposed weight; rows = input features, K = output
    features): S[r, b] = s2d[b, r//16]."""
    s2d = np.asarray(s2d)
    if transposed:
        s2d = s2d.T
    return np.repeat(s2d, 16, axis=0)


def _f32_exact(x: np.ndarray) -> bool:
    return bool(np.all(x.astype(np.float32).astype(np.float64) == x))


def rtz_add_f32(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """float32 a + b rounded toward zero.

    TwoSum in float64 gives s + e == a + b exactly with s = fl64(a + b). Let t be s
    truncated to float32. If t != s, a + b lies strictly between t and the next float32 away
    from zero, so the result is t. If t == s, the result is s unless e is non-zero with the
    opposite sign of s, in which case it is the next float32 toward zero. Overflow
    truncates to the largest finite float32."""
    a64 = np.asarray(a, dtype=np.float32).astype(np.float64)
    b64 = np.asarray(b, dtype=np.float32).astype(np.float64)
    s = a64 + b64
    bb = s - a64
    e = (a64 - (s - bb)) + (b64 - bb)
    with np.errstate(over="ignore"):
        t = s.astype(np.float32)
    away = np.abs(t.astype(np.float64)) > np.abs(s)
    t = np.where(away, np.nextafter(t, np.float32(0)), t)
    exact_f32 = t.astype(np.float64) == s
    step_in = exact_f32 & (e != 0) & (np.sign(e) != np.sign(s))
    return np.where(step_in, np.nextafter(t, np.float32(0)), t).astype(np.float32)


def _exact_sum_rne_f32(terms: list[np.ndarray]) -> np.ndarray:
    """float32 nearest-even of the exact sum of float64 terms (each an exact value)."""
    s = np.zeros_like(terms[0])
    err_any = np.zeros(terms[0].shape, dtype=bool)
    for t in terms:
        n = s + t
        bb = n - s
        e = (s - (n - bb)) + (t - bb)
        err_any |= e != 0
        s = n
    out = s.astype(np.float32)
    if np.any(err_any):
        # rare: float64 itself rounded; redo those elements with exact rationals
        idx = np.argwhere(err_any)
        from .exact import round_fraction_f32
        for ij in map(tuple, idx):
            out[ij] = np.float32(round_fraction_f32(sum(Fraction(float(t[ij])) for t in terms), "rne"))
    return out


def canonicalize(acc: np.ndarray) -> np.ndarray:
    """float32(round_half_even(1024 * acc) / 1024)."""
    acc = np.asarray(acc, dtype=np.float32)
    with np.errstate(over="ignore"):
        return (np.rint((acc * np.float32(1024.0)).astype(np.float32)) / np.float32(1024.0)).astype(np.float32)


def output_scale(g_a, g_b, hadamard_n: int = 0) -> np.float32:
    alpha = np.float32(np.float32(g_a) * np.float32(g_b))
    if hadamard_n:
        alpha = np.float32(alpha * np.float32(1.0 / hadamard_n))
    return alpha


def gemm_model(qa: np.ndarray, sa: np.ndarray, qb: np.ndarray, sb: np.ndarray, block: int,
               alpha=np.float32(1.0), canon: bool = False, reading: str = "sequential",
               return_acc: bool = False) -> np.ndarray:
    """y[m, n] of A[M, K] . B[N, K]^T under the group model.

    qa, qb: decoded payload values (float64, multiples of 0.5); sa [M, K/block], sb [N, K/block]:
    decoded scale values per (row, block)."""
    qa = np.asarray(qa, dtype=np.float64)
    qb = np.asarray(qb, dtype=np.float64)
    sa = np.asarray(sa, dtype=np.float64)
    sb = np.asarray(sb, dtype=np.float64)
    M, K = qa.shape
    N = qb.shape[0]
    if qb.shape[1] != K or K % GROUP or GROUP % block:
        raise ValueError("shapes: K must match and be a multiple of 64; block must divide 64")
    bpg = GROUP // block
    acc = None
    for g in range(K // GROUP):
        T = []
        for j in range(bpg):
            b = g * bpg + j
            ks = slice(b * block, (b + 1) * block)
            I = qa[:, ks] @ qb[:, ks].T          # multiples of 1/4, |I| <= 36*block: exact
            Tb = I * sa[:, b][:, None] * sb[:, b][None, :]   # exact (<= 21 significant bits)
            T.append(Tb + 0.0)        # an exact zero partial is +0 (no signed zero from the BLAS order)
        if reading == "sequential":
            for Tb in T:
                if not _f32_exact(Tb):
                    raise ValueError("block partial outside float32 range (out of contract)")
            G = T[0].astype(np.float32)
            for Tb in T[1:]:
                G = (G + Tb.astype(np.float32)).astype(np.float32)   # float32 add, RNE
        elif reading == "single":
            G = _exact_sum_rne_f32(T)
        else:
            raise ValueError(reading)
        acc = G if acc is None else rtz_add_f32(acc, G)
    if canon:
        acc = canonicalize(acc)
    y = (acc * np.float32(alpha)).astype(np.float32)
    return (y, acc) if return_acc else y


def gemm_fp64(qa, sa, qb, sb, block: int, g_a=1.0, g_b=1.0, hadamard_n: int = 0):
    """float64 product of the decoded operands, and sum |products| per output (for the
    relative tolerance of the group model)."""
    xa = np.asarray(qa, np.float64) * np.repeat(np.asarray(sa, np.float64), block, axis=1) * float(g_a)
    xb = np.asarray(qb, np.float64) * np.repeat(np.asarray(sb, np.float64), block, axis=1) * float(g_b)
    f = 1.0 / hadamard_n if hadamard_n else 1.0
    return (xa @ xb.T) * f, (np.abs(xa) @ np.abs(xb).T) * f


def operand_from_quant(qr, view: str = "1d"):
    """(decoded payload [rows, K], per-(row, block) scale values) of an oracle QuantResult.
    view: '1d' | '2d' (forward weight view) | '2dT' (transposed weight view)."""
    from .formats import decode_e2m1, SCALE_VALUES
    sv = SCALE_VALUES[qr.fmt][qr.scales.astype(np.int64)]
    if view == "1d":
        return decode_e2m1(qr.codes), sv
    if view == "2d":
        return decode_e2m1(qr.codes), expand_2d_scales(sv, transposed=False)
    if view == "2dT":
        return decode_e2m1(np.ascontiguousarray(qr.codes.T)), expand_2d_scales(sv, transposed=True)
    raise ValueError(view)
