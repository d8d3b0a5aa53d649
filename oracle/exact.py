"""Exact-rational reference for tiny shapes (oracle; test infrastructure only).

An independent, element-by-element restatement of the group model with Python
Fractions and an integer rounding routine, used to pin the vectorised oracle in
oracle.gemm (which relies on float32 hardware arithmetic and a TwoSum construction).
Source of the model: "UE5M3 FP4 Block Scaling for Stable Language Model Pretraining",
approach section (접근 방법), software GEMM model bullet.
"""
from __future__ import annotations

import math
from fractions import Fraction

FLT_MAX = Fraction((2 ** 24 - 1) * 2 ** 104)


def round_fraction_f32(x: Fraction, mode: str) -> float:
    """Round an exact dyadic rational to float32 ('rne' or 'rtz'), with subnormals.
    Overflow: 'rne' gives +-inf, 'rtz' gives +-FLT_MAX."""
    x = Fraction(x)
    if x == 0:
        return 0.0
    sign = -1 if x < 0 else 1
    x = abs(x)
    n, d = x.numerator, x.denominator
    if d & (d - 1):
        raise ValueError("not a dyadic rational")
    e = -(d.bit_length() - 1)            # x = n * 2^e
    shift = max(n.bit_length() - 24, -149 - e)
    if shift > 0:
        q = n >> shift
        rem = n - (q << shift)
        half = 1 << (shift - 1)
        if mode == "rne" and (rem > half or (rem == half and q & 1)):
            q += 1
        elif mode not in ("rne", "rtz"):
            raise ValueError(mode)
        n, e = q, e + shift
    v = Fraction(n) * Fraction(2) ** e
    if v > FLT_MAX:
        return sign * (math.inf if mode == "rne" else float(FLT_MAX))
    return sign * float(v)


def gemm_exact(qa, sa, qb, sb, block: int, alpha: float = 1.0, canon: bool = False,
               reading: str = "sequential"):
    """Element-by-element group model with exact arithmetic; qa/qb/sa/sb as nested
    sequences or arrays of exactly representable numbers. Returns a list of lists."""
    M, K = len(qa), len(qa[0])
    N = len(qb)
    bpg = 64 // block
    out = []
    for m in range(M):
        row = []
        for n in range(N):
            acc = None
            for g in range(K // 64):
                parts = []
                for j in range(bpg):
                    b = g * bpg + j
                    s = Fraction(0)
                    for k in range(b * block, (b + 1) * block):
                        s += Fraction(float(qa[m][k])) * Fraction(float(qb[n][k]))
                    parts.append(s * Fraction(float(sa[m][b])) * Fraction(float(sb[n][b])))
                if reading == "sequential":
                    G = parts[0]
                    for t in parts[1:]:
                        G = Fraction(round_fraction_f32(G + t, "rne"))
                    G = Fraction(round_fraction_f32(G, "rne"))
                else:
                    G = Fraction(round_fraction_f32(sum(parts), "rne"))
                acc = G if acc is None else Fraction(round_fraction_f32(acc + G, "rtz"))
            if canon:
                v = acc * 1024
                fl = math.floor(v)
                r = v - fl
                k = fl + 1 if (r > Fraction(1, 2) or (r == Fraction(1, 2) and fl % 2 == 1)) else fl
                acc = Fraction(round_fraction_f32(Fraction(k, 1024), "rne"))
            row.append(round_fraction_f32(acc * Fraction(float(alpha)), "rne"))
        out.append(row)
    return out
