"""Tile-local tensor scales: the CTA-local NVFP4 scale domain (oracle; test infrastructure
only).

Source: "Format-Aware Fusion for Fast FP4 Pretraining", abstract: quantization producers
are co-designed with their scale domain; besides native MXFP4 and global NVFP4 it names a
cooperative-thread-array-local NVFP4, i.e. the second-level (float32) tensor scale is
owned by the producing tile instead of the whole tensor, so quantization needs no global
amax pass.

Reading (listed in the design notes): the operand's rows are cut into stripes of R
consecutive rows (R a power of two from 16 to 128, dividing the GEMM's 128-row tile),
each stripe spanning the whole contraction dimension K. A stripe is quantized exactly
like a global-scale operand (UE5M3 approach rules: s_enc = 6T/A, s_blk = T/A, g = 1/s_enc,
nearest-even saturating block scales with the zero rule, nearest-even E2M1 payload) with A
the stripe's own amax (current scaling). Because a stripe spans K, a GEMM output (m, n)
sees one g per operand, and the epilogue factor becomes
alpha[m, n] = float32(g_a[m / R_a] * g_b[n / R_b]) (times 1/n_H for Hadamard wgrad).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .quantize import quantize_1d, tensor_amax

STRIPES = (16, 32, 64, 128)


@dataclass
class LocalQuant:
    codes: np.ndarray        # uint8 E2M1 codes [rows, K]
    scales: np.ndarray       # uint8 block-scale codes [rows, K/B]
    g: np.ndarray            # float32 [ceil(rows / stripe)] per-stripe decode scales
    amax: np.ndarray         # float32 [ceil(rows / stripe)] per-stripe amax
    fmt: int
    block: int
    stripe: int


def quantize_1d_local(x: np.ndarray, fmt: int, block: int, stripe: int = 16, T: float = 448.0,
                      rounding: str = "rne", seed: int = 0, offset: int = 0) -> LocalQuant:
    """ROW-view quantization of x [rows, K] with one tensor scale per stripe of rows.
    Stochastic rounding draws by the logical element index in the whole operand."""
    if stripe not in STRIPES:
        raise ValueError("stripe must be 16, 32, 64 or 128")
    x = np.asarray(x, dtype=np.float32)
    R, K = x.shape
    n = -(-R // stripe)
    codes = np.zeros((R, K), np.uint8)
    scales = np.zeros((R, K // block), np.uint8)
    g = np.zeros(n, np.float32)
    amax = np.zeros(n, np.float32)
    for i in range(n):
        rows = slice(i * stripe, min(R, (i + 1) * stripe))
        amax[i] = tensor_amax(x[rows])
        qr = quantize_1d(x[rows], fmt, block, amax=amax[i], T=T, rounding=rounding, seed=seed, offset=offset,
                         row0=i * stripe)
        codes[rows], scales[rows], g[i] = qr.codes, qr.scales, qr.g
    return LocalQuant(codes, scales, g, amax, fmt, block, stripe)


def stripe_alpha(g_a, stripe_a, g_b, stripe_b, M: int, N: int, hadamard_n: int = 0) -> np.ndarray:
    """Epilogue factor [M, N]: float32(g_a[m / R_a] * g_b[n / R_b]) [* 1/n], where a stripe
    size of 0 means a single tensor scale (g is one value)."""
    ga = np.asarray(g_a, np.float32).reshape(-1)
    gb = np.asarray(g_b, np.float32).reshape(-1)
    ra = ga[np.arange(M) // stripe_a] if stripe_a else np.full(M, ga[0], np.float32)
    rb = gb[np.arange(N) // stripe_b] if stripe_b else np.full(N, gb[0], np.float32)
    alpha = (ra[:, None] * rb[None, :]).astype(np.float32)
    if hadamard_n:
        alpha = (alpha * np.float32(1.0 / hadamard_n)).astype(np.float32)
    return alpha
