"""Deterministic Hadamard preconditioning of weight-gradient operands (oracle; test infrastructure only).

"技術概要：MXFP4 による大規模言語モデルの事前学習" (MXFP4 pretraining study on MI355X),
method section (手法) and findings (主要な貢献と知見): a fixed 16x16 (H16) or 32x32 (H32)
Hadamard rotation of the weight-gradient path restores stable full-MXFP4 training, where
random rotations and stochastic rounding do not. "Format-Aware Fusion for Fast FP4
Pretraining", abstract: fixed-sign 32-value Hadamard weight-gradient preconditioning.

Reading (the pages give no matrix or order): the Sylvester matrix H_n (no sign diagonal),
applied unnormalised to runs of n consecutive tokens of both wgrad operands, as a fast
Walsh-Hadamard transform with stages h = 1, 2, 4, ..., n/2; each stage maps every pair
(i, i+h) inside a block of 2h to (a+b, a-b) in float32. The factor 1/n is returned to
the weight-gradient GEMM's output scale, because H_n^T H_n = n I.
"""
from __future__ import annotations

import numpy as np


def fwht_tokens(x: np.ndarray, n: int) -> np.ndarray:
    """Blockwise unnormalised FWHT along axis 0 (tokens) in runs of n, float32 arithmetic."""
    if n not in (16, 32):
        raise ValueError("hadamard size must be 16 or 32")
    x = np.asarray(x, dtype=np.float32)
    T = x.shape[0]
    if T % n:
        raise ValueError("token count must be a multiple of the Hadamard size")
    rest = x.shape[1:]
    y = x.reshape((T // n, n) + rest).copy()
    h = 1
    while h < n:
        y = y.reshape((T // n, n // (2 * h), 2, h) + rest)
        a = y[:, :, 0]
        b = y[:, :, 1]
        y = np.stack([a + b, a - b], axis=2)
        h *= 2
    return y.reshape(x.shape).astype(np.float32)
