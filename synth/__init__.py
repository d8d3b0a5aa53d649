"""Seeded synthetic inputs shared by the oracle checks, the GPU parity tests and the benchmark.

This module only draws random tensors with the shapes and value distributions of the
block-scaled FP4 workloads (activations, weights, upstream gradients of LLM linear layers)
and rounds them to bfloat16 storage. It contains none of the quantization or GEMM
arithmetic, and imports neither the oracle nor the HIP library.

Every generator is NumPy ``Generator(PCG64(seed))``; bf16 storage is produced by
round-to-nearest-even on the float32 bit pattern.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "rng", "f32_to_bf16_bits", "bf16_bits_to_f32", "normal", "student_t",
    "scale_channels", "Tensor", "make_config", "CONFIG_NAMES", "LINEARS_8B",
    "C5_TOKENS", "C5_STEPS", "C5_CHECK_STEPS", "layer_base", "step_perm", "step_amp", "drift_np", "drift_torch",
]


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest, ties to even."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal(shape, std: float, seed: int) -> np.ndarray:
    return (rng(seed).standard_normal(shape, dtype=np.float32) * np.float32(std)).astype(np.float32)


def student_t(shape, nu: float, seed: int) -> np.ndarray:
    return rng(seed).standard_t(nu, size=shape).astype(np.float32)


def scale_channels(x: np.ndarray, n_channels: int, factor: float, seed: int) -> tuple[np.ndarray, np.ndarray]:
    """Multiply ``n_channels`` whole columns (the contraction dimension of an activation) by ``factor``."""
    cols = np.sort(rng(seed).choice(x.shape[1], size=n_channels, replace=False))
    y = x.copy()
    y[:, cols] *= np.float32(factor)
    return y, cols


@dataclass
class Tensor:
    """A synthetic input: storage dtype ``dtype`` ('bf16' or 'fp32') and its exact float32 values."""
    name: str
    values: np.ndarray            # float32, exactly the stored values
    dtype: str                    # 'bf16' | 'fp32'
    meta: dict = field(default_factory=dict)

    @property
    def bits(self) -> np.ndarray:
        """Raw storage: uint16 bf16 bits, or the float32 array itself."""
        if self.dtype == "bf16":
            return f32_to_bf16_bits(self.values)
        return self.values


def _as(name, x, dtype, **meta) -> Tensor:
    if dtype == "bf16":
        x = bf16_bits_to_f32(f32_to_bf16_bits(x))
    return Tensor(name, np.ascontiguousarray(x, dtype=np.float32), dtype, meta)


CONFIG_NAMES = {
    1: "tiny 256x256x256 fp32, UE5M3 B=16",
    2: "format sweep 2048^3 bf16 with 0.1% outlier channels",
    3: "Llama-3-8B MLP up-proj fprop 8192x4096 -> 14336",
    4: "Nemotron-H-8B down_proj backward, dY 8192x4096, W 4096x21504",
    5: "8B layer linear set at seq 8192, 100 steps",
}

# (name, in_features, out_features) of one 8B transformer layer's linears
LINEARS_8B = [("qkv", 4096, 6144), ("o", 4096, 4096), ("gate_up", 4096, 28672), ("down", 14336, 4096)]


def make_config(i: int, scale: float = 1.0, rows: int | None = None) -> dict:
    """Inputs of workload ``i`` (1..4). ``rows`` optionally truncates the token dimension
    (a row slice of the same seeded draw is NOT produced; a smaller draw with the same
    seed and distribution is), for quick CPU checks.
    """
    if i == 1:
        X = normal((256, 256), 1.0, 101)
        W = normal((256, 256), 1.0, 102)
        return {"X": _as("X", X, "fp32"), "W": _as("W", W, "fp32")}
    if i == 2:
        n = 2048 if rows is None else rows
        X = normal((n, 2048), 1.0, 201)
        W = normal((2048, 2048), 1.0, 202)
        X, cx = scale_channels(X, 2, 100.0, 203)
        W, cw = scale_channels(W, 2, 100.0, 204)
        return {"X": _as("X", X, "bf16", outlier_cols=cx), "W": _as("W", W, "bf16", outlier_cols=cw)}
    if i == 3:
        m = 8192 if rows is None else rows
        X = student_t((m, 4096), 3.0, 301)
        X, cx = scale_channels(X, 4, 100.0, 302)
        W = normal((14336, 4096), 0.02, 303)
        return {"X": _as("X", X, "bf16", outlier_cols=cx), "W": _as("W", W, "bf16")}
    if i == 4:
        m = 8192 if rows is None else rows
        dY = normal((m, 4096), 1e-3, 401)
        W = normal((4096, 21504), 0.02, 402)
        X = student_t((m, 21504), 3.0, 403)
        return {"dY": _as("dY", dY, "bf16"), "W": _as("W", W, "bf16"), "X": _as("X", X, "bf16")}
    raise ValueError(f"config {i} has per-step inputs; use layer_step_inputs()")


def layer_weight(layer: int, out_f: int, in_f: int) -> Tensor:
    """Fixed weight of linear ``layer`` of the 8B layer set (seed 500 + layer)."""
    return _as(f"W{layer}", normal((out_f, in_f), 0.02, 500 + layer), "bf16")


def layer_step_inputs(layer: int, step: int, tokens: int, in_f: int, out_f: int, drift: float = 1.02) -> dict:
    """Per-step activation X [tokens x in_f] (Student-t nu=3, 4 outlier channels x100) and upstream
    gradient dY [tokens x out_f] (N(0, 1e-3)), both scaled by drift**step."""
    amp = np.float32(drift ** step)
    X = student_t((tokens, in_f), 3.0, 100000 * (layer + 1) + 10 * step + 1)
    X, cx = scale_channels(X, 4, 100.0, 302 + layer)
    dY = normal((tokens, out_f), 1e-3, 100000 * (layer + 1) + 10 * step + 2)
    return {"X": _as("X", X * amp, "bf16", outlier_cols=cx), "dY": _as("dY", dY * amp, "bf16")}


# ---------------------------------------------------------------- 8B layer set at seq 8192
# Per-step inputs of the 8B layer set at its full size. Drawing 570M fresh random numbers per
# step is too slow for a test, so each layer's activation X and upstream gradient dY are one
# draw each (Student-t nu=3 with 4 outlier channels x100, and N(0, 1e-3)); the tensor of step s
# is that draw with its token rows shuffled by a seeded permutation of step s, times the
# amplitude drift**s, rounded to bf16. The shuffle changes which tokens share a weight-gradient
# block and every element's stochastic-rounding index from step to step; the drift moves the
# amax between the samples of a delayed amax cache. The same tensor comes from drift_np (host)
# and drift_torch (device): a row gather, one float32 multiply and a nearest-even bf16 cast.
C5_TOKENS = 8192
C5_STEPS = 100
C5_CHECK_STEPS = (0, 1, 49, 50, 51, 99)
_TENSOR_ID = {"X": 1, "dY": 2}


def layer_base(layer: int, tokens: int, in_f: int, out_f: int) -> dict:
    """The layer's fixed float32 draws: X [tokens x in_f] and dY [tokens x out_f]."""
    X = student_t((tokens, in_f), 3.0, 700000 + 10 * layer + 1)
    X, cx = scale_channels(X, 4, 100.0, 302 + layer)
    dY = normal((tokens, out_f), 1e-3, 700000 + 10 * layer + 2)
    return {"X": X, "dY": dY, "outlier_cols": cx}


def step_perm(layer: int, tensor: str, step: int, tokens: int) -> np.ndarray:
    """Token order of ``tensor`` ('X' or 'dY') of ``layer`` at ``step`` (int64 [tokens])."""
    return rng(800000 + 100000 * layer + 10 * step + _TENSOR_ID[tensor]).permutation(tokens).astype(np.int64)


def step_amp(step: int, drift: float = 1.02) -> np.float32:
    return np.float32(drift ** step)


def drift_np(Z: np.ndarray, perm: np.ndarray, amp) -> Tensor:
    """bf16(Z[perm] * amp) on the host, as a bf16 Tensor."""
    return _as("x", (Z[perm] * np.float32(amp)).astype(np.float32), "bf16")


def drift_torch(Zd, perm_d, amp):
    """The same tensor on the device: Zd float32 [tokens x n] and perm_d int64 device tensors."""
    import torch
    a = torch.tensor(float(np.float32(amp)), dtype=torch.float32, device=Zd.device)
    return (Zd.index_select(0, perm_d) * a).to(torch.bfloat16)
