"""Helpers shared by the GPU parity tests (moving synthetic inputs and oracle results
between NumPy and device tensors; no method arithmetic)."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from oracle import formats as OF


def dev_input(t) -> torch.Tensor:
    """A synth.Tensor as a device tensor of its storage dtype."""
    if t.dtype == "bf16":
        return torch.from_numpy(t.bits.view(np.int16).copy()).view(torch.bfloat16).cuda()
    return torch.from_numpy(t.values.copy()).cuda()


def dev_f32(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def dev_scalar(v) -> torch.Tensor:
    return torch.tensor([np.float32(v)], dtype=torch.float32, device="cuda")


def qtensor_from_oracle(qr: oracle.QuantResult, view: str = "1d"):
    """Upload an oracle quantization as a GEMM operand (the oracle's bytes, not the kernel's)."""
    import fp4_block_scaled_tensor_amd as fp4
    g = dev_scalar(qr.g)
    if view == "1d":
        rows, k = qr.codes.shape
        q = torch.from_numpy(oracle.pack_codes(qr.codes)).cuda()
        s = torch.from_numpy(np.ascontiguousarray(qr.scales)).cuda()
        return fp4.QTensor(q, s, g, qr.fmt, qr.block, fp4.FP4_SCALES_1D, rows, k)
    if view == "2d":
        rows, k = qr.codes.shape
        q = torch.from_numpy(oracle.pack_codes(qr.codes)).cuda()
        s = torch.from_numpy(np.ascontiguousarray(qr.scales)).cuda()
        return fp4.QTensor(q, s, g, qr.fmt, 16, fp4.FP4_SCALES_2D, rows, k)
    if view == "2dT":
        codes_t = np.ascontiguousarray(qr.codes.T)
        rows, k = codes_t.shape
        q = torch.from_numpy(oracle.pack_codes(codes_t)).cuda()
        s = torch.from_numpy(np.ascontiguousarray(qr.scales)).cuda()
        return fp4.QTensor(q, s, g, qr.fmt, 16, fp4.FP4_SCALES_2D_T, rows, k)
    raise ValueError(view)


def assert_bytes_equal(got: torch.Tensor, want: np.ndarray, what: str):
    g = got.cpu().numpy()
    w = np.asarray(want)
    assert g.shape == w.shape, f"{what}: shape {g.shape} != {w.shape}"
    bad = np.argwhere(g != w)
    assert len(bad) == 0, f"{what}: {len(bad)} of {g.size} differ; first at {tuple(bad[0])}: got {g[tuple(bad[0])]}, want {w[tuple(bad[0])]}"


def assert_f32_bits_equal(got, want: np.ndarray, what: str):
    g = got.cpu().numpy() if isinstance(got, torch.Tensor) else np.asarray(got)
    g = np.ascontiguousarray(g, dtype=np.float32).view(np.uint32)
    w = np.ascontiguousarray(want, dtype=np.float32).view(np.uint32)
    assert g.shape == w.shape, f"{what}: shape {g.shape} != {w.shape}"
    bad = np.argwhere(g != w)
    if len(bad):
        i = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} of {g.size} floats differ; first at {i}: got "
                             f"{g[i:][0] if False else np.array(g[i]).view(np.float32)!r} want {np.array(w[i]).view(np.float32)!r}")


def random_operand(rng, rows, K, fmt, block, spread, zero_frac=0.0):
    """An operand built directly in the quantized domain (payload codes, scale codes), for
    GEMM stress cases that the quantizer would rarely produce."""
    codes = rng.integers(0, 16, (rows, K)).astype(np.uint8)
    if zero_frac:
        codes[rng.random((rows, K)) < zero_frac] = 0
    nb = K // block
    if fmt == OF.E8M0:
        sc = (127 + rng.integers(-spread, spread + 1, (rows, nb))).astype(np.uint8)
    else:
        vals = OF.SCALE_VALUES[fmt]
        mid = int(np.searchsorted(vals, 1.0))
        sc = np.clip(mid + rng.integers(-8 * spread, 8 * spread + 1, (rows, nb)), 1, len(vals) - 1).astype(np.uint8)
    return oracle.QuantResult(codes, sc, np.float32(1.0), fmt, block)
