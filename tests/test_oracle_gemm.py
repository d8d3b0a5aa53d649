"""Pins of the oracle's GEMM group model (CPU only)."""
import ctypes
import ctypes.util
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import formats as F
from oracle.exact import gemm_exact, round_fraction_f32
from oracle.gemm import rtz_add_f32, canonicalize, gemm_model, gemm_fp64

FE_TONEAREST, FE_TOWARDZERO = 0x000, 0xC00      # x86 <fenv.h>


def _pairs(n, seed):
    rng = np.random.default_rng(seed)
    a = (rng.standard_normal(n) * np.exp2(rng.integers(-30, 30, n))).astype(np.float32)
    b = (rng.standard_normal(n) * np.exp2(rng.integers(-30, 30, n))).astype(np.float32)
    b[: n // 8] = -a[: n // 8]                          # exact cancellation
    b[n // 8: n // 4] = np.nextafter(-a[n // 8: n // 4], np.float32(0))
    a[-4:] = [3.4e38, -3.4e38, 1e-45, -0.0]
    b[-4:] = [3.4e38, -3.0e38, -1e-45, -0.0]
    return a, b


def test_rtz_add_matches_exact_rounding():
    a, b = _pairs(20000, 1)
    got = rtz_add_f32(a, b)
    for i in range(len(a)):
        ref = round_fraction_f32(Fraction(float(a[i])) + Fraction(float(b[i])), "rtz")
        assert got[i] == np.float32(ref), (a[i], b[i], got[i], ref)


def test_rtz_add_matches_x86_sse_toward_zero():
    """Library/hardware pin: float32 addition under the C library's FE_TOWARDZERO mode."""
    libm = ctypes.CDLL(ctypes.util.find_library("m"))
    a, b = _pairs(200000, 2)
    a, b = a[:-4], b[:-4]
    assert libm.fesetround(FE_TOWARDZERO) == 0
    try:
        hw = np.add(a, b, dtype=np.float32)
    finally:
        libm.fesetround(FE_TONEAREST)
    assert np.array_equal(hw.view(np.uint32), rtz_add_f32(a, b).view(np.uint32))


def test_canonicalize_matches_torch_expression():
    c = np.concatenate([np.random.default_rng(3).standard_normal(100000) * 50,
                        (np.arange(-4096, 4096) + 0.5) / 1024]).astype(np.float32)
    t = torch.from_numpy(c)
    ref = (torch.round(1024 * t) / 1024).numpy()
    assert np.array_equal(canonicalize(c), ref)


def _rand_operand(rng, rows, K, block, fmt, spread):
    q = F.decode_e2m1(rng.integers(0, 16, (rows, K)))
    nb = K // block
    if fmt == F.E8M0:
        s = np.exp2(rng.integers(-spread, spread + 1, (rows, nb)).astype(np.float64))
    else:
        vals = F.SCALE_VALUES[fmt]
        mid = int(np.searchsorted(vals, 1.0))
        s = vals[np.clip(mid + rng.integers(-8 * spread, 8 * spread + 1, (rows, nb)), 1, len(vals) - 1)]
    return q, s


@pytest.mark.parametrize("fmt,block,spread", [(F.UE5M3, 16, 1), (F.UE5M3, 16, 6), (F.E4M3, 16, 4),
                                              (F.UE5M3, 32, 5), (F.E8M0, 32, 2), (F.E8M0, 32, 20)])
@pytest.mark.parametrize("canon", [False, True])
def test_group_model_matches_exact_rationals(fmt, block, spread, canon):
    rng = np.random.default_rng(hash((fmt, block, spread, canon)) % 2 ** 32)
    M, N, K = 5, 6, 256
    qa, sa = _rand_operand(rng, M, K, block, fmt, spread)
    qb, sb = _rand_operand(rng, N, K, block, fmt, spread)
    alpha = np.float32(0.000123)
    for reading in ("sequential", "single"):
        y = gemm_model(qa, sa, qb, sb, block, alpha=alpha, canon=canon, reading=reading)
        ref = np.array(gemm_exact(qa.tolist(), sa.tolist(), qb.tolist(), sb.tolist(), block, float(alpha), canon,
                                  reading), dtype=np.float32)
        assert np.array_equal(y.view(np.uint32), ref.view(np.uint32))


def test_adversarial_rounding_paths_are_exercised():
    """Scale spreads make group partials and cross-group sums inexact; the model must then
    differ from both plain float32 RNE accumulation and from the exact result."""
    rng = np.random.default_rng(11)
    M = N = 16
    K = 1024
    qa, sa = _rand_operand(rng, M, K, 16, F.UE5M3, 6)
    qb, sb = _rand_operand(rng, N, K, 16, F.UE5M3, 6)
    y = gemm_model(qa, sa, qb, sb, 16)
    seq = gemm_model(qa, sa, qb, sb, 16, reading="single")
    y64, _ = gemm_fp64(qa, sa, qb, sb, 16)
    assert np.any(y.astype(np.float64) != y64)
    assert np.any(y != seq)            # the two group readings really differ here


def test_k64_b32_is_correctly_rounded_dot():
    rng = np.random.default_rng(12)
    qa, sa = _rand_operand(rng, 8, 64, 32, F.E8M0, 30)
    qb, sb = _rand_operand(rng, 8, 64, 32, F.E8M0, 30)
    y = gemm_model(qa, sa, qb, sb, 32)
    for m in range(8):
        for n in range(8):
            exact = sum(Fraction(float(qa[m, k] * sa[m, k // 32])) * Fraction(float(qb[n, k] * sb[n, k // 32]))
                        for k in range(64))
            assert y[m, n] == np.float32(round_fraction_f32(exact, "rne"))


def test_unit_scales_give_exact_integer_products():
    rng = np.random.default_rng(13)
    qa = F.decode_e2m1(rng.integers(0, 16, (32, 512)))
    qb = F.decode_e2m1(rng.integers(0, 16, (24, 512)))
    ones_a, ones_b = np.ones((32, 32)), np.ones((24, 32))
    y = gemm_model(qa, ones_a, qb, ones_b, 16)
    ref = (np.round(qa * 2).astype(np.int64) @ np.round(qb * 2).astype(np.int64).T) / 4.0
    assert np.array_equal(y.astype(np.float64), ref)


def test_fp64_tolerance_on_tiny_workload():
    import synth
    cfg = synth.make_config(1)
    X, W = cfg["X"].values, cfg["W"].values
    qx = oracle.quantize_1d(X, F.UE5M3, 16, amax=float(np.abs(X).max()), T=448)
    qw = oracle.quantize_1d(W, F.UE5M3, 16, amax=float(np.abs(W).max()), T=448)
    a, sa = oracle.operand_from_quant(qx)
    b, sb = oracle.operand_from_quant(qw)
    alpha = oracle.output_scale(qx.g, qw.g)
    y = gemm_model(a, sa, b, sb, 16, alpha=alpha)
    y64, sabs = gemm_fp64(a, sa, b, sb, 16, qx.g, qw.g)
    assert np.all(np.abs(y - y64) <= 1e-6 * sabs)
