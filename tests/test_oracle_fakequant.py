"""Pins of the oracle's inference fake quantization (CPU only): decode against exact
rationals, E8M0 fake quant against a brute-force nearest search on the block's scaled
codebook, an error bound for UE5M3 / E4M3, bfloat16 rounding against torch's cast, and
the activation-scale policies' order dependence."""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import formats as F
from oracle.exact import round_fraction_f32
from oracle.fakequant import scale_matrix


def _x(shape, seed, spread=3.0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape) * np.exp(rng.uniform(-spread, spread, (shape[0], 1)))
    return x.astype(np.float32)


@pytest.mark.parametrize("fmt,block,view", [(F.UE5M3, 16, "1d"), (F.E4M3, 32, "1d"), (F.E8M0, 32, "1d"),
                                            (F.UE5M3, 16, "2d"), (F.E4M3, 16, "2dT")])
def test_dequantize_matches_exact_rationals(fmt, block, view):
    x = _x((32, 64), 11)
    A = float(np.max(np.abs(x)))
    if view == "1d":
        qr = oracle.quantize_1d(x, fmt, block, amax=A, T=448)
    else:
        qr = oracle.quantize_2d(x, fmt, amax=A, T=448)
        if view == "2dT":
            qr = oracle.QuantResult(np.ascontiguousarray(qr.codes.T), qr.scales, qr.g, qr.fmt, 16)
    got = oracle.dequantize(qr, view)
    # element by element: the E2M1 value and the scale value from their bit fields, the
    # exact product with g (as the float32 it is), one rounding to float32
    e2m1 = [F._e2m1(c) for c in range(16)]
    scale_of = {F.UE5M3: F._ue5m3, F.E4M3: F._e4m3, F.E8M0: F._e8m0}[fmt]
    R, K = qr.codes.shape
    for r in range(R):
        for k in range(0, K, 7):
            if view == "1d":
                code = qr.scales[r, k // block]
            elif view == "2d":
                code = qr.scales[r // 16, k // 16]
            else:
                code = qr.scales[k // 16, r // 16]
            exact = Fraction(e2m1[qr.codes[r, k]]) * Fraction(scale_of(int(code)))
            if fmt != F.E8M0:
                exact *= Fraction(float(np.float32(qr.g)))
            want = round_fraction_f32(exact, "rne")
            assert np.float32(want) == got[r, k] and np.signbit(got[r, k]) == (qr.codes[r, k] >= 8 or want < 0), (r, k)


def test_e8m0_fake_quant_is_nearest_on_block_grid():
    """MXFP4: x_hat is the nearest point of the block's grid {c * 2^E}, ties to the even
    code, saturating at 6 * 2^E (brute force over the 16 codes)."""
    x = _x((64, 128), 12, spread=8.0)
    x[3, :32] = 0.0
    x[5, 40] = 7.9e-39          # a subnormal input
    y = oracle.fake_quant(x, F.E8M0, 32)
    qr = oracle.quantize_1d(x, F.E8M0, 32)
    E = qr.scales.astype(np.int64) - 127
    grid = np.array([F._e2m1(c) for c in range(16)])
    for r in range(x.shape[0]):
        for k in range(x.shape[1]):
            step = 2.0 ** E[r, k // 32]
            cand = grid * step
            d = np.abs(float(x[r, k]) - cand)
            best = np.flatnonzero(d == d.min())
            got = float(y[r, k])
            assert d.min() == abs(float(x[r, k]) - got), (r, k)
            if len(best) > 1 and cand[best[0]] != cand[best[1]]:
                # a genuine tie between two grid points: the even code wins
                code = [c for c in best if cand[c] == got][0]
                assert code % 2 == 0 or (code & 7) == 0, (r, k)


@pytest.mark.parametrize("fmt,block", [(F.UE5M3, 16), (F.E4M3, 16), (F.UE5M3, 32)])
def test_scaled_fake_quant_error_bound(fmt, block):
    """With the true amax cached, |x - x_hat| <= half the E2M1 step at |r| (0.25 below 2,
    0.5 below 4, 1 above, which also covers the slight overshoot past 6 that a rounded-down
    block scale allows), times S * g, up to float32 rounding of the scale factors."""
    x = _x((48, 128), 13)
    A = float(np.max(np.abs(x)))
    qr = oracle.quantize_1d(x, fmt, block, amax=A, T=448)
    y = oracle.dequantize(qr).astype(np.float64)
    S = scale_matrix(qr)
    g = float(np.float32(qr.g))
    r = np.abs(x.astype(np.float64)) / (S * g)
    half = np.where(r < 2, 0.25, np.where(r < 4, 0.5, 1.0))
    bound = half * S * g * (1 + 2.0 ** -20) + np.abs(x) * 2.0 ** -21
    assert np.all(np.abs(x - y) <= bound)
    # the bound is attained in order of magnitude (a dropped factor of S or g would break it)
    assert np.max(np.abs(x - y) / bound) > 0.5


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(14)
    y = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(1e3),
        (rng.integers(0, 2 ** 16, 4000).astype(np.uint32) << 16 | 0x8000).view(np.float32),   # exact ties
        np.array([0.0, -0.0, 1e-45, -1e-45, 3.0e38, 3.3961e38, 3.3895e38, -3.39e38, 1.0000001], np.float32),
    ])
    y = y[np.isfinite(y)]
    want = torch.from_numpy(y).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.f32_to_bf16_bits(y), want)


def test_policies_and_order_dependence():
    fmt, block = F.UE5M3, 16
    small, big = _x((32, 64), 15, spread=0.1), _x((32, 64), 16, spread=0.1) * np.float32(500.0)
    reqs = [small, big, small, big]
    # current scaling: every request uses its own amax
    cur = oracle.FakeQuantPolicy("current")
    for i, x in enumerate(reqs):
        assert np.array_equal(cur(i, x, fmt, block), oracle.fake_quant(x, fmt, block, amax=oracle.tensor_amax(x)))
    # delayed D=2: samples at requests 0 and 2, held at 1 and 3
    d2 = oracle.FakeQuantPolicy("delayed", D=2)
    amaxes = [oracle.tensor_amax(reqs[0])] * 2 + [oracle.tensor_amax(reqs[2])] * 2
    outs = [d2(i, x, fmt, block) for i, x in enumerate(reqs)]
    for i, x in enumerate(reqs):
        assert np.array_equal(outs[i], oracle.fake_quant(x, fmt, block, amax=amaxes[i]))
    # order dependence: the same big request gives a different result after a small one
    # (stale amax, saturated scales) than when it is sampled itself
    rev = oracle.FakeQuantPolicy("delayed", D=2)
    out_rev = [rev(i, x, fmt, block) for i, x in enumerate([big, small])]
    assert not np.array_equal(outs[1], out_rev[0])
    assert np.array_equal(out_rev[0], oracle.fake_quant(big, fmt, block, amax=oracle.tensor_amax(big)))
    # delayed with D=1 is current scaling; frozen ignores the data's amax
    d1 = oracle.FakeQuantPolicy("delayed", D=1)
    assert all(np.array_equal(d1(i, x, fmt, block), cur(i, x, fmt, block)) for i, x in enumerate(reqs))
    fr = oracle.FakeQuantPolicy("frozen", amax=2.0)
    for i, x in enumerate(reqs):
        assert np.array_equal(fr(i, x, fmt, block), oracle.fake_quant(x, fmt, block, amax=2.0))
