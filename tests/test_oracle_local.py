"""Pins of the oracle's tile-local (CTA-local NVFP4) scale domain (CPU only)."""
import numpy as np
import pytest

import oracle
from oracle import formats as F


def _x(rows, K, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, K)) * np.exp(rng.uniform(-4, 4, (rows, 1)))
    return x.astype(np.float32)


@pytest.mark.parametrize("fmt", [F.E4M3, F.UE5M3])
def test_one_stripe_is_global_current_scaling(fmt):
    x = _x(64, 256, 1)
    lq = oracle.quantize_1d_local(x, fmt, 16, stripe=64)
    qr = oracle.quantize_1d(x, fmt, 16, amax=oracle.tensor_amax(x), T=448)
    assert np.array_equal(lq.codes, qr.codes) and np.array_equal(lq.scales, qr.scales)
    assert lq.g.tolist() == [np.float32(qr.g)]


def test_rescaling_one_stripe_changes_only_its_g():
    """The scale domain is local: multiplying stripe 2 by 2^5 leaves every code and scale of
    every stripe unchanged and multiplies that stripe's g alone by 2^5 (a global scale
    would have moved every other stripe's block scales)."""
    x = _x(96, 128, 2)
    y = x.copy()
    y[32:48] *= np.float32(32.0)
    a = oracle.quantize_1d_local(x, F.E4M3, 16, stripe=16)
    b = oracle.quantize_1d_local(y, F.E4M3, 16, stripe=16)
    assert np.array_equal(a.codes, b.codes) and np.array_equal(a.scales, b.scales)
    ratio = b.g / a.g
    assert ratio[2] == 32.0 and np.all(np.delete(ratio, 2) == 1.0)
    glob_x = oracle.quantize_1d(x, F.E4M3, 16, amax=oracle.tensor_amax(x))
    glob_y = oracle.quantize_1d(y, F.E4M3, 16, amax=oracle.tensor_amax(y))
    assert not np.array_equal(glob_x.scales[:32], glob_y.scales[:32])


@pytest.mark.parametrize("fmt,T", [(F.E4M3, 448), (F.UE5M3, 448), (F.UE5M3, 2048)])
def test_stripe_maximum_block_lands_on_T(fmt, T):
    x = _x(128, 512, 3)
    lq = oracle.quantize_1d_local(x, fmt, 16, stripe=32, T=T)
    sv = F.SCALE_VALUES[fmt][lq.scales.astype(np.int64)]
    for i in range(4):
        blk = np.abs(x[i * 32:(i + 1) * 32]).reshape(32, -1, 16).max(axis=2)
        r, b = np.unravel_index(np.argmax(blk), blk.shape)
        assert sv[i * 32 + r, b] == T
        assert lq.amax[i] == np.max(np.abs(x[i * 32:(i + 1) * 32]))


def test_ragged_last_stripe_and_stripe_alpha_gemm_tolerance():
    xa, xb = _x(80, 256, 4), _x(72, 256, 5)
    qa = oracle.quantize_1d_local(xa, F.E4M3, 16, stripe=32)       # stripes 32, 32, 16
    qb = oracle.quantize_1d_local(xb, F.E4M3, 16, stripe=16)
    assert qa.g.shape == (3,) and qb.g.shape == (5,)
    A, sa = F.decode_e2m1(qa.codes), F.SCALE_VALUES[F.E4M3][qa.scales.astype(np.int64)]
    B, sb = F.decode_e2m1(qb.codes), F.SCALE_VALUES[F.E4M3][qb.scales.astype(np.int64)]
    alpha = oracle.stripe_alpha(qa.g, 32, qb.g, 16, 80, 72)
    assert alpha[33, 17] == np.float32(qa.g[1] * qb.g[1])
    y = oracle.gemm_model(A, sa, B, sb, 16, alpha=alpha)
    xa_hat = A * np.repeat(sa, 16, axis=1) * np.repeat(qa.g.astype(np.float64), 32)[:80, None]
    xb_hat = B * np.repeat(sb, 16, axis=1) * np.repeat(qb.g.astype(np.float64), 16)[:72, None]
    ref = xa_hat @ xb_hat.T
    mag = np.abs(xa_hat) @ np.abs(xb_hat).T
    assert np.all(np.abs(y - ref) <= 1e-6 * mag + 1e-30)
    # the float32 scalar-g path is the single-stripe special case
    a1 = oracle.stripe_alpha([qa.g[0]], 0, [qb.g[0]], 0, 80, 72)
    assert np.all(a1 == oracle.output_scale(qa.g[0], qb.g[0]))
