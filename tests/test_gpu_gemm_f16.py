"""The decode-once route for UE5M3 / E4M3 GEMMs: fp4_decode_f16 and fp4_gemm_f16.

"UE5M3 FP4 Block Scaling for Stable Language Model Pretraining", approach (the software GEMM
model) and limits (no native UE5M3 hardware: an exact software route). The decode writes each
operand once as fp16 E2M1(q) * S * 2^-3; the GEMM over the two decodes follows the same group
model as fp4_gemm_fprop / _dgrad / _wgrad.

Parity: the decoded values equal the oracle's decoded payload times its block-scale values
times 2^-3, exactly, in every scale layout; the GEMM equals the oracle's group model bit for
bit on the stress operands, zero and subnormal scale codes, the tiny workload, the backward
pair (2D weight's transposed view, stochastic dY, H0/H16/H32), tile-local g, and sampled rows
of the full-size up-projection.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import formats as OF
from tests._helpers import assert_f32_bits_equal, dev_input, dev_scalar, qtensor_from_oracle, random_operand

pytestmark = pytest.mark.gpu

fp4 = pytest.importorskip("fp4_block_scaled_tensor_amd")


def _oracle_y(qa, qb, va="1d", vb="1d", canon=False, hadamard_n=0, rows=None):
    a, sa = oracle.operand_from_quant(qa, va)
    b, sb = oracle.operand_from_quant(qb, vb)
    if rows is not None:
        a, sa = a[rows], sa[rows]
    return oracle.gemm_model(a, sa, b, sb, qa.block, alpha=oracle.output_scale(qa.g, qb.g, hadamard_n), canon=canon)


def _decoded(qr, view="1d"):
    """The oracle's decoded operand times 2^-3 (float64), expanded to one value per element."""
    a, sv = oracle.operand_from_quant(qr, view)
    rows, k = a.shape
    B = k // sv.shape[1]
    return a.astype(np.float64) * np.repeat(sv.astype(np.float64), B, axis=1) * 0.125


@pytest.mark.parametrize("fmt,block,rows,K,spread", [
    (OF.UE5M3, 16, 72, 256, 6), (OF.UE5M3, 32, 130, 320, 4), (OF.E4M3, 16, 64, 576, 3), (OF.E4M3, 32, 33, 128, 2)])
def test_decode_f16_1d_exact(fmt, block, rows, K, spread):
    rng = np.random.default_rng(rows + K)
    qr = random_operand(rng, rows, K, fmt, block, spread, zero_frac=0.1)
    qr.scales[:, ::7] = rng.integers(0, 8, qr.scales[:, ::7].shape)      # zero and subnormal codes
    got = fp4.decode_f16(qtensor_from_oracle(qr))
    torch.cuda.synchronize()
    g = got.cpu().numpy().astype(np.float64)
    want = _decoded(qr)
    assert np.array_equal(g, want), f"{int(np.sum(g != want))} decoded values differ"
    assert np.array_equal(np.signbit(g), np.signbit(want)), "signs of zeros differ"


@pytest.mark.parametrize("fmt", [OF.UE5M3, OF.E4M3])
def test_decode_f16_2d_views_exact(fmt):
    W = synth.normal((128, 192), 0.02, 77)      # both views have K a multiple of 64
    rw = oracle.quantize_2d(W, fmt, amax=oracle.tensor_amax(W), T=448)
    for view in ("2d", "2dT"):
        got = fp4.decode_f16(qtensor_from_oracle(rw, view))
        torch.cuda.synchronize()
        assert np.array_equal(got.cpu().numpy().astype(np.float64), _decoded(rw, view)), view


STRESS = [
    # fmt, block, spread, M, N, K, canon
    (OF.UE5M3, 16, 1, 64, 64, 64, False),
    (OF.UE5M3, 16, 6, 200, 136, 320, False),
    (OF.UE5M3, 16, 3, 129, 257, 1024, True),
    (OF.UE5M3, 32, 5, 96, 160, 576, False),
    (OF.E4M3, 16, 4, 130, 70, 448, False),
    (OF.E4M3, 32, 2, 64, 128, 256, True),
    (OF.UE5M3, 16, 2, 128, 256, 320, False),
    (OF.E4M3, 16, 3, 256, 384, 1024, False),
]


@pytest.mark.parametrize("fmt,block,spread,M,N,K,canon", STRESS)
def test_gemm_f16_group_model_stress(fmt, block, spread, M, N, K, canon):
    rng = np.random.default_rng(M * 7 + N * 3 + K + spread)
    qa = random_operand(rng, M, K, fmt, block, spread, zero_frac=0.1)
    qb = random_operand(rng, N, K, fmt, block, spread)
    qa.g, qb.g = np.float32(0.75), np.float32(1.25)
    want = _oracle_y(qa, qb, canon=canon)
    got = fp4.gemm_f16(qtensor_from_oracle(qa), qtensor_from_oracle(qb), canon=canon)
    torch.cuda.synchronize()
    assert_f32_bits_equal(got, want, f"fmt={fmt} B={block} spread={spread} {M}x{N}x{K}")


@pytest.mark.parametrize("fmt", [OF.UE5M3, OF.E4M3])
def test_gemm_f16_zero_and_subnormal_scale_codes(fmt):
    rng = np.random.default_rng(117 + fmt)
    qa = random_operand(rng, 96, 512, fmt, 16, 3)
    qb = random_operand(rng, 80, 512, fmt, 16, 3)
    qa.scales[rng.random(qa.scales.shape) < 0.15] = 0
    qb.scales[:, ::5] = rng.integers(0, 8, qb.scales[:, ::5].shape)
    got = fp4.gemm_f16(qtensor_from_oracle(qa), qtensor_from_oracle(qb))
    torch.cuda.synchronize()
    assert_f32_bits_equal(got, _oracle_y(qa, qb), f"zero/subnormal scale codes fmt={fmt}")


def test_gemm_f16_tiny_end_to_end():
    cfg = synth.make_config(1)
    X, W = cfg["X"], cfg["W"]
    Ax, Aw = oracle.tensor_amax(X.values), oracle.tensor_amax(W.values)
    qx = fp4.quantize(dev_input(X), fp4.UE5M3, 16, fp4.ROW, amax=dev_scalar(Ax), T=448)
    w2, _ = fp4.quantize(dev_input(W), fp4.UE5M3, 16, fp4.TILE2D, amax=dev_scalar(Aw), T=448)
    y = fp4.gemm_f16(qx, w2)
    yc = fp4.gemm_f16(qx, w2, canon=True)
    torch.cuda.synchronize()
    rx = oracle.quantize_1d(X.values, OF.UE5M3, 16, amax=Ax, T=448)
    rw2 = oracle.quantize_2d(W.values, OF.UE5M3, amax=Aw, T=448)
    assert_f32_bits_equal(y, _oracle_y(rx, rw2, vb="2d"), "2D weight")
    assert_f32_bits_equal(yc, _oracle_y(rx, rw2, vb="2d", canon=True), "2D weight, canonicalised")


def test_gemm_f16_backward_dgrad_wgrad():
    T_, Fo, Fi = 512, 256, 384
    dY = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(synth.normal((T_, Fo), 1e-3, 401)))
    W = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(synth.normal((Fo, Fi), 0.02, 402)))
    X = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(synth.student_t((T_, Fi), 3.0, 403)))
    Ady, Aw = oracle.tensor_amax(dY), oracle.tensor_amax(W)
    qdy = fp4.quantize(torch.from_numpy(dY).cuda(), fp4.UE5M3, 16, fp4.ROW, amax=dev_scalar(Ady), T=448,
                       stochastic=True, seed=42, offset=0)
    _, wt = fp4.quantize(torch.from_numpy(W).cuda(), fp4.UE5M3, 16, fp4.TILE2D, amax=dev_scalar(Aw), T=448)
    dx = fp4.gemm_f16(qdy, wt)
    torch.cuda.synchronize()
    rdy = oracle.quantize_1d(dY, OF.UE5M3, 16, amax=Ady, T=448, rounding="sr", seed=42, offset=0)
    rw = oracle.quantize_2d(W, OF.UE5M3, amax=Aw, T=448)
    assert_f32_bits_equal(dx, _oracle_y(rdy, rw, vb="2dT"), "dgrad")
    for hn in (0, 16, 32):
        Ay, Ax = oracle.tensor_amax(dY, hn), oracle.tensor_amax(X, hn)
        qdyt = fp4.quantize(torch.from_numpy(dY).cuda(), fp4.UE5M3, 16, fp4.COL, amax=dev_scalar(Ay), T=2048,
                            stochastic=True, seed=42, offset=1, hadamard_n=hn)
        qxt = fp4.quantize(torch.from_numpy(X).cuda(), fp4.UE5M3, 16, fp4.COL, amax=dev_scalar(Ax), T=448,
                           hadamard_n=hn)
        dw = fp4.gemm_f16(qdyt, qxt, hadamard_n=hn)
        torch.cuda.synchronize()
        rdyt = oracle.quantize_col(dY, OF.UE5M3, 16, amax=Ay, T=2048, rounding="sr", seed=42, offset=1, hadamard_n=hn)
        rxt = oracle.quantize_col(X, OF.UE5M3, 16, amax=Ax, T=448, hadamard_n=hn)
        assert_f32_bits_equal(dw, _oracle_y(rdyt, rxt, hadamard_n=hn), f"wgrad H{hn}")


def test_gemm_f16_tile_local_g():
    """Tile-local operands (one g per 32- and 16-row stripe) through the decode-once route."""
    M, N, K = 200, 176, 512
    xa = synth.normal((M, K), 1.0, 61)
    xb = synth.normal((N, K), 1.0, 62)
    la = oracle.quantize_1d_local(xa, OF.E4M3, 16, stripe=32)
    lb = oracle.quantize_1d_local(xb, OF.E4M3, 16, stripe=16)

    def dev(lq):
        rows, k = lq.codes.shape
        return fp4.QTensor(torch.from_numpy(oracle.pack_codes(lq.codes)).cuda(),
                           torch.from_numpy(np.ascontiguousarray(lq.scales)).cuda(),
                           torch.from_numpy(lq.g.copy()).cuda(), lq.fmt, lq.block, fp4.FP4_SCALES_1D, rows, k,
                           g_stripe=lq.stripe)

    A, sa = OF.decode_e2m1(la.codes), OF.SCALE_VALUES[la.fmt][la.scales.astype(np.int64)]
    B, sb = OF.decode_e2m1(lb.codes), OF.SCALE_VALUES[lb.fmt][lb.scales.astype(np.int64)]
    want = oracle.gemm_model(A, sa, B, sb, 16, alpha=oracle.stripe_alpha(la.g, 32, lb.g, 16, M, N))
    y = fp4.gemm_f16(dev(la), dev(lb))
    torch.cuda.synchronize()
    assert_f32_bits_equal(y, want, "tile-local g")


def test_gemm_f16_up_projection_full_size_sampled():
    """8192 x 4096 -> 14336 with 2D UE5M3 weight scales through the decode-once route: sampled
    rows against the oracle."""
    cfg = synth.make_config(3)
    X, W = cfg["X"], cfg["W"]
    Ax, Aw = oracle.tensor_amax(X.values), oracle.tensor_amax(W.values)
    qx = fp4.quantize(dev_input(X), OF.UE5M3, 16, fp4.ROW, amax=dev_scalar(Ax), T=448)
    qw, _ = fp4.quantize(dev_input(W), OF.UE5M3, 16, fp4.TILE2D, amax=dev_scalar(Aw), T=448)
    y = fp4.gemm_f16(qx, qw)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 127, 128, 2047, 4096, 6143, 8191])
    rx = oracle.quantize_1d(X.values[rows], OF.UE5M3, 16, amax=Ax, T=448)
    rw = oracle.quantize_2d(W.values, OF.UE5M3, amax=Aw, T=448)
    want = _oracle_y(rx, rw, vb="2d")
    assert_f32_bits_equal(y[torch.from_numpy(rows).cuda()].cpu().numpy(), want, "up-projection rows")


def test_gemm_f16_rejects_mxfp4_and_missing_decode():
    rng = np.random.default_rng(9)
    qa = qtensor_from_oracle(random_operand(rng, 64, 128, OF.E8M0, 32, 1))
    qb = qtensor_from_oracle(random_operand(rng, 64, 128, OF.E8M0, 32, 1))
    with pytest.raises(fp4.FP4Error):
        fp4.decode_f16(qa)
    d = torch.zeros((64, 128), dtype=torch.float16, device="cuda")
    with pytest.raises(fp4.FP4Error):
        fp4.gemm_f16(qa, qb, a16=d, b16=d)
