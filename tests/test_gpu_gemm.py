"""GEMM parity: HIP kernels vs the oracle's group model, bit for bit; float64 tolerance."""
import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import formats as OF
from tests._helpers import (assert_f32_bits_equal, dev_input, dev_scalar, qtensor_from_oracle, random_operand)

pytestmark = pytest.mark.gpu

fp4 = pytest.importorskip("fp4_block_scaled_tensor_amd")


def _oracle_y(qa, qb, va="1d", vb="1d", canon=False, hadamard_n=0, rows=None):
    a, sa = oracle.operand_from_quant(qa, va)
    b, sb = oracle.operand_from_quant(qb, vb)
    if rows is not None:
        a, sa = a[rows], sa[rows]
    alpha = oracle.output_scale(qa.g, qb.g, hadamard_n)
    return oracle.gemm_model(a, sa, b, sb, qa.block, alpha=alpha, canon=canon)


STRESS = [
    # fmt, block, spread, M, N, K, canon
    (OF.UE5M3, 16, 1, 64, 64, 64, False),
    (OF.UE5M3, 16, 6, 200, 136, 320, False),
    (OF.UE5M3, 16, 3, 129, 257, 1024, True),
    (OF.UE5M3, 32, 5, 96, 160, 576, False),
    (OF.E4M3, 16, 4, 130, 70, 448, False),
    (OF.E4M3, 32, 2, 64, 128, 256, True),
    (OF.E8M0, 32, 2, 200, 136, 320, False),
    (OF.E8M0, 32, 6, 128, 128, 512, False),
    (OF.E8M0, 32, 24, 160, 96, 1024, True),
    # whole 128 x 128 tiles with a partial last K stage (the clamped, not the interior, form)
    (OF.UE5M3, 16, 2, 128, 256, 320, False),
    (OF.E8M0, 32, 3, 256, 128, 576, False),
]


@pytest.mark.parametrize("fmt,block,spread,M,N,K,canon", STRESS)
def test_group_model_stress(fmt, block, spread, M, N, K, canon):
    """Operands built in the quantized domain with wide scale spreads inside each group,
    ragged M/N and a partial last K stage: every rounding rule of the model is exercised."""
    rng = np.random.default_rng(M * 7 + N * 3 + K + spread)
    qa = random_operand(rng, M, K, fmt, block, spread, zero_frac=0.1)
    qb = random_operand(rng, N, K, fmt, block, spread)
    qa.g, qb.g = np.float32(0.75), np.float32(1.25)
    want = _oracle_y(qa, qb, canon=canon)
    got = fp4.gemm_fprop(qtensor_from_oracle(qa), qtensor_from_oracle(qb), canon=canon)
    torch.cuda.synchronize()
    assert_f32_bits_equal(got, want, f"fmt={fmt} B={block} spread={spread} {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(256, 128, 2048), (200, 136, 1280), (128, 384, 4096)])
def test_mxfp4_outlier_blocks_then_fast_stages(M, N, K):
    """MXFP4 operands with narrow scale spreads except a few K-blocks of A raised by 2^7 (an
    outlier channel): the stages holding them fail the exponent-gap test and run group by
    group, the stages after them pass again. Covers whole-tile shapes (the unclamped interior
    form) and ragged ones."""
    rng = np.random.default_rng(M + N + K)
    qa = random_operand(rng, M, K, OF.E8M0, 32, 1, zero_frac=0.05)
    qb = random_operand(rng, N, K, OF.E8M0, 32, 2)
    nb = K // 32
    for blk in sorted(set(rng.integers(0, nb, 3).tolist()) | {nb // 2 + 1}):
        qa.scales[:, blk] = (qa.scales[:, blk].astype(np.int32) + 7).astype(np.uint8)
    want = _oracle_y(qa, qb)
    got = fp4.gemm_fprop(qtensor_from_oracle(qa), qtensor_from_oracle(qb))
    torch.cuda.synchronize()
    assert_f32_bits_equal(got, want, f"outlier blocks {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K,bad", [
    (128, 256, 256, []), (128, 256, 256, [0]), (128, 128, 768, [1]), (128, 128, 768, [0, 2]),
    (256, 128, 1280, [1, 2]), (128, 256, 2048, [0, 3, 4, 7]), (128, 128, 2048, [6, 7]),
    (200, 136, 1344, [0, 5])])
def test_mxfp4_failing_stages_at_chosen_positions(M, N, K, bad):
    """The fast stage loop runs passing 256-K stages two at a time (even, odd); a failing
    stage runs group by group and the loop re-aligns on the next even stage. Stages made to
    fail at chosen positions (first, last, even, odd, consecutive; one-stage and odd stage
    counts; a partial last stage and a ragged tile in the last case): one group of each bad
    stage has a block of A raised by 2^12, past the exponent-gap bound."""
    rng = np.random.default_rng(M * 3 + N + K + len(bad))
    qa = random_operand(rng, M, K, OF.E8M0, 32, 1)
    qb = random_operand(rng, N, K, OF.E8M0, 32, 1)
    for st in bad:
        blk = 8 * st + 2 * int(rng.integers(0, min(4, K // 64 - 4 * st)))   # K-block 0 of one of its groups
        qa.scales[:, blk] = (qa.scales[:, blk].astype(np.int32) + 12).astype(np.uint8)
    want = _oracle_y(qa, qb)
    got = fp4.gemm_fprop(qtensor_from_oracle(qa), qtensor_from_oracle(qb))
    torch.cuda.synchronize()
    assert_f32_bits_equal(got, want, f"failing stages {bad} {M}x{N}x{K}")


@pytest.mark.parametrize("fmt,block", [(OF.UE5M3, 16), (OF.E8M0, 32)])
def test_empty_k_writes_zeros(fmt, block):
    """K = 0: every output is an empty sum, +0 (the output buffer starts non-zero)."""
    qa = random_operand(np.random.default_rng(3), 64, 0, fmt, block, 1)
    qb = random_operand(np.random.default_rng(4), 40, 0, fmt, block, 1)
    out = torch.full((64, 40), 7.0, dtype=torch.float32, device="cuda")
    got = fp4.gemm_fprop(qtensor_from_oracle(qa), qtensor_from_oracle(qb), out=out)
    torch.cuda.synchronize()
    assert_f32_bits_equal(got, np.zeros((64, 40), np.float32), f"K=0 fmt={fmt}")


@pytest.mark.parametrize("fmt", [OF.UE5M3, OF.E4M3])
def test_zero_and_subnormal_scale_codes(fmt):
    """Hand-built operands whose block-scale codes include 0 (the value 0: the quantizer never
    writes it, the format allows it) and every subnormal code."""
    rng = np.random.default_rng(17 + fmt)
    qa = random_operand(rng, 96, 512, fmt, 16, 3)
    qb = random_operand(rng, 80, 512, fmt, 16, 3)
    qa.scales[rng.random(qa.scales.shape) < 0.15] = 0
    qb.scales[:, ::5] = rng.integers(0, 8, qb.scales[:, ::5].shape)
    want = _oracle_y(qa, qb)
    got = fp4.gemm_fprop(qtensor_from_oracle(qa), qtensor_from_oracle(qb))
    torch.cuda.synchronize()
    assert_f32_bits_equal(got, want, f"zero/subnormal scale codes fmt={fmt}")


def test_same_sign_rtz_drift():
    """All-positive products: every cross-group add truncates in the same direction."""
    rng = np.random.default_rng(5)
    for fmt, block, spread in ((OF.UE5M3, 16, 6), (OF.E8M0, 32, 12)):
        qa = random_operand(rng, 64, 4096, fmt, block, spread)
        qb = random_operand(rng, 64, 4096, fmt, block, spread)
        qa.codes &= 7
        qb.codes &= 7
        want = _oracle_y(qa, qb)
        got = fp4.gemm_fprop(qtensor_from_oracle(qa), qtensor_from_oracle(qb))
        torch.cuda.synchronize()
        assert_f32_bits_equal(got, want, f"drift fmt={fmt}")
        exact, _ = oracle.gemm_fp64(*oracle.operand_from_quant(qa), *oracle.operand_from_quant(qb), block)
        assert np.any(want.astype(np.float64) < exact)    # truncation really happened


def test_tiny_end_to_end():
    """256x256 fp32 X, W ~ N(0,1); UE5M3 block 16, T = 448, nearest-even; Y = X W^T; W both
    with 1D and with 2D 16x16 scales."""
    cfg = synth.make_config(1)
    X, W = cfg["X"], cfg["W"]
    Ax, Aw = oracle.tensor_amax(X.values), oracle.tensor_amax(W.values)
    qx = fp4.quantize(dev_input(X), fp4.UE5M3, 16, fp4.ROW, amax=dev_scalar(Ax), T=448)
    qw = fp4.quantize(dev_input(W), fp4.UE5M3, 16, fp4.ROW, amax=dev_scalar(Aw), T=448)
    w2, w2t = fp4.quantize(dev_input(W), fp4.UE5M3, 16, fp4.TILE2D, amax=dev_scalar(Aw), T=448)
    y1 = fp4.gemm_fprop(qx, qw)
    y2 = fp4.gemm_fprop(qx, w2)
    y3 = fp4.gemm_fprop(qx, w2, canon=True)
    torch.cuda.synchronize()
    rx = oracle.quantize_1d(X.values, OF.UE5M3, 16, amax=Ax, T=448)
    rw = oracle.quantize_1d(W.values, OF.UE5M3, 16, amax=Aw, T=448)
    rw2 = oracle.quantize_2d(W.values, OF.UE5M3, amax=Aw, T=448)
    assert_f32_bits_equal(y1, _oracle_y(rx, rw), "1D weight")
    assert_f32_bits_equal(y2, _oracle_y(rx, rw2, vb="2d"), "2D weight")
    assert_f32_bits_equal(y3, _oracle_y(rx, rw2, vb="2d", canon=True), "2D weight, canonicalised")
    a, sa = oracle.operand_from_quant(rx)
    b, sb = oracle.operand_from_quant(rw)
    y64, sabs = oracle.gemm_fp64(a, sa, b, sb, 16, rx.g, rw.g)
    assert np.all(np.abs(y1.cpu().numpy() - y64) <= 1e-6 * sabs)


@pytest.mark.parametrize("fmt,block", [(OF.UE5M3, 16), (OF.E4M3, 16), (OF.E8M0, 32)])
def test_format_sweep_2048(fmt, block):
    """2048^3 bf16 N(0,1) with 0.1% outlier columns, each format, quantize + GEMM on the GPU:
    every output bit-exact against the oracle's group model and within the tolerance of the
    float64 product."""
    cfg = synth.make_config(2)
    X, W = cfg["X"], cfg["W"]
    Ax, Aw = oracle.tensor_amax(X.values), oracle.tensor_amax(W.values)
    qx = fp4.quantize(dev_input(X), fmt, block, fp4.ROW, amax=dev_scalar(Ax), T=448)
    qw = fp4.quantize(dev_input(W), fmt, block, fp4.ROW, amax=dev_scalar(Aw), T=448)
    y = fp4.gemm_fprop(qx, qw)
    y_again = fp4.gemm_fprop(qx, qw)
    torch.cuda.synchronize()
    y = y.cpu().numpy()
    assert np.array_equal(y.view(np.uint32), y_again.cpu().numpy().view(np.uint32))   # run-to-run
    rx = oracle.quantize_1d(X.values, fmt, block, amax=Ax, T=448)
    rw = oracle.quantize_1d(W.values, fmt, block, amax=Aw, T=448)
    assert_f32_bits_equal(y, _oracle_y(rx, rw), f"fmt {fmt}")
    a, sa = oracle.operand_from_quant(rx)
    b, sb = oracle.operand_from_quant(rw)
    y64, sabs = oracle.gemm_fp64(a, sa, b, sb, block, rx.g, rw.g)
    assert np.all(np.abs(y - y64) <= 1e-6 * sabs)


def test_backward_dgrad_wgrad():
    """dX = dY W (2D weight, transposed copy) and dW = dY^T X (stochastic dY, T = 2048 for the
    wgrad dY view), with and without H16, at a reduced token count."""
    T_, Fo, Fi = 512, 256, 384
    dY = synth.Tensor("dY", synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(synth.normal((T_, Fo), 1e-3, 401))), "bf16")
    W = synth.Tensor("W", synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(synth.normal((Fo, Fi), 0.02, 402))), "bf16")
    X = synth.Tensor("X", synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(synth.student_t((T_, Fi), 3.0, 403))), "bf16")
    Ady, Aw = oracle.tensor_amax(dY.values), oracle.tensor_amax(W.values)
    # dgrad
    qdy = fp4.quantize(dev_input(dY), fp4.UE5M3, 16, fp4.ROW, amax=dev_scalar(Ady), T=448, stochastic=True, seed=42,
                       offset=0)
    _, wt = fp4.quantize(dev_input(W), fp4.UE5M3, 16, fp4.TILE2D, amax=dev_scalar(Aw), T=448)
    dx = fp4.gemm_dgrad(qdy, wt)
    torch.cuda.synchronize()
    rdy = oracle.quantize_1d(dY.values, OF.UE5M3, 16, amax=Ady, T=448, rounding="sr", seed=42, offset=0)
    rw = oracle.quantize_2d(W.values, OF.UE5M3, amax=Aw, T=448)
    assert_f32_bits_equal(dx, _oracle_y(rdy, rw, vb="2dT"), "dgrad")
    # wgrad
    for hn in (0, 16, 32):
        Ay, Ax = oracle.tensor_amax(dY.values, hn), oracle.tensor_amax(X.values, hn)
        qdyt = fp4.quantize(dev_input(dY), fp4.UE5M3, 16, fp4.COL, amax=dev_scalar(Ay), T=2048, stochastic=True,
                            seed=42, offset=1, hadamard_n=hn)
        qxt = fp4.quantize(dev_input(X), fp4.UE5M3, 16, fp4.COL, amax=dev_scalar(Ax), T=448, hadamard_n=hn)
        dw = fp4.gemm_wgrad(qdyt, qxt, hadamard_n=hn)
        torch.cuda.synchronize()
        rdyt = oracle.quantize_col(dY.values, OF.UE5M3, 16, amax=Ay, T=2048, rounding="sr", seed=42, offset=1,
                                   hadamard_n=hn)
        rxt = oracle.quantize_col(X.values, OF.UE5M3, 16, amax=Ax, T=448, hadamard_n=hn)
        assert_f32_bits_equal(dw, _oracle_y(rdyt, rxt, hadamard_n=hn), f"wgrad H{hn}")


def test_mxfp4_backward():
    T_, Fo, Fi = 256, 128, 192
    dY = synth.normal((T_, Fo), 1e-3, 11)
    X = synth.student_t((T_, Fi), 3.0, 12)
    W = synth.normal((Fo, Fi), 0.02, 13)
    qdy = fp4.quantize(torch.from_numpy(dY).cuda(), fp4.E8M0, 32, fp4.ROW, stochastic=True, seed=42, offset=0)
    qwt = fp4.quantize(torch.from_numpy(np.ascontiguousarray(W.T)).cuda(), fp4.E8M0, 32, fp4.ROW)
    qdyt = fp4.quantize(torch.from_numpy(dY).cuda(), fp4.E8M0, 32, fp4.COL, stochastic=True, seed=42, offset=1,
                        hadamard_n=16)
    qxt = fp4.quantize(torch.from_numpy(X).cuda(), fp4.E8M0, 32, fp4.COL, hadamard_n=16)
    dx = fp4.gemm_dgrad(qdy, qwt)
    dw = fp4.gemm_wgrad(qdyt, qxt, hadamard_n=16)
    torch.cuda.synchronize()
    rdy = oracle.quantize_1d(dY, OF.E8M0, 32, rounding="sr", seed=42, offset=0)
    rwt = oracle.quantize_1d(np.ascontiguousarray(W.T), OF.E8M0, 32)
    rdyt = oracle.quantize_col(dY, OF.E8M0, 32, rounding="sr", seed=42, offset=1, hadamard_n=16)
    rxt = oracle.quantize_col(X, OF.E8M0, 32, hadamard_n=16)
    assert_f32_bits_equal(dx, _oracle_y(rdy, rwt), "mx dgrad")
    assert_f32_bits_equal(dw, _oracle_y(rdyt, rxt, hadamard_n=16), "mx wgrad H16")


@pytest.mark.parametrize("fmt,block", [(OF.UE5M3, 16), (OF.E8M0, 32)])
def test_up_projection_full_size_sampled(fmt, block):
    """The 8192 x 4096 -> 14336 up-projection in full on the GPU (UE5M3: 2D weight scales;
    MXFP4: 1D block 32); 16 sampled output rows against the oracle."""
    cfg = synth.make_config(3)
    X, W = cfg["X"], cfg["W"]
    Ax, Aw = oracle.tensor_amax(X.values), oracle.tensor_amax(W.values)
    qx = fp4.quantize(dev_input(X), fmt, block, fp4.ROW, amax=dev_scalar(Ax), T=448)
    if fmt == OF.UE5M3:
        qw, _ = fp4.quantize(dev_input(W), fmt, 16, fp4.TILE2D, amax=dev_scalar(Aw), T=448)
    else:
        qw = fp4.quantize(dev_input(W), fmt, block, fp4.ROW)
    y = fp4.gemm_fprop(qx, qw)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 127, 128, 2047, 4096, 5000, 6143, 7000, 8000, 8100, 8150, 8189, 8190, 8191, 3333])
    y_rows = y[torch.from_numpy(rows).cuda()].cpu().numpy()
    rx = oracle.quantize_1d(X.values[rows], fmt, block, amax=Ax, T=448)
    if fmt == OF.UE5M3:
        rw = oracle.quantize_2d(W.values, fmt, amax=Aw, T=448)
        want = _oracle_y(rx, rw, vb="2d")
    else:
        rw = oracle.quantize_1d(W.values, fmt, block)
        want = _oracle_y(rx, rw)
    assert_f32_bits_equal(y_rows, want, f"up-projection fmt {fmt}")


def test_mxfp4_exact_range_edges_checked_mode():
    """MXFP4 operands whose block exponents reach both edges of the exact range (codes 65 and
    185 on both sides: combined exponents -124 and +116, the smallest nonzero partials 2^-126
    and group sums up to 2304 * 2^116) with wide in-group gaps: fp4_scale_range reports the
    code range, the checked mode accepts it and the GEMM is bit-exact against the oracle
    (including round-toward-zero accumulations that saturate at the largest float32). One
    code past the edge makes the checked mode raise FP4_ERANGE before anything runs."""
    rng = np.random.default_rng(81)
    M, N, K = 96, 64, 512
    pick = np.array([65, 185, 127, 100, 150], dtype=np.uint8)

    def operand(rows):
        codes = rng.integers(0, 16, (rows, K)).astype(np.uint8)
        sc = pick[rng.integers(0, len(pick), (rows, K // 32))]
        sc[0, 0], sc[1, 1] = 65, 185
        codes[2, :], sc[2, :] = 7, 185        # all +6 at the top exponent: output (2, 2) saturates
        return oracle.QuantResult(codes, sc, np.float32(1.0), OF.E8M0, 32)

    qa, qb = operand(M), operand(N)
    A, B = qtensor_from_oracle(qa), qtensor_from_oracle(qb)
    assert fp4.scale_range(A).cpu().tolist() == [65, 185]
    y = fp4.gemm_fprop(A, B, checked=True)
    torch.cuda.synchronize()
    with np.errstate(over="ignore"):
        want = _oracle_y(qa, qb)
    assert_f32_bits_equal(y, want, "MXFP4 at the exact-range edges")
    assert np.any(np.abs(want) == np.finfo(np.float32).max)      # some sums saturate under round-toward-zero
    qb.scales[5, 3] = 186
    with pytest.raises(fp4.FP4Error, match="FP4_ERANGE"):
        fp4.gemm_fprop(A, qtensor_from_oracle(qb), checked=True)
