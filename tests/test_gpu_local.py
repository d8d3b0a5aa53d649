"""Tile-local (CTA-local NVFP4) tensor scales: the stripe quantizer bit-exact against the
oracle, and the three GEMMs with per-stripe g in their epilogue bit-exact against the
oracle's group model with the per-(row-stripe, col-stripe) factor."""
import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import formats as OF
from tests._helpers import assert_bytes_equal, assert_f32_bits_equal, dev_input, dev_scalar, qtensor_from_oracle

pytestmark = pytest.mark.gpu

fp4 = pytest.importorskip("fp4_block_scaled_tensor_amd")


def _tensor(rows, cols, dtype, seed):
    x = synth.student_t((rows, cols), 3.0, seed)
    x = x * np.exp(np.random.default_rng(seed).uniform(-3, 3, (rows, 1))).astype(np.float32)   # per-row magnitudes
    if dtype == "bf16":
        return synth.Tensor("x", synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(x)), "bf16")
    return synth.Tensor("x", x.astype(np.float32), dtype)


CASES = [
    # name, rows, cols, dtype, fmt, block, stripe, sr, T
    ("e4m3_s16", 256, 512, "bf16", OF.E4M3, 16, 16, False, 448),
    ("e4m3_s128_ragged", 200, 256, "bf16", OF.E4M3, 16, 128, False, 448),
    ("ue5m3_s32_fp32", 96, 160, "fp32", OF.UE5M3, 16, 32, False, 448),
    ("ue5m3_b32_s64", 130, 96, "bf16", OF.UE5M3, 32, 64, False, 2048),
    ("e4m3_s16_sr", 64, 1024, "bf16", OF.E4M3, 16, 16, True, 448),
]


@pytest.mark.parametrize("name,rows,cols,dtype,fmt,block,stripe,sr,T", CASES, ids=[c[0] for c in CASES])
def test_quantize_local_matches_oracle(name, rows, cols, dtype, fmt, block, stripe, sr, T):
    t = _tensor(rows, cols, dtype, 6000 + rows + cols)
    ref = oracle.quantize_1d_local(t.values, fmt, block, stripe=stripe, T=T, rounding="sr" if sr else "rne",
                                   seed=42, offset=5)
    obs = torch.empty(len(ref.g), dtype=torch.float32, device="cuda")
    got = fp4.quantize_local(dev_input(t), fmt, block, stripe=stripe, T=T, stochastic=sr, seed=42, offset=5,
                             amax_obs=obs)
    torch.cuda.synchronize()
    assert_bytes_equal(got.q, oracle.pack_codes(ref.codes), f"{name} payload")
    assert_bytes_equal(got.s, ref.scales, f"{name} scales")
    assert_f32_bits_equal(got.g, ref.g, f"{name} g")
    assert_f32_bits_equal(obs, ref.amax, f"{name} amax")


def test_quantize_local_single_and_two_pass_forms():
    """Both launch forms against the oracle: one workgroup per stripe when there are at least
    two stripes per compute unit, and the two-pass form (stripe maxima by (column chunk,
    stripe) workgroups, then the row quantizer with per-stripe scales) below that."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for name, rows, cols, stripe in (("single_pass", 2 * cus * 16, 64, 16), ("two_pass", 384, 2048, 128)):
        t = _tensor(rows, cols, "bf16", 6100 + rows)
        ref = oracle.quantize_1d_local(t.values, OF.E4M3, 16, stripe=stripe, T=448.0)
        obs = torch.empty(len(ref.g), dtype=torch.float32, device="cuda")
        got = fp4.quantize_local(dev_input(t), OF.E4M3, 16, stripe=stripe, amax_obs=obs)
        torch.cuda.synchronize()
        assert_bytes_equal(got.q, oracle.pack_codes(ref.codes), f"{name} payload")
        assert_bytes_equal(got.s, ref.scales, f"{name} scales")
        assert_f32_bits_equal(got.g, ref.g, f"{name} g")
        assert_f32_bits_equal(obs, ref.amax, f"{name} amax")


def _oracle_operand(lq):
    return OF.decode_e2m1(lq.codes), OF.SCALE_VALUES[lq.fmt][lq.scales.astype(np.int64)]


def _dev_local(lq):
    rows, k = lq.codes.shape
    q = torch.from_numpy(oracle.pack_codes(lq.codes)).cuda()
    s = torch.from_numpy(np.ascontiguousarray(lq.scales)).cuda()
    g = torch.from_numpy(lq.g.copy()).cuda()
    return fp4.QTensor(q, s, g, lq.fmt, lq.block, fp4.FP4_SCALES_1D, rows, k, g_stripe=lq.stripe)


@pytest.mark.parametrize("fmt", [OF.E4M3, OF.UE5M3])
@pytest.mark.parametrize("canon", [False, True])
def test_fprop_both_operands_tile_local(fmt, canon):
    M, N, K = 200, 176, 512
    xa = _tensor(M, K, "fp32", 61).values
    xb = _tensor(N, K, "fp32", 62).values
    la = oracle.quantize_1d_local(xa, fmt, 16, stripe=32)
    lb = oracle.quantize_1d_local(xb, fmt, 16, stripe=16)
    A, sa = _oracle_operand(la)
    B, sb = _oracle_operand(lb)
    want = oracle.gemm_model(A, sa, B, sb, 16, alpha=oracle.stripe_alpha(la.g, 32, lb.g, 16, M, N), canon=canon)
    y = fp4.gemm_fprop(_dev_local(la), _dev_local(lb), canon=canon)
    torch.cuda.synchronize()
    assert_f32_bits_equal(y, want, f"fprop fmt={fmt} canon={canon}")


def test_local_activation_with_global_2d_weight_and_dgrad():
    """fprop: tile-local X (stripe 16) x global 2D W; dgrad: tile-local dY x W^T (global
    transposed 2D view): one side per-row g, the other a single g."""
    M, N, K = 256, 192, 320
    x = _tensor(M, K, "fp32", 63).values
    w = synth.normal((N, K), 0.02, 64)
    dy = _tensor(M, N, "fp32", 65).values
    lx = oracle.quantize_1d_local(x, OF.E4M3, 16, stripe=16)
    qw = oracle.quantize_2d(w, OF.E4M3, amax=oracle.tensor_amax(w))
    A, sa = _oracle_operand(lx)
    B, sb = oracle.operand_from_quant(qw, "2d")
    want = oracle.gemm_model(A, sa, B, sb, 16, alpha=oracle.stripe_alpha(lx.g, 16, [qw.g], 0, M, N))
    y = fp4.gemm_fprop(_dev_local(lx), qtensor_from_oracle(qw, "2d"))
    torch.cuda.synchronize()
    assert_f32_bits_equal(y, want, "fprop local x global 2D")
    ldy = oracle.quantize_1d_local(dy, OF.E4M3, 16, stripe=64, rounding="sr", seed=3, offset=1)
    A, sa = _oracle_operand(ldy)
    B, sb = oracle.operand_from_quant(qw, "2dT")
    want = oracle.gemm_model(A, sa, B, sb, 16, alpha=oracle.stripe_alpha(ldy.g, 64, [qw.g], 0, M, K))
    dx = fp4.gemm_dgrad(_dev_local(ldy), qtensor_from_oracle(qw, "2dT"))
    torch.cuda.synchronize()
    assert_f32_bits_equal(dx, want, "dgrad local dY x global W^T")


@pytest.mark.parametrize("fmt,block,cols,extra_rows,sr,T", [(OF.UE5M3, 32, 256, 5, False, 2048.0),
                                                          (OF.E4M3, 16, 512, 0, True, 448.0),
                                                          (OF.UE5M3, 16, 1024, 16, False, 448.0)])
def test_quantize_local_register_form(fmt, block, cols, extra_rows, sr, T):
    """At least two 16-row bf16 stripes per compute unit, each at most 65536 elements: the
    form that keeps a stripe in registers between its maximum and its quantization. Ragged
    last stripe, block 32, stochastic rounding; every byte, g and the stripe maxima."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    rows = 2 * cus * 16 + extra_rows
    t = _tensor(rows, cols, "bf16", 6200 + cols + extra_rows)
    ref = oracle.quantize_1d_local(t.values, fmt, block, stripe=16, T=T, rounding="sr" if sr else "rne",
                                   seed=7, offset=3)
    obs = torch.empty(len(ref.g), dtype=torch.float32, device="cuda")
    got = fp4.quantize_local(dev_input(t), fmt, block, stripe=16, T=T, stochastic=sr, seed=7, offset=3, amax_obs=obs)
    torch.cuda.synchronize()
    assert_bytes_equal(got.q, oracle.pack_codes(ref.codes), "payload")
    assert_bytes_equal(got.s, ref.scales, "scales")
    assert_f32_bits_equal(got.g, ref.g, "g")
    assert_f32_bits_equal(obs, ref.amax, "stripe amax")


def test_full_size_activation_tile_local_sampled():
    """8192 x 4096 activation quantized with stripes of 16 rows (512 stripes) by the
    library; stripes 0-7 and 504-511 checked against the oracle."""
    X = synth.make_config(3, rows=8192)["X"]
    got = fp4.quantize_local(dev_input(X), fp4.E4M3, 16, stripe=16)
    torch.cuda.synchronize()
    for r0 in (0, 8064):
        ref = oracle.quantize_1d_local(X.values[r0:r0 + 128], OF.E4M3, 16, stripe=16)
        assert_bytes_equal(got.q[r0:r0 + 128], oracle.pack_codes(ref.codes), "payload")
        assert_bytes_equal(got.s[r0:r0 + 128], ref.scales, "scales")
        assert_f32_bits_equal(got.g[r0 // 16:r0 // 16 + 8], ref.g, "g")
