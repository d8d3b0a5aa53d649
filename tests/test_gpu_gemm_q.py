"""GEMMs whose epilogue quantizes the output as the next GEMM's ROW-view operand
("Format-Aware Fusion for Fast FP4 Pretraining", abstract: the producer emits the layout its
consumer reads; "Practical FP4 Training for Large-Scale MoE Models on Hopper GPUs",
methodology: FP4 copies instead of a separate round trip).

Parity: the payload, scales and g the GEMM writes equal oracle.quantize_1d applied to the
oracle group model's float32 output (the same cached amax, T, rounding and counter offset),
byte for byte; the float32 output, when also requested, equals the model; the observed amax
and the health counts equal the oracle's. Both GEMM kernels (MXFP4 and the decoded UE5M3 /
E4M3 route) and every output format, on tiles cut by ragged M and N.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import formats as OF
from tests._helpers import assert_bytes_equal, assert_f32_bits_equal, dev_input, dev_scalar, qtensor_from_oracle

pytestmark = pytest.mark.gpu

fp4 = pytest.importorskip("fp4_block_scaled_tensor_amd")


def _model_y(qa, qb, vb="1d", canon=False):
    a, sa = oracle.operand_from_quant(qa)
    b, sb = oracle.operand_from_quant(qb, vb)
    return oracle.gemm_model(a, sa, b, sb, qa.block, alpha=oracle.output_scale(qa.g, qb.g), canon=canon)


def _operands(M, N, K, in_fmt, seed):
    B = 32 if in_fmt == OF.E8M0 else 16
    X = synth.student_t((M, K), 3.0, seed)
    W = synth.normal((N, K), 0.02, seed + 1)
    Ax = None if in_fmt == OF.E8M0 else oracle.tensor_amax(X)
    Aw = None if in_fmt == OF.E8M0 else oracle.tensor_amax(W)
    return (oracle.quantize_1d(X, in_fmt, B, amax=Ax, T=448), oracle.quantize_1d(W, in_fmt, B, amax=Aw, T=448))


CASES = [
    # name, M, N, K, input fmt, output fmt, output block, sr, amax factor, f32 too, canon
    ("mx_to_ue5m3", 256, 384, 256, OF.E8M0, OF.UE5M3, 16, False, 1.0, True, False),
    ("mx_to_mx_sr_ragged", 200, 96, 320, OF.E8M0, OF.E8M0, 32, True, 1.0, False, False),
    ("ue5m3_to_ue5m3_stale", 136, 272, 192, OF.UE5M3, OF.UE5M3, 16, False, 0.004, True, False),
    ("ue5m3_to_e4m3_sr", 128, 160, 128, OF.UE5M3, OF.E4M3, 16, True, 1.3, False, True),
    ("e4m3_to_ue5m3_b32", 72, 224, 256, OF.E4M3, OF.UE5M3, 32, False, 0.5, True, False),
    ("mx_to_e4m3_b32_sr", 264, 128, 128, OF.E8M0, OF.E4M3, 32, True, 2.0, False, False),
]


@pytest.mark.parametrize("name,M,N,K,ifmt,ofmt,oblock,sr,afac,f32,canon", CASES, ids=[c[0] for c in CASES])
def test_fprop_q_matches_oracle(name, M, N, K, ifmt, ofmt, oblock, sr, afac, f32, canon):
    qa, qb = _operands(M, N, K, ifmt, 9100 + M)
    y = _model_y(qa, qb, canon=canon)
    A_true = oracle.tensor_amax(y)
    A = np.float32(A_true * np.float32(afac))        # the cached amax (stale by afac)
    want = oracle.quantize_1d(y, ofmt, oblock, amax=A, T=448.0, rounding="sr" if sr else "rne", seed=5, offset=13)
    obs = torch.empty(1, dtype=torch.float32, device="cuda")
    st = fp4.new_stats()
    got, yf = fp4.gemm_fprop_q(qtensor_from_oracle(qa), qtensor_from_oracle(qb), ofmt, oblock,
                               amax=None if ofmt == OF.E8M0 else dev_scalar(A), T=448.0, stochastic=sr, seed=5,
                               offset=13, canon=canon, want_f32=f32, amax_obs=obs, stats=st)
    torch.cuda.synchronize()
    assert_bytes_equal(got.q, want.packed, f"{name} payload")
    assert_bytes_equal(got.s, want.scales, f"{name} scales")
    assert got.g.item() == np.float32(want.g)
    assert obs.item() == A_true
    assert tuple(int(c) for c in st.cpu().numpy()) == oracle.block_health(y, ofmt, oblock, amax=A, T=448.0)
    if afac < 0.01:
        assert st[0].item() > 0                       # far past the headroom: scales saturate
    if f32:
        assert_f32_bits_equal(yf, y, f"{name} float32 output")
    else:
        assert yf is None


@pytest.mark.parametrize("ifmt", [OF.UE5M3, OF.E8M0])
def test_dgrad_q_with_2d_weight_sr_output(ifmt):
    """dX = dY . W with the output quantized as the previous layer's stochastic dY operand."""
    T_, Fo, Fi = 256, 192, 320
    dY = synth.normal((T_, Fo), 1e-3, 9201)
    W = synth.normal((Fo, Fi), 0.02, 9202)
    if ifmt == OF.E8M0:
        rdy = oracle.quantize_1d(dY, ifmt, 32, rounding="sr", seed=42, offset=0)
        rwt = oracle.quantize_1d(np.ascontiguousarray(W.T), ifmt, 32)
        a, b, vb = qtensor_from_oracle(rdy), qtensor_from_oracle(rwt), "1d"
    else:
        Ady, Aw = oracle.tensor_amax(dY), oracle.tensor_amax(W)
        rdy = oracle.quantize_1d(dY, ifmt, 16, amax=Ady, T=448, rounding="sr", seed=42, offset=0)
        rwt = oracle.quantize_2d(W, ifmt, amax=Aw, T=448)
        a, b, vb = qtensor_from_oracle(rdy), qtensor_from_oracle(rwt, "2dT"), "2dT"
    dx = _model_y(rdy, rwt, vb=vb)
    A = oracle.tensor_amax(dx)
    want = oracle.quantize_1d(dx, OF.UE5M3, 16, amax=A, T=448.0, rounding="sr", seed=42, offset=16)
    got, dxf = fp4.gemm_dgrad_q(a, b, OF.UE5M3, 16, amax=dev_scalar(A), T=448.0, stochastic=True, seed=42,
                                offset=16, want_f32=True)
    torch.cuda.synchronize()
    assert_f32_bits_equal(dxf, dx, "dgrad float32")
    assert_bytes_equal(got.q, want.packed, "dX payload")
    assert_bytes_equal(got.s, want.scales, "dX scales")


@pytest.mark.parametrize("ifmt", [OF.UE5M3, OF.E8M0], ids=["ue5m3", "mxfp4"])
def test_fprop_q_full_size_sampled_rows(ifmt):
    """The up-projection at full size (8192 x 4096 -> 14336) with the output quantized in the
    epilogue (UE5M3 block 16, nearest-even, a cached amax from the previous step): sampled row
    slices of the payload and scales against the oracle's quantization of the model's rows,
    and the float32 output rows against the model."""
    cfg = synth.make_config(3)
    X, W = cfg["X"], cfg["W"]
    E8 = ifmt == OF.E8M0
    B = 32 if E8 else 16
    Ax, Aw = oracle.tensor_amax(X.values), oracle.tensor_amax(W.values)
    qx = fp4.quantize(dev_input(X), ifmt, B, fp4.ROW, amax=None if E8 else dev_scalar(Ax), T=448)
    if E8:
        qw = fp4.quantize(dev_input(W), ifmt, B, fp4.ROW)
    else:
        qw, _ = fp4.quantize(dev_input(W), ifmt, 16, fp4.TILE2D, amax=dev_scalar(Aw), T=448)
    A_out = np.float32(7.5)
    got, y = fp4.gemm_fprop_q(qx, qw, OF.UE5M3, 16, amax=dev_scalar(A_out), T=448.0, want_f32=True)
    torch.cuda.synchronize()
    rw = oracle.quantize_1d(W.values, ifmt, B) if E8 else oracle.quantize_2d(W.values, ifmt, amax=Aw, T=448)
    for r0, r1 in ((0, 4), (4100, 4104), (8188, 8192)):
        rx = oracle.quantize_1d(X.values[r0:r1], ifmt, B, amax=None if E8 else Ax, T=448)
        yr = _model_y(rx, rw, vb="1d" if E8 else "2d")
        assert_f32_bits_equal(y[r0:r1], yr, f"rows {r0}")
        want = oracle.quantize_1d(yr, OF.UE5M3, 16, amax=A_out, T=448.0)
        assert_bytes_equal(got.q[r0:r1], want.packed, f"payload rows {r0}")
        assert_bytes_equal(got.s[r0:r1], want.scales, f"scales rows {r0}")
