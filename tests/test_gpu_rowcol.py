"""Fused ROW + COL quantization (one read of x, both operand layouts): bit-exact against the
oracle's ROW-view and COL-view quantizations of the same tensor, and against the two
separate library calls."""
import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import formats as OF
from tests._helpers import assert_bytes_equal, dev_input, dev_scalar

pytestmark = pytest.mark.gpu

fp4 = pytest.importorskip("fp4_block_scaled_tensor_amd")


def _tensor(rows, cols, dtype, seed):
    x = synth.student_t((rows, cols), 3.0, seed)
    x, _ = synth.scale_channels(x, max(1, cols // 100), 100.0, seed + 1)
    if dtype == "bf16":
        return synth.Tensor("x", synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(x)), "bf16")
    return synth.Tensor("x", x, dtype)


CASES = [
    # name, tokens, features, dtype, fmt, block, sr_row, sr_col, hadamard, T_row, T_col
    ("ue5m3", 512, 208, "bf16", OF.UE5M3, 16, False, False, 0, 448, 448),
    ("ue5m3_h16_ragged", 1008, 208, "bf16", OF.UE5M3, 16, False, False, 16, 448, 448),
    ("ue5m3_h32_sr", 320, 80, "bf16", OF.UE5M3, 16, True, True, 32, 448, 2048),
    ("e4m3_fp32_srcol", 256, 64, "fp32", OF.E4M3, 16, False, True, 0, 448, 448),
    ("e4m3_b32_srrow", 160, 96, "bf16", OF.E4M3, 32, True, False, 16, 2048, 448),
    ("mx_h16", 544, 160, "bf16", OF.E8M0, 32, False, False, 16, 0, 0),
    ("mx_h32_sr", 288, 96, "bf16", OF.E8M0, 32, True, True, 32, 0, 0),
    ("ue5m3_b32_h16", 96, 96, "bf16", OF.UE5M3, 32, False, False, 16, 448, 448),
    ("tiny", 16, 16, "bf16", OF.UE5M3, 16, False, False, 16, 448, 448),
]


@pytest.mark.parametrize("name,tok,feat,dtype,fmt,block,srr,src,hn,Tr,Tc", CASES, ids=[c[0] for c in CASES])
def test_rowcol_matches_oracle(name, tok, feat, dtype, fmt, block, srr, src, hn, Tr, Tc):
    t = _tensor(tok, feat, dtype, 5000 + tok + feat)
    Ar = oracle.tensor_amax(t.values)
    Ac = oracle.tensor_amax(t.values, hn)
    ref_r = oracle.quantize_1d(t.values, fmt, block, amax=Ar, T=Tr, rounding="sr" if srr else "rne", seed=7,
                               offset=2)
    ref_c = oracle.quantize_col(t.values, fmt, block, amax=Ac, T=Tc, rounding="sr" if src else "rne", seed=11,
                                offset=3, hadamard_n=hn)
    x = dev_input(t)
    obs_r = torch.empty(1, dtype=torch.float32, device="cuda")
    obs_c = torch.empty(1, dtype=torch.float32, device="cuda")
    row, col = fp4.quantize_rowcol(x, fmt, block, amax_row=dev_scalar(Ar), amax_col=dev_scalar(Ac), T_row=Tr,
                                   T_col=Tc, stochastic_row=srr, stochastic_col=src, seed_row=7, offset_row=2,
                                   seed_col=11, offset_col=3, hadamard_n=hn, amax_obs_row=obs_r, amax_obs_col=obs_c)
    torch.cuda.synchronize()
    assert_bytes_equal(row.q, ref_r.packed, f"{name} ROW payload")
    assert_bytes_equal(row.s, ref_r.scales, f"{name} ROW scales")
    assert_bytes_equal(col.q, ref_c.packed, f"{name} COL payload")
    assert_bytes_equal(col.s, ref_c.scales, f"{name} COL scales")
    assert row.g.item() == np.float32(ref_r.g) and col.g.item() == np.float32(ref_c.g)
    assert obs_r.item() == Ar and obs_c.item() == Ac
    assert (row.rows, row.k, col.rows, col.k) == (tok, feat, feat, tok)


def test_rowcol_strided_input_matches_separate_calls():
    """x is a column slice of a wider tensor (row stride > cols); the fused call gives the
    bytes of the two separate calls."""
    t = _tensor(384, 320, "bf16", 61)
    full = dev_input(t)
    x = full[:, 64:256]
    A = dev_scalar(oracle.tensor_amax(t.values[:, 64:256]))
    Ah = dev_scalar(oracle.tensor_amax(t.values[:, 64:256], 16))
    row, col = fp4.quantize_rowcol(x, fp4.UE5M3, 16, amax_row=A, amax_col=Ah, T_col=2048, stochastic_col=True,
                                   seed_col=5, offset_col=9, hadamard_n=16)
    r2 = fp4.quantize(x, fp4.UE5M3, 16, fp4.ROW, amax=A)
    c2 = fp4.quantize(x, fp4.UE5M3, 16, fp4.COL, amax=Ah, T=2048, stochastic=True, seed=5, offset=9, hadamard_n=16)
    torch.cuda.synchronize()
    for a, b, what in ((row.q, r2.q, "ROW payload"), (row.s, r2.s, "ROW scales"), (col.q, c2.q, "COL payload"),
                       (col.s, c2.s, "COL scales")):
        assert_bytes_equal(a, b.cpu().numpy(), what)


@pytest.mark.parametrize("fmt", [OF.UE5M3, OF.E8M0])
def test_rowcol_full_size_activation_sampled(fmt):
    """8192 x 4096 Student-t activation with outlier channels, both views quantized in full
    (the launch the step uses); 256 tokens of the ROW view and 64 features of the COL view
    checked against the oracle."""
    X = synth.make_config(3, rows=8192)["X"]
    block = 32 if fmt == OF.E8M0 else 16
    A = oracle.tensor_amax(X.values)
    row, col = fp4.quantize_rowcol(dev_input(X), fmt, block, amax_row=dev_scalar(A), amax_col=dev_scalar(A))
    torch.cuda.synchronize()
    rows = np.r_[0:128, 8064:8192]
    ref = oracle.quantize_1d(X.values[rows], fmt, block, amax=A, T=448)
    idx = torch.from_numpy(rows).cuda()
    assert_bytes_equal(row.q[idx], ref.packed, "ROW payload rows")
    assert_bytes_equal(row.s[idx], ref.scales, "ROW scale rows")
    f0, f1 = 2000, 2064
    ref_c = oracle.quantize_1d(np.ascontiguousarray(X.values[:, f0:f1].T), fmt, block, amax=A, T=448)
    assert_bytes_equal(col.q[f0:f1], ref_c.packed, "COL payload rows")
    assert_bytes_equal(col.s[f0:f1], ref_c.scales, "COL scale rows")


def test_rowcol_empty_writes_g():
    x = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    row, col = fp4.quantize_rowcol(x, fp4.UE5M3, 16, amax_row=dev_scalar(2.0), amax_col=dev_scalar(4.0), T_col=2048)
    torch.cuda.synchronize()
    assert row.q.numel() == 0 and col.q.numel() == 0
    assert row.g.item() == np.float32(oracle.tensor_scales(2.0, 448)[2])
    assert col.g.item() == np.float32(oracle.tensor_scales(4.0, 2048)[2])
