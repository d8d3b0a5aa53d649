"""Quantizer parity: HIP kernels vs the oracle, bit-exact payload bytes, scale codes and g."""
import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import formats as OF
from tests._helpers import assert_bytes_equal, dev_input, dev_scalar

pytestmark = pytest.mark.gpu

fp4 = pytest.importorskip("fp4_block_scaled_tensor_amd")


def _tensor(rows, cols, dtype, seed, kind="normal"):
    if kind == "t":
        x = synth.student_t((rows, cols), 3.0, seed)
        x, _ = synth.scale_channels(x, max(1, cols // 1000), 100.0, seed + 1)
    else:
        x = synth.normal((rows, cols), 1.0, seed)
    t = synth.Tensor("x", x, dtype)
    if dtype == "bf16":
        t = synth.Tensor("x", synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(x)), "bf16")
    return t


ROW_CASES = [
    # name, rows, cols, dtype, fmt, block, sr, T
    ("tiny_fp32_ue5m3", 256, 256, "fp32", OF.UE5M3, 16, False, 448),
    ("ragged_ue5m3", 40, 96, "bf16", OF.UE5M3, 16, False, 448),
    ("ragged_e4m3_b32", 24, 160, "bf16", OF.E4M3, 32, False, 448),
    ("ragged_mx", 33, 96, "bf16", OF.E8M0, 32, False, 0),
    ("sweep_ue5m3", 2048, 2048, "bf16", OF.UE5M3, 16, False, 448),
    ("sweep_e4m3", 2048, 2048, "bf16", OF.E4M3, 16, False, 448),
    ("sweep_mx", 2048, 2048, "bf16", OF.E8M0, 32, False, 0),
    ("sr_ue5m3", 512, 1024, "bf16", OF.UE5M3, 16, True, 2048),
    ("sr_mx", 64, 4096, "fp32", OF.E8M0, 32, True, 0),
    ("ragged_tiles_sr_fp32", 9, 1056, "fp32", OF.E4M3, 16, True, 448),
    ("ragged_tiles_ue5m3_b32", 17, 2080, "bf16", OF.UE5M3, 32, False, 2048),
]


@pytest.mark.parametrize("name,rows,cols,dtype,fmt,block,sr,T", ROW_CASES, ids=[c[0] for c in ROW_CASES])
def test_row_view(name, rows, cols, dtype, fmt, block, sr, T):
    t = _tensor(rows, cols, dtype, 1000 + rows + cols, "t")
    A = oracle.tensor_amax(t.values)
    ref = oracle.quantize_1d(t.values, fmt, block, amax=A, T=T, rounding="sr" if sr else "rne", seed=42, offset=8)
    x = dev_input(t)
    obs = torch.empty(1, dtype=torch.float32, device="cuda")
    got = fp4.quantize(x, fmt, block, fp4.ROW, amax=dev_scalar(A), T=T, stochastic=sr, seed=42, offset=8, amax_obs=obs)
    torch.cuda.synchronize()
    assert_bytes_equal(got.q, ref.packed, f"{name} payload")
    assert_bytes_equal(got.s, ref.scales, f"{name} scales")
    assert got.g.item() == np.float32(ref.g)
    assert obs.item() == A


@pytest.mark.parametrize("dtype,ld", [("bf16", 1096), ("bf16", (1 << 23) + 64), ("fp32", (1 << 22) + 32)],
                         ids=["bf16_ld1096", "bf16_ld_over_2^23", "fp32_ld_over_2^22"])
def test_row_view_strided_input(dtype, ld):
    """x as a view with row stride ld > cols: a short stride, and strides whose row offsets
    no longer fit the 32-bit in-tile addressing (the per-block-thread form runs then)."""
    rows, cols = 5, 1024
    t = _tensor(rows, cols, dtype, 1500 + ld % 97, "t")
    A = oracle.tensor_amax(t.values)
    ref = oracle.quantize_1d(t.values, OF.UE5M3, 16, amax=A, T=448, rounding="sr", seed=9, offset=2)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    base = torch.zeros(rows, ld, dtype=tdt, device="cuda")
    base[:, :cols] = dev_input(t)
    x = base[:, :cols]
    assert x.stride(0) == ld
    got = fp4.quantize(x, OF.UE5M3, 16, fp4.ROW, amax=dev_scalar(A), T=448, stochastic=True, seed=9, offset=2)
    torch.cuda.synchronize()
    assert_bytes_equal(got.q, ref.packed, "payload")
    assert_bytes_equal(got.s, ref.scales, "scales")
    assert got.g.item() == np.float32(ref.g)


def test_row_view_full_size_activation_sampled_rows():
    """8192 x 4096 Student-t activation with outlier channels (the up-projection input),
    quantized in full on the GPU; 256 rows checked against the oracle."""
    cfg = synth.make_config(3, rows=8192)
    X = cfg["X"]
    A = oracle.tensor_amax(X.values)
    got = fp4.quantize(dev_input(X), fp4.UE5M3, 16, fp4.ROW, amax=dev_scalar(A), T=448)
    torch.cuda.synchronize()
    rows = np.r_[0:128, 8064:8192]
    ref = oracle.quantize_1d(X.values[rows], OF.UE5M3, 16, amax=A, T=448)
    assert_bytes_equal(got.q[torch.from_numpy(rows).cuda()], ref.packed, "payload rows")
    assert_bytes_equal(got.s[torch.from_numpy(rows).cuda()], ref.scales, "scale rows")


COL_CASES = [
    # name, tokens, features, dtype, fmt, block, sr, hadamard, T
    ("col_ue5m3", 512, 200, "bf16", OF.UE5M3, 16, False, 0, 448),
    ("col_ue5m3_h16", 512, 200, "bf16", OF.UE5M3, 16, False, 16, 448),
    ("col_ue5m3_h32_sr", 320, 72, "bf16", OF.UE5M3, 16, True, 32, 2048),
    ("col_e4m3_sr", 256, 64, "fp32", OF.E4M3, 16, True, 0, 448),
    ("col_mx_h16", 544, 136, "bf16", OF.E8M0, 32, False, 16, 0),
    ("col_mx_h32_sr", 288, 40, "bf16", OF.E8M0, 32, True, 32, 0),
    ("col_ue5m3_b32_h16", 96, 24, "bf16", OF.UE5M3, 32, False, 16, 448),
]


@pytest.mark.parametrize("name,tok,feat,dtype,fmt,block,sr,hn,T", COL_CASES, ids=[c[0] for c in COL_CASES])
def test_col_view(name, tok, feat, dtype, fmt, block, sr, hn, T):
    t = _tensor(tok, feat, dtype, 2000 + tok + feat, "t")
    A = oracle.tensor_amax(t.values, hn)
    ref = oracle.quantize_col(t.values, fmt, block, amax=A, T=T, rounding="sr" if sr else "rne", seed=42, offset=9,
                              hadamard_n=hn)
    x = dev_input(t)
    obs = torch.empty(1, dtype=torch.float32, device="cuda")
    got = fp4.quantize(x, fmt, block, fp4.COL, amax=dev_scalar(A), T=T, stochastic=sr, seed=42, offset=9,
                       hadamard_n=hn, amax_obs=obs)
    amax_gpu = fp4.tensor_amax(x, hn)
    torch.cuda.synchronize()
    assert_bytes_equal(got.q, ref.packed, f"{name} payload")
    assert_bytes_equal(got.s, ref.scales, f"{name} scales")
    assert obs.item() == A and amax_gpu.item() == A


def test_col_view_backward_gradient_full_size():
    """dY [8192 x 4096] ~ N(0, 1e-3), stochastic rounding (Philox seed 42), T = 2048, the
    wgrad view; 64 features (operand rows) checked against the oracle."""
    cfg = synth.make_config(4, rows=8192)
    dY = cfg["dY"]
    A = oracle.tensor_amax(dY.values)
    got = fp4.quantize(dev_input(dY), fp4.UE5M3, 16, fp4.COL, amax=dev_scalar(A), T=2048, stochastic=True, seed=42,
                       offset=1)
    torch.cuda.synchronize()
    f0, f1 = 1000, 1064
    ref = oracle.quantize_1d(np.ascontiguousarray(dY.values[:, f0:f1].T), OF.UE5M3, 16, amax=A, T=2048,
                             rounding="sr", seed=42, offset=1, row0=f0)
    assert_bytes_equal(got.q[f0:f1], ref.packed, "payload")
    assert_bytes_equal(got.s[f0:f1], ref.scales, "scales")


@pytest.mark.parametrize("fmt,rows,cols,dtype", [(OF.UE5M3, 256, 320, "bf16"), (OF.E4M3, 80, 48, "fp32"),
                                                 (OF.UE5M3, 16, 16, "bf16")])
def test_tile2d(fmt, rows, cols, dtype):
    t = _tensor(rows, cols, dtype, 3000 + rows, "normal")
    A = oracle.tensor_amax(t.values)
    ref = oracle.quantize_2d(t.values, fmt, amax=A, T=448)
    fwd, dgr = fp4.quantize(dev_input(t), fmt, 16, fp4.TILE2D, amax=dev_scalar(A), T=448)
    torch.cuda.synchronize()
    assert_bytes_equal(fwd.q, ref.packed, "forward payload")
    assert_bytes_equal(dgr.q, oracle.pack_codes(np.ascontiguousarray(ref.codes.T)), "transposed payload")
    assert_bytes_equal(fwd.s, ref.scales, "2D scales")
    assert fwd.g.item() == np.float32(ref.g)


def test_tile2d_full_size_weight_sampled():
    """Up-projection weight [14336 x 4096] ~ N(0, 0.02): both payload copies, 1024 rows checked."""
    W = synth.make_config(3, rows=8)["W"]
    A = oracle.tensor_amax(W.values)
    fwd, dgr = fp4.quantize(dev_input(W), fp4.UE5M3, 16, fp4.TILE2D, amax=dev_scalar(A), T=448)
    torch.cuda.synchronize()
    r0, r1 = 7168, 8192
    ref = oracle.quantize_2d(W.values[r0:r1], OF.UE5M3, amax=A, T=448)
    assert_bytes_equal(fwd.q[r0:r1], ref.packed, "forward payload")
    assert_bytes_equal(fwd.s[r0 // 16:r1 // 16], ref.scales, "scales")
    assert_bytes_equal(dgr.q[:, r0 // 2:r1 // 2], oracle.pack_codes(np.ascontiguousarray(ref.codes.T)), "transposed")


def test_zero_and_stale_amax_edges():
    """Zero blocks (scale -> 1), a zero tensor amax (all scales 1), and a stale cached amax
    far below the data (saturated block scales)."""
    x = synth.normal((64, 128), 1.0, 77)
    x[3] = 0
    x[5, 16:32] = 1e-30
    for A in (float(np.max(np.abs(x))), 0.0, 1e-3, float("inf")):
        ref = oracle.quantize_1d(x, OF.UE5M3, 16, amax=A, T=448)
        got = fp4.quantize(torch.from_numpy(x).cuda(), fp4.UE5M3, 16, fp4.ROW, amax=dev_scalar(A), T=448)
        torch.cuda.synchronize()
        assert_bytes_equal(got.q, ref.packed, f"payload A={A}")
        assert_bytes_equal(got.s, ref.scales, f"scales A={A}")
        assert got.g.item() == np.float32(ref.g)


def test_empty_tensor_writes_g():
    x = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    got = fp4.quantize(x, fp4.UE5M3, 16, fp4.ROW, amax=dev_scalar(2.0), T=448)
    torch.cuda.synchronize()
    assert got.q.numel() == 0 and got.g.item() == np.float32(oracle.tensor_scales(2.0, 448)[2])


def test_amax_cache_update_and_reset():
    cache = fp4.AmaxCache(D=3)
    ref = oracle.AmaxCache(3)
    seen = []
    for step in range(8):
        obs = dev_scalar(step + 1.5)
        cache.update(step, obs)
        ref.update(step, step + 1.5)
        torch.cuda.synchronize()
        seen.append(cache.amax.item())
        assert cache.amax.item() == float(ref.amax)
        if step == 4:
            cache.reset()
            ref.reset()
    assert seen == [1.5, 1.5, 1.5, 4.5, 4.5, 6.5, 7.5, 7.5]


@pytest.mark.parametrize("r", [1.3, 3.7, 0.2])
def test_stochastic_rounding_unbiased_over_a_million_draws(r):
    """The whole SR path of the library (Philox draws, the E2M1 decision, packing): 70000 rows
    of 16, each row a block with one element 6 (so that the block scale is 448 and the
    payload multiplier is exactly 1) and 15 elements r. The mean of the 1,050,000 decoded SR
    values lies within 3 sigma (plus the 2^-16 resolution of the draws times the grid step)
    of r, and every value is one of r's two neighbouring codebook values."""
    rows = 70000
    x = np.full((rows, 16), np.float32(r), dtype=np.float32)
    x[:, 0] = 6.0
    amax = dev_scalar(np.float32(6.0))
    got = fp4.quantize(torch.from_numpy(x).cuda(), fp4.UE5M3, 16, fp4.ROW, amax=amax, T=448.0, stochastic=True,
                       seed=42, offset=11)
    torch.cuda.synchronize()
    assert np.all(got.s.cpu().numpy() == OF.encode_scale(np.array([448.0], np.float32), OF.UE5M3)[0])
    q = got.q.cpu().numpy()
    codes = np.stack([q & 15, q >> 4], axis=-1).reshape(rows, 16)
    vals = OF.decode_e2m1(codes[:, 1:]).astype(np.float64).ravel()
    mags = OF.E2M1_MAGS.astype(np.float64)
    lo, hi = mags[mags <= np.float32(r)].max(), mags[mags > np.float32(r)].min()
    assert set(np.unique(vals)) <= {lo, hi}
    f = (np.float64(np.float32(r)) - lo) / (hi - lo)
    sigma = (hi - lo) * np.sqrt(f * (1 - f) / vals.size)
    assert abs(vals.mean() - np.float64(np.float32(r))) <= 3 * sigma + (hi - lo) * 2.0 ** -16


@pytest.mark.parametrize("rows,cols,dtype", [(7001, 12296, "bf16"), (4099, 2056, "fp32"), (9000, 4096, "bf16")])
def test_tensor_amax_grid_stride(rows, cols, dtype):
    """Shapes where the tensor maximum's workgroups each loop over several row groups and
    column pieces (ragged in both); the single largest magnitude is planted in the last rows
    and last columns, then moved to the first element."""
    t = _tensor(rows, cols, dtype, 4000 + rows, "normal")
    v = t.values.copy()
    for r, c in ((rows - 1, cols - 3), (0, 0)):
        w = v.copy()
        w[r, c] = -1000.0
        tt = synth.Tensor("x", w, dtype)
        got = fp4.tensor_amax(dev_input(tt))
        torch.cuda.synchronize()
        assert got.item() == oracle.tensor_amax(w) == np.float32(1000.0), (r, c)
