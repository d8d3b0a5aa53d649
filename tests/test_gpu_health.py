"""Quantizer health counts and the NaN contract of every maximum, on the GPU against the oracle.

Health counts (saturated / zero-scale / non-finite blocks, "UE5M3 FP4 Block Scaling for Stable
Language Model Pretraining", key contributions: the 61440/T headroom of a stale amax) are
compared with oracle.block_health in every view and launch form; with finite inputs the
payload and scale bytes are compared too. NaN contract: a NaN anywhere makes the observed
maximum NaN (as the oracle's float maximum does) in the tensor maximum, the quantizers'
observed amax and all three tile-local forms, whose NaN stripe then gets the degenerate
tensor scale g = 1.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import formats as OF
from tests._helpers import assert_bytes_equal, assert_f32_bits_equal, dev_input, dev_scalar

pytestmark = pytest.mark.gpu

fp4 = pytest.importorskip("fp4_block_scaled_tensor_amd")


def _stats():
    return fp4.new_stats()


def _stressed(rows, cols, seed, gamma=200.0, dtype="bf16"):
    """uniform(-gamma, gamma) data with the cached amax at 1 (so blocks above 61440/T saturate),
    one all-zero ROW block, one ROW block of tiny values (its scale encodes to zero) and one
    all-zero 16x16 tile."""
    rng = np.random.default_rng(seed)
    x = (rng.uniform(-1, 1, (rows, cols)) * gamma).astype(np.float32)
    x[1, 32:64] = 0.0
    x[2, 64:96] = 1e-9
    x[16:32, 128:144] = 0.0
    x[40:48, :] *= np.float32(0.001)         # some rows that stay inside the headroom
    t = synth.Tensor("x", x, dtype)
    if dtype == "bf16":
        t = synth.Tensor("x", synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(x)), "bf16")
    return t


def _with_nonfinite(t):
    v = t.values.copy()
    v[3, 5] = np.inf
    v[10, 200] = np.nan
    v[33, 17] = -np.inf
    v[33, 18] = np.nan
    return synth.Tensor("x", v, t.dtype)


def _counts(st):
    return tuple(int(c) for c in st.cpu().numpy()[:3])


VIEWS = [("row", OF.UE5M3, 16), ("row", OF.E4M3, 32), ("row", OF.E8M0, 32), ("col", OF.UE5M3, 16),
         ("col16", OF.E4M3, 16), ("col", OF.E8M0, 32), ("2d", OF.UE5M3, 16), ("2d", OF.E4M3, 16)]


@pytest.mark.parametrize("view,fmt,block", VIEWS, ids=[f"{v}-{OF.FMT_NAMES[f]}{b}" for v, f, b in VIEWS])
@pytest.mark.parametrize("nonfinite", [False, True], ids=["finite", "inf_nan"])
def test_health_counts_match_oracle(view, fmt, block, nonfinite):
    t = _stressed(128, 512, 71)
    if nonfinite:
        t = _with_nonfinite(t)
    x, T = t.values, 448.0
    amax = dev_scalar(1.0)
    st = _stats()
    obs = torch.empty(1, dtype=torch.float32, device="cuda")
    hn = 16 if view == "col16" else 0
    ov = {"row": "row", "col": "col", "col16": "col", "2d": "2d"}[view]
    fv = {"row": fp4.ROW, "col": fp4.COL, "col16": fp4.COL, "2d": fp4.TILE2D}[view]
    got = fp4.quantize(dev_input(t), fmt, block, fv, amax=amax, T=T, hadamard_n=hn, amax_obs=obs, stats=st)
    torch.cuda.synchronize()
    want = oracle.block_health(x, fmt, block, amax=1.0, T=T, view=ov, hadamard_n=hn)
    assert _counts(st) == want
    assert want[0] > 0 or fmt == OF.E8M0          # the case does saturate
    # and has zero-scale blocks (the rotation mixes them away; E8M0's 32-token COL blocks are
    # wider than the zeroed 16-token run)
    assert want[1] > 0 or view == "col16" or (fmt == OF.E8M0 and view == "col")
    if nonfinite:
        assert want[2] > 0 and np.isnan(obs.item())
        return
    assert obs.item() == oracle.tensor_amax(x, hn)
    if view == "2d":
        ref = oracle.quantize_2d(x, fmt, amax=1.0, T=T)
        got = got[0]
    elif ov == "col":
        ref = oracle.quantize_col(x, fmt, block, amax=1.0, T=T, hadamard_n=hn)
    else:
        ref = oracle.quantize_1d(x, fmt, block, amax=1.0, T=T)
    assert_bytes_equal(got.q, ref.packed, "payload")
    assert_bytes_equal(got.s, ref.scales, "scales")
    assert want[:2] == (ref.n_sat, ref.n_zero)


def test_health_counts_row_wide_stride_form():
    """A row stride above 2^24 bytes takes the per-block-thread ROW kernel; its counts too."""
    t = _stressed(64, 256, 72, dtype="bf16")
    ld = (1 << 23) + 64
    buf = torch.zeros((64, ld), dtype=torch.bfloat16, device="cuda")
    buf[:, :256] = dev_input(t)
    st = _stats()
    got = fp4.quantize(buf[:, :256], OF.UE5M3, 16, fp4.ROW, amax=dev_scalar(1.0), T=448.0, stats=st)
    torch.cuda.synchronize()
    ref = oracle.quantize_1d(t.values, OF.UE5M3, 16, amax=1.0, T=448.0)
    assert_bytes_equal(got.q, ref.packed, "payload")
    assert _counts(st) == oracle.block_health(t.values, OF.UE5M3, 16, amax=1.0, T=448.0) == (ref.n_sat, ref.n_zero, 0)


@pytest.mark.parametrize("fmt,block,sr", [(OF.UE5M3, 16, False), (OF.E8M0, 32, True)])
@pytest.mark.parametrize("nonfinite", [False, True], ids=["finite", "inf_nan"])
def test_health_counts_rowcol(fmt, block, sr, nonfinite):
    t = _stressed(256, 512, 73)
    if nonfinite:
        t = _with_nonfinite(t)
    sr_, sc_ = _stats(), _stats()
    Tr, Tc = 448.0, 2048.0
    fp4.quantize_rowcol(dev_input(t), fmt, block, amax_row=dev_scalar(1.0), amax_col=dev_scalar(1.0), T_row=Tr,
                        T_col=Tc, stochastic_row=sr, stochastic_col=sr, seed_row=1, seed_col=2, hadamard_n=16,
                        stats_row=sr_, stats_col=sc_)
    torch.cuda.synchronize()
    assert _counts(sr_) == oracle.block_health(t.values, fmt, block, amax=1.0, T=Tr, view="row")
    assert _counts(sc_) == oracle.block_health(t.values, fmt, block, amax=1.0, T=Tc, view="col", hadamard_n=16)


def test_health_counts_headroom_edge():
    """The saturation count is zero at growth 137.0 and positive at 137.3 for T = 448 (and at
    30.0 / 30.1 for T = 2048): the headroom edge of the key contributions, seen on the device."""
    rng = np.random.default_rng(74)
    base = rng.uniform(-1, 1, (64, 256)).astype(np.float32)
    base[0, 0] = 1.0
    for T, ok, bad in ((448.0, 137.0, 137.3), (2048.0, 30.0, 30.1)):
        for gamma, expect in ((ok, False), (bad, True)):
            x = (base * np.float32(gamma)).astype(np.float32)
            st = _stats()
            fp4.quantize(torch.from_numpy(x).cuda(), OF.UE5M3, 16, fp4.ROW, amax=dev_scalar(1.0), T=T, stats=st)
            torch.cuda.synchronize()
            c = _counts(st)
            assert c == oracle.block_health(x, OF.UE5M3, 16, amax=1.0, T=T)
            assert (c[0] > 0) == expect, (T, gamma, c)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("hn", [0, 16, 32])
def test_nan_propagates_through_tensor_amax(dtype, hn):
    t = _stressed(256, 1024, 75, gamma=3.0, dtype=dtype)
    v = t.values.copy()
    v[200, 777] = np.nan
    tn = synth.Tensor("x", v, dtype)
    got = fp4.tensor_amax(dev_input(tn), hn)
    clean = fp4.tensor_amax(dev_input(t), hn)
    torch.cuda.synchronize()
    assert np.isnan(got.item()) and np.isnan(oracle.tensor_amax(v, hn))
    assert clean.item() == oracle.tensor_amax(t.values, hn)


def test_nan_propagates_through_tile_local_forms():
    """All three tile-local forms (register-resident 16-row stripes, one workgroup per stripe,
    two-pass): the stripe holding a NaN reports amax NaN and gets g = 1 (the degenerate tensor
    scale, as the oracle's for a non-finite amax); every other stripe matches the oracle."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for name, rows, cols, stripe, dtype in (("register", 2 * cus * 16, 256, 16, "bf16"),
                                            ("single_pass", 2 * cus * 16, 64, 16, "fp32"),
                                            ("two_pass", 384, 2048, 128, "bf16")):
        t = _stressed(rows, cols, 76, gamma=2.0, dtype=dtype)
        v = t.values.copy()
        bad_row = rows // 2 + 3
        v[bad_row, cols - 5] = np.nan
        bad = bad_row // stripe
        ref = oracle.quantize_1d_local(t.values, OF.E4M3, 16, stripe=stripe, T=448.0)
        obs = torch.empty(len(ref.g), dtype=torch.float32, device="cuda")
        got = fp4.quantize_local(dev_input(synth.Tensor("x", v, dtype)), OF.E4M3, 16, stripe=stripe, amax_obs=obs)
        torch.cuda.synchronize()
        g, a = got.g.cpu().numpy(), obs.cpu().numpy()
        assert np.isnan(a[bad]) and g[bad] == 1.0, name
        assert oracle.tensor_scales(np.float32(np.nan), 448.0)[2] == 1.0
        keep = np.arange(len(ref.g)) != bad
        assert_f32_bits_equal(g[keep], ref.g[keep], f"{name} g")
        assert_f32_bits_equal(a[keep], ref.amax[keep], f"{name} amax")
