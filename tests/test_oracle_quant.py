"""Pins of the oracle quantizer: zero-scale rule, headroom edge, nearest-ness, E8M0 rule,
stochastic rounding statistics, 2D and transposed views, the amax cache (CPU only)."""
import math

import numpy as np
import pytest

import oracle
from oracle import formats as F
from oracle.quantize import sr_e2m1, e8m0_block


def test_zero_scale_rule():
    x = np.zeros((4, 64), np.float32)
    x[1, 16:32] = 1e-30          # amax_b * T / A far below half the smallest UE5M3 subnormal
    x[2, :] = np.linspace(-3, 3, 64)
    for fmt, one in ((F.UE5M3, 0x78), (F.E4M3, 0x38)):
        q = oracle.quantize_1d(x, fmt, 16, amax=3.0, T=448)
        assert q.scales[0].tolist() == [one] * 4
        assert q.scales[1, 1] == one
        assert np.all(F.decode_e2m1(q.codes[0]) == 0) and np.all(F.decode_e2m1(q.codes[1]) == 0)
        assert q.n_zero == 12     # rows 0, 1 (incl. the tiny block) and 3
        assert np.all(q.scales[2] != one) or fmt == F.E4M3


@pytest.mark.parametrize("T,gamma_ok,gamma_bad", [(448, 137.0, 137.3), (2048, 30.0, 30.1)])
def test_headroom_edge(T, gamma_ok, gamma_bad):
    """With cached amax A and the true amax grown by gamma, no block scale saturates iff
    gamma * T <= 61440 (headroom about 137x at T=448 and 30x at T=2048)."""
    rng = np.random.default_rng(5)
    base = rng.uniform(-1, 1, (8, 256)).astype(np.float32)
    base[0, 0] = 1.0
    for gamma, expect_sat in ((gamma_ok, False), (gamma_bad, True)):
        x = (base * np.float32(gamma)).astype(np.float32)
        q = oracle.quantize_1d(x, F.UE5M3, 16, amax=1.0, T=T)
        assert (q.n_sat > 0) == expect_sat, (gamma, q.n_sat)


def test_block_scale_and_payload_are_nearest():
    rng = np.random.default_rng(6)
    x = (rng.standard_t(3, (64, 512)) * 0.7).astype(np.float32)
    A = float(np.max(np.abs(x)))
    q = oracle.quantize_1d(x, F.UE5M3, 16, amax=A, T=448)
    s_enc, s_blk, g = oracle.tensor_scales(A, 448)
    amax_b = np.abs(x).reshape(64, 32, 16).max(axis=2)
    v = (amax_b * s_blk).astype(np.float32).astype(np.float64)
    S = F.UE5M3_VALUES[q.scales.astype(int)]
    d = np.abs(F.UE5M3_VALUES[None, :] - v.reshape(-1, 1)).min(axis=1)
    assert np.all(np.abs(S.reshape(-1) - v.reshape(-1)) == d)   # nearest codebook entry
    r = (x.reshape(64, 32, 16) * (s_enc / S.astype(np.float32))[..., None].astype(np.float32)).astype(np.float32)
    dq = np.abs(F.decode_e2m1(q.codes).reshape(64, 32, 16))
    best = np.abs(F.E2M1_MAGS[None, :] - np.abs(r).reshape(-1, 1).astype(np.float64)).min(axis=1)
    assert np.all(np.abs(dq.reshape(-1) - np.abs(r).reshape(-1)) == best)
    # decoded tensor approximates x: error at most half the local E2M1 spacing (<=1) times S*g
    xh = F.decode_e2m1(q.codes).reshape(64, 32, 16) * (S * g)[..., None]
    assert np.all(np.abs(xh - x.reshape(64, 32, 16)) <= 1.0 * (S * g)[..., None] * 1.0000001)


def test_e8m0_rule():
    rng = np.random.default_rng(8)
    x = (rng.standard_normal((32, 256)) * np.exp(rng.uniform(-20, 20, (32, 1)))).astype(np.float32)
    x[3, 32:64] = 0
    q = oracle.quantize_1d(x, F.E8M0, 32)
    amax_b = np.abs(x).reshape(32, 8, 32).max(axis=2)
    for i in range(32):
        for b in range(8):
            a = float(amax_b[i, b])
            E = 0 if a == 0 else max(-127, min(127, math.frexp(a)[1] - 1 - 2))
            assert q.scales[i, b] == E + 127
            mx = np.max(np.abs(F.decode_e2m1(q.codes[i, b * 32:(b + 1) * 32])))
            assert (a == 0 and mx == 0) or mx in (4.0, 6.0)
    assert q.g == 1.0


def test_sr_fixed_points_and_sign():
    vals = np.array(list(F.E2M1_MAGS) + [-x for x in F.E2M1_MAGS], np.float32)
    for u in (0, 1, 32767, 65535):
        c = sr_e2m1(vals, np.full(vals.shape, u, np.uint16))
        assert np.array_equal(F.decode_e2m1(c), vals.astype(np.float64))
    assert int(sr_e2m1(np.float32(7.5), np.uint16(0))) == 7
    assert int(sr_e2m1(np.float32(-0.1), np.uint16(65535))) == 8


@pytest.mark.parametrize("r", [0.3, 1.1, 2.71, 4.9, -0.83, -3.33])
def test_sr_unbiased(r):
    n = 1_000_000
    idx = np.arange(n, dtype=np.uint64)
    u = oracle.philox.sr_uniform16(42, 17, idx)
    vals = F.decode_e2m1(sr_e2m1(np.full(n, r, np.float32), u))
    a = abs(np.float32(r))
    lo = F.E2M1_MAGS[np.searchsorted(F.E2M1_MAGS, a, side="right") - 1]
    hi = F.E2M1_MAGS[np.searchsorted(F.E2M1_MAGS, a, side="right")]
    p = (a - lo) / (hi - lo)
    sigma = (hi - lo) * math.sqrt(p * (1 - p) / n)
    bias_bound = (hi - lo) * 2.0 ** -16
    assert abs(abs(vals.mean()) - float(a)) <= 3 * sigma + bias_bound


def test_sr_reproducible_and_offset_sensitive():
    x = np.random.default_rng(9).standard_normal((16, 128)).astype(np.float32)
    a = oracle.quantize_1d(x, F.UE5M3, 16, amax=4.0, T=448, rounding="sr", seed=42, offset=8)
    b = oracle.quantize_1d(x, F.UE5M3, 16, amax=4.0, T=448, rounding="sr", seed=42, offset=8)
    c = oracle.quantize_1d(x, F.UE5M3, 16, amax=4.0, T=448, rounding="sr", seed=42, offset=9)
    assert np.array_equal(a.codes, b.codes) and not np.array_equal(a.codes, c.codes)
    assert np.array_equal(a.scales, c.scales)


def test_2d_views_share_scales():
    w = np.random.default_rng(10).standard_normal((64, 96)).astype(np.float32) * 0.02
    A = float(np.max(np.abs(w)))
    q = oracle.quantize_2d(w, F.UE5M3, amax=A, T=448)
    assert q.scales.shape == (4, 6)
    tiles = np.abs(w).reshape(4, 16, 6, 16).max(axis=(1, 3))
    _, s_blk, _ = oracle.tensor_scales(A, 448)
    assert np.array_equal(q.scales, F.encode_scale((tiles * s_blk).astype(np.float32), F.UE5M3))
    # every element of a tile is quantized with that tile's scale, in both views
    qa, sa = oracle.operand_from_quant(q, "2d")
    qt, st = oracle.operand_from_quant(q, "2dT")
    assert np.array_equal(qt, qa.T) and np.array_equal(np.repeat(st, 16, axis=1), np.repeat(sa, 16, axis=1).T)


def test_col_view_is_transposed_row_view():
    x = np.random.default_rng(11).standard_normal((64, 48)).astype(np.float32)
    for n in (0, 16, 32):
        A = float(oracle.tensor_amax(x, n))
        q = oracle.quantize_col(x, F.UE5M3, 16, amax=A, T=2048, hadamard_n=n)
        ref = oracle.quantize_1d(oracle.transposed_view(x, n), F.UE5M3, 16, amax=A, T=2048)
        assert q.codes.shape == (48, 64) and np.array_equal(q.codes, ref.codes)


def test_tensor_scales_special_cases():
    for A in (0.0, np.inf, np.nan, 1e-40):
        s = oracle.tensor_scales(A, 448)
        assert all(v == 1.0 for v in s) or A == 1e-40
    s_enc, s_blk, g = oracle.tensor_scales(2.0, 448)
    assert s_enc == np.float32(6 * 448 / 2.0) and s_blk == np.float32(224.0) and g == np.float32(1 / 1344.0)


def test_amax_cache_sample_and_hold():
    c = oracle.AmaxCache(50)
    seen = [float(c.update(s, s + 1)) for s in range(120)]
    assert seen[0] == 1 and seen[49] == 1 and seen[50] == 51 and seen[99] == 51 and seen[100] == 101
    c.reset()                   # a resumed run: cache not checkpointed
    assert float(c.update(123, 7.0)) == 7.0 and float(c.update(124, 9.0)) == 7.0
    d1 = oracle.AmaxCache(1)
    assert [float(d1.update(s, s * 2.0)) for s in range(3)] == [0.0, 2.0, 4.0]


def _max_element_block(view_vals, codes, scale_vals, block, two_d=False):
    """(scale value, E2M1 code) of the block holding the largest |value| of an operand view."""
    i, k = np.unravel_index(np.argmax(np.abs(view_vals)), view_vals.shape)
    s = scale_vals[i // 16, k // 16] if two_d else scale_vals[i, k // block]
    return float(s), int(codes[i, k]), float(view_vals[i, k])


@pytest.mark.parametrize("fmt,T", [(F.UE5M3, 448.0), (F.UE5M3, 2048.0), (F.E4M3, 448.0)])
@pytest.mark.parametrize("sign", [1.0, -1.0])
def test_true_amax_maps_to_scale_T_and_payload_6(fmt, T, sign):
    """Tensor-scale pin, independent of the formula's own restatement. With the cached amax
    equal to the true max|x|, the block holding that element gets block-scale value exactly
    T (the headroom figures 61440/448 and 61440/2048 of the key-contributions section say the
    cached amax sits at scale value T), and the element itself gets E2M1 code +-6 (0x7 /
    0xF), the codebook's largest magnitude, so the payload range is fully used. Its decoded
    value 6 * T * g then reproduces the amax within float32 rounding, which pins g. A
    tensor scale built as T/A instead of 6T/A would give code +-1 here, and a g of 1/s_blk
    a decoded value 6 times too large."""
    rng = np.random.default_rng(31)
    x = (rng.standard_t(3, (128, 256)) * 0.37).astype(np.float32)
    i, k = np.unravel_index(np.argmax(np.abs(x)), x.shape)
    x[i, k] = np.float32(sign) * np.abs(x[i, k])
    want_code = 0x7 | (0x8 if sign < 0 else 0)
    for view in ("row", "col", "col16", "2d"):
        if view == "row":
            A = oracle.tensor_amax(x)
            q = oracle.quantize_1d(x, fmt, 16, amax=A, T=T)
            vals, two_d = x, False
        elif view.startswith("col"):
            hn = 16 if view == "col16" else 0
            A = oracle.tensor_amax(x, hn)
            q = oracle.quantize_col(x, fmt, 16, amax=A, T=T, hadamard_n=hn)
            vals, two_d = oracle.transposed_view(x, hn), False
        else:
            A = oracle.tensor_amax(x)
            q = oracle.quantize_2d(x, fmt, amax=A, T=T)
            vals, two_d = x, True
        if view == "col16":      # the rotated maximum's sign is whatever the FWHT made it
            v_sign = np.sign(vals.ravel()[np.argmax(np.abs(vals))])
            want = 0x7 | (0x8 if v_sign < 0 else 0)
        else:
            want = want_code
        S, code, v = _max_element_block(vals, q.codes, q.scale_values(), 16, two_d)
        assert S == T, (view, S)
        assert code == want, (view, hex(code))
        decoded = 6.0 * T * float(q.g)
        assert abs(decoded - abs(v)) <= 4 * 2.0 ** -24 * abs(v), (view, decoded, v)


def test_block_health_matches_quantizer_counts_and_headroom_edge():
    """The health counts agree with the quantizer's own saturation and zero-scale counts (whose
    saturation edge is pinned at gamma * T = 61440 above), in every view."""
    rng = np.random.default_rng(41)
    base = rng.uniform(-1, 1, (64, 256)).astype(np.float32)
    base[3, 32:48] = 0.0                      # a zero block (ROW view)
    base[0, 0] = 1.0
    for gamma in (1.0, 137.0, 137.3, 300.0):
        x = (base * np.float32(gamma)).astype(np.float32)
        for fmt in (F.UE5M3, F.E4M3):
            q = oracle.quantize_1d(x, fmt, 16, amax=1.0, T=448)
            assert oracle.block_health(x, fmt, 16, amax=1.0, T=448) == (q.n_sat, q.n_zero, 0)
            qc = oracle.quantize_col(x, fmt, 16, amax=1.0, T=448, hadamard_n=16)
            assert oracle.block_health(x, fmt, 16, amax=1.0, T=448, view="col", hadamard_n=16) == \
                (qc.n_sat, qc.n_zero, 0)
            q2 = oracle.quantize_2d(x, fmt, amax=1.0, T=448)
            assert oracle.block_health(x, fmt, 16, amax=1.0, T=448, view="2d") == (q2.n_sat, q2.n_zero, 0)
        sat = oracle.block_health(x, F.UE5M3, 16, amax=1.0, T=448)[0]
        assert (sat > 0) == (gamma * 448 > 61440), gamma
    qm = oracle.quantize_1d(base, F.E8M0, 32)
    assert oracle.block_health(base, F.E8M0, 32) == (0, qm.n_zero, 0) and qm.n_zero == 0
    z = base.copy()
    z[5, 64:96] = 0.0
    assert oracle.block_health(z, F.E8M0, 32) == (0, 1, 0) == (0, oracle.quantize_1d(z, F.E8M0, 32).n_zero, 0)


def test_block_health_counts_nonfinite_blocks():
    """Hand-placed Inf and NaN inputs: each block holding one counts once as non-finite; an Inf
    block's unrounded scale is infinite, so it also counts as saturated (a NaN block does not)."""
    x = np.random.default_rng(42).uniform(-1, 1, (32, 128)).astype(np.float32)
    x[2, 5] = np.inf           # ROW block (2, 0)
    x[2, 7] = np.nan           # same block
    x[9, 100] = -np.inf        # ROW block (9, 6)
    x[17, 40] = np.nan         # ROW block (17, 2)
    assert oracle.block_health(x, F.UE5M3, 16, amax=1.0, T=448) == (1, 0, 3)
    assert oracle.block_health(x, F.E8M0, 32) == (0, 0, 3)
    # COL view: blocks run along 16 tokens of one feature: (feature 5, tokens 0-15),
    # (feature 7, tokens 0-15), (100, 0-15), (40, 16-31)
    assert oracle.block_health(x, F.UE5M3, 16, amax=1.0, T=448, view="col") == (2, 0, 4)
    # 2D tiles: (0, 0) holds the Inf and a NaN (its maximum is NaN: not saturated), (0, 6) the
    # -inf, (1, 2) the NaN
    assert oracle.block_health(x, F.E4M3, 16, amax=1.0, T=448, view="2d") == (1, 0, 3)
    assert np.isnan(oracle.tensor_amax(x))
