"""Pins of the oracle's MXFP4 -> FP8 conversion (CPU only): E4M3 encoding against torch's
float8_e4m3fn cast, the exact value round trip where the page's alignment is lossless, the
chunk scale rule, and hand-worked elements."""
import numpy as np
import pytest
import torch

import oracle
from oracle import formats as F
from oracle.fp8convert import chunk_scale_codes, decode_e4m3_signed, encode_e4m3_signed


def _operand(rows, K, seed, spread):
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 16, (rows, K)).astype(np.uint8)
    base = rng.integers(100, 150, (rows, 1))
    scales = np.clip(base + rng.integers(-spread, spread + 1, (rows, K // 32)), 0, 254).astype(np.uint8)
    return codes, scales


def test_e4m3_encoder_matches_torch_cast():
    rng = np.random.default_rng(1)
    v = np.concatenate([rng.standard_normal(20000) * np.exp(rng.uniform(-12, 6, 20000)),
                        decode_e4m3_signed(np.arange(256)[np.arange(256) % 128 != 127]),      # every code
                        [2.0 ** -10, 3 * 2.0 ** -11, -(2.0 ** -10), 0.0, -0.0, 384.0, 1.5 * 2 ** -9]])
    v = v[np.abs(v) <= 448].astype(np.float32)
    want = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(encode_e4m3_signed(v.astype(np.float64)), want)


@pytest.mark.parametrize("spread", [0, 3, 20])
def test_round_trip_is_exact_within_14_binades(spread):
    codes, scales = _operand(64, 512, 2 + spread, spread)
    y, c8 = oracle.mxfp4_to_fp8(codes, scales)
    x = F.decode_e2m1(codes) * np.ldexp(1.0, np.repeat(scales.astype(np.int64), 32, axis=1) - 127)
    got = oracle.fp8_values(y, c8)
    emax = np.repeat(np.repeat(scales.astype(np.int64), 32, axis=1).reshape(64, 4, 128).max(axis=2), 128, axis=1)
    d = emax - np.repeat(scales.astype(np.int64), 32, axis=1)
    ok = d <= 14
    assert np.array_equal(got[ok], x[ok])
    # beyond 14 binades the value is the E4M3-rounded one: error below half a subnormal step
    step = np.ldexp(1.0, np.repeat(c8.astype(np.int64), 128, axis=1) - 127 - 9)
    assert np.all(np.abs(got[~ok] - x[~ok]) <= step[~ok] / 2)
    assert np.all(np.abs(decode_e4m3_signed(y)) <= 384)
    # transposed output is the same codes, transposed
    yt, c8t = oracle.mxfp4_to_fp8(codes, scales, transpose=True)
    assert np.array_equal(yt, y.T) and np.array_equal(c8t, c8)


def test_chunk_scale_rule_and_worked_elements():
    # chunk with block codes (127, 125, 120, 127): e_max = 127, c = 121
    scales = np.array([[127, 125, 120, 127]], np.uint8)
    assert chunk_scale_codes(scales).tolist() == [[121]]
    # tiny chunk: e_max = 3 -> c = 0 (shift limited to e_max)
    assert chunk_scale_codes(np.array([[3, 1, 0, 2]], np.uint8)).tolist() == [[0]]
    codes = np.zeros((1, 128), np.uint8)
    codes[0, 0] = 0x7        # +6 in block 0 (scale 2^0): 6 * 2^(127-121) = 384 -> E4M3 0x7C (1.5 * 2^8)
    codes[0, 1] = 0xA        # -1 in block 0: -64 -> 0xE8 (sign, exponent field 6+7=13, mantissa 0)
    codes[0, 32] = 0x1       # 0.5 in block 1 (2^-2): 0.5 * 2^(125-121) = 8 -> 0x50
    codes[0, 64] = 0x1       # 0.5 in block 2 (2^-7): 0.5 * 2^-1 = 0.25 -> 0x28
    codes[0, 96] = 0x8       # -0 in block 3 -> 0x80
    y, c8 = oracle.mxfp4_to_fp8(codes, scales)
    assert (y[0, 0], y[0, 1], y[0, 32], y[0, 64], y[0, 96]) == (0x7C, 0xE8, 0x50, 0x28, 0x80)
    assert y[0, 2] == 0 and c8[0, 0] == 121
    # a block 20 binades below its chunk's maximum: 6 * 2^(c-127) * 2^-14 in E4M3 units
    s2 = np.array([[140, 120, 140, 140]], np.uint8)        # c = 134, block 1 shift = -14
    c2 = np.zeros((1, 128), np.uint8)
    c2[0, 32], c2[0, 33], c2[0, 34] = 0x7, 0x1, 0x3          # 6, 0.5, 1.5 times 2^-14
    y2, _ = oracle.mxfp4_to_fp8(c2, s2)
    # 6 * 2^-14 = 1.5 * 2^-12 -> subnormal grid 2^-9: 0.1875 units -> 0; 0.5 * 2^-14 -> 0; 1.5 * 2^-14 -> 0
    assert (y2[0, 32], y2[0, 33], y2[0, 34]) == (0, 0, 0)
    s3 = np.array([[140, 130, 140, 140]], np.uint8)        # shift -4: 6 * 2^-4 = 0.375 = 3 * 2^-3
    y3, _ = oracle.mxfp4_to_fp8(c2, s3)
    assert decode_e4m3_signed(y3[0, 32]) == 0.375 and decode_e4m3_signed(y3[0, 33]) == 2.0 ** -5
