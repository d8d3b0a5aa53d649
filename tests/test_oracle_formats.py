"""Pins of the oracle's codebooks and encoders (CPU only)."""
import os

import numpy as np
import pytest
import torch

from oracle import formats as F

HERE = os.path.dirname(os.path.abspath(__file__))


def page_constants():
    out = {}
    with open(os.path.join(HERE, "golden", "page_constants.txt"), encoding="utf-8") as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            name, val = line.split("|")[0].split()
            out[name] = val
    return out


C = page_constants()


def test_ue5m3_codebook_matches_pages():
    v = F.UE5M3_VALUES
    assert v[-1] == float(C["ue5m3_max"]) == 61440.0
    assert len(v) == 248 and np.all(np.diff(v) > 0)
    assert v[1] == 2.0 ** -17                      # smallest subnormal under the bias-15 reading
    assert F.SCALE_ONE_CODE[F.UE5M3] == 0x78
    # headroom figures: maximum / T, rounded as the page quotes them
    assert round(v[-1] / float(C["T_default"])) == int(C["headroom_T448"])
    assert v[-1] / float(C["T_override"]) == float(C["headroom_T2048"])


def test_e4m3_codebook():
    v = F.E4M3_VALUES
    assert v[-1] == float(C["e4m3_max"]) == 448.0
    assert len(v) == 127 and np.all(np.diff(v) > 0)
    assert v[1] == 2.0 ** -9 and F.SCALE_ONE_CODE[F.E4M3] == 0x38


def test_e4m3_encoder_matches_torch_float8_cast():
    rng = np.random.default_rng(7)
    x = np.concatenate([
        rng.uniform(0, 448, 200000), np.exp(rng.uniform(-25, 6, 200000)),
        (F.E4M3_VALUES[:-1] + F.E4M3_VALUES[1:]) / 2,           # every tie
        F.E4M3_VALUES,
    ]).astype(np.float32)
    x = x[x <= 448]
    ours = F.encode_scale(x, F.E4M3)
    theirs = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, theirs)


def test_e2m1_codebook_by_definition():
    assert list(F.E2M1_MAGS) == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert list(F.E2M1_VALUES[8:]) == [-0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]
    assert len(set(F.E2M1_VALUES.tolist())) == 15   # +0 and -0 compare equal


@pytest.mark.parametrize("x,code", [
    (0.0, 0), (0.25, 0), (0.2500001, 1), (0.5, 1), (0.75, 2), (1.25, 2), (1.2500001, 3), (1.75, 4),
    (2.5, 4), (2.5000002, 5), (3.5, 6), (5.0, 6), (5.0000005, 7), (6.0, 7), (7.9, 7), (1e30, 7),
    (np.inf, 7), (-0.0, 8), (-0.1, 8), (-0.75, 10), (-5.0, 14), (-100.0, 15), (1e-45, 0),
])
def test_e2m1_ties_and_saturation(x, code):
    assert int(F.encode_e2m1(np.float32(x))) == code


def _brute_nearest_even(v, values):
    d = np.abs(values[None, :] - v[:, None])
    best = d.min(axis=1)
    cand = d == best[:, None]
    codes = np.arange(len(values))
    # among equidistant codes prefer the even one
    even = cand & (codes[None, :] % 2 == 0)
    return np.where(even.any(axis=1), np.argmax(even, axis=1), np.argmax(cand, axis=1))


@pytest.mark.parametrize("fmt", [F.UE5M3, F.E4M3])
def test_scale_encoder_is_nearest_even(fmt):
    vals = F.SCALE_VALUES[fmt]
    rng = np.random.default_rng(3)
    v = np.concatenate([np.exp(rng.uniform(-45, 12, 30000)), (vals[:-1] + vals[1:]) / 2, vals]).astype(np.float32)
    v = v[v <= vals[-1]]
    assert np.array_equal(F.encode_scale(v, fmt), _brute_nearest_even(v.astype(np.float64), vals))
    # saturation
    assert int(F.encode_scale(np.float32(vals[-1] * 1.5), fmt)) == len(vals) - 1
    assert int(F.encode_scale(np.float32(np.inf), fmt)) == len(vals) - 1


def test_e2m1_encoder_is_nearest_even():
    rng = np.random.default_rng(4)
    v = np.concatenate([rng.uniform(0, 6, 50000), (F.E2M1_MAGS[:-1] + F.E2M1_MAGS[1:]) / 2]).astype(np.float32)
    assert np.array_equal(F.encode_e2m1(v), _brute_nearest_even(v.astype(np.float64), F.E2M1_MAGS))
