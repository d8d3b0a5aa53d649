"""Device encoders (through fp4_debug_encode) against the oracle's enumerated codebooks."""
import numpy as np
import pytest
import torch

import oracle
from oracle import formats as OF
from oracle.quantize import e8m0_block, sr_e2m1

pytestmark = pytest.mark.gpu

fp4 = pytest.importorskip("fp4_block_scaled_tensor_amd")


def _around(values: np.ndarray) -> np.ndarray:
    """Every codebook midpoint and value, and their float32 neighbours."""
    mids = ((values[:-1] + values[1:]) / 2).astype(np.float32)
    pts = np.concatenate([mids, values.astype(np.float32)])
    return np.concatenate([pts, np.nextafter(pts, np.float32(np.inf)), np.nextafter(pts, np.float32(0))])


def _sweep(lo_exp, hi_exp, n_per_exp, seed):
    rng = np.random.default_rng(seed)
    e = np.repeat(np.arange(lo_exp, hi_exp), n_per_exp)
    m = rng.integers(0, 1 << 23, e.size, dtype=np.uint32)
    bits = ((e + 127).astype(np.uint32) << 23) | m
    return bits.view(np.float32)


def _run(x: np.ndarray, which: int, u16: np.ndarray | None = None) -> np.ndarray:
    dx = torch.from_numpy(np.ascontiguousarray(x, np.float32)).cuda()
    du = torch.from_numpy(u16.view(np.int16).copy()).cuda() if u16 is not None else None
    out = fp4.debug_encode(dx, which, du)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def test_e2m1_payload_encoder():
    pos = np.concatenate([_sweep(-12, 5, 1 << 18, 1), _around(OF.E2M1_MAGS),
                          np.array([0.0, 1e-45, 1e-38, 3e38, np.inf, 7.0, 6.5, 5.5], np.float32)])
    x = np.concatenate([pos, -pos]).astype(np.float32)
    assert np.array_equal(_run(x, 0), OF.encode_e2m1(x))


def test_e2m1_payload_encoder_every_float_in_decision_range():
    """Every float32 with magnitude in [2^-4, 2^4) (all 2^27 bit patterns of those eight
    binades, both signs): every E2M1 decision boundary, tie and the saturation edge lies
    inside this range; outside it the code is 0 or 6 (covered by the sweep above)."""
    mant = np.arange(1 << 23, dtype=np.uint32)
    for e in range(-4, 4):
        for sign in (0, 1):
            bits = (np.uint32(sign << 31) | (np.uint32(e + 127) << np.uint32(23))) | mant
            x = bits.view(np.float32)
            got = _run(x, 0)
            want = OF.encode_e2m1(x)
            if not np.array_equal(got, want):
                bad = np.flatnonzero(got != want)
                raise AssertionError(f"binade 2^{e} sign {sign}: {bad.size} codes differ, first x={x[bad[0]]!r} "
                                     f"got {got[bad[0]]} want {want[bad[0]]}")


@pytest.mark.parametrize("fmt,which,lo,hi", [(OF.UE5M3, 1, -24, 18), (OF.E4M3, 2, -14, 11)])
def test_scale_encoders(fmt, which, lo, hi):
    x = np.concatenate([_sweep(lo, hi, 1 << 15, 2 + which), _around(OF.SCALE_VALUES[fmt]),
                        np.array([0.0, 1e-45, 1e30, np.inf], np.float32)]).astype(np.float32)
    assert np.array_equal(_run(x, which), OF.encode_scale(x, fmt))


def test_e8m0_exponent():
    x = np.concatenate([_sweep(-126, 128, 4096, 5), np.array([0.0, 1e-45, 3e-39, 1e-40, 2.0 ** -126], np.float32)])
    assert np.array_equal(_run(x, 3), e8m0_block(x)[0])


def test_stochastic_e2m1():
    rng = np.random.default_rng(6)
    r = np.concatenate([rng.uniform(-7, 7, 1 << 20), np.repeat(OF.E2M1_VALUES, 64),
                        np.array([0.25, 0.75, 1.75, 3.5, 5.0, -0.0], np.float32).repeat(64)]).astype(np.float32)
    u = rng.integers(0, 1 << 16, r.size).astype(np.uint16)
    assert np.array_equal(_run(r, 4, u), sr_e2m1(r, u))
