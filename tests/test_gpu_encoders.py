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


def test_stochastic_e2m1_decision_boundaries():
    """The rule rounds up iff the draw u < 2^16 f (strict), f the value's fraction within its
    codebook interval. Values whose f is exactly k/2^16, one float step above or below that,
    drawn against u = k - 1, k, k + 1, in every interval and with both signs; and the tiniest
    magnitudes (f = 2|r|, down to the smallest subnormal) against u = 0, 1, 2, 65535."""
    rng = np.random.default_rng(7)
    rs, us = [], []
    for lo, hi in ((0.0, 0.5), (0.5, 1.0), (1.0, 1.5), (1.5, 2.0), (2.0, 3.0), (3.0, 4.0), (4.0, 6.0)):
        for k in rng.integers(1, 65535, 256):
            a = np.float32(lo + (hi - lo) * (int(k) / 65536.0))          # exact: f = k / 2^16
            for aa in (a, np.nextafter(a, np.float32(np.inf)), np.nextafter(a, np.float32(-np.inf))):
                for d in (k - 1, k, k + 1):
                    rs += [aa, -aa]
                    us += [d, d]
    for e in range(14, 150):
        t = np.float32(2.0 ** -e)
        for d in (0, 1, 2, 65535):
            rs += [t, -t]
            us += [d, d]
    r = np.array(rs, np.float32)
    u = np.array(us, np.uint16)
    assert np.array_equal(_run(r, 4, u), sr_e2m1(r, u))


def test_stochastic_e2m1_saturation_and_specials():
    """Magnitudes from 6 up (where the rule gives 6 whatever the draw), the largest float,
    infinities and NaNs of both signs, zeros and the codebook's top interval, each against
    the draws 0, 1, 2^15 and 65535."""
    big = np.array([6.0, np.nextafter(np.float32(6.0), np.float32(np.inf)), 6.5, 7.0, 7.999, 8.0, 11.0, 12.0, 16.0,
                    1e4, 1e30, 3.4028235e38, np.inf, np.nan, 0.0, 4.0, 5.0, 5.999,
                    np.nextafter(np.float32(6.0), np.float32(0))], np.float32)
    r = np.concatenate([big, -big]).astype(np.float32)
    r = np.repeat(r, 4)
    u = np.tile(np.array([0, 1, 1 << 15, 65535], np.uint16), r.size // 4)
    assert np.array_equal(_run(r, 4, u), sr_e2m1(r, u))


def _oracle_code(x: np.ndarray, which: int) -> np.ndarray:
    x = np.asarray(x, np.float32)
    if which == 3:
        return e8m0_block(x)[0].astype(np.int64)
    return OF.encode_scale(x, OF.UE5M3 if which == 1 else OF.E4M3).astype(np.int64)


def _oracle_steps(which: int):
    """(code at +0, [(bit pattern, new code)] of every float32 where the oracle's code differs
    from the previous float's). The candidate points are where a nearest-even encoder can
    change its code (every codebook midpoint and its float neighbours; for E8M0 every power of
    two and the smallest subnormal); the oracle alone decides which of them are steps."""
    if which == 3:
        pts = np.ldexp(np.float64(1.0), np.arange(-149, 128)).astype(np.float32)
    else:
        v = OF.SCALE_VALUES[OF.UE5M3 if which == 1 else OF.E4M3]
        mids = ((v[:-1] + v[1:]) / 2).astype(np.float32)
        pts = np.concatenate([mids, np.nextafter(mids, np.float32(np.inf)), v[1:].astype(np.float32)])
    pts = np.unique(pts[pts > 0])
    prev = np.nextafter(pts, np.float32(0))
    c, cp = _oracle_code(pts, which), _oracle_code(prev, which)
    step = c != cp
    return int(_oracle_code(np.zeros(1, np.float32), which)[0]), \
        sorted(zip(pts[step].view(np.uint32).astype(np.int64).tolist(), c[step].tolist()))


@pytest.mark.parametrize("which,name", [(1, "ue5m3"), (2, "e4m3"), (3, "e8m0")])
def test_scale_encoder_every_nonnegative_float(which, name):
    """Every non-negative float32 that is not a NaN (all 2^31 - 2^23 + 1 bit patterns from +0 to
    +inf, subnormals included), in increasing order through the device scale encoder: its codes
    start at the oracle's code of +0 and change exactly at the oracle's steps, to the oracle's
    codes, and nowhere else. A piecewise-constant function is fixed by its first value and its
    steps, so the device encoder equals the oracle's on every one of those inputs. (A block
    maximum of +inf is outside the E8M0 exponent's contract: that sweep ends at the largest
    finite float.)"""
    start, want = _oracle_steps(which)
    last = 0x7F7FFFFF if which == 3 else 0x7F800000   # +inf is outside the E8M0 exponent's contract
    C = 1 << 27
    steps, prev_code, first = [], None, None
    for c0 in range(0, last + 1, C):
        n = min(C, last + 1 - c0)
        bits = torch.arange(c0, c0 + n, dtype=torch.int64, device="cuda").to(torch.int32)
        codes = fp4.debug_encode(bits.view(torch.float32), which).to(torch.int32)
        if first is None:
            first = int(codes[0].item())
        elif int(codes[0].item()) != prev_code:
            steps.append((c0, int(codes[0].item())))
        idx = torch.nonzero(codes[1:] != codes[:-1]).flatten() + 1
        for i, cd in zip(idx.cpu().tolist(), codes[idx].cpu().tolist()):
            steps.append((c0 + i, cd))
        prev_code = int(codes[-1].item())
        del bits, codes
    assert first == start, (name, first, start)
    assert steps == want, (name, len(steps), len(want),
                           next(((a, b) for a, b in zip(steps, want) if a != b), None))
