"""Pins of the oracle's Philox generator and Hadamard transform (CPU only)."""
import numpy as np
import pytest
import scipy.linalg

from oracle import philox as P
from oracle.hadamard import fwht_tokens


def test_generic_round_structure_matches_numpy_philox4x64():
    """NumPy's Philox bit generator is Philox-4x64-10; it increments the counter before
    generating, so its first block is the function at counter + 1."""
    for ctr, key in (((5, 6, 7, 8), (11, 12)), ((2 ** 64 - 2, 0, 3, 1), (2 ** 63, 99))):
        bg = np.random.Philox(counter=np.array(ctr, dtype=np.uint64), key=np.array(key, dtype=np.uint64))
        raw = [int(bg.random_raw()) for _ in range(4)]
        c1 = list(ctr)
        c1[0] = (c1[0] + 1) % 2 ** 64
        if c1[0] == 0:
            c1[1] += 1
        assert list(P.philox_generic(c1, key, 10, 64, P.PHILOX4x64_M, P.PHILOX4x64_W)) == raw


# Known-answer vectors for Philox-4x32-10 published with the generator (Salmon et al., SC'11,
# Random123 distribution): (counter words, key words) -> output words.
KAT = [
    ((0, 0, 0, 0), (0, 0), (0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8)),
    ((0xFFFFFFFF,) * 4, (0xFFFFFFFF,) * 2, (0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD)),
    ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344), (0xA4093822, 0x299F31D0),
     (0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1)),
]


@pytest.mark.parametrize("ctr,key,out", KAT)
def test_philox4x32_known_answers(ctr, key, out):
    assert P.philox_generic(ctr, key, 10, 32, P.PHILOX4x32_M, P.PHILOX4x32_W) == out
    got = P.philox4x32_10(*[np.array([c], np.uint32) for c in ctr], *key)
    assert tuple(int(g[0]) for g in got) == out


def test_vectorised_equals_generic():
    rng = np.random.default_rng(1)
    c = rng.integers(0, 2 ** 32, (4, 64), dtype=np.uint64)
    k = (0xDEADBEEF, 0x12345678)
    v = P.philox4x32_10(*c, *k)
    for j in range(64):
        g = P.philox_generic([int(c[i, j]) for i in range(4)], k, 10, 32, P.PHILOX4x32_M, P.PHILOX4x32_W)
        assert tuple(int(v[i][j]) for i in range(4)) == g


def test_sr_uniform16_word_mapping():
    seed, offset = (1 << 40) + 42, (3 << 32) + 9
    idx = np.array([0, 1, 2, 7, 8, 13, 2 ** 33 + 5], np.uint64)
    u = P.sr_uniform16(seed, offset, idx)
    for i, ui in zip(idx.tolist(), u.tolist()):
        blk = i >> 3
        out = P.philox_generic((blk & 0xFFFFFFFF, blk >> 32, offset & 0xFFFFFFFF, offset >> 32),
                               (seed & 0xFFFFFFFF, seed >> 32), 10, 32, P.PHILOX4x32_M, P.PHILOX4x32_W)
        assert ui == (out[(i >> 1) & 3] >> (16 * (i & 1))) & 0xFFFF


def test_sr_uniform16_is_uniform():
    u = P.sr_uniform16(42, 0, np.arange(1 << 20, dtype=np.uint64)).astype(np.int64)
    counts = np.bincount(u >> 8, minlength=256)
    e = len(u) / 256
    chi2 = float(np.sum((counts - e) ** 2 / e))
    assert chi2 < 255 + 5 * np.sqrt(2 * 255)          # ~5 sigma of chi2(255)
    r = np.corrcoef(u[:-1], u[1:])[0, 1]
    assert abs(r) < 5 / np.sqrt(len(u))


@pytest.mark.parametrize("n", [16, 32])
def test_fwht_is_sylvester_hadamard(n):
    H = scipy.linalg.hadamard(n).astype(np.float64)
    assert np.array_equal(H @ H.T, n * np.eye(n))
    E = np.eye(n, dtype=np.float32)
    assert np.array_equal(fwht_tokens(E, n), H.astype(np.float32))      # column j = H e_j
    x = np.random.default_rng(2).integers(-50, 50, (4 * n, 7)).astype(np.float32)
    ref = np.concatenate([H @ x[i * n:(i + 1) * n].astype(np.float64) for i in range(4)])
    assert np.array_equal(fwht_tokens(x, n), ref.astype(np.float32))    # exact on small integers
    assert np.array_equal(fwht_tokens(fwht_tokens(x, n), n), n * x)
