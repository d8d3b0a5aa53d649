"""Philox counter-based generator (oracle; test infrastructure only).

The stochastic-rounding recipe draws its random numbers from Philox (the upstream
gradient dY is rounded stochastically with a seeded generator; "UE5M3 FP4 Block Scaling
for Stable Language Model Pretraining", approach section (접근 방법), rounding bullets,
and developer-perspective section (개발자 관점), which warns that random-bit quality
matters). The pages do not define the generator; Philox-4x32-10 is taken from its
publication (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy as 1, 2, 3",
SC'11): the round function multiplies two counter words by fixed constants, swaps the
high and low product halves into the other lanes xor-ed with the key, and the key is
bumped by the Weyl constants between rounds.

The round structure is written once, generic in the word width, so the same code
instantiated at 4x64 can be checked against NumPy's Philox bit generator.
"""
from __future__ import annotations

import numpy as np

PHILOX4x32_M = (0xD2511F53, 0xCD9E8D57)
PHILOX4x32_W = (0x9E3779B9, 0xBB67AE85)
PHILOX4x64_M = (0xD2E7470EE14C6C93, 0xCA5A826395121157)
PHILOX4x64_W = (0x9E3779B97F4A7C15, 0xBB67AE8584CAA73B)


def philox_generic(ctr, key, rounds: int, bits: int, M, W):
    """Philox-4xW on Python ints (any width). ctr: 4 words, key: 2 words."""
    mask = (1 << bits) - 1
    c0, c1, c2, c3 = (int(x) & mask for x in ctr)
    k0, k1 = (int(x) & mask for x in key)
    for r in range(rounds):
        if r > 0:
            k0, k1 = (k0 + W[0]) & mask, (k1 + W[1]) & mask
        p0, p1 = M[0] * c0, M[1] * c2
        hi0, lo0 = p0 >> bits, p0 & mask
        hi1, lo1 = p1 >> bits, p1 & mask
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return c0, c1, c2, c3


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Vectorised Philox-4x32-10 over uint32 arrays (broadcasting). Returns 4 uint32 arrays."""
    m32 = np.uint64(0xFFFFFFFF)
    c = [np.asarray(x, dtype=np.uint64) & m32 for x in (c0, c1, c2, c3)]
    k = [np.uint64(int(k0) & 0xFFFFFFFF), np.uint64(int(k1) & 0xFFFFFFFF)]
    M0, M1 = np.uint64(PHILOX4x32_M[0]), np.uint64(PHILOX4x32_M[1])
    for r in range(10):
        if r > 0:
            k = [(k[0] + np.uint64(PHILOX4x32_W[0])) & m32, (k[1] + np.uint64(PHILOX4x32_W[1])) & m32]
        p0 = M0 * c[0]           # < 2^64, exact in uint64
        p1 = M1 * c[2]
        hi0, lo0 = p0 >> np.uint64(32), p0 & m32
        hi1, lo1 = p1 >> np.uint64(32), p1 & m32
        c = [hi1 ^ c[1] ^ k[0], lo1, hi0 ^ c[3] ^ k[1], lo0]
    return [x.astype(np.uint32) for x in c]


def sr_uniform16(seed: int, offset: int, index: np.ndarray) -> np.ndarray:
    """16-bit uniform draw for logical element ``index`` of a stochastically rounded operand.

    One Philox call serves 8 consecutive elements: counter = (index>>3 as two 32-bit
    words, offset as two 32-bit words), key = seed as two 32-bit words; element takes
    output word (index>>1)&3 and, within it, the low half for even index and the high
    half for odd index. Counter = logical index makes the draws independent of any
    launch geometry; ``offset`` separates steps and operand views.
    """
    index = np.asarray(index, dtype=np.uint64)
    blk = index >> np.uint64(3)
    lo = blk & np.uint64(0xFFFFFFFF)
    hi = blk >> np.uint64(32)
    o = [np.uint64(offset & 0xFFFFFFFF), np.uint64((offset >> 32) & 0xFFFFFFFF)]
    out = philox4x32_10(lo, hi, np.broadcast_to(o[0], lo.shape), np.broadcast_to(o[1], lo.shape),
                        seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF)
    w = ((index >> np.uint64(1)) & np.uint64(3)).astype(np.int64)
    word = np.choose(w, out).astype(np.uint32)
    half = (index & np.uint64(1)).astype(np.uint32)
    return ((word >> (np.uint32(16) * half)) & np.uint32(0xFFFF)).astype(np.uint16)
