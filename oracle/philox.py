"""Oracle noise generator: Philox4x32-10 and the Box-Muller transform, on the CPU.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import this
module; only the tests, the package's smoke check and the benchmark's CPU
baseline call it.

The FlashDP and DP-GRAPE pages say only that Gaussian noise is added to the
clipped sum ("noise addition": FlashDP abstract; DP-GRAPE English explainer,
Methodology).  They name no generator.  The generator here is the one this
library fixes for its noise: Philox4x32-10 as published by Salmon, Moraes,
Dror and Shaw ("Parallel Random Numbers: As Easy as 1, 2, 3", SC'11), with

* key     = (low 32 bits of seed, high 32 bits of seed),
* counter = (low 32 bits of block, high 32 bits of block, 0, 0),
  where block = offset + floor(e / 4) for output element e, and
* lane    = e mod 4 selects one of the four normals of that block.

Uniforms: u = ((w >> 9) + 0.5) * 2**-23, so every u lies strictly inside (0, 1)
and is exact in float32.  Normals: (z0, z1) from (u0, u1) and (z2, z3) from
(u2, u3) by Box-Muller, z = sqrt(-2 ln u_a) * (cos 2 pi u_b, sin 2 pi u_b).

Two forms of the generator are given: a scalar pure-Python one that reads
like the definition, and a numpy one that applies the same rounds to whole
arrays of counters.  Both are plain; neither is tuned.
"""
from __future__ import annotations

import math

import numpy as np

# Round multipliers and key increments of Philox-4x32 (SC'11, Philox section).
PHILOX_M0 = 0xD2511F53
PHILOX_M1 = 0xCD9E8D57
PHILOX_W0 = 0x9E3779B9   # golden ratio
PHILOX_W1 = 0xBB67AE85   # sqrt(3) - 1
ROUNDS = 10
MASK32 = 0xFFFFFFFF


def _round_scalar(ctr, key):
    """One Philox-4x32 round: two 32x32->64 products, then the S-box/permutation."""
    p0 = PHILOX_M0 * ctr[0]
    p1 = PHILOX_M1 * ctr[2]
    hi0, lo0 = p0 >> 32, p0 & MASK32
    hi1, lo1 = p1 >> 32, p1 & MASK32
    return [hi1 ^ ctr[1] ^ key[0], lo1, hi0 ^ ctr[3] ^ key[1], lo0]


def philox4x32_10(counter, key):
    """Scalar Philox4x32-10: counter is 4 words, key is 2 words; returns 4 words."""
    ctr = [int(c) & MASK32 for c in counter]
    k = [int(key[0]) & MASK32, int(key[1]) & MASK32]
    for r in range(ROUNDS):
        if r > 0:
            k = [(k[0] + PHILOX_W0) & MASK32, (k[1] + PHILOX_W1) & MASK32]
        ctr = _round_scalar(ctr, k)
    return ctr


def seed_key(seed: int):
    seed &= (1 << 64) - 1
    return (seed & MASK32, seed >> 32)


def block_counter(block: int):
    block &= (1 << 64) - 1
    return (block & MASK32, block >> 32, 0, 0)


def philox_words_scalar(seed: int, offset: int, nblocks: int):
    """Words of blocks offset .. offset+nblocks-1, as a list of 4-word lists."""
    key = seed_key(seed)
    return [philox4x32_10(block_counter(offset + i), key) for i in range(nblocks)]


def philox_words(seed: int, blocks) -> np.ndarray:
    """Vectorised Philox4x32-10 over an array of 64-bit block indices -> uint32 [n, 4]."""
    blocks = np.asarray(blocks, dtype=np.uint64).reshape(-1)
    m32 = np.uint64(MASK32)
    c0 = blocks & m32
    c1 = blocks >> np.uint64(32)
    c2 = np.zeros_like(c0)
    c3 = np.zeros_like(c0)
    k0, k1 = seed_key(seed)
    for r in range(ROUNDS):
        if r > 0:
            k0 = (k0 + PHILOX_W0) & MASK32
            k1 = (k1 + PHILOX_W1) & MASK32
        p0 = np.uint64(PHILOX_M0) * c0          # < 2**64: no wrap
        p1 = np.uint64(PHILOX_M1) * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & m32
        hi1, lo1 = p1 >> np.uint64(32), p1 & m32
        c0, c1, c2, c3 = (hi1 ^ c1 ^ np.uint64(k0), lo1,
                          hi0 ^ c3 ^ np.uint64(k1), lo0)
    return np.stack([c0, c1, c2, c3], axis=1).astype(np.uint32)


def words_to_uniform(w) -> np.ndarray:
    """u = ((w >> 9) + 0.5) * 2**-23 in float64 (exact; also exact in float32)."""
    w = np.asarray(w, dtype=np.uint64)
    return ((w >> np.uint64(9)).astype(np.float64) + 0.5) * 2.0 ** -23


def box_muller(ua, ub):
    """Two normals from two uniforms: radius sqrt(-2 ln ua), angle 2 pi ub."""
    rad = np.sqrt(-2.0 * np.log(ua))
    ang = 2.0 * np.pi * ub
    return rad * np.cos(ang), rad * np.sin(ang)


def normals_of_words(words: np.ndarray) -> np.ndarray:
    """uint32 [n, 4] Philox words -> float64 [n, 4] normals (z0, z1, z2, z3)."""
    u = words_to_uniform(words)
    z0, z1 = box_muller(u[:, 0], u[:, 1])
    z2, z3 = box_muller(u[:, 2], u[:, 3])
    return np.stack([z0, z1, z2, z3], axis=1)


def gaussian_at(seed: int, offset: int, elements) -> np.ndarray:
    """Normals xi_e for an array of element indices e (float64)."""
    e = np.asarray(elements, dtype=np.uint64).reshape(-1)
    blocks = np.uint64(offset) + e // np.uint64(4)
    lane = (e % np.uint64(4)).astype(np.int64)
    # one Philox call per distinct block
    ub, inv = np.unique(blocks, return_inverse=True)
    z = normals_of_words(philox_words(seed, ub))
    return z[inv.reshape(-1), lane]


def gaussian(seed: int, offset: int, n: int) -> np.ndarray:
    """Normals xi_0 .. xi_{n-1} (float64), four per Philox block starting at ``offset``."""
    nblocks = (n + 3) // 4
    if nblocks == 0:
        return np.zeros(0, dtype=np.float64)
    blocks = np.uint64(offset) + np.arange(nblocks, dtype=np.uint64)
    return normals_of_words(philox_words(seed, blocks)).reshape(-1)[:n]


def gaussian_scalar(seed: int, offset: int, n: int):
    """Pure-Python normals for small n (math module, float64)."""
    out = []
    for w in philox_words_scalar(seed, offset, (n + 3) // 4):
        u = [((x >> 9) + 0.5) * 2.0 ** -23 for x in w]
        for a, b in ((0, 1), (2, 3)):
            rad = math.sqrt(-2.0 * math.log(u[a]))
            out.append(rad * math.cos(2.0 * math.pi * u[b]))
            out.append(rad * math.sin(2.0 * math.pi * u[b]))
    return out[:n]


def noise_blocks(n_elements: int) -> int:
    """Philox blocks one call of n elements consumes: ceil(n / 4)."""
    return (int(n_elements) + 3) // 4
