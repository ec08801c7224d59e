"""Philox4x64-10 and Philox4x32-10 counter-based generators, written from their
published definition.

TEST INFRASTRUCTURE ONLY: part of the CPU oracle.  Only tests, the smoke check
and the benchmark's CPU-baseline leg may import this package.

Source of the generators: J. K. Salmon, M. A. Moraes, R. O. Dror, D. E. Shaw,
"Parallel Random Numbers: As Easy as 1, 2, 3", SC'11 -- the Philox family,
instances N=4 words of W=64 bits and of W=32 bits, R=10 rounds.  One round
maps the counter (x0, x1, x2, x3) under the round key (k0, k1) to

    (hi(M1*x2) ^ x1 ^ k0,  lo(M1*x2),  hi(M0*x0) ^ x3 ^ k1,  lo(M0*x0))

where hi/lo are the upper/lower W bits of the 2W-bit product; between rounds
the key advances by the Weyl constants (golden ratio and sqrt(3)-1 in W-bit
fixed point).  The 4x64 instance is pinned bit-for-bit against numpy's
independent ``numpy.random.Philox`` in the tests, the 4x32 instance against
the known-answer vectors published with the generators.

The pages fix only that the projection is regenerated "from its seed and
metadata" (LoGRA paper text, paperpeel.com, §2.2 "Memory and
synchronization").  Which generator and which bits is this library's choice;
the layout is stated here and in ``include/logra.h``:

* key of a projection: ``(seed, (step << 32) | matrix_id)``;
* sign bits of A (Philox4x32-10): one block per (row j, 128-column group
  c = l >> 7) with 32-bit counter words ``(c, j | 2**31, matrix_id, step)``
  under the 32-bit key words ``(seed & 0xFFFFFFFF, seed >> 32)``; column l
  uses bit ``l & 31`` of output word ``(l & 127) >> 5``; bit 1 means
  sigma = -1, bit 0 means +1 (the top bit of counter word 1 keeps these
  blocks apart from the rounding draws' under an equal seed);
* Gaussian entries (the Gaussian projection variant, Philox4x64-10): one
  block per (row j, 4-column group c = l >> 2) with counter ``(j, c, 2, 0)``;
  column l takes Box-Muller pair ``(l & 3) >> 1`` of the four words, cosine
  for even l, sine for odd l (see ``gaussian_normals``);
* stochastic-rounding draws (Philox4x32-10, a quarter of the 4x64 instance's
  multiplies per draw): element e = (row0 + i) * k + l (logical index) of
  the matrix with projection key ``(sr_seed, (step << 32) | matrix_id)``
  uses the block with 32-bit counter words
  ``(g & 0xFFFFFFFF, g >> 32, matrix_id, step)``, g = e >> 3, under the
  32-bit key words ``(sr_seed & 0xFFFFFFFF, sr_seed >> 32)``, and takes the
  16 bits ``[16*(e & 1), +16)`` of output word ``(e & 7) >> 1``.
"""
from __future__ import annotations

import numpy as np

MASK32 = np.uint64(0xFFFFFFFF)
SHIFT32 = np.uint64(32)

# Multipliers and Weyl increments of Philox4x64 (Salmon et al., SC'11).
PHILOX_M0 = np.uint64(0xD2E7470EE14C6C93)
PHILOX_M1 = np.uint64(0xCA5A826395121157)
PHILOX_W0 = np.uint64(0x9E3779B97F4A7C15)
PHILOX_W1 = np.uint64(0xBB67AE8584CAA73B)
ROUNDS = 10


def _mulhilo64(a: np.ndarray, m: np.uint64):
    """128-bit product of uint64 array ``a`` and constant ``m`` as (hi, lo)."""
    a = np.asarray(a, dtype=np.uint64)
    m = np.uint64(m)
    a_lo, a_hi = a & MASK32, a >> SHIFT32
    m_lo, m_hi = m & MASK32, m >> SHIFT32
    with np.errstate(over="ignore"):
        p00 = a_lo * m_lo
        p01 = a_lo * m_hi
        p10 = a_hi * m_lo
        p11 = a_hi * m_hi
        mid = (p00 >> SHIFT32) + (p01 & MASK32) + (p10 & MASK32)
        lo = (p00 & MASK32) | ((mid & MASK32) << SHIFT32)
        hi = p11 + (p01 >> SHIFT32) + (p10 >> SHIFT32) + (mid >> SHIFT32)
    return hi, lo


def philox4x64_10(ctr, key):
    """Apply Philox4x64-10 to counters ``ctr`` (shape [..., 4]) under ``key``.

    ``key`` is a pair (k0, k1) of uint64 scalars or arrays broadcastable to the
    counter batch.  Returns an array of the same shape as ``ctr`` (uint64).
    """
    x = np.array(ctr, dtype=np.uint64, copy=True)
    if x.shape[-1] != 4:
        raise ValueError("counter must have 4 words")
    k0 = np.asarray(key[0], dtype=np.uint64)
    k1 = np.asarray(key[1], dtype=np.uint64)
    x0, x1, x2, x3 = x[..., 0], x[..., 1], x[..., 2], x[..., 3]
    with np.errstate(over="ignore"):
        for rnd in range(ROUNDS):
            if rnd:
                k0 = k0 + PHILOX_W0
                k1 = k1 + PHILOX_W1
            hi0, lo0 = _mulhilo64(x0, PHILOX_M0)
            hi1, lo1 = _mulhilo64(x2, PHILOX_M1)
            x0, x1, x2, x3 = hi1 ^ x1 ^ k0, lo1, hi0 ^ x3 ^ k1, lo0
    return np.stack([x0, x1, x2, x3], axis=-1)


# Multipliers and Weyl increments of Philox4x32 (Salmon et al., SC'11).
PHILOX32_M0 = np.uint64(0xD2511F53)
PHILOX32_M1 = np.uint64(0xCD9E8D57)
PHILOX32_W0 = np.uint64(0x9E3779B9)
PHILOX32_W1 = np.uint64(0xBB67AE85)


def philox4x32_10(ctr, key):
    """Apply Philox4x32-10 to 32-bit counter words ``ctr`` (shape [..., 4]) under the
    32-bit key words ``key`` = (k0, k1).  Words are carried in uint64 arrays (the
    32x32-bit products fit exactly); returns uint64 words below 2**32."""
    x = np.array(ctr, dtype=np.uint64, copy=True)
    if x.shape[-1] != 4:
        raise ValueError("counter must have 4 words")
    if np.any(x > MASK32):
        raise ValueError("counter words must fit 32 bits")
    k0 = np.asarray(key[0], dtype=np.uint64) & MASK32
    k1 = np.asarray(key[1], dtype=np.uint64) & MASK32
    x0, x1, x2, x3 = x[..., 0], x[..., 1], x[..., 2], x[..., 3]
    for rnd in range(ROUNDS):
        if rnd:
            k0 = (k0 + PHILOX32_W0) & MASK32
            k1 = (k1 + PHILOX32_W1) & MASK32
        p0 = x0 * PHILOX32_M0
        p1 = x2 * PHILOX32_M1
        x0, x1, x2, x3 = (p1 >> SHIFT32) ^ x1 ^ k0, p1 & MASK32, (p0 >> SHIFT32) ^ x3 ^ k1, p0 & MASK32
    return np.stack([x0, x1, x2, x3], axis=-1)


def projection_key(seed: int, matrix_id: int, step: int):
    """Key words of one projection matrix A: (seed, step<<32 | matrix_id)."""
    if not (0 <= matrix_id < 2**32 and 0 <= step < 2**32 and 0 <= seed < 2**64):
        raise ValueError("seed must fit 64 bits, matrix_id and step 32 bits")
    return np.uint64(seed), np.uint64((int(step) << 32) | int(matrix_id))


def sign_bits(seed: int, matrix_id: int, step: int, r: int, k: int) -> np.ndarray:
    """Sign bits of A as a uint8 array [r, k]: 1 means sigma = -1 (Philox4x32-10)."""
    projection_key(seed, matrix_id, step)   # range checks
    if r > 2**31:
        raise ValueError("r must be below 2**31")
    nblk = (k + 127) // 128
    ctr = np.zeros((r, nblk, 4), dtype=np.uint64)
    ctr[..., 0] = np.arange(nblk, dtype=np.uint64)[None, :]
    ctr[..., 1] = np.arange(r, dtype=np.uint64)[:, None] | np.uint64(2**31)
    ctr[..., 2] = matrix_id
    ctr[..., 3] = step
    key = (np.uint64(seed) & MASK32, np.uint64(seed) >> SHIFT32)
    words = philox4x32_10(ctr, key)                     # [r, nblk, 4]
    l = np.arange(k)
    w = words[:, l >> 7, (l & 127) >> 5]                # [r, k]
    return ((w >> (l & 31).astype(np.uint64)) & np.uint64(1)).astype(np.uint8)


def sr_draws(sr_seed: int, matrix_id: int, step: int, d: int, k: int,
             row0: int = 0) -> np.ndarray:
    """16-bit stochastic-rounding draws u as uint32 array [d, k] (Philox4x32-10)."""
    if not (0 <= matrix_id < 2**32 and 0 <= step < 2**32 and 0 <= sr_seed < 2**64):
        raise ValueError("sr_seed must fit 64 bits, matrix_id and step 32 bits")
    e = ((np.arange(d, dtype=np.uint64)[:, None] + np.uint64(row0)) * np.uint64(k)
         + np.arange(k, dtype=np.uint64)[None, :])
    blocks, inv = np.unique(e >> np.uint64(3), return_inverse=True)
    ctr = np.zeros((blocks.size, 4), dtype=np.uint64)
    ctr[:, 0] = blocks & MASK32
    ctr[:, 1] = blocks >> SHIFT32
    ctr[:, 2] = matrix_id
    ctr[:, 3] = step
    key = (np.uint64(sr_seed) & MASK32, np.uint64(sr_seed) >> SHIFT32)
    words = philox4x32_10(ctr, key)                     # [nblocks, 4]
    inv = inv.reshape(e.shape)
    lane = (e & np.uint64(7)).astype(np.int64)
    w = words[inv, lane >> 1]
    return ((w >> (np.uint64(16) * (e & np.uint64(1)))) & np.uint64(0xFFFF)).astype(np.uint32)


def gaussian_normals(seed: int, matrix_id: int, step: int, r: int, k: int) -> np.ndarray:
    """Standard normal entries z [r, k] (fp64) of the Gaussian projection variant.

    Box-Muller (G. E. P. Box and M. E. Muller, "A Note on the Generation of
    Random Normal Deviates", 1958) on the Philox stream: for row j and column
    group c = l >> 2 the block with counter (j, c, 2, 0) gives words w0..w3,
    uniforms u_i = ((w_i >> 11) + 1/2) 2^-53 in (0, 1), and
    z_{4c} = sqrt(-2 ln u0) cos(2 pi u1), z_{4c+1} = sqrt(-2 ln u0) sin(2 pi u1),
    z_{4c+2} = sqrt(-2 ln u2) cos(2 pi u3), z_{4c+3} = sqrt(-2 ln u2) sin(2 pi u3).
    """
    key = projection_key(seed, matrix_id, step)
    ng = (k + 3) // 4
    ctr = np.zeros((r, ng, 4), dtype=np.uint64)
    ctr[..., 0] = np.arange(r, dtype=np.uint64)[:, None]
    ctr[..., 1] = np.arange(ng, dtype=np.uint64)[None, :]
    ctr[..., 2] = 2
    words = philox4x64_10(ctr, key)                                 # [r, ng, 4]
    u = ((words >> np.uint64(11)).astype(np.float64) + 0.5) * 2.0 ** -53
    rho0 = np.sqrt(-2.0 * np.log(u[..., 0]))
    rho1 = np.sqrt(-2.0 * np.log(u[..., 2]))
    z = np.empty((r, ng, 4))
    z[..., 0] = rho0 * np.cos(2.0 * np.pi * u[..., 1])
    z[..., 1] = rho0 * np.sin(2.0 * np.pi * u[..., 1])
    z[..., 2] = rho1 * np.cos(2.0 * np.pi * u[..., 3])
    z[..., 3] = rho1 * np.sin(2.0 * np.pi * u[..., 3])
    return z.reshape(r, 4 * ng)[:, :k]
