"""Philox4x32-10 and the dropout keep-mask built on it.
TEST INFRASTRUCTURE ONLY (see the package header).

The pages name dropout but no generator, no counter layout and no threshold
rule.  The generator is Philox4x32 with 10 rounds as defined by Salmon,
Moraes, Dror and Shaw ("Parallel Random Numbers: As Easy as 1, 2, 3", SC'11):
a 128-bit counter (four 32-bit words) and a 64-bit key (two words); each
round multiplies counter words 0 and 2 by two fixed 32-bit constants, taking
the full 64-bit products, and recombines the halves with the other two words
and the key by XOR; between rounds the key words advance by two Weyl
increments, the 32-bit fractional parts of the golden ratio and of sqrt(3).

Mask layout (a reading the pages leave open):
  element index  e = (row0 + i) * ld + (col0 + j)
  counter        (lo32(e >> 2), hi32(e >> 2), lo32(offset), hi32(offset))
  key            (lo32(seed), hi32(seed))
  word           e & 3 of the block
  threshold      T = floor(p * 2^32) in float64; keep iff word >= T
                 (p >= 1 drops every element, p <= 0 keeps every element).

Parity pins (tests/test_oracle_philox.py): the Weyl increments re-derived from
the golden ratio and sqrt(3) with exact integer arithmetic; rocRAND's
open-source Philox4x32-10 engine (compiled from its header on the host)
for many counters and keys; keep-rate and lane-independence statistics;
p = 0 and p = 1.
"""

from __future__ import annotations

import math

import numpy as np

MASK32 = np.uint64(0xFFFFFFFF)
PHILOX_M0 = np.uint64(0xD2511F53)
PHILOX_M1 = np.uint64(0xCD9E8D57)
PHILOX_W0 = np.uint64(0x9E3779B9)   # frac(golden ratio) * 2^32
PHILOX_W1 = np.uint64(0xBB67AE85)   # frac(sqrt 3) * 2^32
ROUNDS = 10


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Apply the ten-round Philox4x32 bijection.  Arguments are arrays (or
    scalars) of 32-bit values; the result is four uint64 arrays holding
    32-bit values."""
    c0, c1, c2, c3, k0, k1 = (np.asarray(v, dtype=np.uint64) & MASK32
                              for v in (c0, c1, c2, c3, k0, k1))
    for rnd in range(ROUNDS):
        if rnd:
            k0 = (k0 + PHILOX_W0) & MASK32
            k1 = (k1 + PHILOX_W1) & MASK32
        p0 = PHILOX_M0 * c0          # < 2^64: exact in uint64
        p1 = PHILOX_M1 * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & MASK32
        hi1, lo1 = p1 >> np.uint64(32), p1 & MASK32
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return c0, c1, c2, c3


def keep_threshold(p: float) -> int:
    """T = floor(p * 2^32) in float64, clamped to [0, 2^32]."""
    if p <= 0.0:
        return 0
    if p >= 1.0:
        return 1 << 32
    return int(math.floor(p * 4294967296.0))


def element_words(e, seed: int, offset: int) -> np.ndarray:
    """The 32-bit Philox word that decides element index e (array)."""
    e = np.asarray(e, dtype=np.uint64)
    blk = e >> np.uint64(2)
    out = philox4x32_10(blk & MASK32, blk >> np.uint64(32),
                        np.uint64(offset & 0xFFFFFFFF), np.uint64(offset >> 32),
                        np.uint64(seed & 0xFFFFFFFF), np.uint64(seed >> 32))
    words = np.stack(out, axis=-1)
    lane = (e & np.uint64(3)).astype(np.int64)
    return np.take_along_axis(words, lane[..., None], axis=-1)[..., 0]


def keep_mask(rows: int, cols: int, p: float, seed: int, offset: int,
              row0: int = 0, col0: int = 0, ld: int | None = None) -> np.ndarray:
    """Boolean keep-mask of a [rows, cols] block whose element (i, j) has the
    global index (row0 + i) * ld + (col0 + j)."""
    if ld is None:
        ld = col0 + cols
    i = np.arange(rows, dtype=np.uint64)[:, None] + np.uint64(row0)
    j = np.arange(cols, dtype=np.uint64)[None, :] + np.uint64(col0)
    e = i * np.uint64(ld) + j
    t = keep_threshold(p)
    if t >= (1 << 32):
        return np.zeros((rows, cols), dtype=bool)
    return element_words(e, seed, offset) >= np.uint64(t)
