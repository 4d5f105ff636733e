"""Counter-based random numbers for the oracle (test infrastructure).

The pages require only that the projection be regenerable "on the fly from a
seed" ([GRAPE] Methodology, design choice 1); they name no generator. The
method draws two random streams -- the projection P and the privacy noise Z --
and both sides of the parity check implement the same published generator
independently:

* Philox4x32-10: Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy
  as 1, 2, 3", SC'11. A 128-bit counter (c0,c1,c2,c3) and a 64-bit key
  (k0,k1). One round uses the two 32x32->64 products M0*c0 and M1*c2 and maps
  the counter to (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2), hi(M0 c0) ^ c3 ^ k1,
  lo(M0 c0)); the key is bumped by the Weyl constants (W0, W1) between
  rounds; ten rounds.
* Box-Muller (Box & Muller 1958): a pair of uniforms (u1, u2) in (0,1) gives
  R = sqrt(-2 ln u1) and the two normals R cos(2 pi u2), R sin(2 pi u2).

Stream layout (ours; the pages give none):
  key      k0 = seed mod 2^32, k1 = seed >> 32
  counter  c0 = e >> 2 (e = row-major element index in the target matrix),
           c1 = layer_id, c2 = step word (proj_step for P, step for Z),
           c3 = tag (0 = projection, 1 = noise)
  uniform  u(x) = (2 * (x >> 9) + 1) * 2^-24, exact in fp32 and fp64
  normals  Philox outputs (x0,x1,x2,x3) -> pairs (x0,x1), (x2,x3) ->
           (R0 cos t0, R0 sin t0, R1 cos t1, R1 sin t1); element e takes
           entry e & 3 of that 4-vector.

Everything here runs on uint64 numpy arrays, so each 32x32 product is exact.
Parity is pinned by tests/test_oracle_philox.py: the raw counter->4xu32 map
against the open-source rocRAND and ATen Philox4x32-10 headers compiled on the
host, and the normals by moments, a Kolmogorov-Smirnov test and the bound
|z| <= sqrt(48 ln 2).
"""
from __future__ import annotations

import numpy as np

_MASK = np.uint64(0xFFFFFFFF)
_M0 = np.uint64(0xD2511F53)
_M1 = np.uint64(0xCD9E8D57)
_W0 = np.uint64(0x9E3779B9)
_W1 = np.uint64(0xBB67AE85)


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Philox4x32-10 bijection on broadcastable uint32-valued arrays.

    Returns four uint32 arrays (the output words x0..x3)."""
    x0, x1, x2, x3 = (np.asarray(c, dtype=np.uint64) & _MASK
                      for c in (c0, c1, c2, c3))
    k0 = np.asarray(k0, dtype=np.uint64) & _MASK
    k1 = np.asarray(k1, dtype=np.uint64) & _MASK
    for _ in range(10):
        p0 = _M0 * x0            # < 2^64: exact in uint64
        p1 = _M1 * x2
        x0, x1, x2, x3 = ((p1 >> np.uint64(32)) ^ x1 ^ k0,
                          p1 & _MASK,
                          (p0 >> np.uint64(32)) ^ x3 ^ k1,
                          p0 & _MASK)
        k0 = (k0 + _W0) & _MASK
        k1 = (k1 + _W1) & _MASK
    return tuple(x.astype(np.uint32) for x in (x0, x1, x2, x3))


def uniform_open01(x):
    """u(x) = (2*(x>>9)+1) * 2^-24 in (0, 1), as float64 (exact)."""
    x = np.asarray(x, dtype=np.uint64)
    return ((x >> np.uint64(9)) * np.uint64(2) + np.uint64(1)).astype(
        np.float64) * 2.0 ** -24


def philox_words(seed: int, layer_id: int, step_word: int, tag: int,
                 counters) -> tuple:
    """Raw Philox outputs for the given c0 values of one stream."""
    seed = int(seed)
    return philox4x32_10(np.asarray(counters, dtype=np.uint64),
                         np.uint64(layer_id & 0xFFFFFFFF),
                         np.uint64(step_word & 0xFFFFFFFF),
                         np.uint64(tag & 0xFFFFFFFF),
                         np.uint64(seed & 0xFFFFFFFF),
                         np.uint64((seed >> 32) & 0xFFFFFFFF))


def gaussian_stream(seed: int, layer_id: int, step_word: int, tag: int,
                    n: int, start: int = 0) -> np.ndarray:
    """Standard normals z(e) for e in [start, start+n), float64."""
    if n <= 0:
        return np.zeros(0, dtype=np.float64)
    e = np.arange(start, start + n, dtype=np.uint64)
    c_lo = int(e[0] >> np.uint64(2))
    c_hi = int(e[-1] >> np.uint64(2))
    x0, x1, x2, x3 = philox_words(seed, layer_id, step_word, tag,
                                  np.arange(c_lo, c_hi + 1, dtype=np.uint64))
    r0 = np.sqrt(-2.0 * np.log(uniform_open01(x0)))
    t0 = 2.0 * np.pi * uniform_open01(x1)
    r1 = np.sqrt(-2.0 * np.log(uniform_open01(x2)))
    t1 = 2.0 * np.pi * uniform_open01(x3)
    quad = np.stack([r0 * np.cos(t0), r0 * np.sin(t0),
                     r1 * np.cos(t1), r1 * np.sin(t1)], axis=1)
    flat = quad.reshape(-1)             # index (c - c_lo)*4 + comp
    return flat[(e - np.uint64(4 * c_lo)).astype(np.int64)]
