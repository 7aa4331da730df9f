"""Philox4x64-10 counter-based generator, written from its published definition
(Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC'11, the
Philox-4x64 variant with 10 rounds).  Test infrastructure only; see oracle/__init__.py.

The WildCat pages sample each pivot at random from the residual diagonal (page
gist.science/de/paper/2602.10056, "Methodik" part 1, pivoting rule) but fix no generator.
The reading taken here: pivot step t of head h draws one uniform from the block

    (x0, x1, x2, x3) = Philox4x64-10(counter = (t, h, 0, 0), key = (seed, 0))
    u = (x0 >> 40) * 2^-24                       (24-bit dyadic value in [0, 1))

so every (seed, head, step) has its own independent draw and any step can be replayed.
"""
from __future__ import annotations

MASK64 = (1 << 64) - 1
# Round multipliers and key-schedule (Weyl) increments of Philox-4x64.
PHILOX_M0 = 0xD2E7470EE14C6C93
PHILOX_M1 = 0xCA5A826395121157
PHILOX_W0 = 0x9E3779B97F4A7C15
PHILOX_W1 = 0xBB67AE8584CAA73B
ROUNDS = 10


def _mulhilo(a: int, b: int):
    p = a * b
    return p >> 64, p & MASK64


def philox4x64_10(counter, key):
    """One Philox4x64-10 block: 4 x uint64 counter, 2 x uint64 key -> 4 x uint64."""
    x0, x1, x2, x3 = (int(c) & MASK64 for c in counter)
    k0, k1 = (int(k) & MASK64 for k in key)
    for rnd in range(ROUNDS):
        if rnd:
            k0 = (k0 + PHILOX_W0) & MASK64
            k1 = (k1 + PHILOX_W1) & MASK64
        hi0, lo0 = _mulhilo(PHILOX_M0, x0)
        hi1, lo1 = _mulhilo(PHILOX_M1, x2)
        x0, x1, x2, x3 = hi1 ^ x1 ^ k0, lo1, hi0 ^ x3 ^ k1, lo0
    return x0, x1, x2, x3


def pivot_uniform(seed: int, head: int, step: int) -> float:
    """The uniform in [0, 1) used by pivot ``step`` of ``head`` (a multiple of 2^-24)."""
    x0 = philox4x64_10((step, head, 0, 0), (seed, 0))[0]
    return (x0 >> 40) * 2.0 ** -24


def pivot_uniforms(seed: int, head: int, r: int):
    return [pivot_uniform(seed, head, t) for t in range(r)]
