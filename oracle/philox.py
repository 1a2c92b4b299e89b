"""Counter-based random numbers of the verification step: Philox4x64-10.

TEST INFRASTRUCTURE (see the package docstring).

The pages name Philox-seeded trials and a Philox seed for the semi-autoregressive
step, and no more. Reading: the generator is Philox4x64 with 10 rounds, as
defined by Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as easy as
1, 2, 3" (SC'11): per round two 64 x 64 -> 128-bit products of counter words 0
and 2 with fixed multipliers; the high halves are xored with counter words 1
and 3 and the key, and the key is bumped by two Weyl constants between
rounds. Every uniform the step
consumes is addressed by what it decides, not by where it sits in the flattened
batch, so results do not depend on the schedule or on the row order:

  U(seed, step, purpose, r, i) = (word 0 of Philox4x64-10(counter = (i + 1, r, purpose, 0),
                                                          key = (seed, step))  >> 40) * 2**-24

a float32 multiple of 2**-24 in [0, 1), exact. Purposes: 0 keeps or rejects
the draft token at position i of request r; 1 draws the extra token at
position i = a_r (the first rejected row, or the bonus row); 2 draws the
Markov (or RNN) head's token at position i.

Plain Python integers, one block at a time. Pin (tests/test_oracle_philox.py):
numpy.random.Philox, an independent implementation of the same generator,
which generates the block for counter c + 1 when constructed with counter c.
"""
from __future__ import annotations

import numpy as np

MASK = (1 << 64) - 1
# the multipliers and Weyl key increments published for Philox4x64
M0, M1 = 0xD2E7470EE14C6C93, 0xCA5A826395121157
W0, W1 = 0x9E3779B97F4A7C15, 0xBB67AE8584CAA73B

ACCEPT, DRAW, DRAFT = 0, 1, 2


def block(counter, key, rounds: int = 10):
    """Philox4x64-rounds of a 4-word counter under a 2-word key: 4 words."""
    c0, c1, c2, c3 = (int(x) & MASK for x in counter)
    k0, k1 = (int(x) & MASK for x in key)
    for n in range(rounds):
        if n > 0:                                   # the key is bumped before every round but the first
            k0 = (k0 + W0) & MASK
            k1 = (k1 + W1) & MASK
        p0 = M0 * c0                                # 128-bit products
        p1 = M1 * c2
        hi0, lo0 = p0 >> 64, p0 & MASK
        hi1, lo1 = p1 >> 64, p1 & MASK
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return c0, c1, c2, c3


def uniform(seed: int, step: int, purpose: int, r: int, i: int) -> float:
    """U(seed, step, purpose, r, i) as defined in the module docstring."""
    w0 = block((i + 1, r, purpose, 0), (seed, step))[0]
    return float(w0 >> 40) * 2.0 ** -24


def trial_uniforms(seed: int, step: int, r: int, i: int, t: int):
    """The two uniforms of trial t of the residual draw at position i of request
    r: words 0 and 1 of the block at counter (i + 1, r, 1, t), each >> 40 and
    times 2**-24. Trial 0's first uniform is U(seed, step, 1, r, i)."""
    w = block((i + 1, r, DRAW, t), (seed, step))
    return float(w[0] >> 40) * 2.0 ** -24, float(w[1] >> 40) * 2.0 ** -24


def uniforms(seed: int, step: int, purpose: int, R: int, n: int, r0: int = 0) -> np.ndarray:
    """U(seed, step, purpose, r0 + r, i) for r < R, i < n: float64 [R, n] (every
    value is a float32). r0 addresses a slice of a larger batch's requests."""
    out = np.empty((R, n), dtype=np.float64)
    for r in range(R):
        for i in range(n):
            out[r, i] = uniform(seed, step, purpose, r0 + r, i)
    return out
