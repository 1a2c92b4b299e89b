"""Pins of the oracle's counter-based generator (oracle.philox).

1. Philox4x64-10 blocks equal numpy.random.Philox's, an independent
   implementation of the same published generator (numpy generates the block
   for counter c + 1 when constructed with counter c), over random counters
   and keys, carries across counter words included.
2. The uniforms' addressing: U(seed, step, purpose, r, i) is the top 24 bits
   of word 0 of the block at counter (i + 1, r, purpose, 0) under key
   (seed, step), times 2**-24.
3. The uniforms are float32 values in [0, 1) and pass a 64-bin chi-square.
4. A planted mistake (no key bump between rounds, or a swapped key) breaks 1.
"""
import random

import numpy as np
import pytest
from scipy import stats

from oracle import philox

U64 = np.uint64
MASK = (1 << 64) - 1


def _numpy_block_after(counter, key):
    """numpy's block for counter + 1 (its generate-after-increment convention)."""
    g = np.random.Philox(counter=np.array(counter, dtype=U64), key=np.array(key, dtype=U64))
    return [int(x) for x in g.random_raw(4)]


def _plus_one(counter):
    v = sum(int(c) << (64 * i) for i, c in enumerate(counter)) + 1
    v &= (1 << 256) - 1
    return [(v >> (64 * i)) & MASK for i in range(4)]


def test_blocks_equal_numpy():
    rng = random.Random(20251203)
    for n in range(400):
        c = [rng.getrandbits(64) for _ in range(4)]
        k = [rng.getrandbits(64) for _ in range(2)]
        if n % 5 == 0:
            c[0] = MASK                      # carry into word 1
        if n % 11 == 0:
            c[0] = c[1] = MASK               # carry into word 2
        if n % 13 == 0:
            c = [0, 0, 0, 0]
        assert list(philox.block(_plus_one(c), k)) == _numpy_block_after(c, k), (c, k)


@pytest.mark.parametrize("seed", [0, 7, (1 << 63) + 5])
@pytest.mark.parametrize("step", [0, 1, 123456789])
def test_uniform_addressing(seed, step):
    for purpose in (philox.ACCEPT, philox.DRAW, philox.DRAFT):
        for r in (0, 1, 511, 100000):
            for i in (0, 4, 31):
                w0 = _numpy_block_after([i, r, purpose, 0], [seed, step])[0]
                want = float(w0 >> 40) * 2.0 ** -24
                got = philox.uniform(seed, step, purpose, r, i)
                assert got == want
                assert np.float32(got) == got and 0.0 <= got < 1.0


def test_uniforms_grid_matches_scalar():
    u = philox.uniforms(7, 3, philox.ACCEPT, 5, 6)
    for r in range(5):
        for i in range(6):
            assert u[r, i] == philox.uniform(7, 3, philox.ACCEPT, r, i)


def test_uniformity_chisquare():
    vals = []
    for step in range(64):
        for r in range(64):
            for i in range(6):
                vals.append(philox.uniform(11, step, (r + i) % 3, r, i))
    counts = np.bincount((np.array(vals) * 64).astype(np.int64), minlength=64)
    assert stats.chisquare(counts).pvalue > 1e-4


def test_planted_mistakes_break_the_pin(monkeypatch):
    c, k = [3, 9, 2, 0], [7, 42]
    want = _numpy_block_after(c, k)
    assert list(philox.block(_plus_one(c), k)) == want
    monkeypatch.setattr(philox, "W0", 0)
    monkeypatch.setattr(philox, "W1", 0)
    assert list(philox.block(_plus_one(c), k)) != want          # key never bumped
    monkeypatch.undo()
    assert list(philox.block(_plus_one(c), k[::-1])) != want    # (step, seed) instead of (seed, step)
