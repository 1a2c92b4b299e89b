"""Pins of oracle.numerics against library routines and brute force."""
from fractions import Fraction

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

from oracle import numerics


def test_decode_bf16_matches_torch():
    g = np.random.Generator(np.random.Philox(1))
    bits = g.integers(0, 1 << 16, size=50000, dtype=np.int64).astype(np.uint16)
    finite = (bits & 0x7F80) != 0x7F80
    bits = bits[finite]
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    got = numerics.decode(bits, "bf16")
    assert np.array_equal(got, ref)


def test_round_bf16_matches_torch_cast_on_fp32_values():
    g = np.random.Generator(np.random.Philox(2))
    x = (g.standard_normal(200000) * 10.0 ** g.integers(-30, 30, 200000)).astype(np.float32)
    # exact halfway points between neighbouring bf16 values (ties go to even)
    base = g.integers(0, 1 << 15, size=5000, dtype=np.int64).astype(np.uint32) << 16
    base = base[((base >> 23) & 0xFF) < 0xFE]
    half = (base | 0x8000).view(np.float32)
    x = np.concatenate([x, half, -half, np.float32([0.0, -0.0, 1e-40, -3e-39])])
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = numerics.round_bf16(x.astype(np.float64))
    assert np.array_equal(got, ref)


def test_round_bf16_is_nearest_by_brute_force():
    g = np.random.Generator(np.random.Philox(3))
    x = g.standard_normal(3000) * 10.0 ** g.integers(-5, 5, 3000)
    got = numerics.round_bf16(x)
    for v, b in zip(x, got):
        cand = [(int(b) + d) & 0xFFFF for d in (-1, 0, 1)]
        vals = [Fraction(float(numerics.decode(np.array([c], np.uint16), "bf16")[0])) for c in cand]
        err = [abs(val - Fraction(float(v))) for val in vals]
        assert err[1] <= err[0] and err[1] <= err[2]


def test_round_f32_matches_numpy_cast():
    x = np.random.default_rng(4).standard_normal(1000) * 1e3
    assert np.array_equal(numerics.round_f32(x), x.astype(np.float32))


@pytest.mark.parametrize("tau", [1.0, 0.7, 2.5])
def test_softmax_matches_logsumexp(tau):
    g = np.random.Generator(np.random.Philox(5))
    a = 3.0 * g.standard_normal((20, 5000))
    ref = np.exp(a / tau - logsumexp(a / tau, axis=1, keepdims=True))
    got = numerics.softmax(a, tau)
    assert np.max(np.abs(got - ref)) < 1e-12
    assert np.allclose(got.sum(axis=1), 1.0, rtol=0, atol=1e-12)


def test_argmax_first_matches_numpy_with_ties():
    g = np.random.Generator(np.random.Philox(6))
    a = g.integers(-4, 4, size=(1000, 37)).astype(np.float64)
    assert np.array_equal(numerics.argmax_first(a), np.argmax(a, axis=1))
    z = np.array([[0.0, -0.0, 0.0], [-0.0, 0.0, -1.0]])
    assert list(numerics.argmax_first(z)) == [0, 0]


def test_inv_cdf_matches_searchsorted():
    g = np.random.Generator(np.random.Philox(7))
    for _ in range(2000):
        V = int(g.integers(1, 50))
        w = g.random(V) * (g.random(V) < 0.7)
        if w.sum() == 0:
            w[0] = 1.0
        u = float(g.integers(0, 1 << 24)) * 2.0 ** -24
        ref = int(np.searchsorted(np.cumsum(w), u * np.cumsum(w)[-1], side="right"))
        if ref == V:
            ref = int(np.nonzero(w > 0)[0][-1])
        assert numerics.inv_cdf(w, u) == ref


def test_inv_cdf_exact_intervals():
    """With dyadic weights the CDF is exact: each index owns [C_{v-1}, C_v)."""
    w = np.array([1, 0, 3, 4, 0, 8], dtype=np.float64) / 16
    edges = [0, 1, 1, 4, 8, 8, 16]
    for v in range(6):
        for t in range(edges[v], edges[v + 1]):
            assert numerics.inv_cdf(w, t / 16) == v
