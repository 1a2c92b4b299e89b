"""Number formats and the small numerical primitives of the oracle.

TEST INFRASTRUCTURE (see the package docstring).

Pins (tests/test_oracle_numerics.py): bf16 decoding against torch's widening,
bf16 rounding against torch's round-to-nearest-even cast on fp32-representable
values and against brute force over neighbouring bf16 values, softmax against
scipy's logsumexp, first-index argmax against numpy, the inverse-CDF draw
against numpy's searchsorted and against exact Fraction arithmetic.
"""
from __future__ import annotations

import numpy as np


def decode(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of stored logits ("bf16" = uint16 bit patterns, "f32")."""
    if dtype == "bf16":
        bits = np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    raise ValueError(dtype)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to bfloat16, nearest with ties to even; uint16 bits.

    Rounds the float64 value directly (one rounding), so it can differ from a
    float64 -> float32 -> bfloat16 chain, which rounds twice. Finite inputs with
    |x| < 2**128 only.
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    _, e = np.frexp(a)                     # a = m * 2**e with m in [0.5, 1)
    # bf16 keeps 8 significant bits; below 2**-126 the quantum stays 2**-133
    q_exp = np.maximum(e - 8, -133)
    r = np.rint(np.ldexp(a, -q_exp))       # exact scaling, then round half to even
    val = np.ldexp(r, q_exp).astype(np.float32)   # representable by construction
    bits = val.view(np.uint32)
    assert not np.any(bits & np.uint32(0xFFFF))
    sign = np.where(np.signbit(x), np.uint32(0x8000), np.uint32(0))
    return (sign | (bits >> np.uint32(16))).astype(np.uint16)


def round_f32(x: np.ndarray) -> np.ndarray:
    """Round float64 to float32 (nearest, ties to even)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def softmax(logits: np.ndarray, tau: float) -> np.ndarray:
    """softmax(logits / tau) along the last axis, float64."""
    a = np.asarray(logits, dtype=np.float64) / float(tau)
    m = np.max(a, axis=-1, keepdims=True)
    e = np.exp(a - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def argmax_first(values: np.ndarray) -> np.ndarray:
    """Index of the maximum along the last axis; ties go to the lowest index.

    Written as "first index whose value equals the maximum" so that it does not
    simply restate numpy's argmax.
    """
    v = np.asarray(values)
    m = np.max(v, axis=-1, keepdims=True)
    hit = v == m
    return np.argmax(hit, axis=-1)


def inv_cdf(w: np.ndarray, u: float) -> int:
    """Draw from weights w with the uniform u in [0, 1) by inverting the CDF.

    W = sum of w in index order, t = u * W, result = smallest v with
    w_0 + ... + w_v > t. If rounding leaves no such v, the last v with w_v > 0.
    """
    w = np.asarray(w, dtype=np.float64)
    c = np.cumsum(w)
    t = float(u) * float(c[-1])
    above = c > t
    if above.any():
        return int(np.argmax(above))
    pos = np.nonzero(w > 0)[0]
    return int(pos[-1])
