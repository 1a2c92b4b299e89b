"""Pin of the inverse-CDF draw's near sets (oracle.verify.draw_rows).

The GPU parity tests excuse a drawn token that differs from the oracle's only
when it is in the oracle's near set: a token whose CDF interval [C(v-1), C(v))
lies within eps * W of t = u * W. The pin uses dyadic weights, whose every
cumulative sum and every distance is exact in float64, so the expected sets
are worked out by hand below. Planted mistakes (no division by W; the distance
to the upper boundary only; zero-weight tokens admitted) must fail the pin.
"""
import numpy as np
import pytest

from oracle import verify

# weights (W = 8): C = [2, 2, 3, 4, 8]; token 1 has no weight (empty interval)
W8 = np.array([[2.0, 0.0, 1.0, 1.0, 4.0]])

# (u, eps) -> (drawn token, near set). Intervals: 0 [0,2), 2 [2,3), 3 [3,4), 4 [4,8).
# u = 95/256: t = 2.96875, so token 0 is 0.96875 / 8 = 0.12109375 away, token 3
# 0.03125 / 8 = 0.00390625 and token 4 1.03125 / 8 = 0.12890625.
U1 = 95.0 / 256.0
CASES = [
    (U1, 0.0, 2, []),
    (U1, 0.0039, 2, []),
    (U1, 0.00390625, 2, [3]),
    (U1, 0.12109375, 2, [0, 3]),
    (U1, 0.12890625, 2, [0, 3, 4]),
    (0.25, 0.0, 2, []),           # t = 2 exactly: token 2 (C(0) = 2 is not > 2)
    (0.25, 1e-9, 2, [0]),         # token 0's interval ends at t
    (0.0, 0.3, 0, [2]),           # t = 0: token 2 is 2/8 away, token 3 3/8
    (0.0, 0.375, 0, [2, 3]),
    (0.96875, 0.25, 4, []),       # t = 7.75: token 3 is 3.75 / 8 away, token 2 4.75 / 8
    (0.96875, 0.5, 4, [3]),
    (0.96875, 0.75, 4, [0, 2, 3]),
]


def check(draw, u, eps, y_want, near_want):
    y, near = draw(W8, np.array([u]), eps)
    assert int(y[0]) == y_want
    assert list(near[0]) == near_want


@pytest.mark.parametrize("u,eps,y,near", CASES)
def test_near_sets(u, eps, y, near):
    check(verify.draw_rows, u, eps, y, near)


@pytest.mark.parametrize("scale", [1.0 / 8.0, 1.0, 1024.0])
def test_near_sets_scale_free(scale):
    for u, eps, y_want, near_want in CASES:
        y, near = verify.draw_rows(W8 * scale, np.array([u]), eps)
        assert int(y[0]) == y_want and list(near[0]) == near_want


def _no_division_by_W(w, u, eps):
    w = np.asarray(w, dtype=np.float64)
    W = w.sum(axis=1)
    return verify.draw_rows(w, u, eps / W)                      # eps compared with unnormalised distances


def _upper_boundary_only(w, u, eps):
    w = np.asarray(w, dtype=np.float64)
    y, _ = verify.draw_rows(w, u)
    c = np.cumsum(w, axis=1)
    t = u * c[:, -1]
    out = []
    for i in range(w.shape[0]):
        d = np.abs(c[i] - t[i]) / c[i, -1]
        v = np.nonzero((w[i] > 0) & (d <= eps))[0]
        out.append(v[v != y[i]])
    return y, out


def _zero_weight_admitted(w, u, eps):
    w = np.asarray(w, dtype=np.float64)
    y, _ = verify.draw_rows(w, u)
    c = np.cumsum(w, axis=1)
    t = u * c[:, -1]
    out = []
    for i in range(w.shape[0]):
        lo = np.concatenate(([0.0], c[i, :-1]))
        d = np.maximum(np.maximum(lo - t[i], t[i] - c[i]), 0.0) / c[i, -1]
        v = np.nonzero(d <= eps)[0]
        out.append(v[v != y[i]])
    return y, out


@pytest.mark.parametrize("bad", [_no_division_by_W, _upper_boundary_only, _zero_weight_admitted])
def test_planted_mistakes_fail(bad):
    failures = 0
    for u, eps, y, near in CASES:
        try:
            check(bad, u, eps, y, near)
        except AssertionError:
            failures += 1
    assert failures > 0


def test_rows_independent():
    w = np.vstack([W8, W8[:, ::-1]])
    y, near = verify.draw_rows(w, np.array([U1, U1]), 0.00390625)
    assert list(y) == [2, 0] and list(near[0]) == [3] and list(near[1]) == []
