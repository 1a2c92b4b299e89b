"""Pins of oracle.schedule: calibration, survival, the prefix scheduler, flatten."""
import itertools
import json
import os

import numpy as np
import pytest
from scipy.special import expit

from oracle import schedule

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_facts.json")


def test_calibration_is_sigmoid_of_scaled_logit():
    g = np.random.Generator(np.random.Philox(1))
    z = (3 * g.standard_normal((50, 7))).astype(np.float32)
    T = np.linspace(1.0, 2.0, 7).astype(np.float32)
    c = schedule.calibrate(z, T)
    ref = expit(z.astype(np.float64) / T.astype(np.float64))
    assert np.max(np.abs(c - ref) / ref) < 4e-16
    # T = 1: plain sigmoid
    c1 = schedule.calibrate(z, np.ones(7, np.float32))
    assert np.max(np.abs(c1 - expit(z.astype(np.float64))) / c1) < 4e-16
    # larger temperature pulls confidences toward 1/2 (corrects over-confidence)
    zz = np.full((1, 2), 3.0, np.float32)
    cc = schedule.calibrate(zz, np.array([1.0, 2.0], np.float32))
    assert 0.5 < cc[0, 1] < cc[0, 0]


def test_survival_is_cumulative_product():
    g = np.random.Generator(np.random.Philox(2))
    c = g.random((40, 9))
    assert np.array_equal(schedule.survival(c), np.cumprod(c, axis=1))
    S = schedule.survival(c)
    assert (np.diff(S, axis=1) <= 0).all()


def test_quantise_range_and_rounding():
    S = np.array([[0.0, 1.0, 0.5, 2.0 ** -33, 3 * 2.0 ** -34]])
    Q = schedule.quantise(S)
    assert list(Q[0]) == [0, 2 ** 32, 2 ** 31, 1, 1]


def test_throughput_table_interpolation():
    b = np.array([4, 8, 16], np.int32)
    thr = np.array([2.0, 3.0, 3.5])
    assert schedule.throughput(4, b, thr) == 2.0
    assert schedule.throughput(6, b, thr) == 2.5
    assert schedule.throughput(12, b, thr) == 3.25
    assert schedule.throughput(2, b, thr) == 1.0
    assert schedule.throughput(100, b, thr) == 3.5


def _concave_table(g, R, kmax):
    pop = np.arange(1, R * (kmax + 1) + 4)
    n = int(g.integers(2, min(7, len(pop)) + 1))
    pts = np.sort(g.choice(pop, size=n, replace=False)).astype(np.int32)
    # step time t(B) = a + c*B (+ d*B^2): throughput B / t(B) is concave and increasing
    a, c, d = 1.0 + g.random(), g.random() * 0.3, g.random() * 0.01
    thr = np.array([p / (a + c * p + d * p * p) for p in pts])
    return pts, thr


def _exhaustive(Q, kk, R, tb, tt):
    best, arg = None, []
    for Ls in itertools.product(range(kk + 1), repeat=R):
        P = sum(int(Q[r, i]) for r in range(R) for i in range(Ls[r]))
        G = schedule.gain(R, P, sum(Ls), tb, tt)
        if best is None or G > best:
            best, arg = G, [Ls]
        elif G == best:
            arg.append(Ls)
    return best, arg


@pytest.mark.parametrize("seed", range(40))
def test_scan_equals_exhaustive_search(seed):
    g = np.random.Generator(np.random.Philox(1000 + seed))
    R = int(g.integers(1, 5))
    k = int(g.integers(1, 4))
    z = (g.standard_normal((R, k)) * 2 + 1).astype(np.float32)
    if seed % 5 == 0:
        z[:, :] = z[0, 0]                      # equal confidences: ties everywhere
    T = np.linspace(1.0, 2.0, k).astype(np.float32)
    tb, tt = _concave_table(g, R, k)
    out = schedule.schedule(z, T, tb, tt, max_len=k)
    best, args = _exhaustive(out["Q"], k, R, tb, tt)
    assert out["best"] == best                 # bitwise: same integer sums, same formula
    L = tuple(int(v) for v in out["L"])
    assert L in args
    if len(args) == 1:
        assert L == args[0]


def test_flat_step_time_verifies_everything():
    g = np.random.Generator(np.random.Philox(3))
    R, k = 16, 5
    z = g.standard_normal((R, k)).astype(np.float32)
    T = np.ones(k, np.float32)
    tb = np.arange(1, 20, dtype=np.int32) * 8
    tt = tb.astype(np.float64)                 # step time constant: thr proportional to B
    out = schedule.schedule(z, T, tb, tt, max_len=k)
    assert (out["L"] == k).all()


def test_hard_knee_at_R_verifies_nothing():
    g = np.random.Generator(np.random.Philox(4))
    R, k = 16, 5
    z = (g.standard_normal((R, k)) + 3).astype(np.float32)
    T = np.ones(k, np.float32)
    tb = np.array([R, 2 * R, 4 * R], np.int32)
    tt = np.full(3, 100.0)                     # no extra throughput past B = R
    out = schedule.schedule(z, T, tb, tt, max_len=k)
    assert (out["L"] == 0).all()


def test_max_len_limits():
    g = np.random.Generator(np.random.Philox(5))
    R, k = 8, 5
    z = g.standard_normal((R, k)).astype(np.float32)
    T = np.ones(k, np.float32)
    tb = np.arange(1, 9, dtype=np.int32) * 16
    tt = tb.astype(np.float64)
    assert (schedule.schedule(z, T, tb, tt, max_len=-1)["L"] == k).all()
    assert (schedule.schedule(z, T, tb, tt, max_len=0)["L"] == 0).all()
    assert (schedule.schedule(z, T, tb, tt, max_len=2)["L"] == 2).all()


def test_selection_is_prefix_closed_and_sorted():
    g = np.random.Generator(np.random.Philox(6))
    R, k = 64, 5
    z = (g.standard_normal((R, k)) + 1).astype(np.float32)
    T = np.linspace(1, 2, k).astype(np.float32)
    tb = np.array([32, 64, 128, 256, 512], np.int32)
    tt = np.array([32, 64, 110, 170, 220], np.float64)
    out = schedule.schedule(z, T, tb, tt, max_len=k)
    Q, L = out["Q"], out["L"]
    sel = [(r, i) for r in range(R) for i in range(L[r])]
    nsel = [(r, i) for r in range(R) for i in range(L[r], k)]
    if sel and nsel:
        assert min(Q[r, i] for r, i in sel) >= max(Q[r, i] for r, i in nsel)


def _c2_like(R, g):
    dom = np.minimum((np.arange(R) * 3) // R, 2)
    m = np.array([0.92, 0.88, 0.75])[dom]
    raw = g.beta(20 * m[:, None].repeat(5, 1), 20 * (1 - m[:, None].repeat(5, 1)))
    return np.log(raw / (1 - raw)).astype(np.float32)


def test_load_adaptive_lengths_match_pages():
    """Low concurrency: 4-6 batch tokens per request; shrinking as load grows."""
    facts = json.load(open(GOLDEN))
    lo, hi = facts["low_concurrency_verify_tokens"]["value"]
    kmax = facts["max_draft_length"]["value"]
    pts = [32, 64, 128, 192, 256, 384, 512, 768, 1024, 1280, 1536, 2048]
    tb = np.array(pts, np.int32)
    tt = np.array([p / (1.0 if p <= 256 else 1 + 0.5 * (p - 256) / 256) for p in pts])
    T = np.linspace(1, 2, kmax).astype(np.float32)
    means = []
    for R in [1, 2, 4, 8, 16, 32, 64, 128, 256, 512]:
        g = np.random.Generator(np.random.Philox(11))
        z = _c2_like(R, g)
        L = schedule.schedule(z, T, tb, tt, max_len=kmax)["L"]
        means.append(L.mean())
    assert lo <= means[0] + 1 <= hi
    assert all(means[i + 1] <= means[i] + 1e-12 for i in range(len(means) - 1))
    assert means[-1] < means[0]


def test_flatten_layout():
    tags, cu = schedule.flatten(np.array([2, 0, 3]))
    assert list(cu) == [0, 2, 2, 5]
    assert tags.tolist() == [[0, 0], [0, 1], [2, 0], [2, 1], [2, 2], [0, 2], [1, 0], [2, 3]]
    assert schedule.n_rows(cu) == 8
    # every (r, j <= L_r) appears exactly once
    assert sorted(map(tuple, tags.tolist())) == [(0, 0), (0, 1), (0, 2), (1, 0), (2, 0), (2, 1), (2, 2), (2, 3)]
