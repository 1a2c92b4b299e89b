"""Calibration, survival, the hardware-aware prefix scheduler, and flattening.

TEST INFRASTRUCTURE (see the package docstring).

What the pages fix:
  * A confidence head scores each draft token's survival given its prefix, and
    a post-hoc temporal temperature scaling corrects its over-confidence
    ([P1] section "2. 置信度调度验证"). The score of a position is the chance it
    is accepted given that every earlier token was accepted ([P2] section 3.2).
  * The scheduler picks each request's verification length from the system
    load, the per-position confidences and the engine's throughput-vs-batch
    curve ([P2] section 3.2), framed as global throughput maximisation ([P4]
    section "置信度计划、负载感知验证"): sort the drafts of all requests by
    confidence, add them batch by batch while the extra step time per extra
    correct token pays ([P3] section "DSpark的神奇之处").
  * The selected tokens are flattened with a (request, position) tag ([P1]
    engineering table, row "内核利用率暴跌"); the row order is free (see flatten).

Readings where the pages are silent (each listed with its reason in the design
notes):
  calibration   c = sigmoid(z / T_i), one temperature per position.
  survival      S_i = c_0 * c_1 * ... * c_i (conditional scores multiplied).
  quantised     Q = floor(S * 2**32 + 0.5), an integer, so sums are exact.
  batch tokens  B = sum over requests of (L_r + 1): the committed token plus
                the verified drafts; B = R + M when M drafts are selected.
  throughput    thr(B) interpolated linearly between table points, thr_0*B/B_0
                below the first point, the last value beyond the last point.
  objective     expected emitted tokens per unit step time,
                G(M) = (R*2**32 + P(M)) * thr(R+M) / (R+M), P(M) = sum of the
                M largest Q (each request always emits one token; the sum of
                survivals is the expected number of accepted drafts).
  selection     candidates (r, i) with i < min(k, max_len) sorted by Q
                descending, then position, then request; M* = the smallest M
                with the largest G; L_r = number of request r's candidates
                among the first M*. max_len = -1 verifies all k.

Pins (tests/test_oracle_schedule.py): calibration against scipy's expit;
survival against numpy's cumprod; the scan against exhaustive search over all
(k+1)**R length assignments for R <= 4; closed forms (flat step time verifies
everything, a hard knee at B = R verifies nothing); the pages' load behaviour
(long verification at low concurrency, shrinking as requests grow).
"""
from __future__ import annotations

import numpy as np

TWO32 = 2 ** 32


def calibrate(z: np.ndarray, T: np.ndarray) -> np.ndarray:
    """c[r,i] = 1 / (1 + exp(-z[r,i] / T[i])), float64."""
    t = np.asarray(z, dtype=np.float64) / np.asarray(T, dtype=np.float64)[None, :]
    return 1.0 / (1.0 + np.exp(-t))


def survival(c: np.ndarray) -> np.ndarray:
    """S[r,i] = c[r,0] * ... * c[r,i], multiplied left to right."""
    S = np.empty_like(c)
    acc = np.ones(c.shape[0], dtype=np.float64)
    for i in range(c.shape[1]):
        acc = acc * c[:, i]
        S[:, i] = acc
    return S


def quantise(S: np.ndarray) -> np.ndarray:
    """Q = floor(S * 2**32 + 0.5) as int64 (0 <= Q <= 2**32)."""
    return np.floor(np.asarray(S, dtype=np.float64) * float(TWO32) + 0.5).astype(np.int64)


def throughput(bt: int, tbl_tokens, tbl_thr) -> float:
    """Engine throughput at bt batch tokens, from the table (B_j, thr_j)."""
    b = [int(v) for v in tbl_tokens]
    th = [float(v) for v in tbl_thr]
    n = len(b)
    if bt < b[0]:
        return (th[0] * float(bt)) / float(b[0])
    if bt >= b[n - 1]:
        return th[n - 1]
    for j in range(n - 1):
        if b[j] <= bt < b[j + 1]:
            frac = float(bt - b[j]) / float(b[j + 1] - b[j])
            return th[j] + (th[j + 1] - th[j]) * frac
    raise AssertionError("unreachable")


def gain(R: int, P: int, M: int, tbl_tokens, tbl_thr) -> float:
    """G = (R*2**32 + P) * thr(R+M) / (R+M), float64 in this operation order."""
    bt = R + M
    return (float(R * TWO32 + P) * throughput(bt, tbl_tokens, tbl_thr)) / float(bt)


def schedule(z, T, tbl_tokens, tbl_thr, max_len: int, k: int = None) -> dict:
    """Per-request verification lengths. Returns a dict with L [R] and details."""
    z = np.asarray(z)
    R, kz = z.shape
    k = kz if k is None else k
    c = calibrate(z, T)
    S = survival(c)
    Q = quantise(S)
    if max_len < 0:
        return dict(L=np.full(R, k, dtype=np.int64), c=c, S=S, Q=Q, M=R * k, G=None, order=None)
    kk = min(k, max_len)
    cand = [(int(Q[r, i]), i, r) for r in range(R) for i in range(kk)]
    cand.sort(key=lambda e: (-e[0], e[1], e[2]))
    best_g, best_m = None, 0
    G = []
    P = 0
    for M in range(len(cand) + 1):
        if M > 0:
            P += cand[M - 1][0]
        g = gain(R, P, M, tbl_tokens, tbl_thr)
        G.append(g)
        if best_g is None or g > best_g:
            best_g, best_m = g, M
    L = np.zeros(R, dtype=np.int64)
    for (_, i, r) in cand[:best_m]:
        L[r] += 1
    return dict(L=L, c=c, S=S, Q=Q, M=best_m, G=np.array(G), order=cand, best=best_g)


def flatten(L: np.ndarray):
    """The flattened varlen batch for lengths L [R].

    Every row is one element with its tag (r, j). Verified rows come first,
    request-major: rows cu[r] .. cu[r+1]-1 carry (r, 0) .. (r, L_r - 1), with
    cu the exclusive prefix sum of L (cu [R+1], cu[R] = N = sum L). Then one bonus
    row per request: row N + r carries (r, L_r). n_rows = N + R.
    The pages fix no row order (the tag carries the dependency); this one puts
    the rows that need both target and draft logits in one contiguous block.
    """
    L = np.asarray(L, dtype=np.int64)
    R = len(L)
    cu = [0]
    tags = []
    for r in range(R):
        for j in range(int(L[r])):
            tags.append((r, j))
        cu.append(cu[-1] + int(L[r]))
    for r in range(R):
        tags.append((r, int(L[r])))
    return np.array(tags, dtype=np.int64).reshape(-1, 2), np.array(cu, dtype=np.int64)


def n_rows(cu_rows) -> int:
    """Rows of the flattened batch: the verified rows plus one bonus row per request."""
    cu = np.asarray(cu_rows, dtype=np.int64)
    return int(cu[-1]) + len(cu) - 1
