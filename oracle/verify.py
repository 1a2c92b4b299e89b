"""The acceptance rule over a flattened varlen batch, float64.

TEST INFRASTRUCTURE (see the package docstring).

Every selected draft token of every request is one element of a single batch;
a tag (request id, position) per element carries the in-sequence dependency
([P1] engineering table, row "内核利用率暴跌": all tokens are flattened into
independent elements and a tag tensor passes the dependencies). For request r
with scheduled length L_r the batch holds rows tagged (r, 0) .. (r, L_r); rows
j < L_r verify draft token x_j, row L_r only supplies the bonus token. The row
order is schedule.flatten's; everything here is keyed by the tags.

Per verified row (the rule itself is oracle.rule):
  greedy    g = first argmax of the target logits; keep iff g == x_j.
  sampling  p = softmax(target / tau), q = softmax(draft / tau);
            keep iff u[r, j] < min(1, p(x_j) / q(x_j)).
Per request: a_r = first j < L_r not kept, else L_r ([P2] section 一: resample
after the first divergence). Emitted: x_0 .. x_{a_r - 1}, then
  greedy    the target argmax of row a_r;
  sampling  an inverse-CDF draw from max(0, p - q) at row a_r when a_r < L_r
            (from p when that residual has no mass), else from p of row L_r.
The uniforms come from the counter-based generator (oracle.philox), or are
given as an array (see verify()).

The scalar definition in oracle.rule and this vectorised form must agree
element for element on the same uniforms (tests/test_oracle_verify.py); the
vectorisation runs over requests, one position at a time, with no other
reordering. Pins: agreement with oracle.rule; a chi-square test on 10**7
seeded trials that emitted tokens follow the target distribution; negative
controls that a planted mistake fails it.
"""
from __future__ import annotations

import numpy as np

from . import numerics, philox

# Distance (a fraction of the draw's total weight W) within which the tokens a
# draw could produce under rounding are reported (draw_rows' near sets): the
# float32 draws of the GPU path keep t / W and each C(v) / W within this of the
# exact values (relative errors of the weights from the scaled exponent, the
# exponential and the normaliser, and the float32 running sums, each a few
# times 2**-24 times the number of summation levels).
DRAW_EPS = 1e-5


def _first_false(acc: np.ndarray, L: np.ndarray) -> np.ndarray:
    """a_r = smallest j < L_r with acc[r, j] False, else L_r."""
    R, k = acc.shape
    a = np.array(L, dtype=np.int64, copy=True)
    for j in range(k - 1, -1, -1):
        rej = (~acc[:, j]) & (j < L)
        a = np.where(rej, j, a)
    return a


def decide(px: np.ndarray, qx: np.ndarray, u_acc: np.ndarray, L: np.ndarray):
    """Keep flags and accepted lengths from p(x_j), q(x_j) [R,k] and uniforms.

    keep probability = min(1, p/q), 1 where q == 0; keep iff u < that.
    Entries j >= L_r are ignored (False).
    """
    px = np.asarray(px, dtype=np.float64)
    qx = np.asarray(qx, dtype=np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(qx > 0, px / np.where(qx > 0, qx, 1.0), np.inf)
    keep = np.minimum(1.0, ratio)
    acc = np.asarray(u_acc, dtype=np.float64) < keep
    k = px.shape[1]
    acc &= np.arange(k)[None, :] < np.asarray(L)[:, None]
    return acc, _first_false(acc, np.asarray(L)), ratio


def draw_rows(w: np.ndarray, u: np.ndarray, eps: float = 0.0):
    """Inverse-CDF draw per row of weights w [n,V] with uniforms u [n].

    W = sum of the row in index order, t = u * W, C(v) = w_0 + ... + w_v; the
    draw is the smallest v with C(v) > t, else (rounding) the last v with
    w_v > 0. Token v owns the interval [C(v-1), C(v)) of the CDF.

    Returns (index [n], near [n]): near[i] holds, in increasing order, the
    other tokens with positive weight whose interval lies within eps * W of t,
    i.e. the tokens a perturbation of t or of the CDF by at most eps * W could
    draw instead. With eps = 0 every near set is empty.
    """
    w = np.asarray(w, dtype=np.float64)
    c = np.cumsum(w, axis=1)
    W = c[:, -1]
    t = np.asarray(u, dtype=np.float64) * W
    above = c > t[:, None]
    y = np.argmax(above, axis=1)
    none = ~above.any(axis=1)
    if none.any():
        for i in np.nonzero(none)[0]:
            y[i] = np.nonzero(w[i] > 0)[0][-1]
    near = []
    for i in range(w.shape[0]):
        if eps <= 0.0:
            near.append(np.zeros(0, dtype=np.int64))
            continue
        lo = np.concatenate(([0.0], c[i, :-1]))             # C(v - 1)
        dist = np.maximum(np.maximum(lo - t[i], t[i] - c[i]), 0.0)
        v = np.nonzero((w[i] > 0) & (dist <= eps * W[i]))[0]
        near.append(v[v != y[i]].astype(np.int64))
    return y.astype(np.int64), near


# Trials of the rejection draw from the residual before the inverse-CDF fallback.
# All of them are rejected with probability (1 - TV)^64, TV = sum(max(0, p - q)):
# rare even where the draft nearly agrees with the target (TV ~ 0.1).
RESIDUAL_TRIALS = 64


def residual_draw_rejection(p: np.ndarray, q: np.ndarray, trial_u, trials: int = RESIDUAL_TRIALS,
                            near_eps: float = 0.0):
    """One draw from max(0, p - q) / sum(max(0, p - q)) for one row (p, q [V]).

    Trial t takes y ~ p by the inverse CDF with its first uniform u1 and keeps
    it iff its second uniform u2 < 1 - q(y) / p(y); the first kept trial gives
    the token. A proposal from p kept with probability max(0, p - q) / p has
    probability max(0, p(y) - q(y)) of being kept as y, so the kept token has
    exactly the normalised residual's distribution. If all `trials` trials are
    rejected, the token is the inverse-CDF draw from the residual itself (from
    p if it has no mass) with the uniform trial_u(trials)[0]: exact too, since
    that draw does not depend on the rejected trials. trial_u(t) -> (u1, u2).

    Returns (token, kept trial or -1, near): near lists what rounding could
    change on the way: ("draw", t, tokens) for a trial whose proposal has
    other tokens within near_eps (draw_rows' near sets), ("keep", t) for a
    trial with |u2 - (1 - q(y) / p(y))| < 1e-6, ("fallback", tokens) for the
    fallback draw.
    """
    p = np.asarray(p, dtype=np.float64)
    q = np.asarray(q, dtype=np.float64)
    near = []
    for t in range(trials):
        u1, u2 = trial_u(t)
        y, nb = draw_rows(p[None, :], np.array([u1]), near_eps)
        y = int(y[0])
        if len(nb[0]):
            near.append(("draw", t, nb[0]))
        bound = 1.0 - q[y] / p[y]
        if abs(u2 - bound) < 1e-6:
            near.append(("keep", t))
        if u2 < bound:
            return y, t, near
    w = residual_rows(p[None, :], q[None, :])
    y, nb = draw_rows(w, np.array([trial_u(trials)[0]]), near_eps)
    if len(nb[0]):
        near.append(("fallback", nb[0]))
    return int(y[0]), -1, near


def residual_rows(p: np.ndarray, q: np.ndarray) -> np.ndarray:
    """max(0, p - q) per row; p itself for rows where that has no mass."""
    w = np.maximum(p - q, 0.0)
    empty = ~(w.sum(axis=1) > 0)
    w[empty] = p[empty]
    return w


def verify_probs(P: np.ndarray, Qd: np.ndarray, x: np.ndarray, L: np.ndarray, u: np.ndarray):
    """Sampling-mode rule on explicit distributions.

    P [R,k+1,V] target distributions, Qd [R,k,V] draft distributions, x [R,k]
    draft tokens, L [R] lengths, u [R,k+1] uniforms (j < k keep, k resample).
    Returns (a [R], out [R,k+1] padded with -1).
    """
    R, k1, V = P.shape
    k = k1 - 1
    rr = np.arange(R)[:, None]
    jj = np.arange(k)[None, :]
    px = P[rr, jj, x]
    qx = Qd[rr, jj, x]
    _, a, _ = decide(px, qx, u[:, :k], L)
    pa = P[np.arange(R), a]
    qa = Qd[np.arange(R), np.minimum(a, k - 1)]
    w = np.where((a < L)[:, None], residual_rows(pa, qa), pa)
    y, _ = draw_rows(w, u[:, k])
    return a, _emit(a, x, y, k)


def _emit(a, x, y, k):
    R = len(a)
    out = np.full((R, k + 1), -1, dtype=np.int64)
    for j in range(k):
        out[:, j] = np.where(j < a, x[:, j], out[:, j])
    out[np.arange(R), a] = y
    return out


def lengths_from_cu(cu_rows: np.ndarray) -> np.ndarray:
    """L_r from the verified-row offsets of the flattened batch (schedule.flatten)."""
    cu = np.asarray(cu_rows, dtype=np.int64)
    return cu[1:] - cu[:-1]


def verify(mode: str, dtype: str, target: np.ndarray, draft, tokens: np.ndarray,
           tags: np.ndarray, cu_rows: np.ndarray, tau: float, u_verify=None,
           block_rows: int = 64, rng=None, near_eps: float = DRAW_EPS) -> dict:
    """Verify a flattened batch. Shapes: target [R,k+1,V], draft [R,k,V] (sampling
    only), tokens [R,k], tags [B,2] with B = cu_rows[R] + R, cu_rows [R+1]
    (schedule.flatten).

    Uniforms (sampling): rng = (seed, step) takes them from the counter-based
    generator (oracle.philox): U(seed, step, 0, r, j) keeps or rejects row j;
    the draw at a_r is the bonus draw with U(seed, step, 1, r, a_r) when every
    row was kept, else the residual's rejection draw with the trial uniforms
    of (r, a_r) (residual_draw_rejection). rng = (seed, step, r0) addresses
    the requests as r0 + r: a slice of a larger batch gets the uniforms the
    whole batch would. Without rng, u_verify [R,k+1]
    gives them: column j < k keeps or rejects row j, column k drives an
    inverse-CDF draw (from the residual, or from p for the bonus row).

    Returns a dict with accepted_len [R], out_tokens [R,k+1] (-1 after the last
    emitted token) and per-row and per-request diagnostics for parity tests,
    among them the uniforms used (u_accept [R,k], u_draw [R]: the inverse-CDF
    draw's uniform, or the kept trial's first one), the residual mass
    sum(max(0, p - q)) of each rejected row a_r (0 where every row was kept),
    draw_trial [R] (the kept trial of a rejection draw; -1: fallback or no
    rejection draw), draw_by_trials [R] (the draw was a rejection draw) and
    draw_near (draw_rows' near sets at near_eps; for a rejection draw,
    residual_draw_rejection's list).
    """
    R, k1, V = target.shape
    k = k1 - 1
    L = lengths_from_cu(cu_rows)
    tags = np.asarray(tags, dtype=np.int64)
    B = int(cu_rows[-1]) + R
    assert tags.shape[0] >= B
    x = np.asarray(tokens, dtype=np.int64)
    res = dict(L=L)

    if mode == "greedy":
        g_row = np.zeros(B, dtype=np.int64)
        for s in range(0, B, block_rows):
            e = min(B, s + block_rows)
            rows = numerics.decode(target[tags[s:e, 0], tags[s:e, 1]], dtype)
            g_row[s:e] = numerics.argmax_first(rows)
        g = np.full((R, k + 1), -1, dtype=np.int64)
        g[tags[:B, 0], tags[:B, 1]] = g_row
        acc = np.zeros((R, k), dtype=bool)
        for j in range(k):
            acc[:, j] = (j < L) & (g[:, j] == x[:, j])
        a = _first_false(acc, L)
        y = g[np.arange(R), a]
        res.update(accepted_len=a, out_tokens=_emit(a, x, y, k), row_argmax=g_row,
                   accept=acc)
        return res

    if mode != "sample":
        raise ValueError(mode)
    if rng is not None:
        seed, step, r0 = (tuple(rng) + (0,))[:3]
        u_acc = philox.uniforms(seed, step, philox.ACCEPT, R, k, r0)
    else:
        u_acc = np.asarray(u_verify, dtype=np.float64)[:, :k]
    px = np.zeros((R, k), dtype=np.float64)
    qx = np.ones((R, k), dtype=np.float64)
    row_p = np.full(B, np.nan)
    row_q = np.full(B, np.nan)
    ver = tags[:B, 1] < L[tags[:B, 0]]
    vidx = np.nonzero(ver)[0]
    for s in range(0, len(vidx), block_rows):
        t = vidx[s:s + block_rows]
        r, j = tags[t, 0], tags[t, 1]
        xt = x[r, j]
        p = numerics.softmax(numerics.decode(target[r, j], dtype), tau)
        q = numerics.softmax(numerics.decode(draft[r, j], dtype), tau)
        n = np.arange(len(t))
        px[r, j] = p[n, xt]
        qx[r, j] = q[n, xt]
        row_p[t] = p[n, xt]
        row_q[t] = q[n, xt]
    acc, a, ratio = decide(px, qx, u_acc, L)
    if rng is not None:
        u_draw = np.array([philox.uniform(seed, step, philox.DRAW, r0 + r, int(a[r])) for r in range(R)])
    else:
        u_draw = np.asarray(u_verify, dtype=np.float64)[:, k]
    # resample / bonus rows, recomputed one block at a time
    y = np.zeros(R, dtype=np.int64)
    near = [None] * R
    res_mass = np.zeros(R, dtype=np.float64)
    trial = np.full(R, -1, dtype=np.int64)
    by_trials = np.zeros(R, dtype=bool)
    for s in range(0, R, block_rows):
        rs = np.arange(s, min(R, s + block_rows))
        ar = a[rs]
        p = numerics.softmax(numerics.decode(target[rs, ar], dtype), tau)
        w = p.copy()
        rej = ar < L[rs]
        q = None
        if rej.any():
            q = numerics.softmax(numerics.decode(draft[rs[rej], ar[rej]], dtype), tau)
            wr = np.maximum(p[rej] - q, 0.0)
            res_mass[rs[rej]] = wr.sum(axis=1)
            wr = residual_rows(p[rej], q)
            w[rej] = wr
        y[rs], nb = draw_rows(w, u_draw[rs], near_eps)
        for n_, r_ in enumerate(rs):
            near[r_] = nb[n_]
        if rng is not None and rej.any():
            # the residual by rejection from p (the counter-based uniforms' draw)
            for n_, r_ in enumerate(rs[rej]):
                i_ = int(a[r_])
                yy, tt, nn = residual_draw_rejection(
                    p[np.nonzero(rej)[0][n_]], q[n_],
                    lambda t, r_=r_, i_=i_: philox.trial_uniforms(seed, step, r0 + int(r_), i_, t), near_eps=near_eps)
                y[r_], trial[r_], near[r_], by_trials[r_] = yy, tt, nn, True
                u_draw[r_] = philox.trial_uniforms(seed, step, r0 + int(r_), i_, tt if tt >= 0 else RESIDUAL_TRIALS)[0]
    row_ratio = np.full(B, np.nan)
    row_acc = np.zeros(B, dtype=bool)
    row_ratio[vidx] = ratio[tags[vidx, 0], tags[vidx, 1]]
    row_acc[vidx] = acc[tags[vidx, 0], tags[vidx, 1]]
    res.update(accepted_len=a, out_tokens=_emit(a, x, y, k), row_p=row_p, row_q=row_q,
               row_ratio=row_ratio, row_accept=row_acc, accept=acc, draw_near=near,
               residual_mass=res_mass, row_verified=ver, u_accept=u_acc, u_draw=u_draw, draw_trial=trial,
               draw_by_trials=by_trials)
    return res
