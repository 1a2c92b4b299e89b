"""Pins of the float64 batch verifier (oracle.verify).

1. It agrees element for element with the scalar rule (oracle.rule) when both
   take the same uniforms: accept flags, accepted lengths and emitted tokens.
2. Chi-square on 10**7 Philox-seeded trials: the first n = k+1 tokens emitted
   over repeated steps follow the target's autoregressive distribution
   (V = 8, k = 3, 4096 cells). Pre-registered threshold: p > 1e-4.
3. The same test with a planted mistake gives p < 1e-9.
4. Greedy mode on logits equals the scalar greedy rule.
"""
import numpy as np
import pytest
from scipy import stats

from oracle import numerics, rule, schedule, verify

from chisq_harness import LogitModel, chi2_pvalue, run_trials


def _rand_dists(g, shape, V, zeros=0.0):
    a = g.gamma(1.0, size=shape + (V,))
    if zeros:
        a = np.where(g.random(a.shape) < zeros, 0.0, a)
        a[..., 0] += 1e-3
    return a / a.sum(axis=-1, keepdims=True)


@pytest.mark.parametrize("seed", range(6))
def test_batch_equals_scalar_rule(seed):
    g = np.random.Generator(np.random.Philox(100 + seed))
    R, k, V = 300, 4, 6
    P = _rand_dists(g, (R, k + 1), V)
    Qd = _rand_dists(g, (R, k), V, zeros=0.2 if seed % 2 else 0.0)
    if seed == 3:
        Qd[:50] = P[:50, :k]                   # p == q rows: empty residual
    x = np.zeros((R, k), dtype=np.int64)
    for j in range(k):
        c = np.cumsum(Qd[:, j], axis=1)
        x[:, j] = np.minimum((c < g.random(R)[:, None]).sum(axis=1), V - 1)
    L = g.integers(0, k + 1, size=R)
    u = (g.integers(0, 1 << 24, size=(R, k + 1)) * 2.0 ** -24)
    a, out = verify.verify_probs(P, Qd, x, L, u)
    for r in range(R):
        def coin(j, prob, r=r):
            return u[r, j] < prob

        def draw(w, r=r):
            return numerics.inv_cdf(np.array(w, dtype=np.float64), u[r, k])

        ar, em = rule.speculative_step(list(P[r]), list(Qd[r]), list(x[r]), int(L[r]), coin, draw)
        assert ar == a[r]
        assert list(out[r, :ar + 1]) == em
        assert (out[r, ar + 1:] == -1).all()


def test_greedy_batch_equals_scalar_rule():
    g = np.random.Generator(np.random.Philox(7))
    R, k, V = 200, 5, 16
    target = g.integers(-3, 3, size=(R, k + 1, V)).astype(np.float32)    # many ties
    x = g.integers(0, V, size=(R, k)).astype(np.int64)
    agree = g.random((R, k)) < 0.7
    x = np.where(agree, numerics.argmax_first(target[:, :k].astype(np.float64)), x)
    L = g.integers(0, k + 1, size=R)
    tags, cu = schedule.flatten(L)
    res = verify.verify("greedy", "f32", target, None, x, tags, cu, 1.0,
                        np.zeros((R, k + 1), dtype=np.float32))
    for r in range(R):
        ar, em = rule.greedy_step([list(target[r, j]) for j in range(k + 1)], list(x[r]), int(L[r]))
        assert ar == res["accepted_len"][r]
        assert list(res["out_tokens"][r, :ar + 1]) == em


def test_sampling_batch_on_logits_matches_probability_form():
    """verify() on stored logits equals verify_probs() on their float64 softmax."""
    g = np.random.Generator(np.random.Philox(9))
    R, k, V = 64, 3, 40
    tl = (2 * g.standard_normal((R, k + 1, V))).astype(np.float32)
    dl = (tl[:, :k] + g.standard_normal((R, k, V))).astype(np.float32)
    tau = 0.8
    P = numerics.softmax(tl.astype(np.float64), tau)
    Qd = numerics.softmax(dl.astype(np.float64), tau)
    x = np.array([[numerics.inv_cdf(Qd[r, j], g.random()) for j in range(k)] for r in range(R)])
    L = g.integers(0, k + 1, size=R)
    u = (g.integers(0, 1 << 24, size=(R, k + 1)) * 2.0 ** -24).astype(np.float32)
    tags, cu = schedule.flatten(L)
    res = verify.verify("sample", "f32", tl, dl, x, tags, cu, tau, u)
    a, out = verify.verify_probs(P, Qd, x, L, u.astype(np.float64))
    assert (res["accepted_len"] == a).all()
    assert (res["out_tokens"] == out).all()


# ---------------------------------------------------------------------------
# chi-square over repeated steps
# ---------------------------------------------------------------------------

@pytest.fixture(scope="module")
def logit_model():
    return LogitModel(seed=5)


def test_chisquare_1e7_trials(logit_model):
    k = 3
    seqs, pr = logit_model.target_probs(k + 1)
    counts = run_trials(logit_model, 10_000_000, k, seed=2026, verify_fn=verify.verify_probs)
    assert counts.sum() == 10_000_000
    p = chi2_pvalue(counts, pr)
    assert p > 1e-4, p


def _planted_resample_from_p(P, Qd, x, L, u):
    orig = verify.residual_rows
    try:
        verify.residual_rows = lambda p, q: p.copy()
        return verify.verify_probs(P, Qd, x, L, u)
    finally:
        verify.residual_rows = orig


def _planted_inverted_ratio(P, Qd, x, L, u):
    return verify.verify_probs(Qd_pad(Qd, P), P[:, :-1], x, L, u)


def Qd_pad(Qd, P):
    # target rows replaced by draft rows (bonus row kept): keep prob becomes min(1, q/p)
    out = P.copy()
    out[:, :-1] = Qd
    return out


def _planted_no_min(P, Qd, x, L, u):
    # accept iff u < p (the draft probability is ignored)
    R, k1, V = P.shape
    Q1 = np.ones_like(Qd)
    a, _ = verify.verify_probs(P, Q1, x, L, u)
    _, out = verify.verify_probs(P, Qd, x, np.minimum(L, a), u)
    return np.minimum(L, a), out


@pytest.mark.parametrize("bad", [_planted_resample_from_p, _planted_inverted_ratio, _planted_no_min])
def test_chisquare_planted_mistakes_fail(logit_model, bad):
    k = 3
    seqs, pr = logit_model.target_probs(k + 1)
    counts = run_trials(logit_model, 1_000_000, k, seed=77, verify_fn=bad)
    assert chi2_pvalue(counts, pr) < 1e-9


# ---------------------------------------------------------------------------
# uniforms from the counter-based generator (rng = (seed, step))
# ---------------------------------------------------------------------------

def test_rng_uniforms_are_addressed_by_decision():
    """verify(rng=(seed, step)): the keep decisions use U(seed, step, 0, r, j)
    (the same as an array holding them), the bonus draw U(seed, step, 1, r, L_r),
    and the residual draw of a rejecting request is residual_draw_rejection
    with that request's trial uniforms."""
    from oracle import philox
    g = np.random.Generator(np.random.Philox(31))
    R, k, V = 40, 4, 24
    tl = (2 * g.standard_normal((R, k + 1, V))).astype(np.float32)
    dl = (tl[:, :k] + g.standard_normal((R, k, V))).astype(np.float32)
    Qd = numerics.softmax(dl.astype(np.float64), 1.0)
    x = np.array([[numerics.inv_cdf(Qd[r, j], g.random()) for j in range(k)] for r in range(R)])
    L = g.integers(0, k + 1, size=R)
    tags, cu = schedule.flatten(L)
    res = verify.verify("sample", "f32", tl, dl, x, tags, cu, 1.0, rng=(7, 12))
    u = np.zeros((R, k + 1))
    for r in range(R):
        for j in range(k):
            u[r, j] = philox.uniform(7, 12, philox.ACCEPT, r, j)
        u[r, k] = philox.uniform(7, 12, philox.DRAW, r, int(res["accepted_len"][r]))
    ref = verify.verify("sample", "f32", tl, dl, x, tags, cu, 1.0, u)
    assert np.array_equal(res["accepted_len"], ref["accepted_len"])
    assert np.array_equal(res["u_accept"], u[:, :k])
    a = res["accepted_len"]
    bonus = a == L
    assert bonus.any() and (~bonus).any()
    assert np.array_equal(res["out_tokens"][bonus], ref["out_tokens"][bonus])
    P = numerics.softmax(tl.astype(np.float64), 1.0)
    for r in np.nonzero(~bonus)[0]:
        assert np.array_equal(res["out_tokens"][r, :a[r]], x[r, :a[r]])
        yy, tt, _ = verify.residual_draw_rejection(P[r, a[r]], Qd[r, a[r]],
                                                   lambda t, r=r: philox.trial_uniforms(7, 12, r, int(a[r]), t))
        assert res["out_tokens"][r, a[r]] == yy and res["draw_trial"][r] == tt
    # another step gives other decisions
    other = verify.verify("sample", "f32", tl, dl, x, tags, cu, 1.0, rng=(7, 13))
    assert not np.array_equal(other["u_accept"], res["u_accept"])


def _residual_dists(g, V):
    p = g.gamma(1.0, size=V)
    p /= p.sum()
    q = g.gamma(1.0, size=V)
    q /= q.sum()
    res = np.maximum(p - q, 0.0)
    return p, q, res / res.sum()


def _chi2_p(counts, expected):
    """Chi-square p-value; a count in a cell of expected 0 gives 0."""
    from scipy import stats
    zero = expected == 0
    if counts[zero].sum() > 0:
        return 0.0
    return stats.chisquare(counts[~zero], expected[~zero]).pvalue


def test_residual_rejection_draw_is_exact():
    """The rejection draw's tokens follow max(0, p - q) normalised: a
    chi-square on 2e5 draws (V = 8) against it, with few trials so that the
    fallback is exercised too. Planted mistakes fail: keeping with probability
    q / p, keeping every proposal, and a fallback from p."""
    g = np.random.Generator(np.random.Philox(77))
    V = 8
    p, q, res = _residual_dists(g, V)
    n = 100_000
    uu = g.random((n, 4, 2))

    def run(draw, trials):
        ys = np.array([draw(p, q, lambda t, i=i: (uu[i, min(t, 3), 0], uu[i, min(t, 3), 1]), trials)[0]
                       for i in range(n)])
        return np.bincount(ys, minlength=V)

    counts = run(lambda p_, q_, f, T: verify.residual_draw_rejection(p_, q_, f, T), 2)
    assert _chi2_p(counts, res * n) > 1e-4

    def keep_q_over_p(p_, q_, f, T):
        orig = verify.residual_draw_rejection
        for t in range(T):
            u1, u2 = f(t)
            y = int(verify.draw_rows(p_[None, :], np.array([u1]))[0][0])
            if u2 < min(1.0, q_[y] / p_[y]):
                return y, t, []
        return orig(p_, q_, f, 0)

    def keep_all(p_, q_, f, T):
        return int(verify.draw_rows(p_[None, :], np.array([f(0)[0]]))[0][0]), 0, []

    def fallback_from_p(p_, q_, f, T):
        y, t, nn = verify.residual_draw_rejection(p_, q_, f, T)
        if t < 0:
            y = int(verify.draw_rows(p_[None, :], np.array([f(T)[0]]))[0][0])
        return y, t, nn
    for bad in (keep_q_over_p, keep_all):
        assert _chi2_p(run(bad, 2), res * n) < 1e-9
    # the fallback alone (no trials) is the inverse-CDF draw from the residual
    assert _chi2_p(run(lambda p_, q_, f, T: verify.residual_draw_rejection(p_, q_, f, 0), 0), res * n) > 1e-4
    assert _chi2_p(run(fallback_from_p, 0), res * n) < 1e-9


def test_residual_rejection_draw_fallback_and_empty_residual():
    # p == q: no trial can keep; the fallback draws from p
    p = np.array([0.5, 0.25, 0.125, 0.125])
    y, t, near = verify.residual_draw_rejection(p, p.copy(), lambda t: (0.6, 0.0), 16)
    assert t == -1 and y == 1                 # C = [0.5, 0.75, ...]: t = 0.6 falls in token 1
    # a trial keeps iff u2 < 1 - q(y) / p(y)
    q = np.array([0.25, 0.25, 0.25, 0.25])
    y, t, _ = verify.residual_draw_rejection(p, q, lambda t: (0.1, 0.49), 16)   # y = 0: 1 - q/p = 0.5
    assert (y, t) == (0, 0)
    seq = iter([(0.1, 0.51), (0.1, 0.49)])
    y, t, _ = verify.residual_draw_rejection(p, q, lambda t: next(seq), 16)
    assert (y, t) == (0, 1)
    y, t, near = verify.residual_draw_rejection(p, q, lambda t: (0.1, 0.5 - 1e-7), 16)
    assert (y, t) == (0, 0) and ("keep", 0) in near


def test_residual_rejection_default_cap():
    """With p == q no trial can keep: the default draw runs RESIDUAL_TRIALS = 64
    trials, in order, then the fallback takes the first uniform of trial 64."""
    assert verify.RESIDUAL_TRIALS == 64
    p = np.array([0.5, 0.25, 0.125, 0.125])
    seen = []

    def tu(t):
        seen.append(t)
        return (0.6, 0.0)

    y, t, _ = verify.residual_draw_rejection(p, p.copy(), tu)
    assert (y, t) == (1, -1)
    assert seen == list(range(64)) + [64]


def test_rng_chisquare_lossless(logit_model):
    """Trials through verify(rng=(seed, step)), one step per round of the
    harness: the first k+1 emitted tokens follow the target (V = 8, k = 2,
    512 cells). A planted reuse of the keep uniform for the draw must fail."""
    from oracle import philox
    k = 2
    seqs, pr = logit_model.target_probs(k + 1)
    V = logit_model.V
    calls = [0]

    def via_rng(rows, x, L, u, reuse=False):
        R = rows.shape[0]
        tl = logit_model.tl[rows]
        dl = logit_model.dl[rows[:, :k]]
        tags, cu = schedule.flatten(L)
        calls[0] += 1
        if not reuse:
            res = verify.verify("sample", "f32", tl, dl, x, tags, cu, 1.0, rng=(5, calls[0]))
        else:
            uu = np.zeros((R, k + 1))
            uu[:, :k] = philox.uniforms(5, calls[0], philox.ACCEPT, R, k)
            uu[:, k] = uu[:, 0]
            res = verify.verify("sample", "f32", tl, dl, x, tags, cu, 1.0, uu)
        return res["accepted_len"], res["out_tokens"]

    counts = run_trials(logit_model, 60_000, k, seed=99, verify_fn=via_rng, batch=20_000, rows=True)
    assert counts.sum() == 60_000
    assert chi2_pvalue(counts, pr) > 1e-4
    counts = run_trials(logit_model, 60_000, k, seed=98,
                        verify_fn=lambda *a: via_rng(*a, reuse=True), batch=20_000, rows=True)
    assert chi2_pvalue(counts, pr) < 1e-9


def test_rng_request_offset_addresses_a_slice():
    """rng = (seed, step, r0): a slice of requests lo..hi verified on its own
    gets exactly the whole batch's uniforms, decisions and tokens."""
    g = np.random.Generator(np.random.Philox(77))
    R, k, V = 9, 3, 40
    tl = (2.0 * g.standard_normal((R, k + 1, V))).astype(np.float32)
    dl = (tl[:, :k] + g.standard_normal((R, k, V))).astype(np.float32)
    x = g.integers(0, V, size=(R, k))
    L = g.integers(0, k + 1, size=R)
    tags, cu = schedule.flatten(L)
    whole = verify.verify("sample", "f32", tl, dl, x, tags, cu, 1.0, rng=(5, 2))
    lo, hi = 3, 8
    t2, c2 = schedule.flatten(L[lo:hi])
    part = verify.verify("sample", "f32", tl[lo:hi], dl[lo:hi], x[lo:hi], t2, c2, 1.0, rng=(5, 2, lo))
    assert np.array_equal(part["u_accept"], whole["u_accept"][lo:hi])
    assert np.array_equal(part["u_draw"], whole["u_draw"][lo:hi])
    assert np.array_equal(part["accepted_len"], whole["accepted_len"][lo:hi])
    assert np.array_equal(part["out_tokens"], whole["out_tokens"][lo:hi])
    # without the offset the slice would draw other numbers
    other = verify.verify("sample", "f32", tl[lo:hi], dl[lo:hi], x[lo:hi], t2, c2, 1.0, rng=(5, 2))
    assert not np.array_equal(other["u_accept"], whole["u_accept"][lo:hi])
