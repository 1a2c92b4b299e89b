"""Exact pins of the oracle's acceptance rule (oracle.rule).

The rule is run under an enumerator that follows every coin flip and every draw
with its exact probability (Fractions), so the distribution it induces is
computed exactly, not sampled. What is pinned is the property the pages state
for the method: the tokens emitted over repeated draft-and-verify steps follow
the target model's own autoregressive distribution, exactly (lossless
speculative decoding; rejection sampling keeps each emitted token's
distribution equal to the target's).

Planted mistakes (on the CPU, in copies of the rule) must break the equality.
"""
from fractions import Fraction
import itertools
import random

import pytest

from oracle import rule


class _Need(Exception):
    def __init__(self, options):
        self.options = options


def enumerate_outcomes(fn):
    """All results of fn(coin, draw) with their exact probabilities."""
    out = {}
    todo = [((), Fraction(1))]
    while todo:
        forced, pr = todo.pop()
        pos = [0]

        def choose(options):
            i = pos[0]
            if i < len(forced):
                pos[0] += 1
                return forced[i]
            raise _Need(options)

        def coin(j, p):
            p = Fraction(p)
            return choose([(True, p), (False, 1 - p)])

        def draw(w):
            W = sum(w, Fraction(0))
            return choose([(v, Fraction(w[v]) / W) for v in range(len(w)) if w[v] != 0])

        try:
            res = fn(coin, draw)
        except _Need as need:
            for choice, q in need.options:
                if q != 0:
                    todo.append((forced + (choice,), pr * q))
            continue
        out[res] = out.get(res, Fraction(0)) + pr
    return out


class TinyModel:
    """Random rational conditionals p(.|s), q(.|s) for every prefix s."""

    def __init__(self, V, seed, q_zeros=True, equal_rows=False):
        self.V, self.seed, self.q_zeros, self.equal_rows = V, seed, q_zeros, equal_rows
        self._p, self._q = {}, {}

    def _dist(self, s, salt, allow_zero):
        rnd = random.Random(f"{self.seed}/{salt}/{s}")
        w = [rnd.randint(0 if allow_zero else 1, 6) for _ in range(self.V)]
        if sum(w) == 0:
            w[rnd.randrange(self.V)] = 1
        tot = sum(w)
        return [Fraction(a, tot) for a in w]

    def p(self, s):
        s = tuple(s)
        if s not in self._p:
            self._p[s] = self._dist(s, "p", False)
        return self._p[s]

    def q(self, s):
        s = tuple(s)
        if s not in self._q:
            if self.equal_rows and len(s) % 2 == 0:
                self._q[s] = list(self.p(s))       # p == q: residual is empty
            else:
                self._q[s] = self._dist(s, "q", self.q_zeros)
        return self._q[s]


def _step_fn(model, ctx, k, length_policy, step=rule.speculative_step):
    """One draft-and-verify step from context ctx, as a function of (coin, draw)."""

    def fn(coin, draw):
        x = []
        # the draft proposes the whole block; the verify length may depend on
        # what is known before each token is decided
        L = None
        for j in range(k):
            if length_policy.kind == "prefix-stop" and L is None and length_policy.stop(ctx, x):
                L = j
            x.append(draw(model.q(ctx + tuple(x))))
        if length_policy.kind == "context":
            L = length_policy.length(ctx)
        elif length_policy.kind == "prefix-stop":
            L = k if L is None else L
        elif length_policy.kind == "sees-token":
            L = length_policy.length_from_tokens(ctx, x, model)
        p_rows = [model.p(ctx + tuple(x[:j])) for j in range(L + 1)]
        q_rows = [model.q(ctx + tuple(x[:j])) for j in range(L)]
        a, emitted = step(p_rows, q_rows, x, L, coin, draw)
        assert len(emitted) == a + 1
        return tuple(emitted)

    return fn


class Policy:
    def __init__(self, kind, **kw):
        self.kind = kind
        self.__dict__.update(kw)


def emitted_distribution(model, k, n, policy, step=rule.speculative_step):
    """Exact distribution of the first n emitted tokens over repeated steps."""
    frontier = {(): Fraction(1)}
    done = {}
    while frontier:
        nxt = {}
        for ctx, pr in frontier.items():
            for emitted, q in enumerate_outcomes(_step_fn(model, ctx, k, policy, step)).items():
                c2 = ctx + emitted
                if len(c2) >= n:
                    key = c2[:n]
                    done[key] = done.get(key, Fraction(0)) + pr * q
                else:
                    nxt[c2] = nxt.get(c2, Fraction(0)) + pr * q
        frontier = nxt
    return done


def target_distribution(model, n):
    out = {}
    for s in itertools.product(range(model.V), repeat=n):
        pr = Fraction(1)
        for t in range(n):
            pr *= model.p(s[:t])[s[t]]
        out[s] = pr
    return out


def _assert_equal(d1, d2):
    keys = set(d1) | set(d2)
    for key in keys:
        assert d1.get(key, 0) == d2.get(key, 0), (key, d1.get(key, 0), d2.get(key, 0))
    assert sum(d1.values()) == 1


CASES = [
    # (V, k, seed, q_zeros, equal_rows)
    (2, 1, 0, False, False),
    (2, 3, 1, True, False),
    (3, 2, 2, True, False),
    (3, 3, 3, False, True),
    (4, 2, 4, True, False),
]


@pytest.mark.parametrize("V,k,seed,q_zeros,equal_rows", CASES)
def test_lossless_context_lengths(V, k, seed, q_zeros, equal_rows):
    """Verify length chosen from the context (as a scheduler does before the target runs)."""
    model = TinyModel(V, seed, q_zeros, equal_rows)
    n = k + 1
    pol = Policy("context", length=lambda ctx: (len(ctx) * 7 + sum(ctx) + seed) % (k + 1))
    _assert_equal(emitted_distribution(model, k, n, pol), target_distribution(model, n))


@pytest.mark.parametrize("V,k,seed", [(2, 3, 5), (3, 3, 6), (4, 2, 7)])
def test_lossless_prefix_stopping(V, k, seed):
    """Stopping before position j may depend on the drafts x_<j (a prefix scheduler)."""
    model = TinyModel(V, seed)

    def stop(ctx, x):
        return len(x) >= 1 and model.q(ctx + tuple(x[:-1]))[x[-1]] < Fraction(1, 3)

    pol = Policy("prefix-stop", stop=stop)
    n = k + 1
    _assert_equal(emitted_distribution(model, k, n, pol), target_distribution(model, n))


def test_single_step_first_token_is_target():
    model = TinyModel(4, 11)
    for L in range(4):
        pol = Policy("context", length=lambda ctx, L=L: L)
        dist = enumerate_outcomes(_step_fn(model, (), 3, pol))
        first = {}
        for em, pr in dist.items():
            first[em[0]] = first.get(em[0], Fraction(0)) + pr
        for v in range(4):
            assert first.get(v, 0) == model.p(())[v]


def test_verify_length_seeing_the_token_is_not_lossless():
    """Reading recorded in the design notes: the decision to verify position j
    must not depend on x_j itself. A policy that truncates on the drawn token's
    own draft probability biases the output."""
    model = TinyModel(2, 21, q_zeros=False)

    def length_from_tokens(ctx, x, m):
        L = 0
        while L < len(x) and m.q(ctx + tuple(x[:L]))[x[L]] >= Fraction(1, 2):
            L += 1
        return L

    pol = Policy("sees-token", length_from_tokens=length_from_tokens)
    d = emitted_distribution(model, 2, 3, pol)
    t = target_distribution(model, 3)
    assert any(d.get(s, 0) != t[s] for s in t)


def test_greedy_equals_repeated_argmax():
    """Greedy verification reproduces greedy target decoding token for token."""
    rnd = random.Random(3)
    V, k = 5, 4
    for trial in range(200):
        table = {}

        def logits(s):
            s = tuple(s)
            if s not in table:
                table[s] = [rnd.randint(0, 3) for _ in range(V)]   # many ties
            return table[s]

        ctx = ()
        steps = 0
        while len(ctx) < 12:
            # a draft that agrees with the target some of the time
            x = []
            for j in range(k):
                g = rule.first_argmax(logits(ctx + tuple(x)))
                x.append(g if rnd.random() < 0.6 else rnd.randrange(V))
            L = rnd.randint(0, k)
            rows = [logits(ctx + tuple(x[:j])) for j in range(L + 1)]
            a, em = rule.greedy_step(rows, x, L)
            assert len(em) == a + 1 and 0 <= a <= L
            ctx = ctx + tuple(em)
            steps += 1
        ref = ()
        while len(ref) < len(ctx):
            ref = ref + (rule.first_argmax(logits(ref)),)
        assert ref == ctx


# ---- planted mistakes (negative controls) ---------------------------------

def _step_resample_from_p(p_rows, q_rows, x, L, coin, draw):
    for j in range(L):
        if not coin(j, rule.keep_probability(p_rows[j][x[j]], q_rows[j][x[j]])):
            return j, list(x[:j]) + [draw(list(p_rows[j]))]
    return L, list(x[:L]) + [draw(list(p_rows[L]))]


def _step_inverted_ratio(p_rows, q_rows, x, L, coin, draw):
    for j in range(L):
        if not coin(j, rule.keep_probability(q_rows[j][x[j]], p_rows[j][x[j]])):
            return j, list(x[:j]) + [draw(rule.residual(p_rows[j], q_rows[j]))]
    return L, list(x[:L]) + [draw(list(p_rows[L]))]


def _step_bonus_from_draft_row(p_rows, q_rows, x, L, coin, draw):
    for j in range(L):
        if not coin(j, rule.keep_probability(p_rows[j][x[j]], q_rows[j][x[j]])):
            return j, list(x[:j]) + [draw(rule.residual(p_rows[j], q_rows[j]))]
    last = q_rows[L - 1] if L > 0 else p_rows[0]
    return L, list(x[:L]) + [draw(list(last))]


def _step_residual_without_clip(p_rows, q_rows, x, L, coin, draw):
    for j in range(L):
        if not coin(j, rule.keep_probability(p_rows[j][x[j]], q_rows[j][x[j]])):
            w = [abs(a - b) for a, b in zip(p_rows[j], q_rows[j])]
            if sum(w) == 0:
                w = list(p_rows[j])
            return j, list(x[:j]) + [draw(w)]
    return L, list(x[:L]) + [draw(list(p_rows[L]))]


@pytest.mark.parametrize("bad", [_step_resample_from_p, _step_inverted_ratio,
                                 _step_bonus_from_draft_row, _step_residual_without_clip])
def test_planted_mistakes_break_losslessness(bad):
    model = TinyModel(3, 31, q_zeros=False)
    k, n = 2, 3
    pol = Policy("context", length=lambda ctx: 2 if len(ctx) == 0 else 1)
    d = emitted_distribution(model, k, n, pol, step=bad)
    t = target_distribution(model, n)
    assert any(d.get(s, 0) != t[s] for s in t)
