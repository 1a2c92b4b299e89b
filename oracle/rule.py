"""The acceptance rule for one request, written out as a definition.

TEST INFRASTRUCTURE (see the package docstring).

Speculative decoding lets a draft propose a block and the target check the whole
block in one pass; verified tokens are kept and the first disagreement is
replaced by a fresh draw ([P2] section 一; [P4] opening paragraphs: the longest
correct prefix is kept). The replacement keeps the output distribution equal to
the target's ([P3] section "DSpark的神奇之处": rejection sampling guarantees the
distribution of every emitted token).

Sampling form (the standard exact rule):
  for j = 0 .. L-1: keep draft token x_j with probability min(1, p_j(x_j) / q_j(x_j));
  at the first j that is not kept, emit a draw from max(0, p_j - q_j) normalised
  and stop; if all L are kept, emit a draw from the target row p_L (bonus token).
Greedy form: keep x_j iff x_j equals the target argmax of row j (lowest index
on ties); the first mismatch, or row L when all match, emits the target argmax.

The functions take probability vectors in any arithmetic that supports
+, -, *, /, comparison and max (Python floats, numpy float64, Fractions), and
random choices through two callables, so that a test can enumerate every
outcome with its exact probability:
  coin(j, prob) -> bool      True with probability `prob` (keep row j)
  draw(weights) -> int       index v with probability weights[v] / sum(weights)

Pins (tests/test_oracle_rule_exact.py): exhaustive enumeration with Fractions
that the tokens emitted over repeated steps follow the target's autoregressive
distribution exactly; greedy output equals repeated target argmax.
"""
from __future__ import annotations

from typing import Callable, List, Sequence, Tuple


def keep_probability(p_x, q_x):
    """min(1, p(x) / q(x)); a draft token the draft could not have drawn (q = 0) is kept."""
    if q_x == 0:
        return 1
    r = p_x / q_x
    return r if r < 1 else 1


def residual(p_row: Sequence, q_row: Sequence) -> List:
    """max(0, p - q) elementwise; the target row itself when that mass is zero.

    A zero residual means p == q, where a rejection has probability zero; the
    fallback only guards rounding in float arithmetic.
    """
    w = [(a - b) if a > b else (a - a) for a, b in zip(p_row, q_row)]
    total = w[0] - w[0]
    for v in w:
        total = total + v
    if total == 0:
        return list(p_row)
    return w


def speculative_step(p_rows: Sequence[Sequence], q_rows: Sequence[Sequence], x: Sequence[int], L: int,
                     coin: Callable, draw: Callable) -> Tuple[int, List[int]]:
    """One verification of a request whose first L draft tokens were scheduled.

    p_rows: L+1 target distributions (row L feeds the bonus token).
    q_rows: L draft distributions; x: the L draft tokens.
    Returns (accepted length a, emitted tokens x_0..x_{a-1} followed by one more).
    """
    for j in range(L):
        if not coin(j, keep_probability(p_rows[j][x[j]], q_rows[j][x[j]])):
            return j, list(x[:j]) + [draw(residual(p_rows[j], q_rows[j]))]
    return L, list(x[:L]) + [draw(list(p_rows[L]))]


def first_argmax(row: Sequence) -> int:
    best = 0
    for v in range(1, len(row)):
        if row[v] > row[best]:
            best = v
    return best


def greedy_step(target_rows: Sequence[Sequence], x: Sequence[int], L: int) -> Tuple[int, List[int]]:
    """Greedy verification: target_rows are L+1 rows of target logits (or probabilities)."""
    for j in range(L):
        g = first_argmax(target_rows[j])
        if g != x[j]:
            return j, list(x[:j]) + [g]
    return L, list(x[:L]) + [first_argmax(target_rows[L])]
