"""The Markov head of the semi-autoregressive drafter.

TEST INFRASTRUCTURE (see the package docstring).

The drafter keeps a parallel backbone that proposes the whole block in one pass
and adds a light sequential module that injects prefix information token by
token; the default module is a Markov head that depends only on the previous
token ([P1] section "1. 半自回归生成"; [P2] section 3.1).

Reading (the pages give no formula): the head adds a low-rank correction to
the backbone logits of position i, looked up from the previous token,
  dl_i = bk_i + E[x_{i-1}] . P^T,   x_{-1} = the last committed token,
with E [V, d_m] the previous-token embedding and P [V, d_m] the projection (one
d_m row per vocabulary entry). dl_i is computed in float64 and rounded once to
the storage type (bf16 or fp32, nearest-even), and x_i is drawn from the
rounded logits: greedy = first argmax; sampling = inverse-CDF draw from
softmax(dl_i / tau) with uniform u[r, i] = U(seed, step, 2, r, i)
(oracle.philox), or a given array. The draft distribution q that the
verifier uses is the softmax of these same stored logits, so the draw and the
verification see one distribution.

Pins (tests/test_oracle_markov.py): the projection against an exact
Fraction dot product on small bf16 inputs; the rounding against torch's bf16
cast; draws against the first-index argmax and the inverse-CDF pins.
"""
from __future__ import annotations

import numpy as np

from . import numerics, philox


def head_exact(bk_row: np.ndarray, emb: np.ndarray, proj: np.ndarray, prev: np.ndarray,
               dtype: str) -> np.ndarray:
    """bk + E[prev] . P^T for one position, in float64 before any rounding."""
    e = numerics.decode(emb, dtype)[np.asarray(prev, dtype=np.int64)]      # [R, d_m]
    p = numerics.decode(proj, dtype)                                       # [V, d_m]
    return numerics.decode(bk_row, dtype) + e @ p.T


def head_logits(bk_row: np.ndarray, emb: np.ndarray, proj: np.ndarray, prev: np.ndarray,
                dtype: str) -> np.ndarray:
    """Rounded draft logits for one position: round(bk + E[prev] . P^T); stored type."""
    exact = head_exact(bk_row, emb, proj, prev, dtype)
    if dtype == "bf16":
        return numerics.round_bf16(exact)
    return numerics.round_f32(exact)


def draw_position(dl_row: np.ndarray, dtype: str, mode: str, tau: float, u: np.ndarray, near_eps: float = 0.0):
    """Next draft token per request from stored logits [R, V]; also the draws'
    near sets (oracle.verify.draw_rows; None in greedy mode)."""
    vals = numerics.decode(dl_row, dtype)
    if mode == "greedy":
        return numerics.argmax_first(vals).astype(np.int64), None
    from .verify import draw_rows
    return draw_rows(numerics.softmax(vals, tau), np.asarray(u, dtype=np.float64), near_eps)


def draft_uniforms(u_draft, rng, R: int, k: int) -> np.ndarray:
    """The head's sampling uniforms [R, k]: U(seed, step, 2, r0 + r, i) for
    rng = (seed, step) or (seed, step, r0) (oracle.philox; r0 addresses a slice
    of a larger batch's requests), else the given array."""
    if rng is not None:
        seed, step, r0 = (tuple(rng) + (0,))[:3]
        return philox.uniforms(seed, step, philox.DRAFT, R, k, r0)
    return np.asarray(u_draft, dtype=np.float64)


def markov_draft(mode: str, dtype: str, backbone: np.ndarray, emb: np.ndarray, proj: np.ndarray,
                 prev_token: np.ndarray, tau: float, u_draft=None, prev_override=None, rng=None,
                 near_eps: float = 0.0) -> dict:
    """Run the head over the k positions.

    Sampling uniforms: U(seed, step, 2, r, i) for rng = (seed, step), else
    u_draft [R, k]. prev_override (optional [R,k]): previous tokens to use at
    each position instead of the head's own draws, so that one position can be
    checked against another implementation's draws. draw_near[r][i]: the near
    set of the draw at near_eps (oracle.verify.draw_rows).
    """
    R, k, V = backbone.shape
    x = np.zeros((R, k), dtype=np.int64)
    dl = np.zeros(backbone.shape, dtype=backbone.dtype)
    near = [[np.zeros(0, dtype=np.int64)] * k for _ in range(R)]
    u = draft_uniforms(u_draft, rng, R, k) if mode == "sample" else np.zeros((R, k))
    prev = np.asarray(prev_token, dtype=np.int64)
    for i in range(k):
        if prev_override is not None:
            prev = np.asarray(prev_override[:, i], dtype=np.int64)
        dl[:, i] = head_logits(backbone[:, i], emb, proj, prev, dtype)
        xi, nb = draw_position(dl[:, i], dtype, mode, tau, u[:, i], near_eps)
        x[:, i] = xi
        if nb is not None:
            for r in range(R):
                near[r][i] = nb[r]
        prev = xi
    return dict(tokens=x, logits=dl, draw_near=near, u_draft=u)
