"""The RNN head of the semi-autoregressive drafter.

TEST INFRASTRUCTURE (see the package docstring).

The pages name two light sequential modules on top of the parallel backbone:
the default Markov head, which looks only at the previous token, and an RNN
head, which carries the whole prefix of the block in a recurrent state
([P1] section "1. 半自回归生成"; [P2] section 3.1, where it keeps more of the
block's history at a higher cost and for a small gain).

Reading (the pages give no formula): the plainest recurrent form that keeps
the Markov head's low-rank additive correction,
  h_{-1} = 0,
  h_i    = round(tanh(E[x_{i-1}] + A h_{i-1})),      x_{-1} = the last committed token,
  dl_i   = round(bk_i + h_i . P^T),
with E [V, d_m] the token embedding, A [d_m, d_m] the recurrence ((A h)_j =
sum_k A[j, k] h_k) and P [V, d_m] the projection. Each value is computed in
float64 and rounded once to the storage type (bf16 or fp32, nearest-even):
the state because it is the operand of the next products, the logits because
they are the draft distribution the verifier uses. Draws as the Markov head.

Pins (tests/test_oracle_rnn.py): with A = 0 the head is the Markov head on the
table round(tanh(E)); the unrounded recurrence against torch.nn.RNN in
float64 (input weights the identity, no biases); the state's dependence on the
whole prefix (a change of x_{-1} reaches position 2 only through A).
"""
from __future__ import annotations

import numpy as np

from . import numerics
from .markov import draft_uniforms, draw_position


def _round(x: np.ndarray, dtype: str) -> np.ndarray:
    return numerics.round_bf16(x) if dtype == "bf16" else numerics.round_f32(x)


def state_exact(emb: np.ndarray, rec: np.ndarray, prev: np.ndarray, h_prev: np.ndarray, dtype: str) -> np.ndarray:
    """tanh(E[prev] + A h_prev) in float64, before rounding: [R, d_m].
    h_prev holds decoded values (float64)."""
    e = numerics.decode(emb, dtype)[np.asarray(prev, dtype=np.int64)]
    A = numerics.decode(rec, dtype)
    return np.tanh(e + h_prev @ A.T)


def states(emb: np.ndarray, rec: np.ndarray, prev_tokens: np.ndarray, dtype: str, round_state: bool = True) -> np.ndarray:
    """The states h_0 .. h_{k-1} for given previous tokens [R, k] (column i is
    x_{i-1}): float64 [R, k, d_m], rounded to the storage type unless
    round_state is False."""
    R, k = prev_tokens.shape
    d_m = emb.shape[1]
    h = np.zeros((R, d_m))
    out = np.zeros((R, k, d_m))
    for i in range(k):
        s = state_exact(emb, rec, prev_tokens[:, i], h, dtype)
        h = numerics.decode(_round(s, dtype), dtype) if round_state else s
        out[:, i] = h
    return out


def rnn_draft(mode: str, dtype: str, backbone: np.ndarray, emb: np.ndarray, rec: np.ndarray, proj: np.ndarray,
              prev_token: np.ndarray, tau: float, u_draft=None, prev_override=None, state_override=None,
              rng=None, near_eps: float = 0.0) -> dict:
    """Run the head over the k positions.

    Uniforms and draw_near as oracle.markov.markov_draft.

    prev_override (optional [R,k]): previous tokens to use at each position
    instead of the head's own draws; state_override (optional [R,k,d_m],
    stored type): h_{i-1} to use at position i instead of the head's own (so
    that one position can be checked against another implementation's state).
    """
    R, k, V = backbone.shape
    d_m = emb.shape[1]
    x = np.zeros((R, k), dtype=np.int64)
    dl = np.zeros(backbone.shape, dtype=backbone.dtype)
    hs = np.zeros((R, k, d_m), dtype=emb.dtype)
    near = [[np.zeros(0, dtype=np.int64)] * k for _ in range(R)]
    u = draft_uniforms(u_draft, rng, R, k) if mode == "sample" else np.zeros((R, k))
    prev = np.asarray(prev_token, dtype=np.int64)
    h = np.zeros((R, d_m))
    P = numerics.decode(proj, dtype)
    for i in range(k):
        if prev_override is not None:
            prev = np.asarray(prev_override[:, i], dtype=np.int64)
        if state_override is not None and i > 0:
            h = numerics.decode(state_override[:, i - 1], dtype)
        hr = _round(state_exact(emb, rec, prev, h, dtype), dtype)
        hs[:, i] = hr
        h = numerics.decode(hr, dtype)
        dl[:, i] = _round(numerics.decode(backbone[:, i], dtype) + h @ P.T, dtype)
        xi, nb = draw_position(dl[:, i], dtype, mode, tau, u[:, i], near_eps)
        x[:, i] = xi
        if nb is not None:
            for r in range(R):
                near[r][i] = nb[r]
        prev = xi
    return dict(tokens=x, logits=dl, states=hs, draw_near=near, u_draft=u)
