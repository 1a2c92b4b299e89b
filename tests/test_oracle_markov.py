"""Pins of oracle.markov: the head's projection and rounding, and its draws."""
from fractions import Fraction

import numpy as np
import torch

from draft_token_verification_flattened_amd import workloads
from oracle import markov, numerics


def _exact_round_bf16(fr):
    """Nearest bf16 to an exact rational (ties to even), by scanning neighbours."""
    approx = numerics.round_bf16(np.array([float(fr)]))[0]
    best = None
    for d in range(-2, 3):
        b = (int(approx) + d) & 0xFFFF
        if (b & 0x7F80) == 0x7F80:
            continue
        v = Fraction(float(numerics.decode(np.array([b], np.uint16), "bf16")[0]))
        key = (abs(v - fr), b & 1)
        if best is None or key < best[0]:
            best = (key, b)
    return best[1]


def test_head_logits_bf16_exact():
    g = np.random.Generator(np.random.Philox(1))
    R, V, d = 3, 24, 16
    bk = workloads.f32_to_bf16_bits(3 * g.standard_normal((R, V)).astype(np.float32))
    E = workloads.f32_to_bf16_bits(g.standard_normal((V, d)).astype(np.float32))
    P = workloads.f32_to_bf16_bits((0.05 * g.standard_normal((V, d))).astype(np.float32))
    prev = np.array([0, 5, 23])
    got = markov.head_logits(bk, E, P, prev, "bf16")
    Ed = numerics.decode(E, "bf16")
    Pd = numerics.decode(P, "bf16")
    bkd = numerics.decode(bk, "bf16")
    for r in range(R):
        for v in range(V):
            exact = Fraction(float(bkd[r, v])) + sum(
                Fraction(float(Ed[prev[r], t])) * Fraction(float(Pd[v, t])) for t in range(d))
            assert got[r, v] == _exact_round_bf16(exact)


def test_head_logits_f32_close_to_exact():
    g = np.random.Generator(np.random.Philox(2))
    R, V, d = 4, 32, 4
    bk = (2 * g.standard_normal((R, V))).astype(np.float32)
    E = (0.3 * g.standard_normal((V, d))).astype(np.float32)
    P = (0.3 * g.standard_normal((V, d))).astype(np.float32)
    prev = np.array([1, 2, 30, 31])
    got = markov.head_logits(bk, E, P, prev, "f32")
    for r in range(R):
        for v in range(V):
            exact = Fraction(float(bk[r, v])) + sum(
                Fraction(float(E[prev[r], t])) * Fraction(float(P[v, t])) for t in range(d))
            f = float(exact)
            lo, hi = np.nextafter(np.float32(f), np.float32(-np.inf)), np.nextafter(np.float32(f), np.float32(np.inf))
            cands = [lo, np.float32(f), hi]
            errs = [abs(Fraction(float(c)) - exact) for c in cands]
            assert abs(Fraction(float(got[r, v])) - exact) == min(errs)


def test_rounding_matches_torch_on_fp32_sums():
    g = np.random.Generator(np.random.Philox(3))
    x = (5 * g.standard_normal(100000)).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(numerics.round_bf16(x.astype(np.float64)), ref)


def test_draft_draws_follow_rounded_logits():
    w = workloads.make("c0")
    for mode in ("greedy", "sample"):
        out = markov.markov_draft(mode, "f32", w.backbone, w.emb, w.proj, w.prev_token, 1.0, w.u_draft)
        dl = out["logits"].astype(np.float64)
        prev = w.prev_token
        for i in range(w.k):
            ref = markov.head_logits(w.backbone[:, i], w.emb, w.proj, prev, "f32")
            assert np.array_equal(out["logits"][:, i], ref)
            if mode == "greedy":
                assert (out["tokens"][:, i] == np.argmax(dl[:, i], axis=1)).all()
            else:
                p = numerics.softmax(dl[:, i], 1.0)
                for r in range(w.R):
                    ref_tok = np.searchsorted(np.cumsum(p[r]), w.u_draft[r, i] * np.cumsum(p[r])[-1], side="right")
                    assert out["tokens"][r, i] == ref_tok
            prev = out["tokens"][:, i]


def test_prev_override_reproduces_own_draws():
    w = workloads.make("c0")
    a = markov.markov_draft("sample", "f32", w.backbone, w.emb, w.proj, w.prev_token, 1.0, w.u_draft)
    prevs = np.concatenate([w.prev_token[:, None], a["tokens"][:, :-1]], axis=1)
    b = markov.markov_draft("sample", "f32", w.backbone, w.emb, w.proj, w.prev_token, 1.0, w.u_draft,
                            prev_override=prevs)
    assert np.array_equal(a["tokens"], b["tokens"])
    assert np.array_equal(a["logits"], b["logits"])
