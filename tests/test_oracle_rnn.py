"""Pins of the RNN-head oracle (CPU only)."""
import numpy as np
import pytest
import torch

from draft_token_verification_flattened_amd import workloads
from oracle import markov as omarkov
from oracle import numerics
from oracle import rnn as ornn


def _small_bf16(seed=5, R=6, k=4, V=40, d_m=8):
    g = np.random.Generator(np.random.Philox(seed))
    enc = workloads.f32_to_bf16_bits
    bk = enc((2.0 * g.standard_normal((R, k, V))).astype(np.float32))
    emb = enc(g.standard_normal((V, d_m)).astype(np.float32))
    rec = enc((0.5 / np.sqrt(d_m) * g.standard_normal((d_m, d_m))).astype(np.float32))
    proj = enc((0.3 * g.standard_normal((V, d_m))).astype(np.float32))
    prev = g.integers(0, V, size=R)
    u = g.random((R, k)).astype(np.float32)
    return bk, emb, rec, proj, prev, u


def _cases():
    w = workloads.make("c0")
    yield "f32", w.backbone, w.emb, w.rec, w.proj, w.prev_token, w.u_draft
    yield ("bf16",) + _small_bf16()


@pytest.mark.parametrize("mode", ["greedy", "sample"])
def test_zero_recurrence_is_the_markov_head_on_tanh_table(mode):
    """A = 0: h_i = round(tanh(E[x_{i-1}])), so the head is the Markov head with
    the embedding table round(tanh(E)): tokens and stored logits bit for bit."""
    for dt, bk, emb, rec, proj, prev, u in _cases():
        table = numerics.round_bf16(np.tanh(numerics.decode(emb, dt))) if dt == "bf16" else \
            numerics.round_f32(np.tanh(numerics.decode(emb, dt)))
        got = ornn.rnn_draft(mode, dt, bk, emb, np.zeros_like(rec), proj, prev, 1.0, u)
        ref = omarkov.markov_draft(mode, dt, bk, table, proj, prev, 1.0, u)
        assert np.array_equal(got["tokens"], ref["tokens"]), dt
        assert np.array_equal(got["logits"], ref["logits"]), dt


def test_unrounded_recurrence_matches_torch_rnn():
    """Without the storage rounding, the states are an Elman RNN with tanh,
    input weights the identity and no biases: torch.nn.RNN in float64."""
    for dt, bk, emb, rec, proj, prev, u in _cases():
        R, k, V = bk.shape
        d_m = emb.shape[1]
        g = np.random.Generator(np.random.Philox(17))
        toks = g.integers(0, V, size=(R, k))
        ours = ornn.states(emb, rec, toks, dt, round_state=False)
        net = torch.nn.RNN(d_m, d_m, nonlinearity="tanh", bias=False, batch_first=True).double()
        with torch.no_grad():
            net.weight_ih_l0.copy_(torch.eye(d_m, dtype=torch.float64))
            net.weight_hh_l0.copy_(torch.tensor(numerics.decode(rec, dt)))
            x = torch.tensor(numerics.decode(emb, dt)[toks])          # [R, k, d_m]
            ref, _ = net(x)
        assert np.allclose(ours, ref.numpy(), rtol=1e-12, atol=1e-14), dt


def test_state_carries_the_whole_prefix():
    """With the drafted tokens held fixed, the committed token x_{-1} reaches
    position 2 only through the recurrence: it changes the RNN head's logits
    there and leaves the Markov head's unchanged."""
    dt, bk, emb, rec, proj, prev, u = ("bf16",) + _small_bf16(seed=8)
    R, k, V = bk.shape
    fixed = np.random.Generator(np.random.Philox(3)).integers(0, V, size=(R, k))
    other = (prev + 1 + np.arange(R)) % V
    ov_a, ov_b = fixed.copy(), fixed.copy()           # column i: the token before position i
    ov_a[:, 0], ov_b[:, 0] = prev, other
    ra = ornn.rnn_draft("greedy", dt, bk, emb, rec, proj, prev, 1.0, u, prev_override=ov_a)
    rb = ornn.rnn_draft("greedy", dt, bk, emb, rec, proj, other, 1.0, u, prev_override=ov_b)
    ma = omarkov.markov_draft("greedy", dt, bk, emb, proj, prev, 1.0, u, prev_override=ov_a)
    mb = omarkov.markov_draft("greedy", dt, bk, emb, proj, other, 1.0, u, prev_override=ov_b)
    assert np.array_equal(ma["logits"][:, 2], mb["logits"][:, 2])
    assert not np.array_equal(ra["logits"][:, 2], rb["logits"][:, 2])
    # and with A = 0 the RNN head forgets it too
    z = np.zeros_like(rec)
    za = ornn.rnn_draft("greedy", dt, bk, emb, z, proj, prev, 1.0, u, prev_override=ov_a)
    zb = ornn.rnn_draft("greedy", dt, bk, emb, z, proj, other, 1.0, u, prev_override=ov_b)
    assert np.array_equal(za["logits"][:, 2], zb["logits"][:, 2])


def test_state_override_with_own_states_is_identity():
    for dt, bk, emb, rec, proj, prev, u in _cases():
        a = ornn.rnn_draft("sample", dt, bk, emb, rec, proj, prev, 1.0, u)
        b = ornn.rnn_draft("sample", dt, bk, emb, rec, proj, prev, 1.0, u, prev_override=np.concatenate(
            [np.asarray(prev)[:, None], a["tokens"][:, :-1]], axis=1), state_override=a["states"])
        assert np.array_equal(a["tokens"], b["tokens"]) and np.array_equal(a["logits"], b["logits"])
