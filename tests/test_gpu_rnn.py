"""rnn_draft (the RNN head) against the float64 oracle, stage by stage.

At every position the oracle takes the kernel's own inputs of that stage (the
previous token drawn and the previous state stored by the GPU), so that a
rounding difference at one position does not make every later one differ:

  state   h_i = round(tanh(E[x_{i-1}] + A h_{i-1})). The kernel accumulates
          d_m + 1 terms in float32 (error at most (d_m + 1) u m, u = 2^-24,
          m = |E| + sum |A h|; tanh has slope at most 1) and evaluates tanh in
          float32 (within 4 ulp here, 2^-21 relative); the stored value must lie
          within that plus half a storage spacing of the exact value.
  logits  dl_i = round(bk_i + h_i . P^T) with the kernel's h_i: within
          (d_m + 2) u (|bk| + sum |h P|) plus half a spacing, as the Markov head.
  tokens  the oracle's draw from the kernel's stored logits must give the
          kernel's token (sampling: unless within 1e-5 of a CDF boundary).

The whole trajectory is also compared with the oracle's own run and the share
of positions that agree is printed.
"""
import numpy as np
import pytest
import torch

from draft_token_verification_flattened_amd import binding as B
from draft_token_verification_flattened_amd import workloads
from draft_token_verification_flattened_amd.pipeline import to_device
from oracle import markov as omarkov
from oracle import numerics
from oracle import rnn as ornn

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


def say(*a):
    print("[gpu]", *a, flush=True)


def _spacing(x, dtype):
    e = np.floor(np.log2(np.maximum(np.abs(x), 1e-300)))
    return 2.0 ** (e - (7 if dtype == "bf16" else 23))


def _gpu_rnn(mode, bk, emb, rec, proj, prev, tau, u, keep_state=True):
    R, k, V = bk.shape
    d_m = emb.shape[1]
    dev = "cuda"
    tb = to_device(bk, dev)
    toks = torch.zeros(R, k, dtype=torch.int32, device=dev)
    logits = torch.zeros(R, k, V, dtype=tb.dtype, device=dev)
    st = torch.zeros(R, k, d_m, dtype=tb.dtype, device=dev) if keep_state else None
    ws = B.workspace(B.rnn_workspace_bytes(R, k, V, d_m), dev)
    B.rnn_draft(B.SAMPLE if mode == "sample" else B.GREEDY, tb, to_device(emb, dev), to_device(rec, dev),
                to_device(proj, dev), to_device(prev, dev), tau, to_device(u, dev), toks, logits, ws, state_out=st)
    torch.cuda.synchronize()

    def host(t):
        a = t.cpu().numpy()
        return a.view(np.uint16) if a.dtype == np.int16 else a
    return host(toks), host(logits), (host(st) if st is not None else None), B.read_status(ws)


def check_rnn(dtype, mode, tau, bk, emb, rec, proj, prev0, u, gt, gl, gs, rows=None):
    R, k, V = gl.shape
    d_m = emb.shape[1]
    rows = np.arange(R) if rows is None else np.asarray(rows)
    E, A, P = (numerics.decode(x, dtype) for x in (emb, rec, proj))
    worst_s = worst_l = 0.0
    for i in range(k):
        prev = prev0[rows] if i == 0 else gt[rows, i - 1]
        hp = np.zeros((len(rows), d_m)) if i == 0 else numerics.decode(gs[rows, i - 1], dtype)
        # state
        pre = E[prev] + hp @ A.T
        exact = np.tanh(pre)
        m = np.abs(E[prev]) + np.abs(hp) @ np.abs(A).T
        eps = (d_m + 1) * U * m + 2.0 ** -21 * np.abs(exact) + 1e-30
        h = numerics.decode(gs[rows, i], dtype)
        allowed = eps + 0.5 * _spacing(np.abs(exact) + eps, dtype)
        err = np.abs(h - exact)
        worst_s = max(worst_s, float(np.max(err / allowed)))
        assert np.all(err <= allowed), ("state", i, float(np.max(err / allowed)))
        # logits, with the kernel's state
        ex = numerics.decode(bk[rows, i], dtype) + h @ P.T
        mag = np.abs(numerics.decode(bk[rows, i], dtype)) + np.abs(h) @ np.abs(P).T
        delta = (d_m + 2) * U * mag
        g = numerics.decode(gl[rows, i], dtype)
        allowed = delta + 0.5 * _spacing(np.maximum(np.abs(g), np.abs(ex)) + delta, dtype)
        err = np.abs(g - ex)
        worst_l = max(worst_l, float(np.max(err / allowed)))
        assert np.all(err <= allowed), ("logits", i, float(np.max(err / allowed)))
        # token, from the kernel's logits
        xo, margin = omarkov.draw_position(gl[rows, i], dtype, mode, tau, u[rows, i])
        bad = np.nonzero(xo != gt[rows, i])[0]
        for n in bad:
            assert mode == "sample" and margin[n] < 1e-5, ("token", int(rows[n]), i)
    say(f"rnn: worst state error / bound {worst_s:.3f}, logits {worst_l:.3f}")


def _trajectory_agreement(gt, ref_tokens):
    same = np.cumprod(gt == ref_tokens, axis=1).astype(bool)
    return float(same.mean())


@pytest.mark.parametrize("mode", ["greedy", "sample"])
def test_rnn_c0(mode):
    w = workloads.make("c0")
    say("rnn c0", mode)
    gt, gl, gs, st = _gpu_rnn(mode, w.backbone, w.emb, w.rec, w.proj, w.prev_token, w.tau, w.u_draft)
    assert st == 0
    check_rnn("f32", mode, w.tau, w.backbone, w.emb, w.rec, w.proj, w.prev_token, w.u_draft, gt, gl, gs)
    ref = ornn.rnn_draft(mode, "f32", w.backbone, w.emb, w.rec, w.proj, w.prev_token, w.tau, w.u_draft)
    say("rnn c0 trajectory agreement", _trajectory_agreement(gt, ref["tokens"]))


RNN_SMALL = [
    # R, k, V, d_m, mode
    (16, 2, 64, 32, "greedy"),        # one MFMA tile
    (70, 3, 1000, 64, "sample"),      # partial request block, V % 64 != 0
    (130, 2, 1001, 96, "greedy"),     # ragged V: scalar epilogue
    (64, 5, 5000, 256, "sample"),
    (33, 6, 700, 480, "sample"),      # largest bf16 d_m
]


@pytest.mark.parametrize("R,k,V,d_m,mode", RNN_SMALL)
def test_rnn_bf16_small(R, k, V, d_m, mode):
    g = np.random.Generator(np.random.Philox(R + V + 7))
    enc = workloads.f32_to_bf16_bits
    bk = enc((3 * g.standard_normal((R, k, V))).astype(np.float32))
    emb = enc(g.standard_normal((V, d_m)).astype(np.float32))
    rec = enc((0.5 / np.sqrt(d_m) * g.standard_normal((d_m, d_m))).astype(np.float32))
    proj = enc((0.5 / np.sqrt(d_m) * g.standard_normal((V, d_m))).astype(np.float32))
    prev = g.integers(0, V, size=R).astype(np.int32)
    u = (g.integers(0, 1 << 24, size=(R, k)) * 2.0 ** -24).astype(np.float32)
    say("rnn bf16", R, k, V, d_m, mode)
    gt, gl, gs, st = _gpu_rnn(mode, bk, emb, rec, proj, prev, 1.0, u)
    assert st == 0
    check_rnn("bf16", mode, 1.0, bk, emb, rec, proj, prev, u, gt, gl, gs)
    ref = ornn.rnn_draft(mode, "bf16", bk, emb, rec, proj, prev, 1.0, u)
    say("rnn bf16 trajectory agreement", _trajectory_agreement(gt, ref["tokens"]))
    # without state_out the states live in the workspace: same tokens and logits
    gt2, gl2, _, _ = _gpu_rnn(mode, bk, emb, rec, proj, prev, 1.0, u, keep_state=False)
    assert np.array_equal(gt2, gt) and np.array_equal(gl2, gl)


def test_rnn_zero_recurrence_equals_markov_on_tanh_table():
    """A = 0 through the GPU: the same tokens and logits as markov_draft run on
    the table round(tanh(E)) (the oracle's pin, here between two entry points)."""
    R, k, V, d_m = 40, 4, 3000, 64
    g = np.random.Generator(np.random.Philox(77))
    enc = workloads.f32_to_bf16_bits
    bk = enc((3 * g.standard_normal((R, k, V))).astype(np.float32))
    emb = enc(g.standard_normal((V, d_m)).astype(np.float32))
    proj = enc((0.5 / np.sqrt(d_m) * g.standard_normal((V, d_m))).astype(np.float32))
    prev = g.integers(0, V, size=R).astype(np.int32)
    u = (g.integers(0, 1 << 24, size=(R, k)) * 2.0 ** -24).astype(np.float32)
    table = numerics.round_bf16(np.tanh(numerics.decode(emb, "bf16")))
    say("rnn A=0 vs markov")
    gt, gl, gs, _ = _gpu_rnn("sample", bk, emb, np.zeros((d_m, d_m), np.uint16), proj, prev, 1.0, u)
    dev = "cuda"
    toks = torch.zeros(R, k, dtype=torch.int32, device=dev)
    logits = torch.zeros(R, k, V, dtype=torch.int16, device=dev)
    ws = B.workspace(B.markov_workspace_bytes(R, k, V, d_m), dev)
    B.markov_draft(B.SAMPLE, to_device(bk, dev), to_device(table, dev), to_device(proj, dev), to_device(prev, dev),
                   1.0, to_device(u, dev), toks, logits, ws)
    torch.cuda.synchronize()
    mt, ml = toks.cpu().numpy(), logits.cpu().numpy().view(np.uint16)
    # Where the kernel's states equal the exact table rows of the tokens it
    # drew (its float32 tanh may round an element differently), the two entry
    # points run the same projection on the same operands: identical bits.
    prevs = np.concatenate([prev[:, None], gt[:, :-1]], axis=1)
    same_state = np.all(gs == table[prevs], axis=(1, 2))
    assert same_state.sum() > 0
    for r in np.nonzero(same_state)[0]:
        assert np.array_equal(gt[r], mt[r]) and np.array_equal(gl[r], ml[r]), r
    say("rnn A=0: requests whose states match the table and equal the Markov head", int(same_state.sum()), "of", R)


def test_rnn_c4_sampled():
    """R = 512, k = 5, V = 151936, d_m = 256, bf16 (the semi-autoregressive
    workload with the RNN head): every stage checked on 24 sampled requests."""
    w = workloads.make("c4")
    say("rnn c4 sample")
    gt, gl, gs, st = _gpu_rnn("sample", w.backbone, w.emb, w.rec, w.proj, w.prev_token, w.tau, w.u_draft)
    assert st == 0
    rows = np.random.Generator(np.random.Philox(4)).choice(w.R, 24, replace=False)
    check_rnn("bf16", "sample", w.tau, w.backbone, w.emb, w.rec, w.proj, w.prev_token, w.u_draft, gt, gl, gs, rows)
