"""rnn_draft (the RNN head) against the float64 oracle's own run.

The oracle (oracle.rnn.rnn_draft) runs the head on its own draws with the same
uniforms; it never takes a GPU output. Position by position, over the requests
whose tokens have agreed so far:

  state   h_i = round(tanh(E[x_{i-1}] + A h_{i-1})). The kernel accumulates
          d_m + 1 terms in float32 (error at most (d_m + 1) u m, u = 2^-24,
          m = |E| + sum |A h|) and evaluates tanh in float32 (within 4 ulp here,
          2^-21 relative). It starts from its own h_{i-1}, which may differ from
          the oracle's by rounding; tanh has slope at most 1, so that moves the
          exact value by at most |A| dh, dh = |h_{i-1} - h'_{i-1}| measured at
          the previous position. The stored value must lie within the sum of
          these plus half a storage spacing of the oracle's exact value.
  logits  dl_i = round(bk_i + h_i . P^T): within (d_m + 2) u (|bk| + sum |h P|)
          + |P| dh_i plus half a spacing of the oracle's exact value.
  tokens  equal to the oracle's; where the two logit rows are identical, a
          sampled token may differ only inside the oracle's near set
          (oracle.verify.draw_rows); where they differ by rounding, inside the
          near set widened by the L1 distance of the two distributions
          (sampling), or within the rows' differences of the maximum (greedy).
          A request whose token differed leaves the comparison.
"""
import numpy as np
import pytest
import torch

from draft_token_verification_flattened_amd import binding as B
from draft_token_verification_flattened_amd import workloads
from draft_token_verification_flattened_amd.pipeline import to_device
from oracle import numerics
from oracle import rnn as ornn
from oracle import verify as overify

import parity_log

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


def say(*a):
    print("[gpu]", *a, flush=True)


def _spacing(x, dtype):
    e = np.floor(np.log2(np.maximum(np.abs(x), 1e-300)))
    return 2.0 ** (e - (7 if dtype == "bf16" else 23))


def _softmax_rows(x, tau):
    a = x / tau
    a = a - a.max(axis=1, keepdims=True)
    e = np.exp(a)
    return e / e.sum(axis=1, keepdims=True)


def _gpu_rnn(mode, bk, emb, rec, proj, prev, tau, u, keep_state=True, seed=0, step=0):
    R, k, V = bk.shape
    d_m = emb.shape[1]
    dev = "cuda"
    tb = to_device(bk, dev)
    toks = torch.zeros(R, k, dtype=torch.int32, device=dev)
    logits = torch.zeros(R, k, V, dtype=tb.dtype, device=dev)
    st = torch.zeros(R, k, d_m, dtype=tb.dtype, device=dev) if keep_state else None
    ws = B.workspace(B.rnn_workspace_bytes(R, k, V, d_m), dev)
    B.rnn_draft(B.SAMPLE if mode == "sample" else B.GREEDY, tb, to_device(emb, dev), to_device(rec, dev),
                to_device(proj, dev), to_device(prev, dev), tau, None if u is None else to_device(u, dev), toks,
                logits, ws, state_out=st, seed=seed, step=step)
    torch.cuda.synchronize()

    def host(t):
        a = t.cpu().numpy()
        return a.view(np.uint16) if a.dtype == np.int16 else a
    return host(toks), host(logits), (host(st) if st is not None else None), B.read_status(ws)


def check_rnn(dtype, mode, tau, bk, emb, rec, proj, prev0, ref, gt, gl, gs, case):
    R, k, V = gl.shape
    d_m = emb.shape[1]
    E, A, P = (numerics.decode(x, dtype) for x in (emb, rec, proj))
    absA, absP = np.abs(A), np.abs(P)
    alive = np.ones(R, dtype=bool)
    dh = np.zeros((R, d_m))
    worst_s = worst_l = 0.0
    n_pos = n_state_diff = n_logit_diff = n_tok = n_near = 0
    for i in range(k):
        rows = np.nonzero(alive)[0]
        if len(rows) == 0:
            break
        n_pos += len(rows)
        prev = prev0[rows] if i == 0 else ref["tokens"][rows, i - 1]
        ho_prev = np.zeros((len(rows), d_m)) if i == 0 else numerics.decode(ref["states"][rows, i - 1], dtype)
        hg_prev = np.zeros((len(rows), d_m)) if i == 0 else numerics.decode(gs[rows, i - 1], dtype)
        # state
        exact = np.tanh(E[prev] + ho_prev @ A.T)
        m = np.abs(E[prev]) + np.abs(hg_prev) @ absA.T
        eps = (d_m + 1) * U * m + 2.0 ** -21 * np.abs(exact) + dh[rows] @ absA.T + 1e-30
        h = numerics.decode(gs[rows, i], dtype)
        allowed = eps + 0.5 * _spacing(np.abs(exact) + eps, dtype)
        err = np.abs(h - exact)
        worst_s = max(worst_s, float(np.max(err / allowed)))
        assert np.all(err <= allowed), ("state", i, float(np.max(err / allowed)))
        ho = numerics.decode(ref["states"][rows, i], dtype)
        dh[rows] = np.abs(h - ho)
        n_state_diff += int((h != ho).sum())
        # logits
        ex = numerics.decode(bk[rows, i], dtype) + ho @ P.T
        mag = np.abs(numerics.decode(bk[rows, i], dtype)) + np.abs(h) @ absP.T
        delta = (d_m + 2) * U * mag + dh[rows] @ absP.T
        g = numerics.decode(gl[rows, i], dtype)
        o = numerics.decode(ref["logits"][rows, i], dtype)
        allowed = delta + 0.5 * _spacing(np.maximum(np.abs(g), np.abs(ex)) + delta, dtype)
        err = np.abs(g - ex)
        worst_l = max(worst_l, float(np.max(err / allowed)))
        assert np.all(err <= allowed), ("logits", i, float(np.max(err / allowed)))
        rowdiff = np.any(g != o, axis=1)
        n_logit_diff += int((g != o).sum())
        # tokens
        diff = np.nonzero(gt[rows, i] != ref["tokens"][rows, i])[0]
        for n in diff:
            r = rows[n]
            a, b = int(gt[r, i]), int(ref["tokens"][r, i])
            if mode == "greedy":
                assert rowdiff[n], ("token", r, i)
                dd = np.abs(g[n] - o[n])
                assert o[n, b] - o[n, a] <= dd[a] + dd[b], ("token", r, i)
            elif not rowdiff[n]:
                assert a in ref["draw_near"][r][i], ("token", r, i, a, b)
                n_near += 1
            else:
                l1 = np.abs(_softmax_rows(g[n:n + 1], tau) - _softmax_rows(o[n:n + 1], tau)).sum()
                _, nb = overify.draw_rows(_softmax_rows(o[n:n + 1], tau), np.array([ref["u_draft"][r, i]]),
                                          l1 + overify.DRAW_EPS)
                assert a in nb[0], ("token", r, i, a, b, l1)
        n_tok += len(diff)
        alive[rows[diff]] = False
    assert n_near <= max(2, int(0.02 * n_pos)), (n_near, n_pos)
    rec = parity_log.record("rnn", case, positions=n_pos, state_diffs=n_state_diff, logit_diffs=n_logit_diff,
                            token_diffs=n_tok, token_diffs_same_row=n_near, worst_state_over_bound=worst_s,
                            worst_logit_over_bound=worst_l, requests_whole_block=int(alive.sum()))
    say("parity", rec)
    return rec


@pytest.mark.parametrize("mode", ["greedy", "sample"])
def test_rnn_c0(mode):
    w = workloads.make("c0")
    say("rnn c0", mode)
    gt, gl, gs, st = _gpu_rnn(mode, w.backbone, w.emb, w.rec, w.proj, w.prev_token, w.tau, w.u_draft)
    assert st == 0
    ref = ornn.rnn_draft(mode, "f32", w.backbone, w.emb, w.rec, w.proj, w.prev_token, w.tau, w.u_draft,
                         near_eps=overify.DRAW_EPS)
    check_rnn("f32", mode, w.tau, w.backbone, w.emb, w.rec, w.proj, w.prev_token, ref, gt, gl, gs, f"c0 {mode}")


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
    ref = ornn.rnn_draft(mode, "bf16", bk, emb, rec, proj, prev, 1.0, u, near_eps=overify.DRAW_EPS)
    check_rnn("bf16", mode, 1.0, bk, emb, rec, proj, prev, ref, gt, gl, gs, f"R={R} k={k} V={V} d_m={d_m} {mode}")
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


def test_rnn_c4():
    """R = 512, k = 5, V = 151936, d_m = 256, bf16 (the semi-autoregressive
    workload with the RNN head), every request, uniforms from the library's
    generator (seed 7) against the oracle's."""
    w = workloads.make("c4")
    say("rnn c4 sample, Philox seed 7")
    gt, gl, gs, st = _gpu_rnn("sample", w.backbone, w.emb, w.rec, w.proj, w.prev_token, w.tau, None, seed=7, step=1)
    assert st == 0
    ref = ornn.rnn_draft("sample", "bf16", w.backbone, w.emb, w.rec, w.proj, w.prev_token, w.tau, rng=(7, 1),
                         near_eps=overify.DRAW_EPS)
    rec = check_rnn("bf16", "sample", w.tau, w.backbone, w.emb, w.rec, w.proj, w.prev_token, ref, gt, gl, gs,
                    "c4 philox")
    assert rec["positions"] >= w.R
