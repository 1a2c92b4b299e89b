"""Lagged scheduling (spec_verify_ex) and its HIP graph, checked against the
plain sequential path and the oracle's schedule.

The lengths of round t come from the confidences of round t - 2; round t+1's
schedule runs inside round t's verify launches. Every round must give exactly
what a sequential schedule-then-verify of the same inputs gives (same
kernels, so bit for bit), and the lengths must match the oracle's schedule of
the lagged confidences. A captured run of rounds is replayed several times,
with eager work between the replays, and every replay is compared with the
eager results. A job too large for one workgroup, or with fixed lengths, is
launched after the decisions instead; its results must equal spec_schedule's.
"""
import numpy as np
import pytest
import torch

from draft_token_verification_flattened_amd import binding as B
from draft_token_verification_flattened_amd import workloads
from draft_token_verification_flattened_amd.pipeline import DeviceStep, LaggedStep, to_device
from oracle import schedule as osched

pytestmark = pytest.mark.gpu

ROUNDS = 6


def _sequential(d, z_t, mode):
    """Schedule from z_t, then verify, one after the other on one stream."""
    w = d.w
    R, k = w.R, w.k
    i32 = dict(dtype=torch.int32, device="cuda")
    L = torch.zeros(R, **i32)
    tags = torch.zeros(R * (k + 1), 2, **i32)
    cu = torch.zeros(R + 1, **i32)
    nr = torch.zeros(1, **i32)
    B.spec_schedule(z_t, d.T, d.tbl_b, d.tbl_t, k, L, tags, cu, nr, d.ws_sched)
    acc = torch.zeros(R, **i32)
    out = torch.zeros(R, k + 1, **i32)
    dl, tk = d.drafts(mode)
    B.spec_verify(mode, d.target, dl, tk, tags, cu, nr, w.tau, d.u_verify, acc, out, d.ws_verify)
    torch.cuda.synchronize()
    return L.cpu().numpy(), acc.cpu().numpy(), out.cpu().numpy()


@pytest.fixture(scope="module")
def setup():
    w = workloads.make("c1")
    d = DeviceStep(w)
    zr = workloads.conf_rounds(w, ROUNDS)
    return w, d, zr, to_device(zr, "cuda")


@pytest.mark.parametrize("mode", [B.SAMPLE, B.GREEDY])
def test_lagged_rounds_match_sequential(setup, mode):
    w, d, zr, zdev = setup
    print(f"[gpu] lagged eager rounds, mode {mode}", flush=True)
    ls = LaggedStep(d, zdev)
    ls.start(0)
    got = []
    for t in range(ROUNDS):
        ls.step(mode)
        s = t % 2
        torch.cuda.synchronize()
        got.append((ls.lengths[s].cpu().numpy(), ls.acc_len[s].cpu().numpy(), ls.out_tokens[s].cpu().numpy()))
        # the side stream may still be scheduling round t+1 into the other slot; fine
    torch.cuda.synchronize()
    for t in range(ROUNDS):
        zt = zdev[(t - 2) % ROUNDS]
        L, acc, out = _sequential(d, zt, mode)
        ref = osched.schedule(zr[(t - 2) % ROUNDS], w.pos_temp, w.tbl_tokens, w.tbl_thr, w.k)
        assert np.array_equal(got[t][0], ref["L"]), t
        assert np.array_equal(got[t][0], L), t
        assert np.array_equal(got[t][1], acc), t
        assert np.array_equal(got[t][2], out), t


def test_lagged_graph_replays(setup):
    w, d, zr, zdev = setup
    mode = B.SAMPLE
    print("[gpu] lagged graph capture and replays", flush=True)
    ls = LaggedStep(d, zdev)
    ls.start(0)
    eager = []
    for t in range(2):
        ls.step(mode)
        torch.cuda.synchronize()
        eager.append((ls.acc_len[t % 2].clone(), ls.out_tokens[t % 2].clone()))
    # capture rounds 0 and 1 again (the schedule of round 0 must be in place)
    ls.start(0)
    torch.cuda.synchronize()
    g = ls.capture(mode, 2)
    for rep in range(3):
        ls.start(0)                              # round 0's schedule, eager
        g.replay()
        torch.cuda.synchronize()
        for t in range(2):
            assert torch.equal(ls.acc_len[t % 2], eager[t][0]), (rep, t)
            assert torch.equal(ls.out_tokens[t % 2], eager[t][1]), (rep, t)
        _sequential(d, zdev[3], B.GREEDY)         # eager work between replays


@pytest.mark.parametrize("R,k,max_len", [(2048, 8, 8), (64, 5, -1), (64, 5, 0), (3, 5, 2)])
def test_verify_ex_job_matches_schedule(setup, R, k, max_len):
    w, d, zr, zdev = setup
    print(f"[gpu] spec_verify_ex job R={R} k={k} max_len={max_len}", flush=True)
    g = np.random.Generator(np.random.Philox(R * 31 + k))
    z = to_device((g.standard_normal((R, k)) * 1.5 + 1).astype(np.float32), "cuda")
    T = to_device(np.linspace(1, 2, k).astype(np.float32), "cuda")
    pts = np.array([max(1, R // 2), R, 2 * R, 4 * R, 8 * R, 33 * R], np.int32)
    thr = np.array([p / (1.0 + 0.6 * max(0, p - R) / R) for p in pts])
    tb, tt = to_device(pts, "cuda"), to_device(thr, "cuda")
    i32 = dict(dtype=torch.int32, device="cuda")
    outs = []
    for use_ex in (False, True):
        L = torch.zeros(R, **i32)
        tags = torch.zeros(R * (k + 1), 2, **i32)
        cu = torch.zeros(R + 1, **i32)
        nr = torch.zeros(1, **i32)
        sv = torch.zeros(R, k, dtype=torch.float64, device="cuda")
        ws = B.workspace(B.schedule_workspace_bytes(R, k), "cuda")
        if use_ex:
            job = B.schedule_job(z, T, tb, tt, max_len, L, tags, cu, nr, ws, sv)
            d.schedule(w.k)
            d.verify(B.SAMPLE)
            torch.cuda.synchronize()
            ref_acc, ref_out = d.host("acc_len"), d.host("out_tokens")
            dl, tk = d.drafts(B.SAMPLE)
            B.spec_verify(B.SAMPLE, d.target, dl, tk, d.tags, d.cu_rows, d.n_rows, w.tau, d.u_verify, d.acc_len,
                          d.out_tokens, d.ws_verify, next_job=job)
            torch.cuda.synchronize()
            assert np.array_equal(d.host("acc_len"), ref_acc)
            assert np.array_equal(d.host("out_tokens"), ref_out)
        else:
            B.spec_schedule(z, T, tb, tt, max_len, L, tags, cu, nr, ws, sv)
            torch.cuda.synchronize()
        outs.append([x.cpu().numpy() for x in (L, tags, cu, nr, sv)])
    for a, b in zip(outs[0], outs[1]):
        assert np.array_equal(a, b)
