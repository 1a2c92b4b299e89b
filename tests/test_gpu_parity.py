"""GPU parity: libspecv (HIP, gfx950) against the CPU oracle, stage by stage.

Tolerances:
  greedy        accepted lengths, emitted tokens, per-row argmax: bit-exact.
  scheduler     lengths, offsets and tags: bit-exact; survival within 1e-14
                relative (device and host exp may differ in the last bit).
  sampling      p(x), q(x), p/q within 1e-5 relative (fp32 accumulation over
                the vocabulary); keep decisions identical except where
                |u - p/q| < 1e-6 (counted); resampled / bonus tokens identical
                except where the oracle's draw is within 1e-5 * W of a CDF
                boundary (counted).
  Markov head   stored logits within the float32 accumulation bound plus half
                a storage spacing of the exact value (check_markov); tokens
                identical except where rounding differences can move them.
Inputs flow one way only: the oracle never consumes a GPU output. Where a later
stage needs an earlier one (tags, draft logits), the GPU is fed the oracle's.
"""
import numpy as np
import pytest
import torch

from draft_token_verification_flattened_amd import binding as B
from draft_token_verification_flattened_amd import workloads
from draft_token_verification_flattened_amd.pipeline import DeviceStep, to_device
from oracle import markov as omarkov
from oracle import numerics
from oracle import schedule as osched
from oracle import verify as overify

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

_W, _DEV = {}, {}


def W(name):
    if name not in _W:
        _W[name] = workloads.make(name)
    return _W[name]


def D(name):
    if name not in _DEV:
        _DEV[name] = DeviceStep(W(name))
    return _DEV[name]


def say(*a):
    print("[gpu]", *a, flush=True)


def ref_schedule(w, max_len):
    return osched.schedule(w.conf_logit, w.pos_temp, w.tbl_tokens, w.tbl_thr, max_len)


_MK = {}


def ref_markov(name, mode):
    key = (name, mode)
    if key not in _MK:
        w = W(name)
        _MK[key] = omarkov.markov_draft(mode, w.dtype, w.backbone, w.emb, w.proj, w.prev_token, w.tau, w.u_draft)
    return _MK[key]


def drafts_for(name, mode):
    """(host draft logits, host tokens) the oracle uses; the GPU gets the same."""
    w = W(name)
    if w.backbone is not None:
        m = ref_markov(name, mode)
        return m["logits"], m["tokens"]
    return w.draft, (w.tokens_sample if mode == "sample" else w.tokens_greedy)


# ---------------------------------------------------------------------------
# scheduler
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["c0", "c1", "c2", "c3", "c4"])
@pytest.mark.parametrize("max_len", [None, -1, 0, 2])
def test_schedule_bit_exact(name, max_len):
    w = W(name)
    ml = w.k if max_len is None else max_len
    d = D(name)
    say("schedule", name, "max_len", ml)
    d.schedule(ml)
    torch.cuda.synchronize()
    ref = ref_schedule(w, ml)
    L = d.host("lengths")
    assert np.array_equal(L, ref["L"]), (L, ref["L"])
    tags, cu = osched.flatten(ref["L"])
    assert np.array_equal(d.host("cu_rows"), cu)
    assert int(d.host("n_rows")[0]) == osched.n_rows(cu)
    assert np.array_equal(d.host("tags")[:osched.n_rows(cu)], tags)
    S = d.host("survival")
    assert np.max(np.abs(S - ref["S"]) / ref["S"]) < 1e-14


@pytest.mark.parametrize("R,k", [(2048, 8), (16384, 1), (512, 32), (1, 5)])
def test_schedule_limits(R, k):
    g = np.random.Generator(np.random.Philox(R * 100 + k))
    z = (g.standard_normal((R, k)) * 1.5 + 1).astype(np.float32)
    T = np.linspace(1, 2, k).astype(np.float32)
    pts = np.array([max(1, R // 2), R, 2 * R, 4 * R, 8 * R, 33 * R], np.int32)
    thr = np.array([p / (1.0 + 0.6 * max(0, p - R) / R) for p in pts])
    say("schedule limits R", R, "k", k)
    dev = lambda a: to_device(a, "cuda")   # noqa: E731
    L = torch.zeros(R, dtype=torch.int32, device="cuda")
    tags = torch.zeros(R * (k + 1), 2, dtype=torch.int32, device="cuda")
    cu = torch.zeros(R + 1, dtype=torch.int32, device="cuda")
    nr = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = B.workspace(B.schedule_workspace_bytes(R, k), "cuda")
    B.spec_schedule(dev(z), dev(T), dev(pts), dev(thr), k, L, tags, cu, nr, ws)
    torch.cuda.synchronize()
    ref = osched.schedule(z, T, pts, thr, k)
    assert np.array_equal(L.cpu().numpy(), ref["L"])
    rt, rc = osched.flatten(ref["L"])
    assert np.array_equal(cu.cpu().numpy(), rc)
    assert np.array_equal(tags.cpu().numpy()[:osched.n_rows(rc)], rt)


@pytest.mark.parametrize("R,k", [(512, 8), (683, 6), (3, 5)])
@pytest.mark.parametrize("pattern", ["equal", "saturated", "few", "decay", "vanishing"])
def test_schedule_ties(R, k, pattern):
    """Heavy ties in Q: identical confidences in every request ("equal"), all
    survivals 1.0 ("saturated"), or confidences from four values ("few");
    survivals falling through many octaves below 1/4 ("decay"), and survivals
    that quantise to Q = 0 ("vanishing"). R*k = 4096 and 4098 sit on both sides
    of the single-workgroup size limit."""
    g = np.random.Generator(np.random.Philox(R * 7 + k))
    if pattern == "equal":
        z = np.tile((g.standard_normal(k) + 1.5).astype(np.float32), (R, 1))
    elif pattern == "saturated":
        z = np.full((R, k), 60.0, np.float32)
    elif pattern == "decay":
        z = (np.linspace(3.0, -9.0, k)[None, :] + 0.5 * g.standard_normal((R, k))).astype(np.float32)
    elif pattern == "vanishing":
        z = np.full((R, k), -60.0, np.float32)
    else:
        z = g.choice(np.array([-1.0, 0.5, 1.0, 2.0], np.float32), size=(R, k))
    T = np.linspace(1, 2, k).astype(np.float32)
    pts = np.array([max(1, R // 2), R, 2 * R, 4 * R, 8 * R, 33 * R], np.int32)
    thr = np.array([p / (1.0 + 0.6 * max(0, p - R) / R) for p in pts])
    say("schedule ties R", R, "k", k, pattern)
    dev = lambda a: to_device(a, "cuda")   # noqa: E731
    L = torch.zeros(R, dtype=torch.int32, device="cuda")
    tags = torch.zeros(R * (k + 1), 2, dtype=torch.int32, device="cuda")
    cu = torch.zeros(R + 1, dtype=torch.int32, device="cuda")
    nr = torch.zeros(1, dtype=torch.int32, device="cuda")
    surv = torch.zeros(R, k, dtype=torch.float64, device="cuda")
    ws = B.workspace(B.schedule_workspace_bytes(R, k), "cuda")
    for ml in (k, max(1, k // 2)):
        B.spec_schedule(dev(z), dev(T), dev(pts), dev(thr), ml, L, tags, cu, nr, ws, survival_out=surv)
        torch.cuda.synchronize()
        ref = osched.schedule(z, T, pts, thr, ml)
        assert np.array_equal(L.cpu().numpy(), ref["L"]), (pattern, ml)
        rt, rc = osched.flatten(ref["L"])
        assert np.array_equal(cu.cpu().numpy(), rc)
        assert np.array_equal(tags.cpu().numpy()[:osched.n_rows(rc)], rt)
        assert np.max(np.abs(surv.cpu().numpy() - ref["S"]) / ref["S"]) < 1e-14


def test_flatten_matches_oracle():
    g = np.random.Generator(np.random.Philox(5))
    for R, k in [(1, 1), (7, 5), (100000, 4)]:
        Ls = g.integers(-1, k + 2, size=R).astype(np.int32)     # out of range values are clamped
        say("flatten R", R, "k", k)
        tags = torch.zeros(R * (k + 1), 2, dtype=torch.int32, device="cuda")
        cu = torch.zeros(R + 1, dtype=torch.int32, device="cuda")
        nr = torch.zeros(1, dtype=torch.int32, device="cuda")
        B.spec_flatten(to_device(Ls, "cuda"), k, tags, cu, nr)
        torch.cuda.synchronize()
        rt, rc = osched.flatten(np.clip(Ls, 0, k))
        assert np.array_equal(cu.cpu().numpy(), rc)
        assert int(nr.item()) == osched.n_rows(rc)
        assert np.array_equal(tags.cpu().numpy()[:osched.n_rows(rc)], rt)


# ---------------------------------------------------------------------------
# verification
# ---------------------------------------------------------------------------

def _run_verify(name, mode, max_len):
    """GPU verify on the oracle's flattening and the oracle's drafts."""
    w = W(name)
    d = D(name)
    ref_s = ref_schedule(w, max_len)
    tags, cu = osched.flatten(ref_s["L"])
    dl_host, tok_host = drafts_for(name, mode)
    mode_c = B.SAMPLE if mode == "sample" else B.GREEDY
    say("verify", name, mode, "max_len", max_len, "rows", osched.n_rows(cu))
    d.flatten(to_device(ref_s["L"].astype(np.int32), "cuda"))
    d.verify(mode_c, draft=to_device(dl_host, "cuda") if mode == "sample" else None,
             tokens=to_device(tok_host.astype(np.int32), "cuda"))
    torch.cuda.synchronize()
    status = B.read_status(d.ws_verify)
    assert status == 0, status
    ref = overify.verify(mode, w.dtype, w.target, dl_host if mode == "sample" else None, tok_host, tags, cu,
                         w.tau, w.u_verify)
    return d, ref, tags, cu


GREEDY_CASES = [("c0", 5), ("c0", -1), ("c1", 5), ("c2", 5), ("c2", -1), ("c3", 16)]


@pytest.mark.parametrize("name,max_len", GREEDY_CASES)
def test_verify_greedy_bit_exact(name, max_len):
    d, ref, tags, cu = _run_verify(name, "greedy", max_len)
    Bn = osched.n_rows(cu)
    assert np.array_equal(d.host("acc_len"), ref["accepted_len"])
    assert np.array_equal(d.host("out_tokens"), ref["out_tokens"])
    diag = d.host("diag")[:Bn]
    assert np.array_equal(diag[:, 0].astype(np.int64), ref["row_argmax"])


def check_sampling(d, ref, tags, cu, u, tol=1e-5):
    """Sampling-mode parity with near-tie accounting; returns counts."""
    Bn = osched.n_rows(cu)
    diag = d.host("diag")[:Bn].astype(np.float64)
    ver = ref["row_verified"]
    for col, key in [(0, "row_p"), (1, "row_q"), (2, "row_ratio")]:
        g, o = diag[ver, col], ref[key][ver]
        rel = np.abs(g - o) / np.abs(o)
        assert rel.max(initial=0) < tol, (key, rel.max())
    gpu_acc = diag[ver, 3] == 1.0
    ref_acc = ref["row_accept"][ver]
    uu = u[tags[:Bn][ver, 0], tags[:Bn][ver, 1]].astype(np.float64)
    near = np.abs(uu - np.minimum(1.0, ref["row_ratio"][ver])) < 1e-6
    assert np.array_equal(gpu_acc[~near], ref_acc[~near])
    n_near_accept = int((gpu_acc != ref_acc).sum())
    # per request
    R = len(cu) - 1
    row_req = tags[:Bn][ver, 0]
    flip_req = np.zeros(R, dtype=bool)
    flip_req[row_req[near]] = True
    a_g, a_r = d.host("acc_len"), ref["accepted_len"]
    ok = ~flip_req
    assert np.array_equal(a_g[ok], a_r[ok])
    out_g, out_r = d.host("out_tokens"), ref["out_tokens"]
    same = ok & (a_g == a_r)
    near_draw = ref["draw_margin"] < 1e-5
    n_draw_diff = 0
    for r in np.nonzero(same)[0]:
        a = a_r[r]
        assert np.array_equal(out_g[r, :a], out_r[r, :a])
        assert (out_g[r, a + 1:] == -1).all()
        if out_g[r, a] != out_r[r, a]:
            assert near_draw[r], (r, out_g[r, a], out_r[r, a], ref["draw_margin"][r])
            n_draw_diff += 1
    say(f"near-tie accept flips {n_near_accept}, near-boundary draws {n_draw_diff}, "
        f"requests with |u-ratio|<1e-6: {int(flip_req.sum())}")
    return n_near_accept, n_draw_diff


SAMPLE_CASES = [("c0", 5), ("c1", 5), ("c2", 5), ("c2", -1), ("c3", 16), ("c3", -1), ("c4", 5)]


@pytest.mark.parametrize("name,max_len", SAMPLE_CASES)
def test_verify_sampling_within_tolerance(name, max_len):
    w = W(name)
    d, ref, tags, cu = _run_verify(name, "sample", max_len)
    check_sampling(d, ref, tags, cu, w.u_verify)


def test_verify_deterministic():
    d, ref, tags, cu = _run_verify("c2", "sample", -1)
    a1, o1, g1 = d.host("acc_len"), d.host("out_tokens"), d.host("diag")
    say("verify repeat c2")
    d.verify(B.SAMPLE, draft=to_device(W("c2").draft, "cuda"), tokens=to_device(W("c2").tokens_sample, "cuda"))
    torch.cuda.synchronize()
    assert np.array_equal(a1, d.host("acc_len"))
    assert np.array_equal(o1, d.host("out_tokens"))
    assert np.array_equal(g1, d.host("diag"))


# ---------------------------------------------------------------------------
# edge cases on small synthetic inputs
# ---------------------------------------------------------------------------

def _small(R, k, V, dtype, seed, ties=False, scale=3.0):
    g = np.random.Generator(np.random.Philox(seed))
    if ties:
        tl = g.integers(-2, 3, size=(R, k + 1, V)).astype(np.float32)
        dl = g.integers(-2, 3, size=(R, k, V)).astype(np.float32)
    else:
        tl = (scale * g.standard_normal((R, k + 1, V))).astype(np.float32)
        dl = (tl[:, :k] + 1.5 * g.standard_normal((R, k, V))).astype(np.float32)
    if dtype == "bf16":
        tl, dl = workloads.f32_to_bf16_bits(tl), workloads.f32_to_bf16_bits(dl)
    dd = numerics.decode(dl, dtype)
    x = np.argmax(dd + g.gumbel(size=dd.shape), axis=-1).astype(np.int32)
    if ties:
        x = np.where(g.random((R, k)) < 0.5, numerics.argmax_first(numerics.decode(tl[:, :k], dtype)), x)
    u = (g.integers(0, 1 << 24, size=(R, k + 1)) * 2.0 ** -24).astype(np.float32)
    L = g.integers(0, k + 1, size=R).astype(np.int32)
    return tl, dl, x.astype(np.int32), u, L


def _gpu_verify(mode, tl, dl, x, u, L, tau, offset=0):
    R, k1, V = tl.shape
    k = k1 - 1
    dev = "cuda"

    def up(a):
        t = to_device(a, dev)
        if offset:                               # misaligned copy: view into a padded buffer
            big = torch.zeros(t.numel() + offset, dtype=t.dtype, device=dev)
            big[offset:] = t.reshape(-1)
            t = big[offset:].view(t.shape)
        return t

    tags = torch.zeros(R * k1, 2, dtype=torch.int32, device=dev)
    cu = torch.zeros(R + 1, dtype=torch.int32, device=dev)
    nr = torch.zeros(1, dtype=torch.int32, device=dev)
    B.spec_flatten(to_device(L, dev), k, tags, cu, nr)
    acc = torch.zeros(R, dtype=torch.int32, device=dev)
    out = torch.zeros(R, k1, dtype=torch.int32, device=dev)
    diag = torch.zeros(R * k1, 4, dtype=torch.float32, device=dev)
    ws = B.workspace(B.verify_workspace_bytes(mode, R, k, V), dev)
    B.spec_verify(mode, up(tl), up(dl) if mode == B.SAMPLE else None, to_device(x, dev), tags, cu, nr, tau,
                  to_device(u, dev), acc, out, ws, row_diag=diag)
    torch.cuda.synchronize()
    return acc.cpu().numpy(), out.cpu().numpy(), diag.cpu().numpy(), B.read_status(ws)


class _Res:
    def __init__(self, acc, out, diag):
        self.acc_len, self.out_tokens, self.diag = acc, out, diag

    def host(self, n):
        return getattr(self, n)


EDGE = [
    # R, k, V, dtype, ties, offset, tau
    (64, 5, 1000, "bf16", False, 0, 1.0),      # V % 8 == 0, ragged last chunk
    (64, 5, 1001, "bf16", False, 0, 1.0),      # V % 8 != 0: scalar path
    (33, 5, 4096, "bf16", False, 1, 0.7),      # 2-byte misaligned rows: scalar path
    (40, 32, 300, "f32", False, 0, 1.3),       # k = 32
    (50, 4, 5000, "f32", False, 0, 1.0),       # fp32, V % 4 == 0
    (50, 4, 4097, "f32", False, 0, 1.0),       # fp32, ragged
    (300, 3, 64, "bf16", True, 0, 1.0),        # integer logits: many argmax ties
    (1, 5, 151936, "bf16", False, 0, 1.0),     # one request, full vocabulary
]


@pytest.mark.parametrize("R,k,V,dtype,ties,offset,tau", EDGE)
@pytest.mark.parametrize("mode", ["greedy", "sample"])
def test_verify_edges(R, k, V, dtype, ties, offset, tau, mode):
    tl, dl, x, u, L = _small(R, k, V, dtype, seed=R * 7 + V, ties=ties)
    if mode == "greedy":
        x = np.where(np.random.default_rng(1).random((R, k)) < 0.5,
                     numerics.argmax_first(numerics.decode(tl[:, :k], dtype)), x).astype(np.int32)
    say("verify edge", R, k, V, dtype, "ties" if ties else "", "offset", offset, mode)
    mc = B.SAMPLE if mode == "sample" else B.GREEDY
    acc, out, diag, st = _gpu_verify(mc, tl, dl, x, u, L, tau, offset)
    assert st == 0
    tags, cu = osched.flatten(L)
    ref = overify.verify(mode, dtype, tl, dl if mode == "sample" else None, x, tags, cu, tau, u)
    if mode == "greedy":
        assert np.array_equal(acc, ref["accepted_len"])
        assert np.array_equal(out, ref["out_tokens"])
        assert np.array_equal(diag[:osched.n_rows(cu), 0].astype(np.int64), ref["row_argmax"])
    else:
        check_sampling(_Res(acc, out, diag), ref, tags, cu, u)


def test_verify_nothing_scheduled():
    tl, dl, x, u, _ = _small(20, 5, 2048, "bf16", seed=3)
    L = np.zeros(20, np.int32)
    for mode, mc in (("greedy", B.GREEDY), ("sample", B.SAMPLE)):
        say("verify L=0", mode)
        acc, out, diag, st = _gpu_verify(mc, tl, dl, x, u, L, 1.0)
        tags, cu = osched.flatten(L)
        ref = overify.verify(mode, "bf16", tl, dl, x, tags, cu, 1.0, u)
        assert (acc == 0).all()
        assert (out[:, 1:] == -1).all()
        if mode == "greedy":
            assert np.array_equal(out, ref["out_tokens"])


def test_verify_reports_bad_tokens():
    tl, dl, x, u, _ = _small(8, 4, 512, "bf16", seed=4)
    L = np.full(8, 4, np.int32)
    x[2, 1] = 512
    x[5, 0] = -3
    say("verify bad tokens")
    acc, out, diag, st = _gpu_verify(B.SAMPLE, tl, dl, x, u, L, 1.0)
    assert st & B.STATUS_BAD_TOKEN
    assert acc[2] <= 1 and acc[5] == 0


# ---------------------------------------------------------------------------
# Markov head
# ---------------------------------------------------------------------------

def _spacing(a, dtype):
    """Distance between adjacent stored values at magnitude a (bf16: 8
    significant bits, fp32: 24), never below the smallest subnormal step."""
    mant, qmin = (8, -133) if dtype == "bf16" else (24, -149)
    e = np.frexp(np.maximum(np.abs(a), 2.0 ** -140))[1]
    return np.ldexp(1.0, np.maximum(e - mant, qmin))


def _softmax_rows(x, tau):
    a = x / tau
    a = a - a.max(axis=1, keepdims=True)
    e = np.exp(a)
    return e / e.sum(axis=1, keepdims=True)


def check_markov(dtype, gl, gt, ref, u, tau, mode, bk, emb, proj, prev0):
    """Position by position, over requests whose earlier tokens agree.

    Logits: the kernel accumulates d_m products and the backbone value in
    float32 in its own order, then rounds once to the storage type. With
    u = 2**-24 and m = |bk| + sum_d |E[prev, d] * P[v, d]|, the float32 value
    lies within delta = (d_m + 2) * u * m of the exact sum, so the stored value
    must lie within delta + half a storage spacing of it.
    Tokens: with identical rows the draw must agree (sampling: unless the
    oracle's draw is within 1e-5 of a CDF boundary); where rows differ by
    rounding, greedy may pick another token only if the two values are within
    the rows' differences, and sampling only if the oracle's draw margin is
    below the total-variation distance of the two rows' distributions.
    """
    R, k, V = gl.shape
    d_m = emb.shape[1]
    E = numerics.decode(emb, dtype)
    P = numerics.decode(proj, dtype)
    alive = np.ones(R, dtype=bool)
    n_diff_logits = 0
    n_tok_diff = 0
    worst = 0.0
    for i in range(k):
        rows = np.nonzero(alive)[0]
        if len(rows) == 0:
            break
        prev = prev0[rows] if i == 0 else ref["tokens"][rows, i - 1]
        exact = omarkov.head_exact(bk[rows, i], emb, proj, prev, dtype)
        mag = np.abs(numerics.decode(bk[rows, i], dtype)) + np.abs(E[prev]) @ np.abs(P).T
        delta = (d_m + 2) * 2.0 ** -24 * mag
        g = numerics.decode(gl[rows, i], dtype)
        o = numerics.decode(ref["logits"][rows, i], dtype)
        err = np.abs(g - exact)
        allowed = delta + 0.5 * _spacing(np.maximum(np.abs(g), np.abs(exact)) + delta, dtype)
        worst = max(worst, float(np.max(err / allowed)))
        assert np.all(err <= allowed), float(np.max(err / allowed))
        rowdiff = np.any(g != o, axis=1)
        n_diff_logits += int((g != o).sum())
        diff = np.nonzero(gt[rows, i] != ref["tokens"][rows, i])[0]
        for n in diff:
            r = rows[n]
            assert rowdiff[n] or (mode == "sample" and ref["draw_margin"][r, i] < 1e-5), (r, i)
            if mode == "greedy":
                a, b = int(gt[r, i]), int(ref["tokens"][r, i])
                dd = np.abs(g[n] - o[n])
                assert o[n, b] - o[n, a] <= dd[a] + dd[b], (r, i)
            else:
                tv = np.abs(_softmax_rows(g[n:n + 1], tau) - _softmax_rows(o[n:n + 1], tau)).sum()
                assert ref["draw_margin"][r, i] < tv + 1e-5, (r, i, ref["draw_margin"][r, i], tv)
        n_tok_diff += len(diff)
        alive[rows[diff]] = False
    say(f"markov: {n_diff_logits} stored logits differ from the oracle's rounding "
        f"(worst error / bound {worst:.3f}), {n_tok_diff} token differences")
    return n_diff_logits, n_tok_diff


def _gpu_markov(mode, bk, emb, proj, prev, tau, u):
    R, k, V = bk.shape
    d_m = emb.shape[1]
    dev = "cuda"
    tb = to_device(bk, dev)
    toks = torch.zeros(R, k, dtype=torch.int32, device=dev)
    logits = torch.zeros(R, k, V, dtype=tb.dtype, device=dev)
    ws = B.workspace(B.markov_workspace_bytes(R, k, V, d_m), dev)
    B.markov_draft(B.SAMPLE if mode == "sample" else B.GREEDY, tb, to_device(emb, dev), to_device(proj, dev),
                   to_device(prev, dev), tau, to_device(u, dev), toks, logits, ws)
    torch.cuda.synchronize()
    lg = logits.cpu().numpy()
    if lg.dtype == np.int16:
        lg = lg.view(np.uint16)
    return toks.cpu().numpy(), lg, B.read_status(ws)


@pytest.mark.parametrize("mode", ["greedy", "sample"])
def test_markov_c0(mode):
    w = W("c0")
    say("markov c0", mode)
    gt, gl, st = _gpu_markov(mode, w.backbone, w.emb, w.proj, w.prev_token, w.tau, w.u_draft)
    assert st == 0
    ref = ref_markov("c0", mode)
    check_markov("f32", gl, gt, ref, w.u_draft, w.tau, mode, w.backbone, w.emb, w.proj, w.prev_token)


MARKOV_SMALL = [
    # R, k, V, d_m, mode
    (16, 2, 64, 32, "greedy"),        # one MFMA tile
    (70, 3, 1000, 64, "sample"),      # partial request block, V % 64 != 0
    (130, 2, 1001, 96, "greedy"),     # ragged V: scalar epilogue
    (64, 5, 5000, 256, "sample"),
    (600, 2, 3000, 256, "greedy"),    # three request groups of the persistent projection
    (40, 2, 2001, 256, "sample"),     # V % 8 != 0: scalar backbone loads and stores
    (3, 2, 300000, 32, "sample"),     # more than 4096 slices: one wavefront per request picks
    (2, 2, 270000, 32, "greedy"),
]


@pytest.mark.parametrize("R,k,V,d_m,mode", MARKOV_SMALL)
def test_markov_bf16_small(R, k, V, d_m, mode):
    g = np.random.Generator(np.random.Philox(R + V))
    bk = workloads.f32_to_bf16_bits((3 * g.standard_normal((R, k, V))).astype(np.float32))
    emb = workloads.f32_to_bf16_bits(g.standard_normal((V, d_m)).astype(np.float32))
    proj = workloads.f32_to_bf16_bits((0.5 / np.sqrt(d_m) * g.standard_normal((V, d_m))).astype(np.float32))
    prev = g.integers(0, V, size=R).astype(np.int32)
    u = (g.integers(0, 1 << 24, size=(R, k)) * 2.0 ** -24).astype(np.float32)
    say("markov bf16", R, k, V, d_m, mode)
    gt, gl, st = _gpu_markov(mode, bk, emb, proj, prev, 1.0, u)
    assert st == 0
    ref = omarkov.markov_draft(mode, "bf16", bk, emb, proj, prev, 1.0, u)
    check_markov("bf16", gl, gt, ref, u, 1.0, mode, bk, emb, proj, prev)


def test_markov_c4():
    w = W("c4")
    say("markov c4 sample")
    d = D("c4")
    d.markov(B.SAMPLE)
    torch.cuda.synchronize()
    assert B.read_status(d.ws_markov) == 0
    gt = d.host("draft_tokens")
    gl = d.draft_logits.cpu().numpy().view(np.uint16)
    ref = ref_markov("c4", "sample")
    check_markov("bf16", gl, gt, ref, w.u_draft, w.tau, "sample", w.backbone, w.emb, w.proj, w.prev_token)


# ---------------------------------------------------------------------------
# losslessness through the GPU: chi-square on 10**7 seeded trials
# ---------------------------------------------------------------------------

def test_gpu_chisquare_1e7_trials():
    from chisq_harness import LogitModel, chi2_pvalue, run_trials
    model = LogitModel(seed=5)
    k = 3
    V = model.V
    tl_dev = torch.from_numpy(model.tl).cuda()
    dl_dev = torch.from_numpy(model.dl).cuda()
    bufs = {}

    def gpu_verify(rows, x, L, u):
        A = rows.shape[0]
        if A not in bufs:
            bufs[A] = dict(
                tags=torch.zeros(A * (k + 1), 2, dtype=torch.int32, device="cuda"),
                cu=torch.zeros(A + 1, dtype=torch.int32, device="cuda"),
                nr=torch.zeros(1, dtype=torch.int32, device="cuda"),
                acc=torch.zeros(A, dtype=torch.int32, device="cuda"),
                out=torch.zeros(A, k + 1, dtype=torch.int32, device="cuda"),
                ws=B.workspace(B.verify_workspace_bytes(B.SAMPLE, A, k, V), "cuda"))
        b = bufs[A]
        r = torch.from_numpy(rows).cuda()
        tl = tl_dev[r].contiguous()
        dl = dl_dev[r[:, :k]].contiguous()
        B.spec_flatten(torch.from_numpy(L.astype(np.int32)).cuda(), k, b["tags"], b["cu"], b["nr"])
        B.spec_verify(B.SAMPLE, tl, dl, torch.from_numpy(x.astype(np.int32)).cuda(), b["tags"], b["cu"], b["nr"],
                      1.0, torch.from_numpy(u.astype(np.float32)).cuda(), b["acc"], b["out"], b["ws"])
        return b["acc"].cpu().numpy().astype(np.int64), b["out"].cpu().numpy().astype(np.int64)

    say("gpu chi-square 1e7")
    seqs, pr = model.target_probs(k + 1)
    counts = run_trials(model, 10_000_000, k, seed=4242, verify_fn=gpu_verify, rows=True)
    p = chi2_pvalue(counts, pr)
    say("gpu chi-square p =", p)
    assert p > 1e-4
