"""GPU parity: libspecv (HIP, gfx950) against the CPU oracle, stage by stage.

Tolerances:
  greedy        accepted lengths, emitted tokens, per-row argmax: bit-exact.
  scheduler     lengths, offsets and tags: bit-exact; survival within 1e-14
                relative (device and host exp may differ in the last bit).
  sampling      the uniforms the kernel used equal the oracle's bit for bit
                (its own Philox, or the given array); p(x), q(x), p/q and the
                residual mass within 1e-5 relative (fp32 accumulation over the
                vocabulary; the residual mass also within 2e-6 absolute, the
                cancellation in p - q); keep decisions identical except where
                |u - p/q| < 1e-6; resampled / bonus tokens identical except
                where the kernel's token is in the oracle's near set (its CDF
                interval within 1e-5 * W of t = u W, oracle.verify.draw_rows);
                residual draws by rejection trials (the library's uniforms):
                the same kept trial and token, except where the oracle marked
                a trial at or before the earlier side's last one as near (a
                proposal near set, or |u2 - (1 - q/p)| < 1e-6); at most
                DRAW_EXEMPT_LIMIT excused draws per case.
  Markov head   stored logits within the float32 accumulation bound plus half
                a storage spacing of the exact value (check_markov); tokens
                identical except where rounding differences can move them.
Every excused difference is counted and recorded (parity_log).
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
from oracle import philox as ophilox
from oracle import schedule as osched
from oracle import verify as overify

import parity_log

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
        _MK[key] = omarkov.markov_draft(mode, w.dtype, w.backbone, w.emb, w.proj, w.prev_token, w.tau, w.u_draft,
                                        near_eps=overify.DRAW_EPS)
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

def _run_verify(name, mode, max_len, rng=None):
    """GPU verify on the oracle's flattening and the oracle's drafts. rng =
    (seed, step): both sides take the counter-based uniforms; else the
    workload's uniform array."""
    w = W(name)
    d = D(name)
    ref_s = ref_schedule(w, max_len)
    tags, cu = osched.flatten(ref_s["L"])
    dl_host, tok_host = drafts_for(name, mode)
    mode_c = B.SAMPLE if mode == "sample" else B.GREEDY
    say("verify", name, mode, "max_len", max_len, "rows", osched.n_rows(cu), "rng", rng)
    d.flatten(to_device(ref_s["L"].astype(np.int32), "cuda"))
    if rng is None:
        d.rng = False
    else:
        d.rng, d.seed, d.step_no = True, rng[0], rng[1]
    d.verify(mode_c, draft=to_device(dl_host, "cuda") if mode == "sample" else None,
             tokens=to_device(tok_host.astype(np.int32), "cuda"))
    d.rng = False
    torch.cuda.synchronize()
    status = B.read_status(d.ws_verify)
    assert status == 0, status
    ref = overify.verify(mode, w.dtype, w.target, dl_host if mode == "sample" else None, tok_host, tags, cu,
                         w.tau, None if rng else w.u_verify, rng=rng)
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


def DRAW_EXEMPT_LIMIT(draws):
    """Most draws a case may excuse, fixed before the runs. A correct float32
    path moves a draw only when t / W lies within about 1e-6 of a CDF boundary,
    which at these vocabularies happens for well under 1% of draws (those that
    land on tokens of probability below ~2e-6); an off-by-one or a lost
    normaliser moves most draws."""
    return max(2, int(0.02 * draws))


def _first_false(keep, L):
    R, k = keep.shape
    a = L.copy()
    for j in range(k - 1, -1, -1):
        a = np.where((~keep[:, j]) & (j < L), j, a)
    return a


def _trials_explain(near, T, tok_g):
    """A rejection draw that differs between the kernel and the oracle (token or
    kept trial) is excused iff the oracle saw a rounding-sensitive step at or
    before T = the earlier of the two sides' last trials (RESIDUAL_TRIALS for a
    fallback): a proposal or keep decision of trial <= T, or the fallback draw
    with the kernel's token in its near set."""
    for e in near:
        if e[0] in ("draw", "keep") and e[1] <= T:
            return True
        if e[0] == "fallback" and T == overify.RESIDUAL_TRIALS and tok_g in e[1]:
            return True
    return False


def check_sampling(d, ref, tags, cu, case, tol=1e-5, rng=None):
    """Sampling-mode parity (see the module docstring); records and returns the
    exemption counts. rng = (seed, step) of the counter-based uniforms when the
    kernel drew them."""
    Bn = osched.n_rows(cu)
    R = len(cu) - 1
    N = int(cu[-1])
    L = np.diff(np.asarray(cu, dtype=np.int64))
    out_g, out_o = d.host("out_tokens"), ref["out_tokens"]
    k = out_g.shape[1] - 1
    diag = d.host("diag")[:Bn]
    ver = ref["row_verified"]
    rr, jj = tags[:Bn][ver, 0], tags[:Bn][ver, 1]
    worst = {}
    for col, key in [(0, "row_p"), (1, "row_q"), (2, "row_ratio")]:
        g, o = diag[ver, col].astype(np.float64), ref[key][ver]
        rel = np.abs(g - o) / np.abs(o)
        worst[key] = float(rel.max(initial=0))
        assert worst[key] < tol, (key, worst[key])
    # the uniforms the kernel used: the oracle's, bit for bit
    u_g = diag[ver, 3]
    u_o = ref["u_accept"][rr, jj]
    assert np.array_equal(u_g.astype(np.float64), u_o), "acceptance uniforms differ"
    # the kernel's keep decisions, in its own float32 arithmetic, give its accepted lengths
    keep_g = u_g < np.minimum(np.float32(1.0), diag[ver, 2])
    kg = np.zeros((R, k), dtype=bool)
    kg[rr, jj] = keep_g
    a_g, a_o = d.host("acc_len").astype(np.int64), ref["accepted_len"]
    assert np.array_equal(a_g, _first_false(kg, L))
    keep_o = ref["row_accept"][ver]
    near = np.abs(u_o - np.minimum(1.0, ref["row_ratio"][ver])) < 1e-6
    assert np.array_equal(keep_g[~near], keep_o[~near])
    flips = keep_g != keep_o
    flip_req = np.zeros(R, dtype=bool)
    flip_req[rr[flips]] = True
    assert np.array_equal(a_g[~flip_req], a_o[~flip_req])
    # draws, where both sides stopped at the same row
    bon = diag[N:N + R].astype(np.float64)
    same = a_g == a_o
    n_exempt = 0
    worst_res = 0.0
    n_res = 0
    n_trials = 0
    trials_used = 0
    NT = overify.RESIDUAL_TRIALS
    for r in np.nonzero(same)[0]:
        a = int(a_o[r])
        assert np.array_equal(out_g[r, :a], out_o[r, :a])
        assert (out_g[r, a + 1:] == -1).all()
        assert int(bon[r, 1]) == a and int(bon[r, 2]) == out_g[r, a], ("bonus record", r)
        if ref["draw_by_trials"][r]:
            # the residual by rejection trials: the kernel's kept trial (-(t+1) in
            # column 0; a mass >= 0 there: the fallback) and token against the oracle's
            t_g = int(-bon[r, 0]) - 1 if bon[r, 0] < 0 else -1
            t_o = int(ref["draw_trial"][r])
            if t_g >= 0:
                n_trials += 1
                trials_used += t_g + 1
            if t_g == t_o and out_g[r, a] == out_o[r, a]:
                assert bon[r, 3] == ref["u_draw"][r], ("draw uniform", r)
            else:
                T = min(t_g if t_g >= 0 else NT, t_o if t_o >= 0 else NT)
                assert _trials_explain(ref["draw_near"][r], T, int(out_g[r, a])), \
                    (r, t_g, t_o, out_g[r, a], out_o[r, a], ref["draw_near"][r])
                assert rng is not None
                want = ophilox.trial_uniforms(rng[0], rng[1], int(r), a, t_g if t_g >= 0 else NT)[0]
                assert bon[r, 3] == want, ("draw uniform", r)
                n_exempt += 1
            if t_g >= 0:
                continue
        else:
            assert bon[r, 3] == ref["u_draw"][r], ("draw uniform", r)
            if out_g[r, a] != out_o[r, a]:
                assert out_g[r, a] in ref["draw_near"][r], (r, out_g[r, a], out_o[r, a], ref["draw_near"][r])
                n_exempt += 1
        if a < L[r]:
            m_o, m_g = ref["residual_mass"][r], bon[r, 0]
            assert abs(m_g - m_o) <= tol * m_o + 2e-6, ("residual mass", r, m_g, m_o)
            if m_o > 0:
                worst_res = max(worst_res, abs(m_g - m_o) / m_o)
            n_res += 1
        else:
            assert bon[r, 0] == 0.0
    draws = int(same.sum())
    assert n_exempt <= DRAW_EXEMPT_LIMIT(draws), (n_exempt, draws)
    rec = parity_log.record("verify", case, rows=int(ver.sum()), near_keep=int(near.sum()),
                            keep_flips=int(flips.sum()), draws=draws, draw_exempt=n_exempt,
                            residual_rows=n_res, trial_draws=n_trials,
                            mean_trials=trials_used / n_trials if n_trials else 0.0,
                            worst_p=worst["row_p"], worst_q=worst["row_q"],
                            worst_ratio=worst["row_ratio"], worst_residual=worst_res)
    say("parity", rec)
    return rec


SAMPLE_CASES = [("c0", 5), ("c1", 5), ("c2", 5), ("c2", -1), ("c3", 16), ("c3", -1), ("c4", 5)]


@pytest.mark.parametrize("name,max_len", SAMPLE_CASES)
@pytest.mark.parametrize("source", ["array", "philox"])
def test_verify_sampling_within_tolerance(name, max_len, source):
    rng = (int(workloads.CONFIGS[name]["seed"]), 3) if source == "philox" else None
    d, ref, tags, cu = _run_verify(name, "sample", max_len, rng=rng)
    check_sampling(d, ref, tags, cu, f"{name} max_len={max_len} {source}", rng=rng)


@pytest.mark.parametrize("seed,step", [(0, 0), (7, 1), ((1 << 64) - 1, (1 << 63) + 11), (12345, (1 << 32) + 7)])
def test_philox_uniforms_bit_exact(seed, step):
    """The kernel's uniforms: U(seed, step, 0, r, j) for every verified row,
    U(seed, step, 1, r, a_r) for every bonus draw and the kept trial's (or the
    fallback's) first uniform for every residual draw, bit for bit the oracle's
    Philox (pinned to numpy.random.Philox), at 64-bit keys too; and the whole
    result against the oracle with those uniforms."""
    R, k, V = 48, 6, 3000
    tl, dl, x, _, L = _small(R, k, V, "bf16", seed=41)
    L[:] = k
    say("philox uniforms", seed, step)
    acc, out, diag, st = _gpu_verify(B.SAMPLE, tl, dl, x, None, L, 1.0, seed=seed, step=step)
    assert st == 0
    rows = diag[:R * k].reshape(R, k, 4)
    want = ophilox.uniforms(seed, step, ophilox.ACCEPT, R, k)
    assert np.array_equal(rows[:, :, 3].astype(np.float64), want)
    bonus = diag[R * k:R * k + R]
    for r in range(R):
        a = int(acc[r])
        assert int(bonus[r, 1]) == a
        if a == k:
            assert float(bonus[r, 3]) == ophilox.uniform(seed, step, ophilox.DRAW, r, a)
        else:
            t = int(-bonus[r, 0]) - 1 if bonus[r, 0] < 0 else overify.RESIDUAL_TRIALS
            assert float(bonus[r, 3]) == ophilox.trial_uniforms(seed, step, r, a, t)[0]
    tags, cu = osched.flatten(L)
    ref = overify.verify("sample", "bf16", tl, dl, x, tags, cu, 1.0, rng=(seed, step), near_eps=overify.DRAW_EPS)
    check_sampling(_Res(acc, out, diag), ref, tags, cu, f"philox uniforms seed={seed} step={step}",
                   rng=(seed, step))


def test_philox_residual_fallback():
    """Rows whose q is close to p (residual mass about 0.04) and draft tokens
    that q overrates, so that rejections are frequent and the rejection trials
    often need more than one round of 16 and for some requests all 64 fail: the
    later rounds and the fallback, an inverse-CDF draw from the residual with
    the first uniform of trial 64, against the oracle over 40 steps (fp32 rows,
    V = 600); at least 8 fallbacks and 8 draws kept after the first round."""
    R, k, V = 16, 3, 600
    g = np.random.Generator(np.random.Philox(5))
    tl = (2.0 * g.standard_normal((R, k + 1, V))).astype(np.float32)
    dl = (tl[:, :k] + 0.1 * g.standard_normal((R, k, V))).astype(np.float32)
    x = np.argmax(dl - tl[:, :k], axis=2).astype(np.int32)
    L = np.full(R, k, np.int32)
    tags, cu = osched.flatten(L)
    N = int(cu[-1])
    fallbacks = late = 0
    say("philox residual fallback")
    for step in range(40):
        acc, out, diag, st = _gpu_verify(B.SAMPLE, tl, dl, x, None, L, 1.0, seed=11, step=step)
        assert st == 0
        ref = overify.verify("sample", "f32", tl, dl, x, tags, cu, 1.0, rng=(11, step), near_eps=overify.DRAW_EPS)
        check_sampling(_Res(acc, out, diag), ref, tags, cu, f"fallback seed=11 step={step}", rng=(11, step))
        bon = diag[N:N + R]
        fallbacks += int(((acc < L) & (bon[:, 0] >= 0)).sum())
        late += int(((acc < L) & (bon[:, 0] <= -17)).sum())
    say("fallbacks", fallbacks, "kept after the first round", late)
    assert fallbacks >= 8, fallbacks
    assert late >= 8, late


def test_verify_deterministic():
    d, ref, tags, cu = _run_verify("c2", "sample", -1, rng=(2, 5))
    a1, o1, g1 = d.host("acc_len"), d.host("out_tokens"), d.host("diag")
    say("verify repeat c2")
    d.rng, d.seed, d.step_no = True, 2, 5
    d.verify(B.SAMPLE, draft=to_device(W("c2").draft, "cuda"), tokens=to_device(W("c2").tokens_sample, "cuda"))
    d.rng = False
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


def _gpu_verify(mode, tl, dl, x, u, L, tau, offset=0, seed=0, step=0):
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
    ws = B.workspace(B.verify_workspace_bytes(R, k, V), dev)
    B.spec_verify(mode, up(tl), up(dl) if mode == B.SAMPLE else None, to_device(x, dev), tags, cu, nr, tau,
                  None if u is None else to_device(u, dev), acc, out, ws, row_diag=diag, seed=seed, step=step)
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
        check_sampling(_Res(acc, out, diag), ref, tags, cu, f"edge R={R} k={k} V={V} {dtype}")


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


@pytest.mark.parametrize("mode", ["greedy", "sample"])
def test_verify_nonfinite_rows(mode):
    """NaN and +inf logits void their request (accepted length 0, no tokens)
    and set SPECV_STATUS_NONFINITE; -inf logits are valid (tokens that cannot
    be drawn); every other request matches the oracle."""
    R, k, V = 12, 4, 3000
    tl, dl, x, u, L = _small(R, k, V, "bf16", seed=13)
    L[:] = k
    NAN, PINF, NINF = 0x7FC0, 0x7F80, 0xFF80
    tl[1, 2, 100] = NAN                   # a verified target row
    tl[3, k, 7] = PINF                    # a bonus row
    tl[5, 0, :50] = NINF                  # valid
    tl[9, 1, 2047:2049] = NAN             # across a chunk boundary
    void = {1, 3, 9}
    if mode == "sample":
        dl[6, 1, 2999] = NAN              # a draft row, last element (ragged chunk)
        dl[8, 0, :] = NINF                # a draft row of -inf only: no distribution
        dl[10, 2, :1000] = NINF           # valid
        void |= {6, 8}
    mc = B.SAMPLE if mode == "sample" else B.GREEDY
    say("verify nonfinite", mode)
    acc, out, diag, st = _gpu_verify(mc, tl, dl, x, u, L, 1.0)
    assert st & B.STATUS_NONFINITE
    good = np.array([r for r in range(R) if r not in void])
    for r in void:
        assert acc[r] == 0 and (out[r] == -1).all(), r
    tags, cu = osched.flatten(L[good])
    ref = overify.verify(mode, "bf16", tl[good], dl[good] if mode == "sample" else None, x[good], tags, cu, 1.0,
                         u[good], near_eps=overify.DRAW_EPS)
    assert np.array_equal(acc[good], ref["accepted_len"])
    for n, r in enumerate(good):
        a = int(acc[r])
        assert np.array_equal(out[r, :a], ref["out_tokens"][n, :a])
        if out[r, a] != ref["out_tokens"][n, a]:
            assert mode == "sample" and out[r, a] in ref["draw_near"][n], r
    # the same inputs without the planted values: no status bit
    clean = _small(R, k, V, "bf16", seed=13)
    _, _, _, st2 = _gpu_verify(mc, clean[0], clean[1], x, u, L, 1.0)
    assert st2 == 0


def test_markov_nonfinite_status():
    R, k, V, d_m = 16, 2, 1000, 32
    g = np.random.Generator(np.random.Philox(3))
    enc = workloads.f32_to_bf16_bits
    bk = enc((3 * g.standard_normal((R, k, V))).astype(np.float32))
    emb = enc(g.standard_normal((V, d_m)).astype(np.float32))
    proj = enc((0.1 * g.standard_normal((V, d_m))).astype(np.float32))
    prev = g.integers(0, V, size=R).astype(np.int32)
    say("markov nonfinite")
    _, _, st = _gpu_markov("sample", bk, emb, proj, prev, 1.0, None)
    assert st == 0
    bk[4, 1, 500] = 0x7FC0
    _, _, st = _gpu_markov("sample", bk, emb, proj, prev, 1.0, None)
    assert st & B.STATUS_NONFINITE


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


def check_markov(dtype, gl, gt, ref, tau, mode, bk, emb, proj, prev0, case=""):
    """Position by position, over requests whose earlier tokens agree.

    Logits: the kernel accumulates d_m products and the backbone value in
    float32 in its own order, then rounds once to the storage type. With
    u = 2**-24 and m = |bk| + sum_d |E[prev, d] * P[v, d]|, the float32 value
    lies within delta = (d_m + 2) * u * m of the exact sum, so the stored value
    must lie within delta + half a storage spacing of it.
    Tokens: with identical rows the draw must agree (sampling: unless the
    kernel's token is in the oracle's near set); where rows differ by
    rounding, greedy may pick another token only if the two values are within
    the rows' differences, and sampling only if the kernel's token is in the
    oracle's near set widened by the L1 distance of the two rows'
    distributions (each C(v) / W moves by at most that much).
    """
    R, k, V = gl.shape
    d_m = emb.shape[1]
    E = numerics.decode(emb, dtype)
    P = numerics.decode(proj, dtype)
    alive = np.ones(R, dtype=bool)
    n_diff_logits = 0
    n_tok_diff = 0
    n_same_row = 0
    worst = 0.0
    compared = 0
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
        compared += len(rows)
        diff = np.nonzero(gt[rows, i] != ref["tokens"][rows, i])[0]
        for n in diff:
            r = rows[n]
            a, b = int(gt[r, i]), int(ref["tokens"][r, i])
            if mode == "greedy":
                assert rowdiff[n], (r, i)
                dd = np.abs(g[n] - o[n])
                assert o[n, b] - o[n, a] <= dd[a] + dd[b], (r, i)
            elif not rowdiff[n]:
                assert a in ref["draw_near"][r][i], (r, i, a, b)
                n_same_row += 1
            else:
                tv = np.abs(_softmax_rows(g[n:n + 1], tau) - _softmax_rows(o[n:n + 1], tau)).sum()
                _, nb = overify.draw_rows(_softmax_rows(o[n:n + 1], tau), np.array([ref["u_draft"][r, i]]),
                                          tv + overify.DRAW_EPS)
                assert a in nb[0], (r, i, a, b, tv)
        n_tok_diff += len(diff)
        alive[rows[diff]] = False
    assert n_same_row <= DRAW_EXEMPT_LIMIT(compared), (n_same_row, compared)
    rec = parity_log.record("markov", case, positions=compared, logits_1ulp=n_diff_logits,
                            worst_logit_over_bound=worst, token_diffs=n_tok_diff,
                            token_diffs_same_row=n_same_row)
    say("parity", rec)
    return n_diff_logits, n_tok_diff


def _gpu_markov(mode, bk, emb, proj, prev, tau, u, seed=0, step=0):
    R, k, V = bk.shape
    d_m = emb.shape[1]
    dev = "cuda"
    tb = to_device(bk, dev)
    toks = torch.zeros(R, k, dtype=torch.int32, device=dev)
    logits = torch.zeros(R, k, V, dtype=tb.dtype, device=dev)
    ws = B.workspace(B.markov_workspace_bytes(R, k, V, d_m), dev)
    B.markov_draft(B.SAMPLE if mode == "sample" else B.GREEDY, tb, to_device(emb, dev), to_device(proj, dev),
                   to_device(prev, dev), tau, None if u is None else to_device(u, dev), toks, logits, ws, seed=seed,
                   step=step)
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
    check_markov("f32", gl, gt, ref, w.tau, mode, w.backbone, w.emb, w.proj, w.prev_token, f"c0 {mode}")


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
    ref = omarkov.markov_draft(mode, "bf16", bk, emb, proj, prev, 1.0, u, near_eps=overify.DRAW_EPS)
    check_markov("bf16", gl, gt, ref, 1.0, mode, bk, emb, proj, prev, f"R={R} k={k} V={V} d_m={d_m} {mode}")


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
    check_markov("bf16", gl, gt, ref, w.tau, "sample", w.backbone, w.emb, w.proj, w.prev_token, "c4 array")


def test_markov_philox():
    """markov_draft with its own uniforms U(seed, step, 2, r, i) against the
    oracle's head with the same (seed, step) (c4 recipe at R = 96)."""
    w = workloads.make("c4", R=96)
    say("markov philox R=96")
    dev = "cuda"
    R, k, V = w.R, w.k, w.V
    toks = torch.zeros(R, k, dtype=torch.int32, device=dev)
    logits = torch.zeros(R, k, V, dtype=torch.int16, device=dev)
    ws = B.workspace(B.markov_workspace_bytes(R, k, V, w.d_m), dev)
    B.markov_draft(B.SAMPLE, to_device(w.backbone, dev), to_device(w.emb, dev), to_device(w.proj, dev),
                   to_device(w.prev_token, dev), w.tau, None, toks, logits, ws, seed=7, step=42)
    torch.cuda.synchronize()
    assert B.read_status(ws) == 0
    ref = omarkov.markov_draft("sample", "bf16", w.backbone, w.emb, w.proj, w.prev_token, w.tau, rng=(7, 42),
                               near_eps=overify.DRAW_EPS)
    check_markov("bf16", logits.cpu().numpy().view(np.uint16), toks.cpu().numpy(), ref, w.tau, "sample",
                 w.backbone, w.emb, w.proj, w.prev_token, "c4 R=96 philox")


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
                ws=B.workspace(B.verify_workspace_bytes(A, k, V), "cuda"))
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


def test_gpu_chisquare_1e7_trials_philox():
    """The same 10**7 trials with the kernel drawing its own uniforms: one
    (seed, step) per call, step advancing from call to call."""
    from chisq_harness import LogitModel, chi2_pvalue, run_trials
    model = LogitModel(seed=5)
    k = 3
    V = model.V
    tl_dev = torch.from_numpy(model.tl).cuda()
    dl_dev = torch.from_numpy(model.dl).cuda()
    bufs = {}
    calls = [0]

    def gpu_verify(rows, x, L, u):
        A = rows.shape[0]
        if A not in bufs:
            bufs[A] = dict(
                tags=torch.zeros(A * (k + 1), 2, dtype=torch.int32, device="cuda"),
                cu=torch.zeros(A + 1, dtype=torch.int32, device="cuda"),
                nr=torch.zeros(1, dtype=torch.int32, device="cuda"),
                acc=torch.zeros(A, dtype=torch.int32, device="cuda"),
                out=torch.zeros(A, k + 1, dtype=torch.int32, device="cuda"),
                ws=B.workspace(B.verify_workspace_bytes(A, k, V), "cuda"))
        b = bufs[A]
        r = torch.from_numpy(rows).cuda()
        tl = tl_dev[r].contiguous()
        dl = dl_dev[r[:, :k]].contiguous()
        calls[0] += 1
        B.spec_flatten(torch.from_numpy(L.astype(np.int32)).cuda(), k, b["tags"], b["cu"], b["nr"])
        B.spec_verify(B.SAMPLE, tl, dl, torch.from_numpy(x.astype(np.int32)).cuda(), b["tags"], b["cu"], b["nr"],
                      1.0, None, b["acc"], b["out"], b["ws"], seed=2027, step=calls[0])
        return b["acc"].cpu().numpy().astype(np.int64), b["out"].cpu().numpy().astype(np.int64)

    say("gpu chi-square 1e7, device Philox")
    seqs, pr = model.target_probs(k + 1)
    counts = run_trials(model, 10_000_000, k, seed=4243, verify_fn=gpu_verify, rows=True)
    p = chi2_pvalue(counts, pr)
    say("gpu chi-square (device Philox) p =", p)
    assert p > 1e-4


# ---------------------------------------------------------------------------
# the draft head's statistics in place of the pass over the draft rows
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name,head", [("c0", "markov"), ("c4", "markov"), ("c4", "rnn")])
def test_draft_stats_route(name, head):
    """spec_verify_ex with the draft head's statistics against spec_verify on
    the same drafts (the logits route, which the tests above pin to the
    oracle). The statistics must describe the stored draft rows: the drawn
    token and its stored logit exactly, the scale c = log2(e) / tau bit for
    bit, z 2^m = sum of exp2(logit c) within 1e-5 relative. The two routes
    must give p(x), q(x), p/q within 1e-5 relative, the same uniforms, the same
    keep decisions except where |u - min(1, p/q)| < 1e-6, and the same tokens
    except for at most DRAW_EXEMPT_LIMIT draws (the residual's normaliser comes
    from a different float32 summation order)."""
    w = W(name)
    d = D(name) if head == "markov" else DeviceStep(w, head="rnn")
    say("draft stats route", name, head)
    d.rng, d.step_no = True, 5
    d.markov(B.SAMPLE)
    d.schedule(w.k)
    d.use_stats = False
    d.verify(B.SAMPLE)
    torch.cuda.synchronize()
    assert B.read_status(d.ws_verify) == 0
    a1, o1, g1 = d.host("acc_len"), d.host("out_tokens"), d.host("diag").copy()
    d.use_stats = True
    d.verify(B.SAMPLE)
    torch.cuda.synchronize()
    assert B.read_status(d.ws_verify) == 0
    a2, o2, g2 = d.host("acc_len"), d.host("out_tokens"), d.host("diag").copy()
    d.rng = False
    R, k = w.R, w.k
    # the statistics
    st = d.draft_stats.cpu().numpy()
    tok = st[..., 4].copy().view(np.int32)
    x = d.host("draft_tokens")
    assert np.array_equal(tok, x)
    assert np.all(st[..., 3] == np.float32(1.4426950408889634 / w.tau))
    dl = d.draft_logits.cpu().numpy()
    if dl.dtype == np.int16:
        dl = dl.view(np.uint16)
    c = float(np.float32(1.4426950408889634 / w.tau))
    worst = 0.0
    for i in range(k):
        row = numerics.decode(dl[:, i], w.dtype)
        assert np.array_equal(st[:, i, 2].astype(np.float64), row[np.arange(R), x[:, i]])
        a = row * c
        m = a.max(axis=1)
        ztrue = np.exp2(a - m[:, None]).sum(axis=1)
        zgot = st[:, i, 1].astype(np.float64) * np.exp2(st[:, i, 0].astype(np.float64) - m)
        worst = max(worst, float(np.max(np.abs(zgot - ztrue) / ztrue)))
    assert worst < 1e-5, worst
    # the two routes
    N = int(d.host("cu_rows")[-1])
    ver = slice(0, N)
    for col in range(3):
        rel = np.abs(g2[ver, col].astype(np.float64) - g1[ver, col]) / np.abs(g1[ver, col].astype(np.float64))
        assert rel.max(initial=0) < 1e-5, (col, rel.max())
    assert np.array_equal(g1[ver, 3], g2[ver, 3])
    near = np.abs(g1[ver, 3].astype(np.float64) - np.minimum(1.0, g1[ver, 2].astype(np.float64))) < 1e-6
    tags = d.host("tags")[:N]
    near_req = np.zeros(R, dtype=bool)
    near_req[tags[near, 0]] = True
    assert np.array_equal(a1[~near_req], a2[~near_req])
    same = a1 == a2
    diff_draw = int((o1[same] != o2[same]).any(axis=1).sum())
    assert diff_draw <= DRAW_EXEMPT_LIMIT(int(same.sum())), diff_draw
    parity_log.record("stats", f"{name} {head}", rows=N, near_keep=int(near.sum()), draws=int(same.sum()),
                      draw_diffs=diff_draw, worst_z=worst)


def test_draft_stats_must_match_the_call():
    """Statistics made at another temperature, or for another token than the
    one verified, void their requests and set SPECV_STATUS_BAD_STATS."""
    w = W("c0")
    d = D("c0")
    say("draft stats mismatch")
    d.rng, d.step_no = True, 6
    d.markov(B.SAMPLE)
    d.schedule(-1)                              # every request verifies all k rows
    d.rng = False
    acc = torch.zeros(w.R, dtype=torch.int32, device="cuda")
    out = torch.zeros(w.R, w.k + 1, dtype=torch.int32, device="cuda")
    B.spec_verify(B.SAMPLE, d.target, d.draft_logits, d.draft_tokens, d.tags, d.cu_rows, d.n_rows, 0.9, None, acc,
                  out, d.ws_verify, seed=0, step=6, draft_stats=d.draft_stats)
    assert B.read_status(d.ws_verify) & B.STATUS_BAD_STATS
    assert (acc.cpu().numpy() == 0).all() and (out.cpu().numpy() == -1).all()
    toks = d.draft_tokens.clone()
    toks[1, 2] = (toks[1, 2] + 1) % w.V
    B.spec_verify(B.SAMPLE, d.target, d.draft_logits, toks, d.tags, d.cu_rows, d.n_rows, w.tau, None, acc, out,
                  d.ws_verify, seed=0, step=6, draft_stats=d.draft_stats)
    assert B.read_status(d.ws_verify) == B.STATUS_BAD_STATS
    a = acc.cpu().numpy()
    assert a[1] == 0 and (out.cpu().numpy()[1] == -1).all()
