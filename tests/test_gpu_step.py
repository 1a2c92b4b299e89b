"""spec_step (this round's schedule beside the stream of the rows (r, 0), then
the verification of the batch it wrote) against spec_schedule followed by
spec_verify on the same inputs: the same results bit for bit, lengths, batch,
survival, accepted lengths, tokens and row records, in both modes, with the
library's own uniforms and (semi-autoregressive workload) the draft head's
statistics. The sequential paths it falls back to (fixed lengths; schedules
beyond one workgroup) are covered too."""
import numpy as np
import pytest
import torch

from draft_token_verification_flattened_amd import binding as B
from draft_token_verification_flattened_amd import workloads
from draft_token_verification_flattened_amd.pipeline import DeviceStep, to_device

pytestmark = pytest.mark.gpu

_W = {}


def W(name):
    if name not in _W:
        _W[name] = workloads.make(name)
    return _W[name]


def say(*a):
    print("[gpu]", *a, flush=True)


NAMES = ["lengths", "tags", "cu_rows", "n_rows", "survival", "acc_len", "out_tokens", "diag"]


def _outputs(d):
    n = int(d.host("n_rows")[0])
    out = {k: d.host(k).copy() for k in NAMES}
    out["tags"] = out["tags"][:n]
    out["diag"] = out["diag"][:n]
    return out


def _clear(d):
    for k in NAMES:
        getattr(d, k).fill_(-3)


CASES = [("c0", "greedy", None), ("c0", "sample", None), ("c1", "sample", None), ("c1", "greedy", None),
         ("c2", "sample", None), ("c2", "greedy", None), ("c2", "sample", -1), ("c2", "sample", 2),
         ("c3", "sample", None), ("c4", "sample", None)]


@pytest.mark.parametrize("name,mode,max_len", CASES)
def test_spec_step_equals_schedule_then_verify(name, mode, max_len):
    w = W(name)
    d = DeviceStep(w, rng=True)
    mc = B.SAMPLE if mode == "sample" else B.GREEDY
    say("spec_step", name, mode, "max_len", max_len)
    d.step_no = 11
    if w.backbone is not None:
        d.markov(mc)
    _clear(d)
    d.schedule(max_len)
    d.verify(mc, diag=True)
    torch.cuda.synchronize()
    assert B.read_status(d.ws_verify) == 0
    ref = _outputs(d)
    _clear(d)
    d.schedule_verify(mc, max_len, diag=True)
    torch.cuda.synchronize()
    assert B.read_status(d.ws_verify) == 0
    got = _outputs(d)
    for k in NAMES:
        assert np.array_equal(got[k], ref[k]), k
    del d
    torch.cuda.empty_cache()


@pytest.mark.parametrize("mode", ["sample", "greedy"])
def test_spec_step_any_workspace_contents_and_graph_replays(mode):
    """The streaming launch waits for the schedule's completion mark, which is
    unique per call: a workspace full of arbitrary bytes gives the same results,
    and so does every replay of a captured spec_step (each call's decisions
    clear the mark for the next one), with eager work between the replays."""
    w = W("c2")
    d = DeviceStep(w, rng=True)
    mc = B.SAMPLE if mode == "sample" else B.GREEDY
    d.step_no = 5
    say("spec_step eager", mode)
    _clear(d)
    d.schedule_verify(mc, diag=True)
    torch.cuda.synchronize()
    assert B.read_status(d.ws_verify) == 0
    ref = _outputs(d)
    for fill in (0xFF, None):
        say("spec_step on a workspace of", "0xff bytes" if fill is not None else "random bytes")
        if fill is None:
            g = torch.Generator(device="cpu").manual_seed(3)
            d.ws_verify.copy_(torch.randint(0, 256, d.ws_verify.shape, generator=g, dtype=torch.uint8))
        else:
            d.ws_verify.fill_(fill)
        _clear(d)
        d.schedule_verify(mc, diag=True)
        torch.cuda.synchronize()
        assert B.read_status(d.ws_verify) == 0
        got = _outputs(d)
        for key in NAMES:
            assert np.array_equal(got[key], ref[key]), key
    say("spec_step graph capture", mode)
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            d.schedule_verify(mc, diag=True)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(3):
        _clear(d)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        say("replay", rep)
        assert B.read_status(d.ws_verify) == 0
        got = _outputs(d)
        for key in NAMES:
            assert np.array_equal(got[key], ref[key]), (rep, key)
    del graph, d
    torch.cuda.empty_cache()


@pytest.mark.parametrize("R,k,V,dtype", [(1, 5, 151936, "bf16"), (7, 3, 1001, "bf16"), (40, 6, 5000, "f32"),
                                         (16, 1, 3000, "bf16"), (1024, 8, 256, "bf16")])
def test_spec_step_small_and_beyond_one_workgroup(R, k, V, dtype):
    """One request at full V; ragged V (scalar loads); fp32; one draft per
    request (the target rows (r, 1) streamed beside the schedule are bonus rows
    only); and R * k = 8192, whose schedule needs the multi-workgroup kernel
    (sequential path)."""
    g = np.random.Generator(np.random.Philox(R * 31 + V))
    tl = (3 * g.standard_normal((R, k + 1, V))).astype(np.float32)
    dl = (tl[:, :k] + 1.5 * g.standard_normal((R, k, V))).astype(np.float32)
    if dtype == "bf16":
        tl, dl = workloads.f32_to_bf16_bits(tl), workloads.f32_to_bf16_bits(dl)
    x = g.integers(0, V, size=(R, k)).astype(np.int32)
    z = (g.standard_normal((R, k)) + 1.0).astype(np.float32)
    T = np.linspace(1, 2, k).astype(np.float32)
    pts = np.array([max(1, R // 2), R, 2 * R, 4 * R, 8 * R], np.int32)
    thr = np.array([p / (1.0 + 0.6 * max(0, p - R) / R) for p in pts])
    dev = "cuda"
    t = dict(z=to_device(z, dev), T=to_device(T, dev), pts=to_device(pts, dev), thr=to_device(thr, dev),
             tl=to_device(tl, dev), dl=to_device(dl, dev), x=to_device(x, dev))
    i32 = dict(dtype=torch.int32, device=dev)

    def bufs():
        return dict(L=torch.full((R,), -3, **i32), tags=torch.full((R * (k + 1), 2), -3, **i32),
                    cu=torch.full((R + 1,), -3, **i32), nr=torch.full((1,), -3, **i32),
                    acc=torch.full((R,), -3, **i32), out=torch.full((R, k + 1), -3, **i32),
                    diag=torch.zeros(R * (k + 1), 4, dtype=torch.float32, device=dev),
                    ws_s=B.workspace(B.schedule_workspace_bytes(R, k), dev),
                    ws_v=B.workspace(B.verify_workspace_bytes(R, k, V), dev))
    for mc in (B.SAMPLE, B.GREEDY):
        say("spec_step small", R, k, V, dtype, mc)
        a, b = bufs(), bufs()
        B.spec_schedule(t["z"], t["T"], t["pts"], t["thr"], k, a["L"], a["tags"], a["cu"], a["nr"], a["ws_s"])
        B.spec_verify(mc, t["tl"], t["dl"], t["x"], a["tags"], a["cu"], a["nr"], 0.8, None, a["acc"], a["out"],
                      a["ws_v"], row_diag=a["diag"], seed=4, step=2)
        job = B.schedule_job(t["z"], t["T"], t["pts"], t["thr"], k, b["L"], b["tags"], b["cu"], b["nr"], b["ws_s"])
        B.spec_step(job, mc, t["tl"], t["dl"], t["x"], 0.8, None, b["acc"], b["out"], b["ws_v"], row_diag=b["diag"],
                    seed=4, step=2)
        torch.cuda.synchronize()
        assert B.read_status(a["ws_v"]) == 0 and B.read_status(b["ws_v"]) == 0
        n = int(a["nr"].item())
        for key in ("L", "cu", "nr", "acc", "out"):
            assert torch.equal(a[key], b[key]), key
        assert torch.equal(a["tags"][:n], b["tags"][:n])
        assert torch.equal(a["diag"][:n], b["diag"][:n])


def test_spec_step_rejects_bad_arguments_before_enqueueing():
    w = W("c0")
    d = DeviceStep(w)
    job = B.schedule_job(d.z, d.T, d.tbl_b, d.tbl_t, w.k, d.lengths, d.tags, d.cu_rows, d.n_rows, d.ws_sched)
    with pytest.raises(B.SpecvError) as e:
        B.spec_step(job, B.SAMPLE, d.target, d.draft_logits, d.draft_tokens, 0.0, None, d.acc_len, d.out_tokens,
                    d.ws_verify)
    assert "temperature" in str(e.value)
    bad = B.schedule_job(d.z, d.T, d.tbl_b, d.tbl_t, w.k + 1, d.lengths, d.tags, d.cu_rows, d.n_rows, d.ws_sched)
    with pytest.raises(B.SpecvError) as e:
        B.spec_step(bad, B.SAMPLE, d.target, d.draft_logits, d.draft_tokens, 1.0, None, d.acc_len, d.out_tokens,
                    d.ws_verify)
    assert "spec_step (schedule)" in str(e.value)
