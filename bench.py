"""Benchmark of the confidence-scheduled, flattened verification step on one GPU.

One step = one pass of the hot path over one batch of synthetic input:
  (Markov head, for the Markov workloads) -> calibration, survival, prefix
  schedule and flatten -> verification pass, first-reject, resample and emit.

Default workload: R = 256 requests, k = 5, V = 151936, bf16 logits, sampling at
tau = 1, throughput table with a knee at 256 batch tokens (the scheduler
truncates), math/code/chat confidence profiles. The metric is verified draft
tokens per second (N = sum of scheduled lengths per step, divided by the step
time) and the HBM bandwidth the verification kernel achieves against the
8 TB/s peak of MI355X.

  python bench.py [--steps K] [--warmup W] [--config c2] [--mode sample]
                  [--max-len k|-1] [--no-cpu] [--variants] [--copies 3]

Prints one JSON line. Inputs are resident in HBM before timing starts; the
logits exist in `--copies` copies used in turn, so that no step is served from
the Infinity Cache by the step before it.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "verified draft tokens/s at V=151936, k=5, 256 req; achieved HBM GB/s % peak"
HBM_PEAK = 8.0e12
MFMA_BF16_PEAK = 2.5e15   # dense bf16 MFMA, MI355X
DOMINANT = "verify_stream"              # spec_verify; spec_step's is verify_step_stream


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="c2")
    ap.add_argument("--mode", default="sample", choices=["sample", "greedy"])
    ap.add_argument("--max-len", default="k")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--variants", action="store_true",
                    help="also time greedy and verify-all variants of the workload")
    ap.add_argument("--sweep", action="store_true",
                    help="only run the load sweep over R = 1..512 and print its table as one JSON line")
    ap.add_argument("--lagged", action="store_true",
                    help="also time the lagged schedule (two streams, HIP graph) on rotating confidence rounds")
    ap.add_argument("--attention", action="store_true",
                    help="time spec_attention (tag-masked flattened attention over a paged KV cache) instead")
    ap.add_argument("--split-keys", type=int, default=0, help="spec_attention keys per work item (0: automatic)")
    ap.add_argument("--kv-layout", default="head", choices=["head", "position"],
                    help="spec_attention page layout: head-major [Hkv, page, D] or position-major [page, Hkv, D]")
    ap.add_argument("--head", default="markov", choices=["markov", "rnn"],
                    help="the drafter's sequential module for the semi-autoregressive workload (c4)")
    ap.add_argument("--copies", type=int, default=3,
                    help="input copies rotated over the steps (no step reads logits cached by the previous one)")
    ap.add_argument("--copy-probe", type=float, default=0.0,
                    help="only run a device copy of this many GiB (counter calibration) and exit")
    return ap.parse_args()


def source_hash(files=("common.h", "verify.hip")) -> str:
    h = hashlib.sha256()
    for f in files:
        h.update(open(os.path.join(ROOT, "draft_token_verification_flattened_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


# Counter summaries (profiles/) per dominant kernel and workload: the file and
# the sources its kernel is built from (the workload the counters were taken on
# is recorded in the file).
_VERIFY_SRC = ("common.h", "verify.hip")
TRAFFIC = {
    ("verify_step_stream", cfg): (os.path.join(ROOT, "profiles", f"verify_step_stream_{cfg}_traffic.txt"), _VERIFY_SRC)
    for cfg in ("c1", "c2", "c3")
}
TRAFFIC[("markov_logits", "c4")] = (os.path.join(ROOT, "profiles", "markov_logits_c4_traffic.txt"),
                                    ("common.h", "markov.hip"))


def workload_key(args, max_len) -> str:
    return f"{args.config} {args.mode} max_len={max_len} head={args.head}"


def committed_traffic(kernel, wkey):
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary, if it was taken on the current kernel source and on this workload."""
    key = (kernel, wkey.split()[0])
    if key not in TRAFFIC:
        return None, None
    path, files = TRAFFIC[key]
    if not os.path.exists(path):
        return None, None
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("source_hash") != source_hash(files) or vals.get("workload") != wkey:
        return None, vals.get("source_hash")
    try:
        return float(vals["hbm_bytes_per_launch"]), vals.get("source_hash")
    except (KeyError, ValueError):
        return None, None


def markov_bytes_flops(w):
    """Per position: P read once (2 d_m V), the gathered operand rows
    (2 R d_m), the backbone read and the draft logits written (2 R V each);
    2 R d_m V flops."""
    es = 2 if w.dtype == "bf16" else 4
    d_m = w.emb.shape[1]
    nbytes = es * (d_m * w.V + w.R * d_m + 2 * w.R * w.V)
    return nbytes, 2.0 * w.R * d_m * w.V


def algorithmic_bytes(w, mode, N, R, draft_rows=True):
    """Logit bytes the verification must read once: every target row of the
    flattened batch (N verified + R bonus), plus the N draft rows when
    sampling, unless the draft head hands over their softmax states
    (draft_rows=False)."""
    esize = 2 if w.dtype == "bf16" else 4
    rows = (2 * N + R) if (mode == "sample" and draft_rows) else (N + R)
    return rows * w.V * esize


def verify_kernel_bytes(w, mode, N, R, draft_rows, fused):
    """Algorithmic bytes per launch of the verification's streaming kernel:
    verify_step_stream (spec_step: the schedule beside the target rows (r, 0),
    then the other rows) or verify_stream (spec_verify)."""
    return {("verify_step_stream" if fused else "verify_stream"): algorithmic_bytes(w, mode, N, R, draft_rows)}


def run_variant(d, w, mode_c, mode, max_len, steps, warmup, B, torch):
    """Warm up, then run `steps` steps twice: first with the library recording
    start/stop events from each kernel's own dispatch (per-kernel durations;
    the events cost the step some time), then uninstrumented (the step time
    and the throughput)."""
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        d.step(mode_c, max_len)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    B.timing_reset()
    B.timing_enable(True)
    t0.record(stream)
    for _ in range(steps):
        d.step(mode_c, max_len)
    t1.record(stream)
    torch.cuda.synchronize()
    B.timing_enable(False)
    ms_step = t0.elapsed_time(t1) / steps
    kern = {}
    for name in ("rnn_state", "markov_logits", "markov_pick", "schedule", "verify_step_stream", "verify_stream",
                 "verify_decide"):
        n, tot = B.timing_read(name)
        if n:
            kern[name] = dict(launches_per_step=n / steps, avg_us=1000.0 * tot / n)
    B.timing_reset()
    t0.record(stream)
    for _ in range(steps):
        d.step(mode_c, max_len)
    t1.record(stream)
    torch.cuda.synchronize()
    ms_plain = t0.elapsed_time(t1) / steps
    # per-step spread: one event between consecutive steps (a pass of its own)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    evs[0].record(stream)
    for i in range(steps):
        d.step(mode_c, max_len)
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    per = sorted(1000.0 * evs[i].elapsed_time(evs[i + 1]) for i in range(steps))
    pct = {f"p{q}": per[min(steps - 1, int(round(q / 100.0 * (steps - 1))))] for q in (10, 50, 90)}
    L = d.host("lengths")
    N = int(L.sum())
    R = w.R
    draft_rows = d.stats_for(mode_c) is None
    fused = "verify_step_stream" in kern
    dom_name = "verify_step_stream" if fused else DOMINANT
    nbytes = algorithmic_bytes(w, mode, N, R, draft_rows)
    per_kernel = verify_kernel_bytes(w, mode, N, R, draft_rows, fused)
    dom = kern.get(dom_name)
    achieved = per_kernel[dom_name] / (dom["avg_us"] * 1e-6) if dom else None
    for name, nb in per_kernel.items():
        if name in kern:
            kern[name]["algorithmic_bytes"] = nb
            kern[name]["hbm_frac"] = nb / (kern[name]["avg_us"] * 1e-6) / HBM_PEAK
    # the verification's time: its kernels (with spec_step, the streaming launch
    # also holds the schedule, so the fraction is a lower bound)
    verify_us = sum(kern[k]["avg_us"] * kern[k]["launches_per_step"]
                    for k in ("verify_step_stream", "verify_stream", "verify_decide") if k in kern)
    return dict(mode=mode, max_len=max_len, ms_per_step=ms_plain, ms_per_step_instrumented=ms_step, N=N,
                rows=int(d.host("n_rows")[0]), tokens_per_s=N / (ms_plain * 1e-3), verify_us=verify_us,
                verify_tokens_per_s=N / (verify_us * 1e-6) if verify_us else None,
                algorithmic_bytes=nbytes, dominant_kernel=dom_name, dominant_bytes=per_kernel[dom_name],
                fused_schedule=fused,
                draft_rows_read=draft_rows, dominant_gbps=achieved / 1e9 if achieved else None,
                dominant_frac=achieved / HBM_PEAK if achieved else None, kernels=kern, step_us_percentiles=pct)


def run_lagged(d, w, mode_c, steps, warmup, B, torch, copies):
    """Lagged scheduling over n_rounds rotating confidence rounds: round t
    verifies lengths scheduled from round t-2's confidences, and the next
    round's schedule runs inside round t's verify launches (spec_verify_ex).
    Timed eagerly and as a replayed HIP graph, next to the synchronous
    schedule-then-verify of the same rounds.
    Goodput: expected emitted tokens per step (R + the current round's survival
    summed over the verified drafts) per unit step time."""
    import numpy as np
    from draft_token_verification_flattened_amd import workloads
    from draft_token_verification_flattened_amd.pipeline import LaggedStep, to_device
    per = 2 * copies if copies % 2 else copies               # batch slots and input copies line up
    n_rounds = per * max(1, 8 // per)                        # the graph replays this many rounds, in a cycle
    n_long = 24                                              # the lag's effect, from a run without wrap-around
    zlong = to_device(workloads.conf_rounds(w, n_long), "cuda")
    zdev = zlong[:n_rounds].contiguous()
    R, k = w.R, w.k
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    stream = torch.cuda.current_stream()

    # per-round lengths and current-round survival (for the goodput)
    i32 = dict(dtype=torch.int32, device="cuda")
    L = torch.zeros(R, **i32)
    tags = torch.zeros(R * (k + 1), 2, **i32)
    cu = torch.zeros(R + 1, **i32)
    nr = torch.zeros(1, **i32)
    sv = torch.zeros(R, k, dtype=torch.float64, device="cuda")
    Ls, Ss = [], []
    for t in range(n_long):
        B.spec_schedule(zlong[t], d.T, d.tbl_b, d.tbl_t, k, L, tags, cu, nr, d.ws_sched, sv)
        torch.cuda.synchronize()
        Ls.append(L.cpu().numpy().copy())
        Ss.append(sv.cpu().numpy().copy())

    def emitted(lengths, S):
        m = np.arange(k)[None, :] < lengths[:, None]
        return R + float((S * m).sum())

    sync_n = [int(Ls[t].sum()) for t in range(n_rounds)]                 # the timed cycle
    lag_n = [int(Ls[(t - 2) % n_rounds].sum()) for t in range(n_rounds)]
    sync_e = [emitted(Ls[t], Ss[t]) for t in range(2, n_long)]
    lag_e = [emitted(Ls[t - 2], Ss[t]) for t in range(2, n_long)]

    # synchronous: [draft(t),] schedule(t) then verify(t), one stream; the same work
    # as a lagged round, which drafts too when the workload has a sequential head
    def sync_step(t):
        d.step_no = t
        if len(d._copies) > 1:
            d.use_copy(t)
        if d.w.backbone is not None:
            d.markov(mode_c)
        d.schedule_verify(mode_c, z=zdev[t % n_rounds])
    for t in range(warmup):
        sync_step(t)
    torch.cuda.synchronize()
    ev0.record(stream)
    for t in range(steps):
        sync_step(t)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms_sync = ev0.elapsed_time(ev1) / steps

    ls = LaggedStep(d, zdev)
    ls.start(0)
    for _ in range(warmup):
        ls.step(mode_c)
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(steps):
        ls.step(mode_c)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms_eager = ev0.elapsed_time(ev1) / steps

    rounds = n_rounds
    ls.start(0)
    g = ls.capture(mode_c, rounds)
    reps = max(1, steps // rounds)
    for _ in range(2):
        ls.start(0)
        g.replay()
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(reps):
        g.replay()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms_graph = ev0.elapsed_time(ev1) / (reps * rounds)
    mean = lambda v: float(np.mean(v))  # noqa: E731
    return dict(
        rounds_timed=n_rounds, rounds_goodput=n_long - 2, lag=2,
        ms_per_step_sync=ms_sync, ms_per_step_lagged=ms_eager, ms_per_step_lagged_graph=ms_graph,
        verified_per_step_sync=mean(sync_n), verified_per_step_lagged=mean(lag_n),
        tokens_per_s_sync=mean(sync_n) / (ms_sync * 1e-3),
        tokens_per_s_lagged_graph=mean(lag_n) / (ms_graph * 1e-3),
        expected_emitted_per_step_sync=mean(sync_e), expected_emitted_per_step_lagged=mean(lag_e),
        goodput_sync=mean(sync_e) / (ms_sync * 1e-3), goodput_lagged_graph=mean(lag_e) / (ms_graph * 1e-3),
        emitted_lost_to_lag=1.0 - mean(lag_e) / mean(sync_e),
    )


def run_sweep(args, B, torch):
    """Load sweep: for R = 1, 2, 4, ..., 512 requests of the c2 recipe (the
    first R requests of one R = 512 draw, so every R sees the same requests),
    8 rounds of drifting confidences, each a synchronous schedule-then-verify
    (spec_step, with the library's counter-based uniforms).
    Per R: mean verified length per request, mean step time, verified draft
    tokens/s and expected emitted tokens/s (R + survival over the verified
    drafts, per unit measured step time)."""
    import dataclasses
    import numpy as np
    from draft_token_verification_flattened_amd import workloads
    from draft_token_verification_flattened_amd.pipeline import DeviceStep, to_device
    full = workloads.make("c2", R=512)
    rounds = 8
    rows = []
    for R in [1, 2, 4, 8, 16, 32, 64, 128, 256, 512]:
        cut = lambda a: None if a is None else np.ascontiguousarray(a[:R])  # noqa: E731
        w = dataclasses.replace(full, R=R, conf_logit=cut(full.conf_logit), target=cut(full.target),
                                draft=cut(full.draft), tokens_sample=cut(full.tokens_sample),
                                tokens_greedy=cut(full.tokens_greedy), u_verify=cut(full.u_verify))
        d = DeviceStep(w, rng=True)
        z = to_device(workloads.conf_rounds(w, rounds), "cuda")
        k = w.k
        Ls, Ss = [], []
        for t in range(rounds):                               # lengths and survival per round
            B.spec_schedule(z[t], d.T, d.tbl_b, d.tbl_t, k, d.lengths, d.tags, d.cu_rows, d.n_rows, d.ws_sched,
                            d.survival)
            torch.cuda.synchronize()
            Ls.append(d.host("lengths").copy())
            Ss.append(d.host("survival").copy())

        def step(t):
            d.step_no += 1
            d.schedule_verify(B.SAMPLE, z=z[t % rounds])
        for t in range(args.warmup):
            step(t)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        n = max(rounds, args.steps // rounds * rounds)
        e0.record()
        for t in range(n):
            step(t)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / n
        meanL = float(np.mean([L.mean() for L in Ls]))
        N = float(np.mean([L.sum() for L in Ls]))
        emitted = float(np.mean([R + float((S * (np.arange(k)[None, :] < L[:, None])).sum())
                                 for L, S in zip(Ls, Ss)]))
        rows.append(dict(R=R, mean_verify_len=meanL, verified_per_step=N, us_per_step=ms * 1e3,
                         verified_tokens_per_s=N / (ms * 1e-3), expected_emitted_per_step=emitted,
                         goodput=emitted / (ms * 1e-3)))
        print(json.dumps(dict(sweep_row=rows[-1])), file=sys.stderr, flush=True)
        del d, z
        torch.cuda.empty_cache()
    print(json.dumps(dict(sweep="c2 recipe, first R of 512 requests, 8 drifting confidence rounds, sampling",
                          rows=rows)))


def run_attention(args, B, torch):
    """spec_attention at R = 256, k = 5 with Qwen3-4B-like heads (32 query heads
    over 8 KV heads, D = 128), 64-key pages drawn from a shuffled pool (head-major
    unless --kv-layout position), contexts uniform in 1024..3072, verified
    lengths uniform in 0..5, flattened by spec_flatten. Algorithmic bytes per
    call: every request's K and V over its visible positions (ctx + L + 1 per KV
    head), the queries and the output."""
    import numpy as np
    from draft_token_verification_flattened_amd import workloads
    from draft_token_verification_flattened_amd.pipeline import to_device
    head = args.kv_layout == "head"
    ai = workloads.make_attention(256, 5, seed=11, head_major=head)
    dev = "cuda"
    R, k = ai.R, ai.k
    q, kc, vc = (to_device(x, dev) for x in (ai.q, ai.k_cache, ai.v_cache))
    pt, ctx = to_device(ai.page_table, dev), to_device(ai.ctx_len, dev)
    i32 = dict(dtype=torch.int32, device=dev)
    tags = torch.zeros(R * (k + 1), 2, **i32)
    cu = torch.zeros(R + 1, **i32)
    nr = torch.zeros(1, **i32)
    B.spec_flatten(to_device(ai.lengths, dev), k, tags, cu, nr)
    out = torch.zeros(R * (k + 1), ai.Hq, ai.D, dtype=torch.float32, device=dev)
    ws = B.workspace(B.attention_workspace_bytes(R, k, ai.Hq, ai.Hkv, ai.page_size, ai.page_table.shape[1],
                                                 args.split_keys), dev)

    def call():
        B.spec_attention(k, ai.page_size, q, kc, vc, pt, ctx, tags, cu, nr, out, ws,
                         kv_layout=B.KV_HEAD_MAJOR if head else B.KV_POSITION_MAJOR, split_keys=args.split_keys)
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    B.timing_reset()
    B.timing_enable(True)
    for _ in range(args.steps):
        call()
    torch.cuda.synchronize()
    B.timing_enable(False)
    kern = {}
    for name in ("attn_partial", "attn_combine"):
        n, tot = B.timing_read(name)
        if n:
            kern[name] = dict(launches_per_call=n / args.steps, avg_us=1000.0 * tot / n)
    B.timing_reset()
    e0.record()
    for _ in range(args.steps):
        call()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / args.steps
    assert B.read_status(ws) == 0
    L = ai.lengths.astype(np.int64)
    rows = int(L.sum()) + R
    kv = int(2 * ai.Hkv * ai.D * 2 * (ai.ctx_len.astype(np.int64) + L + 1).sum())
    qo = rows * ai.Hq * ai.D * (2 + 4)
    nbytes = kv + qo
    part = kern["attn_partial"]["avg_us"]
    print(json.dumps(dict(attention=dict(
        workload=f"R=256, k=5, Hq=32, Hkv=8, D=128, page 64 ({args.kv_layout}-major), ctx 1024..3072, L uniform 0..5",
        rows=rows, us_per_call=us, rows_per_s=rows / (us * 1e-6), algorithmic_bytes=nbytes,
        kv_bytes=kv, call_gbps=nbytes / (us * 1e-6) / 1e9,
        roofline=dict(bound="hbm", kernel="attn_partial", achieved=nbytes / (part * 1e-6) / 1e9,
                      peak=HBM_PEAK / 1e9, unit="GB/s", frac=nbytes / (part * 1e-6) / HBM_PEAK,
                      avg_launch_us=part),
        split_keys=args.split_keys, kernels=kern))))


_CPU = {}


def _oracle_share(job):
    """One worker's share of an oracle step: (Markov head and) verification of
    a contiguous range of requests, on the batch the parent scheduled. Runs in
    a forked worker; the workload sits in _CPU, inherited from the parent."""
    lo, hi, L = job
    import numpy as np
    from oracle import markov as omarkov
    from oracle import schedule as osched
    from oracle import verify as overify
    w, mode, key = _CPU["w"], _CPU["mode"], _CPU["key"]
    sl = slice(lo, hi)
    # the library's counter-based uniforms, as the timed GPU step draws them
    # (requests addressed as in the whole batch)
    rng = (key[0], key[1], lo)
    if w.backbone is not None:
        m = omarkov.markov_draft(mode, w.dtype, w.backbone[sl], w.emb, w.proj, w.prev_token[sl], w.tau, rng=rng)
        dl, tok = m["logits"], m["tokens"]
    else:
        dl = w.draft[sl] if mode == "sample" else None
        tok = (w.tokens_sample if mode == "sample" else w.tokens_greedy)[sl]
    tags, cu = osched.flatten(np.asarray(L[sl]))
    r = overify.verify(mode, w.dtype, w.target[sl], dl, tok, tags, cu, w.tau, rng=rng)
    return int(np.sum(r["accepted_len"]))


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, mode, max_len, min_seconds=10.0):
    """The oracle, as it stands, on the same workload and the host's cores.

    Each step: the schedule (one process), then (the Markov head and)
    verification split over requests among worker processes, one per core
    (fork, before this process touches the GPU), whole steps repeated for at
    least `min_seconds`. A single-core figure times whole steps in one
    process, on a prefix of the requests when the batch is large (at least
    `min_seconds` / 3). The uniforms are the library's counter-based ones, as
    the timed GPU step uses them, addressed by request in the whole batch, so
    every share computes exactly what the whole batch would."""
    import multiprocessing as mp
    import numpy as np
    from oracle import schedule as osched
    try:
        import threadpoolctl
        limit = threadpoolctl.threadpool_limits(1)         # one BLAS thread per process (workers inherit it)
    except Exception:
        limit = None
    cores = max(1, min(16, len(os.sched_getaffinity(0))))
    from draft_token_verification_flattened_amd import workloads
    _CPU.update(w=w, mode=mode, key=(int(workloads.CONFIGS[w.name]["seed"]), 1))
    R = w.R

    def schedule():
        return osched.schedule(w.conf_logit, w.pos_temp, w.tbl_tokens, w.tbl_thr, max_len)["L"]

    # single core: whole steps over the first R1 requests (schedule of the whole batch)
    R1 = min(R, 32)
    reps1, t = 0, time.perf_counter()
    while True:
        L = schedule()
        _oracle_share((0, R1, L))
        reps1 += 1
        dt1 = time.perf_counter() - t
        if dt1 >= min_seconds / 3:
            break
    N1 = int(np.sum(L[:R1]))
    one_core = N1 * reps1 / dt1
    # all cores: the batch split into `cores` request ranges
    edges = np.linspace(0, R, cores + 1).astype(int)
    ctx = mp.get_context("fork")
    with ctx.Pool(cores) as pool:
        reps, t = 0, time.perf_counter()
        while True:
            L = schedule()
            pool.map(_oracle_share, [(int(edges[i]), int(edges[i + 1]), L) for i in range(cores)
                                     if edges[i + 1] > edges[i]])
            reps += 1
            dt = time.perf_counter() - t
            if dt >= min_seconds:
                break
    if limit is not None:
        limit.restore_original_limits()
    N = int(np.sum(L))
    many = N * reps / dt
    sample = (f"{reps} full steps of the workload (R={R}, N={N} verified drafts per step) in {dt:.1f} s: "
              f"the schedule in one process, then the requests split over {cores} worker processes; "
              f"single core: {reps1} steps over the first {R1} requests ({N1} verified drafts) in {dt1:.1f} s")
    # the faster of the two is the baseline (tiny batches lose to the workers' start-up)
    if one_core > many:
        return dict(value=one_core, unit="verified draft tokens/s", cores=1, kind="oracle",
                    cpu_model=_cpu_model(), multi_core_value=many, multi_core_cores=cores,
                    sample=sample + "; one core was faster")
    return dict(value=many, unit="verified draft tokens/s", cores=cores, kind="oracle",
                cpu_model=_cpu_model(), single_core_value=one_core, sample=sample)


def copy_probe(gib):
    import torch
    n = int(gib * (1 << 30))
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n, "copies": 3}))


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus > 1 or world > 1:
        print("bench.py runs on one GPU only: the verification step is measured on a single MI355X; "
              "multi-GPU runs are not part of this build", file=sys.stderr)
        sys.exit(2)
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return

    import numpy as np  # noqa: F401
    import torch
    from draft_token_verification_flattened_amd import binding as B
    from draft_token_verification_flattened_amd import workloads
    from draft_token_verification_flattened_amd.pipeline import DeviceStep

    if torch.cuda.device_count() < 1:          # counts devices without initialising one
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if not os.path.exists(B.LIB_PATH):         # fail loudly if the HIP library is missing
        raise RuntimeError(f"{B.LIB_PATH} is not built: run python -m draft_token_verification_flattened_amd.build")
    if args.sweep:
        B.lib()
        run_sweep(args, B, torch)
        return
    if args.attention:
        B.lib()
        run_attention(args, B, torch)
        return
    w = workloads.make(args.config)
    max_len = w.k if args.max_len == "k" else int(args.max_len)
    # the oracle baseline first: its worker processes are forked before this
    # process touches the GPU
    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(w, args.mode, max_len)
        print(json.dumps(dict(cpu_baseline=cpu)), file=sys.stderr, flush=True)
    B.lib()
    d = DeviceStep(w, copies=args.copies, head=args.head, rng=True)
    mode_c = B.SAMPLE if args.mode == "sample" else B.GREEDY
    main_res = run_variant(d, w, mode_c, args.mode, max_len, args.steps, args.warmup, B, torch)

    extra = {}
    if args.variants:
        for mode in (["sample", "greedy"] if w.backbone is None else ["sample"]):
            for ml in (w.k, -1):
                if mode == args.mode and ml == max_len:
                    continue
                mc = B.SAMPLE if mode == "sample" else B.GREEDY
                r = run_variant(d, w, mc, mode, ml, args.steps, args.warmup, B, torch)
                extra[f"{mode}_{'scheduled' if ml == w.k else 'verify_all'}"] = r

    lagged = None
    if args.variants or args.lagged:
        lagged = run_lagged(d, w, mode_c, args.steps, args.warmup, B, torch, args.copies)

    kern = main_res["kernels"]
    dom_name = main_res["dominant_kernel"]
    ver = kern.get(dom_name, {})
    mk = kern.get("markov_logits")
    roofline = {
        "bound": "hbm",
        "achieved": main_res["dominant_gbps"],
        "peak": HBM_PEAK / 1e9,
        "unit": "GB/s",
        "frac": main_res["dominant_frac"],
        "traffic": committed_traffic(dom_name, workload_key(args, max_len))[0],
        "kernel": dom_name,
        "avg_launch_us": ver.get("avg_us"),
        "algorithmic_bytes_per_launch": main_res["dominant_bytes"],
    }
    markov_roof = None
    if mk and w.dtype == "bf16":
        # the Markov projection: HBM-bound (about 102 flop per byte at d_m = 256,
        # below the bf16 ridge of 2.5e15 / 8e12 = 312), MFMA use reported beside it
        nb, fl = markov_bytes_flops(w)
        t = mk["avg_us"] * 1e-6
        markov_roof = {
            "bound": "hbm", "achieved": nb / t / 1e9, "peak": HBM_PEAK / 1e9, "unit": "GB/s",
            "frac": nb / t / HBM_PEAK,
            "traffic": committed_traffic("markov_logits", workload_key(args, max_len))[0],
            "kernel": "markov_logits", "avg_launch_us": mk["avg_us"], "algorithmic_bytes_per_launch": nb,
            "mfma": {"achieved": fl / t / 1e12, "peak": MFMA_BF16_PEAK / 1e12, "unit": "TFLOP/s",
                     "frac": fl / t / MFMA_BF16_PEAK, "flops_per_launch": fl},
        }
        # the dominant kernel of the step is the one with the larger share of its time
        if mk["avg_us"] * mk["launches_per_step"] > ver.get("avg_us", 0.0) * ver.get("launches_per_step", 0.0):
            roofline, markov_roof = markov_roof, roofline
    out = {
        "metric": METRIC,
        "value": main_res["tokens_per_s"],
        "unit": "verified draft tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"{args.config}: {workloads.CONFIGS[args.config]['desc']}"
                        + (", RNN head" if args.head == "rnn" and w.backbone is not None else ""),
            "R": w.R, "k": w.k, "V": w.V, "storage": w.dtype, "mode": args.mode,
            "tau": w.tau, "max_len": max_len, "verified_drafts_per_step": main_res["N"],
            "flattened_rows_per_step": main_res["rows"], "parallelism": "single GPU",
            "input_copies": args.copies,
        },
        "roofline": roofline,
        "roofline_other": markov_roof,
        "cpu_baseline": cpu,
        "verify_only": {"us_per_step": main_res["verify_us"], "tokens_per_s": main_res["verify_tokens_per_s"],
                        "hbm_frac": (main_res["algorithmic_bytes"] / (main_res["verify_us"] * 1e-6) / HBM_PEAK
                                     if main_res["verify_us"] else None),
                        "algorithmic_bytes": main_res["algorithmic_bytes"],
                        "kernels": [k for k in ("verify_step_stream", "verify_stream", "verify_decide")
                                    if k in main_res["kernels"]]},
        "kernels": main_res["kernels"],
        "ms_per_step_instrumented": main_res["ms_per_step_instrumented"],
        "step_us_percentiles": main_res["step_us_percentiles"],
        "variants": {k: {kk: v[kk] for kk in ("ms_per_step", "ms_per_step_instrumented", "N", "rows",
                                                "tokens_per_s", "verify_us", "verify_tokens_per_s",
                                                "dominant_gbps", "dominant_frac")}
                     for k, v in extra.items()},
        "lagged_schedule": lagged,
        "source_hash": source_hash(),
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
