"""The multi-step load sweep through the GPU, against the oracle and the pages.

For R = 1, 8, 64, 256 and 512 requests of the saturated workload's recipe (the
first R of one 512-request draw; 8 rounds of drifting confidences each, as
bench.py --sweep runs them):
  - spec_schedule's lengths, offsets and tags equal the oracle's, bit for bit,
    every round;
  - the pages' load behaviour ("刚融完500亿创始人亲自下场写代码…", section
    "不止是算法更是“工业级”的系统魔改"): at R = 1 the mean verification length
    L + 1 lies in [4, 6] (tests/golden/pages_facts.json), and the mean length
    does not increase with R;
  - one sampling verify per R (at V = 4096, the recipe otherwise unchanged,
    uniforms from the library's generator) matches the oracle within the
    parity tolerances, so the decide launch shapes of every load (four, two
    and one workgroups per request, 512-thread workgroups above the compute
    unit count) are exercised on scheduled batches.
"""
import dataclasses
import json
import os

import numpy as np
import pytest
import torch

from draft_token_verification_flattened_amd import binding as B
from draft_token_verification_flattened_amd import workloads
from draft_token_verification_flattened_amd.pipeline import DeviceStep, to_device
from oracle import schedule as osched
from oracle import verify as overify

from test_gpu_parity import check_sampling

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "pages_facts.json")
ROUNDS = 8
LOADS = [1, 8, 64, 256, 512]


def say(*a):
    print("[gpu]", *a, flush=True)


@pytest.fixture(scope="module")
def full():
    return workloads.make("c2", R=512, V=4096)


def _cut(full, R):
    cut = lambda a: None if a is None else np.ascontiguousarray(a[:R])  # noqa: E731
    return dataclasses.replace(full, R=R, conf_logit=cut(full.conf_logit), target=cut(full.target),
                               draft=cut(full.draft), tokens_sample=cut(full.tokens_sample),
                               tokens_greedy=cut(full.tokens_greedy), u_verify=cut(full.u_verify))


def test_sweep_schedule_and_verify(full):
    facts = json.load(open(GOLDEN))
    lo, hi = facts["low_concurrency_verify_tokens"]["value"]
    means = []
    for R in LOADS:
        w = _cut(full, R)
        d = DeviceStep(w)
        z = workloads.conf_rounds(w, ROUNDS)
        zd = to_device(z, "cuda")
        Ls = []
        for t in range(ROUNDS):
            say("sweep schedule R", R, "round", t)
            B.spec_schedule(zd[t], d.T, d.tbl_b, d.tbl_t, w.k, d.lengths, d.tags, d.cu_rows, d.n_rows, d.ws_sched)
            torch.cuda.synchronize()
            ref = osched.schedule(z[t], w.pos_temp, w.tbl_tokens, w.tbl_thr, w.k)
            L = d.host("lengths")
            assert np.array_equal(L, ref["L"]), (R, t)
            tags, cu = osched.flatten(ref["L"])
            assert np.array_equal(d.host("cu_rows"), cu)
            assert np.array_equal(d.host("tags")[:osched.n_rows(cu)], tags)
            Ls.append(L)
        means.append(float(np.mean(Ls)))
        # one verify of the last round's batch, with the library's uniforms
        say("sweep verify R", R)
        d.rng, d.step_no = True, 9
        d.verify(B.SAMPLE)
        torch.cuda.synchronize()
        assert B.read_status(d.ws_verify) == 0
        ref = overify.verify("sample", w.dtype, w.target, w.draft, w.tokens_sample, tags, cu, w.tau,
                             rng=(d.seed, 9))
        check_sampling(d, ref, tags, cu, f"sweep R={R} V=4096 philox", rng=(d.seed, 9))
        del d
        torch.cuda.empty_cache()
    say("sweep mean lengths", dict(zip(LOADS, means)))
    assert lo <= means[0] + 1 <= hi, means[0]
    assert all(means[i + 1] <= means[i] + 1e-12 for i in range(len(means) - 1)), means
    assert means[-1] < means[0]
