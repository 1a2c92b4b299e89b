"""Device buffers for one workload and the calls of one speculative step.

Holds the inputs of a workload in HBM and the outputs of each call, and strings
the library calls together: (Markov draft) -> schedule -> verify. Marshalling
only; all computation happens in libspecv's kernels.
"""
from __future__ import annotations

import numpy as np
import torch

from . import binding as B
from .workloads import CONFIGS, Workload


def to_device(a: np.ndarray, device) -> torch.Tensor:
    if a.dtype == np.uint16:                         # bf16 bit patterns
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


class DeviceStep:
    """`copies` > 1 keeps that many copies of the large read-only inputs (target
    logits, draft logits, Markov backbone logits) and moves to the next copy at
    every step, so that no step finds the previous step's logits in the 256 MB
    Infinity Cache.

    rng=False: the calls take the workload's uniform arrays. rng=True: the
    library draws its own counter-based uniforms keyed by (seed, step), seed =
    the workload's seed and step = a counter that step() advances, so every
    step makes fresh decisions."""

    def __init__(self, w: Workload, device="cuda", copies: int = 1, head: str = "markov", rng: bool = False):
        self.w = w
        self.device = device
        self.rng = rng
        self.fused = True                   # step(): schedule and verification in one spec_step call
        self.seed = int(CONFIGS[w.name]["seed"])
        self.step_no = 0
        R, k, V = w.R, w.k, w.V
        dev = lambda a: None if a is None else to_device(a, device)   # noqa: E731
        self.target = dev(w.target)
        self.draft_in = dev(w.draft)
        self.tok_greedy = dev(w.tokens_greedy)
        self.tok_sample = dev(w.tokens_sample)
        self.z = dev(w.conf_logit)
        self.T = dev(w.pos_temp)
        self.tbl_b = dev(w.tbl_tokens)
        self.tbl_t = dev(w.tbl_thr)
        self.u_verify = dev(w.u_verify)
        self.u_draft = dev(w.u_draft)
        self.backbone = dev(w.backbone)
        self.emb = dev(w.emb)
        self.proj = dev(w.proj)
        self.prev = dev(w.prev_token)
        self.head = head                                 # "markov" or "rnn": the sequential module
        self.rec = dev(w.rec) if head == "rnn" else None
        big = ("target", "draft_in", "backbone")
        self._copies = [{n: getattr(self, n) for n in big}]
        for _ in range(max(1, int(copies)) - 1):
            self._copies.append({n: None if getattr(self, n) is None else getattr(self, n).clone() for n in big})
        self._turn = 0
        i32 = dict(dtype=torch.int32, device=device)
        self.lengths = torch.zeros(R, **i32)
        self.tags = torch.zeros(R * (k + 1), 2, **i32)
        self.cu_rows = torch.zeros(R + 1, **i32)
        self.n_rows = torch.zeros(1, **i32)
        self.survival = torch.zeros(R, k, dtype=torch.float64, device=device)
        self.acc_len = torch.zeros(R, **i32)
        self.out_tokens = torch.zeros(R, k + 1, **i32)
        self.diag = torch.zeros(R * (k + 1), 4, dtype=torch.float32, device=device)
        self.ws_verify = B.workspace(B.verify_workspace_bytes(R, k, V), device)
        self.ws_sched = B.workspace(B.schedule_workspace_bytes(R, k), device)
        # the draft head's per-row softmax states (sampling): spec_verify_ex then
        # skips the pass over the draft rows (use_stats)
        self.use_stats = True
        self.draft_stats = None
        if w.backbone is not None:
            self.draft_tokens = torch.zeros(R, k, **i32)
            self.draft_logits = torch.zeros(R, k, V, dtype=self.backbone.dtype, device=device)
            self.draft_stats = torch.zeros(R, k, B.DRAFT_STAT_WORDS, dtype=torch.float32, device=device)
            nbytes = (B.rnn_workspace_bytes if head == "rnn" else B.markov_workspace_bytes)(R, k, V, w.d_m)
            self.ws_markov = B.workspace(nbytes, device)

    # -- calls ---------------------------------------------------------------
    def schedule(self, max_len=None, stream=None):
        max_len = self.w.k if max_len is None else max_len
        B.spec_schedule(self.z, self.T, self.tbl_b, self.tbl_t, max_len, self.lengths, self.tags, self.cu_rows,
                        self.n_rows, self.ws_sched, self.survival, stream=stream)

    def flatten(self, lengths: torch.Tensor, stream=None):
        B.spec_flatten(lengths, self.w.k, self.tags, self.cu_rows, self.n_rows, stream=stream)

    def uniforms(self, which):
        """Keyword arguments that select the uniforms of a call: the workload's
        array `which`, or (rng) the library's generator at (seed, step_no)."""
        if self.rng:
            return dict(uniforms=None, seed=self.seed, step=self.step_no)
        return dict(uniforms=getattr(self, which), seed=self.seed, step=self.step_no)

    def markov(self, mode, stream=None):
        """The drafter's sequential module: the Markov head, or the RNN head."""
        u = self.uniforms("u_draft")
        if self.head == "rnn":
            B.rnn_draft(mode, self.backbone, self.emb, self.rec, self.proj, self.prev, self.w.tau, u["uniforms"],
                        self.draft_tokens, self.draft_logits, self.ws_markov, stream=stream, seed=u["seed"],
                        step=u["step"], stats_out=self.draft_stats)
        else:
            B.markov_draft(mode, self.backbone, self.emb, self.proj, self.prev, self.w.tau, u["uniforms"],
                           self.draft_tokens, self.draft_logits, self.ws_markov, stream=stream, seed=u["seed"],
                           step=u["step"], stats_out=self.draft_stats)

    def stats_for(self, mode, draft=None, tokens=None):
        """The draft statistics to hand to verification: the head's, when it
        verifies the head's own drafts in sampling mode and use_stats is on."""
        if mode == B.SAMPLE and self.use_stats and self.draft_stats is not None and draft is None and tokens is None:
            return self.draft_stats
        return None

    def drafts(self, mode):
        """(draft logits, draft tokens) the verifier uses for this workload and mode."""
        if self.w.backbone is not None:
            return self.draft_logits, self.draft_tokens
        return self.draft_in, (self.tok_sample if mode == B.SAMPLE else self.tok_greedy)

    def verify(self, mode, draft=None, tokens=None, diag=True, stream=None):
        d, t = self.drafts(mode)
        st = self.stats_for(mode, draft, tokens)
        d = d if draft is None else draft
        t = t if tokens is None else tokens
        u = self.uniforms("u_verify")
        B.spec_verify(mode, self.target, d, t, self.tags, self.cu_rows, self.n_rows, self.w.tau, u["uniforms"],
                      self.acc_len, self.out_tokens, self.ws_verify, row_diag=self.diag if diag else None,
                      stream=stream, seed=u["seed"], step=u["step"], draft_stats=st)

    def use_copy(self, i: int):
        for n, t in self._copies[i % len(self._copies)].items():
            setattr(self, n, t)

    def schedule_verify(self, mode, max_len=None, diag=False, stream=None, z=None):
        """This round's schedule (from the confidence logits z, default the
        workload's), then its verification, in one spec_step call (the schedule
        beside the stream of the rows (r, 0), in the same launch)."""
        max_len = self.w.k if max_len is None else max_len
        job = B.schedule_job(self.z if z is None else z, self.T, self.tbl_b, self.tbl_t, max_len, self.lengths, self.tags, self.cu_rows,
                             self.n_rows, self.ws_sched, self.survival)
        d, t = self.drafts(mode)
        u = self.uniforms("u_verify")
        B.spec_step(job, mode, self.target, d, t, self.w.tau, u["uniforms"], self.acc_len, self.out_tokens,
                    self.ws_verify, row_diag=self.diag if diag else None, stream=stream, seed=u["seed"],
                    step=u["step"], draft_stats=self.stats_for(mode))

    def step(self, mode, max_len=None, diag=False, stream=None):
        """One pass of the hot path: (Markov draft,) schedule + flatten, verify;
        with fused (the default) the schedule and the verification are one
        spec_step call."""
        self.step_no += 1
        if len(self._copies) > 1:
            self._turn += 1
            self.use_copy(self._turn)
        if self.w.backbone is not None:
            self.markov(mode, stream=stream)
        if self.fused:
            self.schedule_verify(mode, max_len, diag=diag, stream=stream)
        else:
            self.schedule(max_len, stream=stream)
            self.verify(mode, diag=diag, stream=stream)

    # -- readback ------------------------------------------------------------
    def host(self, name) -> np.ndarray:
        return getattr(self, name).cpu().numpy()


class LaggedStep:
    """Asynchronous lagged scheduling over a run of rounds.

    The lengths verified in round t come from the confidences of round
    t - lag (lag = 2: the schedule for round t+1 is made while round t is
    verified, from the confidences known before round t). Each round is one
    spec_verify_ex call: it verifies round t from batch slot t % 2 and, as one
    more workgroup of its decide launch, schedules round t+1 into slot
    (t+1) % 2, so the schedule leaves the critical path without a second
    stream or any event. Every launch has a fixed capacity (R (k+1) rows), so
    a run of rounds can be captured into a HIP graph and replayed (capture()).
    Marshalling only.
    """

    def __init__(self, d: DeviceStep, z_rounds: torch.Tensor, lag: int = 2):
        self.d = d
        self.z = z_rounds                     # f32 [n, R, k] on the device
        self.n = int(z_rounds.shape[0])
        self.lag = lag
        w, dev = d.w, d.device
        R, k = w.R, w.k
        i32 = dict(dtype=torch.int32, device=dev)
        self.lengths = [torch.zeros(R, **i32) for _ in range(2)]
        self.tags = [torch.zeros(R * (k + 1), 2, **i32) for _ in range(2)]
        self.cu_rows = [torch.zeros(R + 1, **i32) for _ in range(2)]
        self.n_rows = [torch.zeros(1, **i32) for _ in range(2)]
        self.survival = [torch.zeros(R, k, dtype=torch.float64, device=dev) for _ in range(2)]
        self.acc_len = [torch.zeros(R, **i32) for _ in range(2)]
        self.out_tokens = [torch.zeros(R, k + 1, **i32) for _ in range(2)]
        self.t = 0

    def _job(self, slot: int, rnd: int):
        d = self.d
        return B.schedule_job(self.z[rnd % self.n], d.T, d.tbl_b, d.tbl_t, d.w.k, self.lengths[slot],
                              self.tags[slot], self.cu_rows[slot], self.n_rows[slot], d.ws_sched,
                              self.survival[slot])

    def start(self, t0: int = 0):
        """Schedule round t0 (from the confidences lag rounds before it); round
        t0 is the next to verify."""
        self.t = t0
        d, s = self.d, t0 % 2
        B.spec_schedule(self.z[(t0 - self.lag) % self.n], d.T, d.tbl_b, d.tbl_t, d.w.k, self.lengths[s],
                        self.tags[s], self.cu_rows[s], self.n_rows[s], d.ws_sched, self.survival[s])

    def step(self, mode, diag=False):
        """Verify round t; schedule round t+1 in the same launches."""
        d, t = self.d, self.t
        s, o = t % 2, (t + 1) % 2
        if len(d._copies) > 1:
            d.use_copy(t)
        d.step_no = t
        if d.w.backbone is not None:
            d.markov(mode)
        dl, tk = d.drafts(mode)
        u = d.uniforms("u_verify")
        B.spec_verify(mode, d.target, dl, tk, self.tags[s], self.cu_rows[s], self.n_rows[s], d.w.tau,
                      u["uniforms"], self.acc_len[s], self.out_tokens[s], d.ws_verify,
                      row_diag=d.diag if diag else None, next_job=self._job(o, t + 1 - self.lag), seed=u["seed"],
                      step=u["step"], draft_stats=d.stats_for(mode))
        self.t = t + 1

    def capture(self, mode, rounds: int):
        """A HIP graph of `rounds` consecutive rounds (even, so the batch slots
        line up on replay) starting at the current round; each round keeps its
        own confidence round on every replay."""
        assert rounds % 2 == 0
        t0 = self.t
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(rounds):
                self.step(mode)
        self.t = t0
        return g
