"""Repeated draft-and-verify trials on a tiny prefix-dependent model, for
chi-square tests of losslessness (test code: drafts are drawn here from q)."""
import numpy as np
from scipy import stats

from oracle import numerics


class LogitModel:
    """Prefix-dependent target and draft logits for V = 8; prefixes longer than
    3 share one row (they cannot affect the first 4 emitted tokens)."""

    def __init__(self, V=8, depth=3, seed=0):
        g = np.random.Generator(np.random.Philox(seed))
        self.V, self.depth = V, depth
        self.offsets = [0]
        for l in range(depth):
            self.offsets.append(self.offsets[-1] + V ** l)
        n_rows = self.offsets[-1] + V ** depth + 1
        self.tl = (1.2 * g.standard_normal((n_rows, V))).astype(np.float32)
        self.dl = (self.tl + 0.9 * g.standard_normal((n_rows, V))).astype(np.float32)
        self.shared = n_rows - 1

    def code(self, toks, lens):
        """Row of each prefix toks[i, :lens[i]]."""
        V = self.V
        code = np.full(len(lens), self.shared, dtype=np.int64)
        for l in range(self.depth + 1):
            sel = lens == l
            if not sel.any():
                continue
            c = np.zeros(sel.sum(), dtype=np.int64)
            for t in range(l):
                c = c * V + toks[sel, t]
            code[sel] = self.offsets[l] + c
        return code

    def target_probs(self, n):
        """Exact (float64) probability of every length-n sequence."""
        P = numerics.softmax(self.tl.astype(np.float64), 1.0)
        seqs = np.array(np.meshgrid(*[np.arange(self.V)] * n, indexing="ij")).reshape(n, -1).T
        pr = np.ones(len(seqs))
        for t in range(n):
            rows = self.code(seqs, np.full(len(seqs), t))
            pr *= P[rows, seqs[:, t]]
        return seqs, pr


def run_trials(model, n_trials, k, seed, verify_fn, batch=1_000_000, rows=False):
    """Draft from q, verify, repeat until n = k+1 tokens are emitted; count the
    first n emitted tokens of every trial. verify_fn(P, Qd, x, L, u) -> (a, out),
    or with rows=True verify_fn(row_codes [A,k+1], x, L, u) -> (a, out) so that a
    verifier working on logits can look the rows up itself."""
    V, n = model.V, k + 1
    g = np.random.Generator(np.random.Philox(seed))
    Pt = numerics.softmax(model.tl.astype(np.float64), 1.0)
    Qt = numerics.softmax(model.dl.astype(np.float64), 1.0)
    counts = np.zeros(V ** n, dtype=np.int64)
    for s in range(0, n_trials, batch):
        T = min(batch, n_trials - s)
        ctx = np.zeros((T, n + k + 1), dtype=np.int64)
        lens = np.zeros(T, dtype=np.int64)
        active = np.arange(T)
        while len(active):
            A = len(active)
            toks = np.zeros((A, n + k + 1), dtype=np.int64)
            toks[:] = ctx[active]
            ln = lens[active].copy()
            x = np.zeros((A, k), dtype=np.int64)
            rows_p = np.zeros((A, k + 1), dtype=np.int64)
            for j in range(k + 1):
                code = model.code(toks, ln + j)
                rows_p[:, j] = code
                if j < k:
                    c = np.cumsum(Qt[code], axis=1)
                    x[:, j] = np.minimum((c <= g.random(A)[:, None]).sum(axis=1), V - 1)
                    toks[np.arange(A), ln + j] = x[:, j]
            L = g.integers(0, k + 1, size=A)
            u = (g.integers(0, 1 << 24, size=(A, k + 1)) * 2.0 ** -24)
            if rows:
                a, out = verify_fn(rows_p, x, L, u)
            else:
                a, out = verify_fn(Pt[rows_p], Qt[rows_p[:, :k]], x, L, u)
            for j in range(k + 1):
                put = (j <= a) & (lens[active] + j < n + k + 1)
                idx = active[put]
                ctx[idx, lens[idx] + j] = out[put, j]
            lens[active] += a + 1
            active = active[lens[active] < n]
        code = np.zeros(T, dtype=np.int64)
        for t in range(n):
            code = code * V + ctx[:, t]
        counts += np.bincount(code, minlength=V ** n)
    return counts


def chi2_pvalue(counts, probs, min_expected=5.0):
    """Pearson chi-square p-value; cells expected below min_expected are pooled."""
    exp = probs / probs.sum() * counts.sum()
    small = exp < min_expected
    obs = np.concatenate([counts[~small], [counts[small].sum()]])
    ex = np.concatenate([exp[~small], [exp[small].sum()]])
    if ex[-1] == 0:
        obs, ex = obs[:-1], ex[:-1]
    return stats.chisquare(obs, ex).pvalue
