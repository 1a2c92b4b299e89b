"""Seeded synthetic inputs for the speculative verification path.

This module only draws random numbers and lays them out. It holds none of the
method's arithmetic: no softmax, no acceptance test, no schedule. Both the HIP
path (through the tests and bench.py) and the CPU oracle (through the tests)
consume what it returns; neither imports the other.

Five workloads are defined, sized after the DSpark pages' serving setting
(maximum draft length 5; a Qwen3-like vocabulary of 151936 entries; math, code
and chat traffic with decreasing acceptance). The pages measure on public
math/code/chat suites; those are not used here. The three "domain" profiles of
the saturated workload stand in for them, keeping the pages' ordering of
accepted length (math > code > chat).

Every array comes from numpy's Philox bit generator keyed by the workload seed:
small arrays from one stream in the order written below, the large logit and
weight arrays in blocks of rows, each block from its own stream keyed by
(seed, array, block). A workload is reproducible bit for bit on any host. bf16 arrays are the round-to-nearest-even encoding of fp32 samples and
are stored as their uint16 bit patterns.

Random numbers the method itself consumes (the acceptance uniforms, the
resampling uniform, the Markov head's sampling uniforms) are drawn here as
inputs, float32 values k * 2**-24 in [0, 1).
"""
from __future__ import annotations

import concurrent.futures
import dataclasses
import os
from typing import Optional

import numpy as np

__all__ = ["CONFIGS", "Workload", "make", "f32_to_bf16_bits", "bf16_bits_to_f32",
           "step_time_table"]


# ---------------------------------------------------------------------------
# encoding helpers (storage only)
# ---------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 samples to bfloat16 (nearest, ties to even); uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ---------------------------------------------------------------------------
# workload definitions
# ---------------------------------------------------------------------------

def _table(points, step_time):
    b = np.asarray(points, dtype=np.int32)
    thr = np.array([float(p) / float(step_time(float(p))) for p in points], dtype=np.float64)
    return b, thr


def step_time_table(name: str):
    """Engine throughput table (batch tokens B_j, tokens per unit time thr_j)."""
    if name == "c0":       # concave: step time 1 + 0.08 B
        return _table([4 * j for j in range(1, 9)], lambda b: 1.0 + 0.08 * b)
    if name == "c1":       # flat step time up to 512 tokens
        return _table([64 * j for j in range(1, 9)], lambda b: 1.0)
    if name == "c2":       # soft knee at 256 tokens
        pts = [32, 64, 128, 192, 256, 384, 512, 768, 1024, 1280, 1536, 2048]
        return _table(pts, lambda b: 1.0 if b <= 256 else 1.0 + 0.5 * (b - 256) / 256)
    if name == "c3":       # 16 points up to 4096 tokens
        return _table([256 * j for j in range(1, 17)], lambda b: 1.0 + b / 1024.0)
    if name == "c4":
        pts = [128, 256, 512, 768, 1024, 1536, 2048, 2560, 3072]
        return _table(pts, lambda b: 1.0 if b <= 1024 else 1.0 + 0.5 * (b - 1024) / 1024)
    raise KeyError(name)


CONFIGS = {
    "c0": dict(name="c0", desc="tiny CPU-checkable step: R=4, k=5, V=32, fp32, Markov head rank 4",
               seed=0, R=4, k=5, V=32, dtype="f32", markov=True, d_m=4, tau=1.0,
               modes=("greedy", "sample")),
    "c1": dict(name="c1", desc="light load: R=64, k=5, V=151936, bf16, flat step time to 512 tokens",
               seed=1, R=64, k=5, V=151936, dtype="bf16", markov=False, tau=1.0,
               modes=("greedy", "sample")),
    "c2": dict(name="c2", desc="saturated load: R=256, k=5, V=151936, bf16, knee at 256 batch tokens, "
                                "math/code/chat profiles",
               seed=2, R=256, k=5, V=151936, dtype="bf16", markov=False, tau=1.0,
               modes=("greedy", "sample")),
    "c3": dict(name="c3", desc="long parallel blocks: R=128, k=16, V=129280, bf16, suffix decay, tau=0.7",
               seed=3, R=128, k=16, V=129280, dtype="bf16", markov=False, tau=0.7,
               modes=("sample",)),
    "c4": dict(name="c4", desc="full semi-autoregressive step: R=512, k=5, V=151936, d_m=256, bf16",
               seed=7, R=512, k=5, V=151936, dtype="bf16", markov=True, d_m=256, tau=1.0,
               modes=("sample",)),
}


@dataclasses.dataclass
class Workload:
    name: str
    R: int
    k: int
    V: int
    dtype: str                      # "bf16" (uint16 bit arrays) or "f32"
    tau: float
    conf_logit: np.ndarray          # f32 [R,k]   raw confidence-head logits z
    pos_temp: np.ndarray            # f32 [k]     per-position temperatures
    tbl_tokens: np.ndarray          # i32 [n]
    tbl_thr: np.ndarray             # f64 [n]
    target: np.ndarray              # [R,k+1,V]
    u_verify: np.ndarray            # f32 [R,k+1]  j<k: acceptance; k: resample
    draft: Optional[np.ndarray] = None          # [R,k,V]  (absent for Markov workloads)
    tokens_sample: Optional[np.ndarray] = None  # i32 [R,k] drafts drawn from q at tau
    tokens_greedy: Optional[np.ndarray] = None  # i32 [R,k] argmax of the draft logits
    backbone: Optional[np.ndarray] = None       # [R,k,V]   parallel backbone logits
    emb: Optional[np.ndarray] = None            # [V,d_m]   previous-token embedding
    proj: Optional[np.ndarray] = None           # [V,d_m]   projection, one d_m row per vocab entry
    prev_token: Optional[np.ndarray] = None     # i32 [R]
    rec: Optional[np.ndarray] = None            # [d_m,d_m] RNN-head recurrence A ((A h)_j = sum_k A[j,k] h_k)
    u_draft: Optional[np.ndarray] = None        # f32 [R,k]
    d_m: int = 0


def _recurrence(seed: int, d_m: int, dtype: str) -> np.ndarray:
    """RNN-head recurrence A [d_m, d_m]: N(0, (0.5 / sqrt(d_m))^2) entries (spectral
    radius about 0.5, so the state neither dies out nor saturates over a block),
    from a stream of its own so the workload's other arrays are unchanged."""
    gr = _stream(seed, 3, 0)
    a = np.float32(0.5 / np.sqrt(d_m)) * gr.standard_normal((d_m, d_m), dtype=np.float32)
    return _enc(a, dtype)


def _enc(x32: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return f32_to_bf16_bits(x32)
    return np.ascontiguousarray(x32, dtype=np.float32)


def _dec(x: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_bits_to_f32(x) if dtype == "bf16" else x


def _sample_rows(g: np.random.Generator, logits32: np.ndarray, tau: float) -> np.ndarray:
    """Draw one index per row with probability proportional to exp(logit / tau).

    Gumbel-max: argmax(logit / tau + G), G standard Gumbel.
    """
    rows = logits32.reshape(-1, logits32.shape[-1])
    out = np.empty(rows.shape[0], dtype=np.int32)
    inv_tau = 1.0 / tau
    for i in range(rows.shape[0]):
        u = g.random(rows.shape[1], dtype=np.float64)
        gum = -np.log(-np.log(np.maximum(u, 1e-300)))
        out[i] = np.argmax(rows[i].astype(np.float64) * inv_tau + gum)
    return out.reshape(logits32.shape[:-1])


def _uniform24(g: np.random.Generator, shape) -> np.ndarray:
    # float32 multiples of 2**-24 in [0, 1)
    return (g.integers(0, 1 << 24, size=shape, dtype=np.int64).astype(np.float64) * 2.0 ** -24).astype(np.float32)


# Large arrays are drawn in blocks of rows, each block from its own Philox
# stream keyed by (workload seed, array id, block index), so the result does not
# depend on how many threads fill it.
_BLOCK = 4


def _stream(seed: int, array_id: int, block: int) -> np.random.Generator:
    return np.random.Generator(np.random.Philox(key=(int(seed) << 64) | (int(array_id) << 32) | int(block)))


def _parallel_blocks(n: int, fn):
    blocks = [(b, b * _BLOCK, min(n, (b + 1) * _BLOCK)) for b in range((n + _BLOCK - 1) // _BLOCK)]
    workers = max(1, min(16, os.cpu_count() or 1, len(blocks)))
    if workers == 1:
        for blk in blocks:
            fn(*blk)
        return
    with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as ex:
        list(ex.map(lambda blk: fn(*blk), blocks))


def make(name: str, *, R: Optional[int] = None, V: Optional[int] = None) -> Workload:
    """Build workload `name` ("c0".."c4"). R and V may be shrunk for quick tests;
    the recipe is otherwise unchanged."""
    cfg = dict(CONFIGS[name])
    if R is not None:
        cfg["R"] = R
    if V is not None:
        cfg["V"] = V
    R_, k, V_, dt, tau, seed = cfg["R"], cfg["k"], cfg["V"], cfg["dtype"], cfg["tau"], cfg["seed"]
    g = np.random.Generator(np.random.Philox(seed))
    tbl_b, tbl_thr = step_time_table(name)
    pos_temp = np.linspace(1.0, 2.0, k).astype(np.float32)
    w = dict(name=name, R=R_, k=k, V=V_, dtype=dt, tau=tau, tbl_tokens=tbl_b, tbl_thr=tbl_thr,
             pos_temp=pos_temp)
    st = np.uint16 if dt == "bf16" else np.float32

    if name == "c0":
        tl32 = (2.0 * g.standard_normal((R_, k + 1, V_), dtype=np.float32)).astype(np.float32)
        bk32 = (tl32[:, :k] + g.standard_normal((R_, k, V_), dtype=np.float32)).astype(np.float32)
        sd = np.float32(np.sqrt(0.1))        # N(0, 0.1): variance 0.1
        emb = (sd * g.standard_normal((V_, cfg["d_m"]), dtype=np.float32)).astype(np.float32)
        proj = (sd * g.standard_normal((V_, cfg["d_m"]), dtype=np.float32)).astype(np.float32)
        prev = g.integers(0, V_, size=R_, dtype=np.int64).astype(np.int32)
        z = (1.0 + g.standard_normal((R_, k), dtype=np.float32)).astype(np.float32)
        w.update(target=_enc(tl32, dt), backbone=_enc(bk32, dt), emb=emb, proj=proj,
                 prev_token=prev, conf_logit=z, d_m=cfg["d_m"], rec=_recurrence(seed, cfg["d_m"], dt))
    elif name in ("c1", "c2", "c3"):
        target = np.empty((R_, k + 1, V_), dtype=st)
        draft = np.empty((R_, k, V_), dtype=st)
        tok_g = np.empty((R_, k), dtype=np.int32)
        tok_s = np.empty((R_, k), dtype=np.int32)
        if name == "c3":
            sig = (0.5 + 3.5 * np.arange(k) / (k - 1)).astype(np.float32)   # suffix decay
        else:
            sig = np.full(k, 1.5, dtype=np.float32)

        def fill(b, lo, hi):
            gb = _stream(seed, 1, b)
            tl32 = np.float32(3.0) * gb.standard_normal((hi - lo, k + 1, V_), dtype=np.float32)
            target[lo:hi] = _enc(tl32, dt)
            d32 = tl32[:, :k] + sig[None, :, None] * gb.standard_normal((hi - lo, k, V_), dtype=np.float32)
            draft[lo:hi] = _enc(d32, dt)
            dd = _dec(draft[lo:hi], dt)
            tok_g[lo:hi] = np.argmax(dd, axis=-1)
            tok_s[lo:hi] = _sample_rows(gb, dd, tau)

        _parallel_blocks(R_, fill)
        if name == "c3":
            mu = np.linspace(1.5, -2.5, k)
            z = (mu[None, :] + 0.5 * g.standard_normal((R_, k))).astype(np.float32)
        else:
            if name == "c1":
                m = np.broadcast_to(0.9 * 0.85 ** np.arange(k), (R_, k))
            else:
                # math / code / chat thirds of the requests
                dom = np.minimum((np.arange(R_) * 3) // max(R_, 1), 2)
                m = np.broadcast_to(np.array([0.92, 0.88, 0.75])[dom][:, None], (R_, k))
            raw = np.clip(g.beta(20.0 * m, 20.0 * (1.0 - m)), 1e-12, 1.0 - 1e-12)
            z = np.log(raw / (1.0 - raw)).astype(np.float32)
        w.update(target=target, draft=draft, tokens_greedy=tok_g, tokens_sample=tok_s, conf_logit=z)
    elif name == "c4":
        d_m = cfg["d_m"]
        target = np.empty((R_, k + 1, V_), dtype=st)
        backbone = np.empty((R_, k, V_), dtype=st)
        emb = np.empty((V_, d_m), dtype=st)
        proj = np.empty((V_, d_m), dtype=st)

        def fill_rows(b, lo, hi):
            gb = _stream(seed, 1, b)
            tl32 = np.float32(3.0) * gb.standard_normal((hi - lo, k + 1, V_), dtype=np.float32)
            target[lo:hi] = _enc(tl32, dt)
            bk32 = tl32[:, :k] + np.float32(1.5) * gb.standard_normal((hi - lo, k, V_), dtype=np.float32)
            backbone[lo:hi] = _enc(bk32, dt)

        def fill_vocab(b, lo, hi):
            lo, hi = lo * 1024, min(V_, hi * 1024)
            gb = _stream(seed, 2, b)
            emb[lo:hi] = _enc(gb.standard_normal((hi - lo, d_m), dtype=np.float32), dt)
            proj[lo:hi] = _enc(np.float32(0.5 / 16) * gb.standard_normal((hi - lo, d_m), dtype=np.float32), dt)

        _parallel_blocks(R_, fill_rows)
        _parallel_blocks((V_ + 1023) // 1024, fill_vocab)
        prev = g.integers(0, V_, size=R_, dtype=np.int64).astype(np.int32)
        z = (1.0 + g.standard_normal((R_, k), dtype=np.float32)).astype(np.float32)
        w.update(target=target, backbone=backbone, emb=emb, proj=proj, prev_token=prev,
                 conf_logit=z, d_m=d_m, rec=_recurrence(seed, d_m, dt))
    else:
        raise KeyError(name)

    w["u_verify"] = _uniform24(g, (R_, k + 1))
    w["u_draft"] = _uniform24(g, (R_, k))
    return Workload(**w)


def conf_rounds(w: Workload, n_rounds: int, rho: float = 0.8, sigma: float = 0.75,
                seed: int = 99) -> np.ndarray:
    """Confidence-head logits for n_rounds consecutive rounds of the same
    requests, f32 [n_rounds, R, k]: round 0 is w.conf_logit, and each later
    round adds a stationary AR(1) drift, d_t = rho d_(t-1) + sqrt(1 - rho^2)
    sigma e_t (e standard normal, Philox keyed by the workload seed and `seed`),
    so a schedule made from older confidences sees a different state than the
    round it is used for."""
    g = _stream(int(CONFIGS[w.name]["seed"]), seed, 0)
    R, k = w.conf_logit.shape
    out = np.empty((n_rounds, R, k), dtype=np.float32)
    d = np.zeros((R, k), dtype=np.float64)
    s = float(np.sqrt(1.0 - rho * rho)) * sigma
    for t in range(n_rounds):
        if t > 0:
            d = rho * d + s * g.standard_normal((R, k))
        out[t] = (w.conf_logit.astype(np.float64) + d).astype(np.float32)
    return out


@dataclasses.dataclass
class AttnInputs:
    """Inputs of the tag-masked attention over a flattened batch."""
    R: int
    k: int
    Hq: int
    Hkv: int
    D: int
    page_size: int
    lengths: np.ndarray             # i32 [R]   verified drafts per request (the batch to flatten)
    ctx_len: np.ndarray             # i32 [R]   cached positions before the block
    q: np.ndarray                   # bf16 bits [R*(k+1), Hq, D]   one query per flattened row
    k_cache: np.ndarray             # bf16 bits [pages, page_size, Hkv, D]
    v_cache: np.ndarray             # bf16 bits [pages, page_size, Hkv, D]
    page_table: np.ndarray          # i32 [R, max_pages]
    head_major: bool = False        # pools [pages, Hkv, page_size, D] instead of [pages, page_size, Hkv, D]


def make_attention(R: int, k: int, *, Hq: int = 32, Hkv: int = 8, D: int = 128, page_size: int = 64,
                   ctx_range=(1024, 3072), lengths: Optional[np.ndarray] = None, seed: int = 11,
                   head_major: bool = False) -> AttnInputs:
    """Synthetic attention inputs: N(0, 1) queries, keys and values in bf16;
    context lengths uniform in ctx_range; each request's pages drawn without
    replacement from a shuffled pool with room for ctx + k + 1 positions; per
    request verified lengths uniform in 0 .. k unless given. head_major: pools
    [pages, Hkv, page_size, D] instead of [pages, page_size, Hkv, D]."""
    g = np.random.Generator(np.random.Philox(key=(int(seed) << 64) | 0xA77))
    if lengths is None:
        lengths = g.integers(0, k + 1, size=R).astype(np.int32)
    ctx = g.integers(ctx_range[0], ctx_range[1] + 1, size=R).astype(np.int32)
    need = (ctx.astype(np.int64) + k + 1 + page_size - 1) // page_size
    max_pages = int(need.max())
    n_pages = int(need.sum())
    perm = g.permutation(n_pages).astype(np.int32)
    table = np.zeros((R, max_pages), dtype=np.int32)
    o = 0
    for r in range(R):
        table[r, :need[r]] = perm[o:o + need[r]]
        o += int(need[r])
    q = f32_to_bf16_bits(g.standard_normal((R * (k + 1), Hq, D), dtype=np.float32))

    def pool(array_id):
        shape = (Hkv, page_size, D) if head_major else (page_size, Hkv, D)
        out = np.empty((n_pages,) + shape, dtype=np.uint16)

        def fill(b, lo, hi):
            gg = _stream(seed, array_id, b)
            out[lo:hi] = f32_to_bf16_bits(gg.standard_normal((hi - lo,) + shape, dtype=np.float32))
        _parallel_blocks(n_pages, fill)
        return out
    return AttnInputs(R=R, k=k, Hq=Hq, Hkv=Hkv, D=D, page_size=page_size, lengths=lengths, ctx_len=ctx,
                      q=q, k_cache=pool(40), v_cache=pool(41), page_table=table, head_major=head_major)
