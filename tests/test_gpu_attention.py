"""spec_attention (tag-masked attention of the flattened rows over a paged KV
cache) against the float64 oracle.

Tolerance, from the arithmetic: the scores and sums are float32 over exact
bf16 products, and each softmax weight enters the weighted sum of values
rounded to bf16 (relative error at most 2^-8), so per output element
|out - ref| <= 2^-8 * sum_p w_p |v_p| plus float32 accumulation and score
rounding, which stay far below 2^-12 of the same sum for these sizes. The
bound sum_p w_p |v_p| is the oracle itself run on |V|. The tags and row
offsets come from the oracle's flatten, not from the library.
"""
import numpy as np
import pytest
import torch

from draft_token_verification_flattened_amd import binding as B
from draft_token_verification_flattened_amd import workloads
from draft_token_verification_flattened_amd.pipeline import to_device
from oracle import attention as oatt
from oracle import schedule as osched

pytestmark = pytest.mark.gpu

REL = 2.0 ** -8 + 2.0 ** -12


def _batch(ai, lengths):
    """Flattened tags (padded to R*(k+1) rows), cu_rows, n_rows from the oracle's flatten."""
    tags, cu = osched.flatten(lengths)
    n = osched.n_rows(cu)
    full = np.zeros((ai.R * (ai.k + 1), 2), dtype=np.int32)
    full[:n] = tags
    return full, cu.astype(np.int32), n


def _run(ai, tags, cu, n, split_keys=0, page_table=None, ctx_len=None):
    dev = "cuda"
    pt = ai.page_table if page_table is None else page_table
    ctx = ai.ctx_len if ctx_len is None else ctx_len
    q, kc, vc = (to_device(x, dev) for x in (ai.q, ai.k_cache, ai.v_cache))
    out = torch.full((ai.R * (ai.k + 1), ai.Hq, ai.D), float("nan"), dtype=torch.float32, device=dev)
    ws = B.workspace(B.attention_workspace_bytes(ai.R, ai.k, ai.Hq, ai.Hkv, ai.page_size, pt.shape[1],
                                                 split_keys), dev)
    B.spec_attention(ai.k, ai.page_size, q, kc, vc, to_device(pt, dev), to_device(ctx, dev),
                     to_device(tags, dev), to_device(cu, dev), to_device(np.array([n], np.int32), dev), out, ws,
                     kv_layout=B.KV_HEAD_MAJOR if ai.head_major else B.KV_POSITION_MAJOR, split_keys=split_keys)
    status = B.read_status(ws)
    return out.cpu().numpy().astype(np.float64), status


def _oracle(ai, tags, rows, ctx_len=None):
    ctx = ai.ctx_len if ctx_len is None else ctx_len
    q = ai.q[rows]
    t = tags[rows]
    ref = oatt.flat_attention(q, ai.k_cache, ai.v_cache, ai.page_table, ctx, t, len(rows), ai.page_size,
                              head_major=ai.head_major)
    bound = oatt.flat_attention(q, ai.k_cache, ai.v_cache & np.uint16(0x7FFF), ai.page_table, ctx, t,
                                len(rows), ai.page_size, head_major=ai.head_major)
    return ref, bound


def _check(got, ref, bound, what):
    err = np.abs(got - ref)
    tol = REL * bound + 1e-6
    bad = err > tol
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {bad.size} outside tolerance; worst excess "
                           f"{float((err - tol).max()):.3g}, max err {float(err.max()):.3g}")


CASES = {
    # name: (R, k, Hq, Hkv, page_size, ctx_range, lengths)
    "gqa4_small_pages": (6, 5, 8, 2, 32, (0, 150), [0, 5, 3, 1, 5, 2]),
    "mha_g1": (4, 3, 4, 4, 64, (30, 200), [3, 0, 2, 3]),
    "long_block_chunks": (3, 16, 8, 2, 32, (0, 100), [16, 0, 9]),
    "qwen_heads": (5, 5, 32, 8, 64, (100, 400), [0, 5, 3, 5, 1]),
}


@pytest.mark.parametrize("name", sorted(CASES))
@pytest.mark.parametrize("split_keys", [0, 32, 96])
@pytest.mark.parametrize("head_major", [False, True])
def test_attention_matches_oracle(name, split_keys, head_major):
    R, k, Hq, Hkv, ps, cr, lengths = CASES[name]
    print(f"[gpu] spec_attention {name} split_keys={split_keys} head_major={head_major}", flush=True)
    ai = workloads.make_attention(R, k, Hq=Hq, Hkv=Hkv, page_size=ps, ctx_range=cr,
                                  lengths=np.array(lengths, np.int32), seed=5, head_major=head_major)
    ai.ctx_len[0] = 0                      # a row that sees one key only (L_0 = 0) or a short block
    tags, cu, n = _batch(ai, ai.lengths)
    got, status = _run(ai, tags, cu, n, split_keys)
    assert status == 0
    ref, bound = _oracle(ai, tags, np.arange(n))
    _check(got[:n], ref, bound, name)
    assert np.isnan(got[n:]).all()         # rows past n_rows untouched


@pytest.mark.parametrize("head_major", [True, False])
def test_attention_bench_size_sampled(head_major):
    """R = 256, k = 5, 32 query heads over 8 KV heads, D = 128, 64-key pages,
    contexts 1024..3072: the launch configuration of the benchmark (head-major
    pages); sampled rows against the oracle, every row finite, repeat calls
    bit-identical."""
    print(f"[gpu] spec_attention bench size head_major={head_major}", flush=True)
    ai = workloads.make_attention(256, 5, seed=11, head_major=head_major)
    tags, cu, n = _batch(ai, ai.lengths)
    got, status = _run(ai, tags, cu, n)
    again, _ = _run(ai, tags, cu, n)
    assert status == 0
    assert np.isfinite(got[:n]).all()
    assert np.array_equal(got[:n], again[:n])
    g = np.random.default_rng(3)
    longest = int(np.argmax(ai.ctx_len))
    rows = set(g.choice(n, 40, replace=False).tolist())
    rows |= {n - 1, int(cu[-1]) + longest}                     # last bonus row, the longest context's bonus row
    rows = np.array(sorted(rows))
    ref, bound = _oracle(ai, tags, rows)
    _check(got[rows], ref, bound, "bench size")


def test_attention_data_errors():
    """A row with a wrong tag is written as zeros (BAD_TAG); a request with a
    page id out of range, a context overrunning its page-table row, or a
    negative context is written as zeros (BAD_PAGE); the other rows are exact."""
    print("[gpu] spec_attention data errors", flush=True)
    ai = workloads.make_attention(6, 5, Hq=8, Hkv=2, page_size=32, ctx_range=(40, 120),
                                  lengths=np.array([2, 5, 0, 3, 4, 1], np.int32), seed=8)
    tags, cu, n = _batch(ai, ai.lengths)
    ref, bound = _oracle(ai, tags, np.arange(n))
    bad_row = int(cu[1]) + 2               # request 1, position 2
    t2 = tags.copy()
    t2[bad_row, 1] = 4
    got, status = _run(ai, t2, cu, n)
    assert status == B.STATUS_BAD_TAG
    assert (got[bad_row] == 0).all()
    keep = np.array([t for t in range(n) if t != bad_row])
    _check(got[keep], ref[keep], bound[keep], "bad tag, other rows")

    def rows_of(r):
        return [t for t in range(n) if tags[t, 0] == r]

    pt = ai.page_table.copy()
    pt[3, 1] = ai.k_cache.shape[0] + 7     # request 3, its second page
    ctx = ai.ctx_len.copy()
    ctx[4] = ai.page_table.shape[1] * ai.page_size        # overruns the row
    ctx[5] = -1
    got, status = _run(ai, tags, cu, n, page_table=pt, ctx_len=ctx)
    assert status == B.STATUS_BAD_PAGE
    zero = rows_of(3) + rows_of(4) + rows_of(5)
    assert (got[zero] == 0).all()
    keep = np.array([t for t in range(n) if t not in zero])
    _check(got[keep], ref[keep], bound[keep], "bad pages, other rows")
