"""spec_verify_noalloc (the static-scratch variant of spec_verify) through the C
ABI, against spec_verify with a workspace: the same kernels, so every output
must be bit-identical. Two calls in a row, the second with a smaller batch (the
scratch keeps the first call's contents), a status word through status_out,
and a batch above the scratch limit, which must be refused before anything is
enqueued."""
import numpy as np
import pytest
import torch

from draft_token_verification_flattened_amd import binding as B
from draft_token_verification_flattened_amd import workloads
from draft_token_verification_flattened_amd.pipeline import to_device

pytestmark = pytest.mark.gpu


def say(*a):
    print("[gpu]", *a, flush=True)


def _inputs(R, k, V, seed):
    g = np.random.Generator(np.random.Philox(seed))
    tl = workloads.f32_to_bf16_bits((3 * g.standard_normal((R, k + 1, V))).astype(np.float32))
    dl = workloads.f32_to_bf16_bits((workloads.bf16_bits_to_f32(tl[:, :k])
                                     + 1.5 * g.standard_normal((R, k, V))).astype(np.float32))
    x = g.integers(0, V, size=(R, k)).astype(np.int32)
    L = g.integers(0, k + 1, size=R).astype(np.int32)
    return tl, dl, x, L


def _run(noalloc, mode, tl, dl, x, L, seed, step):
    R, k1, V = tl.shape
    k = k1 - 1
    dev = "cuda"
    tags = torch.zeros(R * k1, 2, dtype=torch.int32, device=dev)
    cu = torch.zeros(R + 1, dtype=torch.int32, device=dev)
    nr = torch.zeros(1, dtype=torch.int32, device=dev)
    B.spec_flatten(to_device(L, dev), k, tags, cu, nr)
    acc = torch.full((R,), -7, dtype=torch.int32, device=dev)
    out = torch.full((R, k1), -7, dtype=torch.int32, device=dev)
    diag = torch.zeros(R * k1, 4, dtype=torch.float32, device=dev)
    tt, dd, xx = to_device(tl, dev), to_device(dl, dev), to_device(x, dev)
    if noalloc:
        st = torch.full((1,), 12345, dtype=torch.int32, device=dev)
        B.spec_verify_noalloc(mode, tt, dd if mode == B.SAMPLE else None, xx, tags, cu, nr, 1.0, None, acc, out,
                              row_diag=diag, status_out=st, seed=seed, step=step)
        torch.cuda.synchronize()
        status = int(st.item())
    else:
        ws = B.workspace(B.verify_workspace_bytes(R, k, V), dev)
        B.spec_verify(mode, tt, dd if mode == B.SAMPLE else None, xx, tags, cu, nr, 1.0, None, acc, out, ws,
                      row_diag=diag, seed=seed, step=step)
        torch.cuda.synchronize()
        status = B.read_status(ws)
    n = int(nr.item())
    return acc.cpu().numpy(), out.cpu().numpy(), diag.cpu().numpy()[:n], status


CALLS = [
    # R, k, V, mode, input seed, (seed, step)
    (256, 5, 151936, B.SAMPLE, 1, (2, 1)),       # the saturated workload's size
    (24, 3, 5001, B.SAMPLE, 2, (2, 2)),          # then a smaller batch, ragged V (scalar path)
    (40, 4, 4096, B.GREEDY, 3, (0, 0)),
    (8, 2, 1000, B.SAMPLE, 4, (9, 7)),
]


def test_noalloc_matches_spec_verify_twice_in_a_row():
    for R, k, V, mode, s_in, (seed, step) in CALLS:
        say("noalloc", R, k, V, "sample" if mode == B.SAMPLE else "greedy")
        tl, dl, x, L = _inputs(R, k, V, s_in)
        a = _run(True, mode, tl, dl, x, L, seed, step)
        b = _run(False, mode, tl, dl, x, L, seed, step)
        assert a[3] == b[3] == 0
        for u, v in zip(a[:3], b[:3]):
            assert np.array_equal(u, v)


def test_noalloc_status_out_reports_nonfinite():
    R, k, V = 16, 4, 3000
    tl, dl, x, L = _inputs(R, k, V, 5)
    L[:] = k
    tl[3, 1, 10] = 0x7FC0                        # a NaN logit voids request 3
    say("noalloc status")
    a = _run(True, B.SAMPLE, tl, dl, x, L, 1, 1)
    b = _run(False, B.SAMPLE, tl, dl, x, L, 1, 1)
    assert a[3] == b[3] == B.STATUS_NONFINITE
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    assert a[0][3] == 0


def test_noalloc_refuses_batches_above_the_scratch():
    R, k, V = 4096, 8, 151936
    assert B.verify_workspace_bytes(R, k, V) > B.NOALLOC_SCRATCH_BYTES
    fake = 1 << 20
    rc = B.lib().spec_verify_noalloc(B.SAMPLE, B.BF16, R, k, V, fake, fake, fake, fake, fake, fake, 1.0, 0, 0, None,
                                     fake, fake, None, None, None)
    assert rc == B.EUNSUPPORTED
    assert "scratch" in B.last_error()
