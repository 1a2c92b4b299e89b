"""Pins of the tag-masked attention oracle (CPU only)."""
import numpy as np
import torch

from draft_token_verification_flattened_amd import workloads
from oracle import attention as oatt
from oracle import schedule as osched
from oracle.numerics import decode


def _small(seed=3, R=5, k=4, Hq=4, Hkv=2, D=16, ps=32, ctx=(20, 70)):
    a = workloads.make_attention(R, k, Hq=Hq, Hkv=Hkv, D=D, page_size=ps, ctx_range=ctx, seed=seed)
    tags, cu = osched.flatten(a.lengths)
    return a, np.asarray(tags, dtype=np.int32), osched.n_rows(cu)


def test_matches_dense_sdpa():
    a, tags, nr = _small()
    out = oatt.flat_attention(a.q, a.k_cache, a.v_cache, a.page_table, a.ctx_len, tags, nr, a.page_size)
    Q, K, V = (decode(x, "bf16") for x in (a.q, a.k_cache, a.v_cache))
    G = a.Hq // a.Hkv
    for t in range(nr):
        r, j = tags[t]
        n = a.ctx_len[r] + j + 1
        P = a.page_table[r].size * a.page_size
        pos = np.arange(P)
        Kd = K[a.page_table[r, pos // a.page_size], pos % a.page_size]      # [P, Hkv, D]
        Vd = V[a.page_table[r, pos // a.page_size], pos % a.page_size]
        mask = torch.tensor(pos < n)
        for h in range(a.Hq):
            ref = torch.nn.functional.scaled_dot_product_attention(
                torch.tensor(Q[t, h][None, None, None, :]), torch.tensor(Kd[:, h // G][None, None]),
                torch.tensor(Vd[:, h // G][None, None]), attn_mask=mask[None, None, None, :])
            assert np.allclose(out[t, h], ref.numpy()[0, 0, 0], rtol=1e-10, atol=1e-12)


def test_equal_keys_give_mean_of_visible_values():
    a, tags, nr = _small(seed=4)
    kc = np.full_like(a.k_cache, a.k_cache.flat[0])
    out = oatt.flat_attention(a.q, kc, a.v_cache, a.page_table, a.ctx_len, tags, nr, a.page_size)
    V = decode(a.v_cache, "bf16")
    G = a.Hq // a.Hkv
    for t in range(nr):
        r, j = tags[t]
        n = a.ctx_len[r] + j + 1
        pos = np.arange(n)
        Vr = V[a.page_table[r, pos // a.page_size], pos % a.page_size]
        for h in range(a.Hq):
            assert np.allclose(out[t, h], Vr[:, h // G].mean(axis=0), rtol=1e-12, atol=1e-12)


def test_single_visible_key_returns_its_value():
    a, _, _ = _small(seed=5)
    ctx = np.zeros_like(a.ctx_len)
    tags = np.array([[r, 0] for r in range(a.R)], dtype=np.int32)
    out = oatt.flat_attention(a.q, a.k_cache, a.v_cache, a.page_table, ctx, tags, a.R, a.page_size)
    V = decode(a.v_cache, "bf16")
    G = a.Hq // a.Hkv
    for r in range(a.R):
        for h in range(a.Hq):
            assert np.array_equal(out[r, h], V[a.page_table[r, 0], 0, h // G])


def test_page_permutation_invariance():
    a, tags, nr = _small(seed=6)
    out = oatt.flat_attention(a.q, a.k_cache, a.v_cache, a.page_table, a.ctx_len, tags, nr, a.page_size)
    perm = np.random.default_rng(0).permutation(a.k_cache.shape[0])
    inv = np.argsort(perm)
    out2 = oatt.flat_attention(a.q, a.k_cache[perm], a.v_cache[perm], inv[a.page_table].astype(np.int32),
                               a.ctx_len, tags, nr, a.page_size)
    assert np.array_equal(out, out2)


def test_common_key_shift_changes_nothing():
    a, tags, nr = _small(seed=7)
    kf = decode(a.k_cache, "bf16").astype(np.float32)
    vf = decode(a.v_cache, "bf16").astype(np.float32)
    qf = decode(a.q, "bf16").astype(np.float32)
    # a dyadic shift (multiples of 1/8 in [-2, 2)): k + u and every score are exact,
    # so each query's scores move by the same q . u
    u = (np.random.default_rng(1).integers(-16, 16, a.D) / 8.0).astype(np.float32)
    out = oatt.flat_attention(qf, kf, vf, a.page_table, a.ctx_len, tags, nr, a.page_size, dtype="f32")
    out2 = oatt.flat_attention(qf, kf + u, vf, a.page_table, a.ctx_len, tags, nr, a.page_size, dtype="f32")
    assert np.allclose(out, out2, rtol=1e-12, atol=1e-12)


def test_tag_mask_hides_later_positions():
    a, tags, nr = _small(seed=8)
    out = oatt.flat_attention(a.q, a.k_cache, a.v_cache, a.page_table, a.ctx_len, tags, nr, a.page_size)
    t = int(np.argmax(tags[:, 1] == 0))                  # a row with j = 0
    r = int(tags[t, 0])
    hidden, seen = int(a.ctx_len[r]) + 1, int(a.ctx_len[r])  # the position after the row, and the row itself
    for pos, changes in ((hidden, False), (seen, True)):
        kc = a.k_cache.copy()
        # lowest exponent bit: every key value of that position doubles or halves (finite, nonzero)
        kc[a.page_table[r, pos // a.page_size], pos % a.page_size] ^= np.uint16(0x0080)
        o2 = oatt.flat_attention(a.q, kc, a.v_cache, a.page_table, a.ctx_len, tags, nr, a.page_size)
        assert np.array_equal(o2[t], out[t]) != changes


def test_head_major_storage_is_the_same_cache():
    """The head-major pool holds the same cache as the position-major one, with
    the head and position axes of each page swapped: the outputs agree bit for
    bit (a wrong axis in either gather would mix heads and positions)."""
    a, tags, nr = _small(seed=9, Hkv=2, Hq=4)
    ref = oatt.flat_attention(a.q, a.k_cache, a.v_cache, a.page_table, a.ctx_len, tags, nr, a.page_size)
    kh = np.ascontiguousarray(a.k_cache.transpose(0, 2, 1, 3))
    vh = np.ascontiguousarray(a.v_cache.transpose(0, 2, 1, 3))
    got = oatt.flat_attention(a.q, kh, vh, a.page_table, a.ctx_len, tags, nr, a.page_size, head_major=True)
    assert np.array_equal(got, ref)
    # and reading the head-major pool as position-major is a different cache
    if a.page_size != a.Hkv:
        wrong = oatt.flat_attention(a.q, np.ascontiguousarray(kh.reshape(a.k_cache.shape)),
                                    np.ascontiguousarray(vh.reshape(a.v_cache.shape)), a.page_table,
                                    a.ctx_len, tags, nr, a.page_size)
        assert not np.allclose(wrong, ref)
