"""Pins of the oracle's attention (CPU only): pure-Python brute force on tiny
shapes, textbook closed forms and invariants."""
import math

import numpy as np
import pytest

from oracle import attention as att
from oracle import brute


def _rand(rng, shape, scale=1.0):
    return (rng.standard_normal(shape) * scale).astype(np.float16)


def test_prefill_matches_brute_force_with_mask_and_lengths():
    rng = np.random.default_rng(0)
    B, Hq, Hkv, L, D = 2, 4, 2, 300, 16
    q = _rand(rng, (B, Hq, L, D))
    k = _rand(rng, (B, Hkv, L, D)).astype(np.float64)
    v = _rand(rng, (B, Hkv, L, D)).astype(np.float64)
    lens = np.array([300, 171])
    mask = np.tril(np.ones((3, 3), np.uint8))
    mask[2, 1] = 0
    mask[1, 0] = 0
    ours = att.prefill(q, k, v, lens, mask=mask, heads=[(0, 0), (0, 3), (1, 2)])
    ref = brute.prefill(q.astype(np.float64), k, v, lens, Hq, Hkv, mask=mask)
    for b, h in [(0, 0), (0, 3), (1, 2)]:
        np.testing.assert_allclose(ours[b, h], np.array(ref[b][h]), rtol=0, atol=1e-12)
    # row 130 of batch 0: tile (1,0) dropped, so it only sees keys 128..130
    # rows >= n_b of batch 1 are padding: zero
    assert not ours[1, 2, 171:].any()


def test_decode_matches_brute_force():
    rng = np.random.default_rng(1)
    B, Hq, Hkv, cap, D = 3, 8, 2, 384, 16
    q = _rand(rng, (B, Hq, D))
    k = _rand(rng, (B, Hkv, cap, D)).astype(np.float64)
    v = _rand(rng, (B, Hkv, cap, D)).astype(np.float64)
    lens = np.array([384, 1, 250])
    mask = np.ones((B, 3), np.uint8)
    mask[0, 1] = 0
    mask[2, 0] = 0
    ours = att.decode(q, k, v, lens, mask=mask)
    ref = np.array(brute.decode(q.astype(np.float64), k, v, lens, Hq, Hkv, mask=mask))
    np.testing.assert_allclose(ours, ref, rtol=0, atol=1e-12)
    ours_nomask = att.decode(q, k, v, lens)
    ref_nomask = np.array(brute.decode(q.astype(np.float64), k, v, lens, Hq, Hkv))
    np.testing.assert_allclose(ours_nomask, ref_nomask, rtol=0, atol=1e-12)


def test_rows_sum_to_one():
    rng = np.random.default_rng(2)
    p = att.probabilities(rng.standard_normal((50, 64)), rng.standard_normal((900, 64)), 0.125)
    np.testing.assert_allclose(p.sum(1), 1.0, rtol=0, atol=1e-13)
    assert (p >= 0).all()


def test_uniform_v_gives_that_value():
    rng = np.random.default_rng(3)
    B, Hq, Hkv, L, D = 1, 4, 1, 260, 32
    q = _rand(rng, (B, Hq, L, D), 3.0)
    k = _rand(rng, (B, Hkv, L, D), 3.0).astype(np.float64)
    row = rng.standard_normal(D)
    v = np.broadcast_to(row, (B, Hkv, L, D)).copy()
    mask = np.tril(np.ones((3, 3), np.uint8))
    mask[2, 0] = 0
    o = att.prefill(q, k, v, [L], mask=mask)
    np.testing.assert_allclose(o, np.broadcast_to(row, o.shape), rtol=0, atol=1e-12)
    od = att.decode(q[:, :, 7], k, v, [200])
    np.testing.assert_allclose(od, np.broadcast_to(row, od.shape), rtol=0, atol=1e-12)


def test_constant_k_gives_means():
    """All keys equal -> uniform weights -> running mean of V over A(i)."""
    rng = np.random.default_rng(4)
    B, Hq, Hkv, L, D = 1, 2, 1, 300, 8
    q = _rand(rng, (B, Hq, L, D))
    k = np.broadcast_to(rng.standard_normal(D), (B, Hkv, L, D)).copy()
    v = rng.standard_normal((B, Hkv, L, D))
    o = att.prefill(q, k, v, [L])
    csum = np.cumsum(v[0, 0], axis=0) / np.arange(1, L + 1)[:, None]
    np.testing.assert_allclose(o[0, 1], csum, rtol=0, atol=1e-12)
    # with a mask: row i in tile 2 with tile (2,1) dropped -> mean of keys
    # 0..127 and 256..i
    mask = np.tril(np.ones((3, 3), np.uint8))
    mask[2, 1] = 0
    om = att.prefill(q, k, v, [L], mask=mask)
    for i in (256, 270, 299):
        keys = list(range(128)) + list(range(256, i + 1))
        np.testing.assert_allclose(om[0, 0, i], v[0, 0, keys].mean(0), rtol=0, atol=1e-12)
    # ragged decode: mean over the first n keys
    od = att.decode(q[:, :, 0], k, v, [137])
    np.testing.assert_allclose(od[0, 1], v[0, 0, :137].mean(0), rtol=0, atol=1e-12)


def test_one_hot_k_closed_form():
    """One key alpha*e_c, all others zero: p* = e^a / (e^a + |A| - 1),
    a = tau*alpha*q_c, and o = p* v* + (1 - p*) mean(other v)."""
    rng = np.random.default_rng(5)
    D, n = 16, 150
    q = _rand(rng, (1, 1, D))
    k = np.zeros((1, 1, n, D))
    jstar, c, alpha = 127, 5, 3.0
    k[0, 0, jstar, c] = alpha
    v = rng.standard_normal((1, 1, n, D))
    tau = 1 / math.sqrt(D)
    a = tau * alpha * float(q[0, 0, c])
    ps = math.exp(a) / (math.exp(a) + n - 1)
    others = np.delete(v[0, 0], jstar, axis=0).mean(0)
    want = ps * v[0, 0, jstar] + (1 - ps) * others
    o = att.decode(q, k, v, [n])
    np.testing.assert_allclose(o[0, 0], want, rtol=0, atol=1e-12)


def test_single_key_row_zero():
    rng = np.random.default_rng(6)
    q = _rand(rng, (1, 2, 5, 8))
    k = rng.standard_normal((1, 1, 5, 8))
    v = rng.standard_normal((1, 1, 5, 8))
    o = att.prefill(q, k, v, [5])
    np.testing.assert_array_equal(o[0, :, 0], np.broadcast_to(v[0, 0, 0], (2, 8)))


def test_gqa_equals_repeated_mha():
    rng = np.random.default_rng(7)
    B, Hq, Hkv, L, D = 1, 8, 2, 64, 16
    q = _rand(rng, (B, Hq, L, D))
    k = rng.standard_normal((B, Hkv, L, D))
    v = rng.standard_normal((B, Hkv, L, D))
    o = att.prefill(q, k, v, [L])
    k_rep = np.repeat(k, Hq // Hkv, axis=1)
    v_rep = np.repeat(v, Hq // Hkv, axis=1)
    o_mha = att.prefill(q, k_rep, v_rep, [L])
    np.testing.assert_array_equal(o, o_mha)
    # identical queries within a group give identical outputs
    q2 = q.copy()
    q2[:, 1:4] = q2[:, 0:1]
    o2 = att.prefill(q2, k, v, [L])
    for h in range(1, 4):
        np.testing.assert_array_equal(o2[0, h], o2[0, 0])


def test_decode_key_permutation_invariance():
    rng = np.random.default_rng(8)
    q = _rand(rng, (1, 2, 32))
    k = rng.standard_normal((1, 1, 200, 32))
    v = rng.standard_normal((1, 1, 200, 32))
    perm = rng.permutation(200)
    o1 = att.decode(q, k, v, [200])
    o2 = att.decode(q, k[:, :, perm], v[:, :, perm], [200])
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-13)


def test_empty_rows_and_lengths_are_zero():
    rng = np.random.default_rng(9)
    q = _rand(rng, (2, 2, 3, 8))
    k = rng.standard_normal((2, 1, 3, 8))
    v = rng.standard_normal((2, 1, 3, 8))
    o = att.prefill(q, k, v, [0, 3], mask=np.zeros((1, 1), np.uint8))
    assert not o.any()
    od = att.decode(q[:, :, 0], k, v, [0, 2])
    assert not od[0].any() and od[1].any()


def test_worker_pool_gives_same_result():
    rng = np.random.default_rng(10)
    q = _rand(rng, (1, 4, 200, 16))
    k = rng.standard_normal((1, 2, 200, 16))
    v = rng.standard_normal((1, 2, 200, 16))
    o1 = att.prefill(q, k, v, [200])
    o2 = att.prefill(q, k, v, [200], workers=3)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-12)


# --- chunked prefill (rows at positions n_b - Lq + i) --------------------------

def test_chunk_matches_brute_force_with_mask_and_padding():
    rng = np.random.default_rng(11)
    B, Hq, Hkv, Lq, cap, D = 3, 4, 2, 40, 300, 16
    q = _rand(rng, (B, Hq, Lq, D))
    k = _rand(rng, (B, Hkv, cap, D)).astype(np.float64)
    v = _rand(rng, (B, Hkv, cap, D)).astype(np.float64)
    lens = np.array([300, 150, 25])          # batch 2: 15 padding rows
    mask = np.tril(np.ones((3, 3), np.uint8))
    mask[2, 0] = 0
    mask[1, 1] = 0                           # the chunk of batch 1 straddles tiles 0 / 1
    ours = att.prefill_chunk(q, k, v, lens, mask=mask)
    ref = np.array(brute.prefill_chunk(q.astype(np.float64), k, v, lens, Hq, Hkv, mask=mask))
    np.testing.assert_allclose(ours, ref, rtol=0, atol=1e-12)
    assert not ours[2, :, :15].any() and ours[2, :, 15:].any()


def test_chunk_equals_the_same_rows_of_a_full_prefill():
    rng = np.random.default_rng(12)
    B, Hq, Hkv, L, D, Lq = 2, 4, 1, 520, 32, 72
    qf = _rand(rng, (B, Hq, L, D))
    k = _rand(rng, (B, Hkv, L, D)).astype(np.float64)
    v = _rand(rng, (B, Hkv, L, D)).astype(np.float64)
    lens = np.array([520, 333])
    mask = np.ones((5, 5), np.uint8)
    mask[3, 1] = 0
    mask[4, 2] = 0
    full = att.prefill(qf, k, v, lens, mask=mask)
    for b in range(B):
        n = int(lens[b])
        qc = np.zeros((B, Hq, Lq, D), np.float16)
        qc[b] = qf[b, :, n - Lq:n]
        got = att.prefill_chunk(qc, k, v, lens, mask=mask, heads=[(b, h) for h in range(Hq)])
        np.testing.assert_allclose(got[b], full[b, :, n - Lq:n], rtol=0, atol=1e-12)


def test_chunk_of_one_row_is_decode():
    rng = np.random.default_rng(13)
    B, Hq, Hkv, cap, D = 3, 8, 2, 400, 16
    q = _rand(rng, (B, Hq, D))
    k = _rand(rng, (B, Hkv, cap, D)).astype(np.float64)
    v = _rand(rng, (B, Hkv, cap, D)).astype(np.float64)
    lens = np.array([400, 1, 257])
    dec = att.decode(q, k, v, lens)
    chk = att.prefill_chunk(q[:, :, None, :], k, v, lens)
    np.testing.assert_allclose(chk[:, :, 0], dec, rtol=0, atol=1e-13)


def test_per_kv_head_mask_selects_the_group_mask():
    # a [B][Hkv][nq][nk] mask gives query head h of batch b the mask of KV head
    # h // (Hq / Hkv): each (b, h) equals the run with that one [nq][nk] mask
    # (the shared-mask path is pinned by brute force above)
    rng = np.random.default_rng(11)
    B, Hq, Hkv, L, D = 2, 4, 2, 300, 16
    q = _rand(rng, (B, Hq, L, D))
    k = _rand(rng, (B, Hkv, L, D)).astype(np.float64)
    v = _rand(rng, (B, Hkv, L, D)).astype(np.float64)
    lens = np.array([300, 260])
    m = np.tile(np.tril(np.ones((3, 3), np.uint8)), (B, Hkv, 1, 1))
    m[0, 1, 2, 1] = 0
    m[1, 0, 1, 0] = 0
    m[1, 1, 2, 0] = 0
    m[1, 1, 2, 1] = 0
    ours = att.prefill(q, k, v, lens, mask=m)
    for b in range(B):
        for h in range(Hq):
            one = att.prefill(q, k, v, lens, mask=m[b, h // 2], heads=[(b, h)])
            np.testing.assert_array_equal(ours[b, h], one[b, h])
    # the four masks differ, so a swapped index would change some head
    assert len({m[b, g].tobytes() for b in range(B) for g in range(Hkv)}) == 4
    chunk = att.prefill_chunk(q[:, :, 200:], k, v, lens, mask=m)
    for b in range(B):
        for h in range(Hq):
            one = att.prefill_chunk(q[:, :, 200:], k, v, lens, mask=m[b, h // 2], heads=[(b, h)])
            np.testing.assert_array_equal(chunk[b, h], one[b, h])
