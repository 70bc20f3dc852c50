"""Pins of the oracle's training-free tile-mask generator (CPU only)."""
from fractions import Fraction

import numpy as np
import pytest

from oracle import maskgen as mg


def _inputs(rng, B=2, Hq=4, Hkv=2, L=900, D=16):
    q = rng.standard_normal((B, Hq, L, D)).astype(np.float16)
    # dequantised-like keys: integer multiples of a power-of-two step
    k = rng.integers(-300, 300, (B, Hkv, L, D)).astype(np.float64) * 2.0 ** -8
    return q, k


def test_structure_and_exact_drop_counts():
    rng = np.random.default_rng(1)
    q, k = _inputs(rng)
    lens = [900, 333]
    for spm in (0, 100, 250, 500, 999, 1000):
        m = mg.generate(q, k, lens, spm)
        assert m.shape == (2, 2, 8, 8)
        for b, n in enumerate(lens):
            nt = (n + 127) // 128
            for g in range(2):
                mb = m[b, g]
                assert not mb[nt:].any()                       # rows past the sequence
                assert not np.triu(mb, 1).any()                # above the diagonal
                for i in range(nt):
                    assert mb[i, 0] == 1 and mb[i, i] == 1
                    if i >= 2:
                        kept = int(mb[i, 1:i].sum())
                        assert kept == (i - 1) - ((i - 1) * spm) // 1000


def test_zero_skip_is_dense_causal_and_full_skip_keeps_first_and_diagonal():
    rng = np.random.default_rng(2)
    q, k = _inputs(rng, B=1, L=1100)
    nt = 9
    dense = mg.generate(q, k, [1100], 0)[0, 0]
    assert np.array_equal(dense, np.tril(np.ones((nt, nt), np.uint8)))
    sparse = mg.generate(q, k, [1100], 1000)[0, 1]
    want = np.eye(nt, dtype=np.uint8)
    want[:, 0] = 1
    assert np.array_equal(sparse, want)


def test_planted_tile_is_kept():
    rng = np.random.default_rng(3)
    B, Hq, Hkv, L, D = 1, 2, 1, 1280, 16
    q = np.abs(rng.standard_normal((B, Hq, L, D))).astype(np.float16)   # positive queries
    k = rng.integers(-20, 20, (B, Hkv, L, D)).astype(np.float64) * 2.0 ** -8
    k[0, 0, 5 * 128:6 * 128] = 4.0                                       # tile 5 aligns with q
    m = mg.generate(q, k, [L], 800)[0, 0]
    for i in range(6, 10):
        assert m[i, 5] == 1
    assert m[9, 1:9].sum() == 8 - (8 * 800) // 1000


def test_power_of_two_rescaling_does_not_change_the_mask():
    rng = np.random.default_rng(4)
    q, k = _inputs(rng, B=1, L=1000)
    m0 = mg.generate(q, k, [1000], 300)
    assert np.array_equal(m0, mg.generate((q.astype(np.float32) * 2).astype(np.float16), k, [1000], 300))
    assert np.array_equal(m0, mg.generate(q, k * 4.0, [1000], 300))


def test_importance_closed_form():
    qsum = np.array([1 << 24, 2 << 24], dtype=np.int64)          # q = (1, 2)
    ksum = np.array([[3 << 24, 0], [0, 8 << 24]], dtype=np.int64)  # means (3,0)/1 and (0,8)/2
    cnt = np.array([1, 2])
    # Qsum stays in units of 2^-24: importance = 2^24 * (q . kmean)
    np.testing.assert_array_equal(mg.importance(qsum, ksum, cnt), [3.0 * 2 ** 24, 8.0 * 2 ** 24])


def test_ranking_matches_exact_rational_evaluation():
    rng = np.random.default_rng(5)
    B, Hq, Hkv, L, D = 1, 2, 1, 1408, 8
    q = rng.standard_normal((B, Hq, L, D)).astype(np.float16)
    k = rng.integers(-100, 100, (B, Hkv, L, D)).astype(np.float64) * 2.0 ** -6
    spm = 400
    m = mg.generate(q, k, [L], spm)[0, 0]
    qsum, ksum, kcnt = mg.pooled(q, k, [L], Hkv)
    nt = L // 128
    for i in range(2, nt):
        exact = []
        for j in range(1, i):
            s = sum(Fraction(int(qsum[0, 0, i, d])) * Fraction(int(ksum[0, 0, j, d]), int(kcnt[0, j]))
                    for d in range(D))
            exact.append((s, j))
        vals = sorted(v for v, _ in exact)
        gaps = [b - a for a, b in zip(vals, vals[1:])]
        if gaps and min(gaps) == 0:
            pytest.skip("exact tie in the test data")
        drop = {j for _, j in sorted(exact)[:((i - 1) * spm) // 1000]}
        for j in range(1, i):
            assert m[i, j] == (0 if j in drop else 1), (i, j)
