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


# ---- per-turn masks (one turn of a multi-turn prefill) -----------------------

def _turn(q_full, lens, Lq, rng):
    """The last Lq positions of each sequence as a turn's q (row i of entry b
    at position n_b - Lq + i); rows at negative positions get random values,
    which the generator must ignore."""
    B, Hq, L, D = q_full.shape
    qc = rng.standard_normal((B, Hq, Lq, D)).astype(np.float16) * 50
    for b, n in enumerate(lens):
        for i in range(Lq):
            p = n - Lq + i
            if p >= 0:
                qc[b, :, i] = q_full[b, :, p]
    return qc


def test_turn_that_is_the_whole_sequence_equals_generate():
    rng = np.random.default_rng(11)
    q, k = _inputs(rng, B=2, L=900)
    lens = [900, 333]
    qc = _turn(q, lens, 900, rng)
    for spm in (0, 250, 700, 1000):
        assert np.array_equal(mg.generate_chunk(qc, k, lens, spm, 900),
                              mg.generate(q, k, lens, spm, 900))


def test_tile_aligned_turn_rows_equal_generate():
    rng = np.random.default_rng(12)
    q, k = _inputs(rng, B=2, L=1000)
    lens = [1000, 744]            # the turn of 616 rows starts at positions 384 and 128
    qc = _turn(q, lens, 616, rng)
    for spm in (250, 600):
        got = mg.generate_chunk(qc, k, lens, spm, 1000)
        full = mg.generate(q, k, lens, spm, 1000)
        for b, n in enumerate(lens):
            t0, t1 = (n - 616) // 128, (n - 1) // 128
            assert np.array_equal(got[b, :, t0:t1 + 1], full[b, :, t0:t1 + 1])
            assert not got[b, :, :t0].any() and not got[b, :, t1 + 1:].any()


@pytest.mark.parametrize("Lq", [1, 100, 300, 1000, 1200])
def test_turn_structure_and_exact_drop_counts(Lq):
    rng = np.random.default_rng(13 + Lq)
    q, k = _inputs(rng, B=3, L=1200)
    lens = [1200, 640, 0]
    qc = rng.standard_normal((3, 4, Lq, 16)).astype(np.float16)
    for spm in (0, 333, 1000):
        m = mg.generate_chunk(qc, k, lens, spm, 1200)
        assert m.shape == (3, 2, 10, 10)
        assert not np.triu(m, 1).any()
        for b, n in enumerate(lens):
            rows = set()
            if n > 0:
                rows = set(range(max(n - Lq, 0) // 128, (n - 1) // 128 + 1))
            for g in range(2):
                for i in range(10):
                    if i not in rows:
                        assert not m[b, g, i].any(), (b, i)
                        continue
                    assert m[b, g, i, 0] == 1 and m[b, g, i, i] == 1
                    if i >= 2:
                        assert int(m[b, g, i, 1:i].sum()) == (i - 1) - ((i - 1) * spm) // 1000


def test_shared_tile_is_ranked_from_the_turns_rows_only():
    """The turn starts inside query tile 10: the earlier rows of that tile
    (the previous turn's) are given a direction that would rank the tiles
    differently; the turn's row for tile 10 follows an exact rational
    evaluation over the turn's own rows, and differs from the row that the
    whole prompt would give, while tile 11 (wholly in the turn) matches it."""
    rng = np.random.default_rng(14)
    B, Hq, Hkv, L, D = 1, 2, 1, 1536, 8
    q = rng.standard_normal((B, Hq, L, D)).astype(np.float16)
    k = rng.integers(-100, 100, (B, Hkv, L, D)).astype(np.float64) * 2.0 ** -6
    start = 10 * 128 + 40                      # the turn: positions 1320 .. 1535
    q[0, :, 10 * 128:start] = (k[0, 0, 5 * 128:6 * 128].mean(axis=0) * 60).astype(np.float16)
    qc = np.ascontiguousarray(q[:, :, start:])
    spm = 500
    got = mg.generate_chunk(qc, k, [L], spm, L)[0, 0]
    full = mg.generate(q, k, [L], spm)[0, 0]
    assert not got[:10].any()
    i = 10
    qs = [sum(Fraction(float(q[0, h, p, d])) for h in range(Hq) for p in range(start, 11 * 128))
          for d in range(D)]
    exact = []
    for j in range(1, i):
        km = [sum(Fraction(int(round(k[0, 0, t, d] * 64)), 64) for t in range(j * 128, (j + 1) * 128)) / 128
              for d in range(D)]
        exact.append((sum(qs[d] * km[d] for d in range(D)), j))
    vals = sorted(v for v, _ in exact)
    assert min(b - a for a, b in zip(vals, vals[1:])) > 0
    drop = {j for _, j in sorted(exact)[:((i - 1) * spm) // 1000]}
    for j in range(1, i):
        assert got[i, j] == (0 if j in drop else 1), j
    assert not np.array_equal(got[i], full[i])
    assert np.array_equal(got[11], full[11])
