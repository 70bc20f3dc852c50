"""Training-free KV-tile mask generator.  TEST INFRASTRUCTURE ONLY.

Policy (section 2.3 of "分块稀疏注意力与KV Cache量化：长文本推理显存优化实践",
xdnf.cn): a coarse pattern of skipped blocks with dense local blocks, the
skipped share capped so that no block is starved; the page's predictor is a
learned head, for which this module substitutes a data-only importance score
(no weights).  Reading taken, per batch entry b and KV head g, over 128x128
tiles of a causal prefill of n_b tokens (nt = ceil(n_b / 128) tiles):

* query tile i < nt keeps KV tile 0 (the first tile) and tile i (the
  diagonal); tiles j > i and every tile of rows i >= nt are 0;
* of the eligible tiles 1 <= j <= i-1 it drops the
  m_i = floor((i-1) * skip_per_mille / 1000) with the lowest importance
  (ties: the lower j first) and keeps the rest;
* importance(i, j) = sum_d Qsum_i[d] * Kmean_j[d], where Qsum_i is the sum of
  the query rows of tile i (rows < n_b) over the Hq/Hkv query heads of KV
  head g, kept in units of 2^-24 (a positive factor per row that leaves every
  ranking unchanged), and Kmean_j the mean of the dequantised keys of tile j
  (keys < n_b).

Because the decision is taken by floating point, the arithmetic is fixed so
that any implementation reproduces it bit for bit: Qsum and Ksum are exact
integer sums of the values times 2^24 (every fp16 value and every
dequantised value (c - z) * s is an integer multiple of 2^-24);
Kmean_j[d] = float64(Ksum_j[d]) / cnt_j / 2^24 (two correctly rounded fp64
operations, in that order); the importance is accumulated over d = 0..D-1 in
that order as fp64 multiply then fp64 add (no fused multiply-add).

Pins (tests/test_oracle_maskgen.py): exact drop counts per row, forced tiles,
skip 0 = the dense causal mask, skip 1000 = first + diagonal only, a planted
high-importance tile always kept, power-of-two rescaling invariance, and a
pure-Python evaluation with Fractions on inputs without near-ties.  The
per-turn variant (generate_chunk) is pinned by equality with generate() when
the turn is the whole sequence and, for turns that start on a tile boundary,
on the turn's rows; by its row structure and drop counts; and by a Fraction
evaluation of a tile shared with the previous turn, whose ranking comes from
the turn's rows alone.
"""
from __future__ import annotations

import numpy as np

TILE = 128
SHIFT = 24          # values are integer multiples of 2^-24


def _q_int(q16: np.ndarray) -> np.ndarray:
    """fp16 array -> exact int64 multiples of 2^-24."""
    return np.rint(q16.astype(np.float64) * (1 << SHIFT)).astype(np.int64)


def pooled(q, k_hat, seq_lens, Hkv):
    """Exact pooled sums.  q fp16 [B][Hq][L][D]; k_hat fp64 [B][Hkv][cap][D]
    (dequantised, integer multiples of 2^-24).  Returns (qsum int64
    [B][Hkv][nq][D], ksum int64 [B][Hkv][nq][D], kcnt int64 [B][nq]) with
    nq = ceil(L / 128)."""
    B, Hq, L, D = q.shape
    r = Hq // Hkv
    nq = (L + TILE - 1) // TILE
    qsum = np.zeros((B, Hkv, nq, D), dtype=np.int64)
    ksum = np.zeros((B, Hkv, nq, D), dtype=np.int64)
    kcnt = np.zeros((B, nq), dtype=np.int64)
    for b in range(B):
        n = int(seq_lens[b])
        for t in range(nq):
            lo, hi = t * TILE, min((t + 1) * TILE, n)
            if hi <= lo:
                continue
            kcnt[b, t] = hi - lo
            for g in range(Hkv):
                qsum[b, g, t] = _q_int(q[b, g * r:(g + 1) * r, lo:hi]).sum(axis=(0, 1))
                kv = np.rint(k_hat[b, g, lo:hi] * (1 << SHIFT)).astype(np.int64)
                ksum[b, g, t] = kv.sum(axis=0)
    return qsum, ksum, kcnt


def importance(qsum_row: np.ndarray, ksum: np.ndarray, cnt: np.ndarray) -> np.ndarray:
    """Importance of one query tile against tiles j (rows of ksum, counts cnt):
    fp64, d in order, multiply then add."""
    kmean = (ksum.astype(np.float64) / cnt.astype(np.float64)[:, None]) / float(1 << SHIFT)
    qv = qsum_row.astype(np.float64)
    s = np.zeros(ksum.shape[0], dtype=np.float64)
    for d in range(qv.shape[0]):
        s = s + kmean[:, d] * qv[d]
    return s


def _fill_row(row: np.ndarray, i: int, qsum_row, ksum, kcnt, skip_per_mille: int) -> None:
    """Mask row of query tile i: tile 0 and the diagonal kept; of tiles
    1 .. i-1 the floor((i-1) * skip / 1000) of lowest importance dropped
    (ties: the lower j first), the rest kept."""
    row[0] = 1
    row[i] = 1
    if i < 2:
        return
    js = np.arange(1, i)
    m = (len(js) * skip_per_mille) // 1000
    row[1:i] = 1
    if m == 0:
        return
    s = importance(qsum_row, ksum[1:i], kcnt[1:i])
    order = np.lexsort((js, s))          # by importance, then j
    row[js[order[:m]]] = 0


def generate(q, k_hat, seq_lens, skip_per_mille: int, max_seq_len: int | None = None):
    """Tile mask uint8 [B][Hkv][nt][nt], nt = ceil(max_seq_len / 128)
    (max_seq_len defaults to q's length)."""
    B, Hq, L, D = q.shape
    Hkv = k_hat.shape[1]
    if not 0 <= skip_per_mille <= 1000:
        raise ValueError("skip_per_mille must lie in [0, 1000]")
    L = L if max_seq_len is None else max_seq_len
    nt_all = (L + TILE - 1) // TILE
    qsum, ksum, kcnt = pooled(q, k_hat, seq_lens, Hkv)
    mask = np.zeros((B, Hkv, nt_all, nt_all), dtype=np.uint8)
    for b in range(B):
        nt = (int(seq_lens[b]) + TILE - 1) // TILE
        for g in range(Hkv):
            for i in range(nt):
                _fill_row(mask[b, g, i], i, qsum[b, g, i], ksum[b, g], kcnt[b], skip_per_mille)
    return mask


def generate_chunk(q, k_hat, seq_lens, skip_per_mille: int, max_seq_len: int):
    """Mask rows for one turn of a multi-turn prefill (section 4.2 of the
    xdnf.cn page: a new turn reads the quantised history).  q fp16
    [B][Hq][Lq][D] holds the last Lq positions of each sequence: row i of
    batch entry b sits at position n_b - Lq + i (rows at negative positions
    are padding), and the cache holds keys 0 .. n_b - 1 (the turn's own keys
    included).  Reading taken: every query tile t that holds at least one of
    the turn's positions gets the row generate() gives it, with Qsum_t the sum
    of the turn's own rows in tile t (rows of earlier turns that share the
    tile are not part of this call); every other row is 0.  Returns uint8
    [B][Hkv][nt][nt], nt = ceil(max_seq_len / 128), indexed by positions as
    the chunked prefill reads it."""
    B, Hq, Lq, D = q.shape
    Hkv = k_hat.shape[1]
    if not 0 <= skip_per_mille <= 1000:
        raise ValueError("skip_per_mille must lie in [0, 1000]")
    if not 0 <= Lq <= max_seq_len:
        raise ValueError("the turn's length must lie in [0, max_seq_len]")
    nt_all = (max_seq_len + TILE - 1) // TILE
    # the turn's rows at their positions: a tile's pooled sum then covers
    # exactly the turn's rows in it
    qpos = np.zeros((B, Hq, max_seq_len, D), dtype=np.float16)
    for b in range(B):
        n = int(seq_lens[b])
        p0 = n - Lq
        i0 = max(0, -p0)
        if n > 0 and Lq > i0:
            qpos[b, :, p0 + i0:n] = q[b, :, i0:]
    qsum, ksum, kcnt = pooled(qpos, k_hat, seq_lens, Hkv)
    mask = np.zeros((B, Hkv, nt_all, nt_all), dtype=np.uint8)
    for b in range(B):
        n = int(seq_lens[b])
        if n <= 0 or Lq == 0:
            continue
        t_first, t_last = max(n - Lq, 0) // TILE, (n - 1) // TILE
        for g in range(Hkv):
            for i in range(t_first, t_last + 1):
                _fill_row(mask[b, g, i], i, qsum[b, g, i], ksum[b, g], kcnt[b], skip_per_mille)
    return mask
