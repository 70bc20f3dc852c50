"""Causal scaled-dot-product attention with GQA, fp64.  TEST INFRASTRUCTURE ONLY.

Definition followed: softmax(Q K^T / sqrt(d_k)) V, the scaled dot-product
attention formula of the Space Bunny inference-stack article (m.xxqk.cn),
section 3.1, over the dequantised cache of "分块稀疏注意力与KV Cache量化：
长文本推理显存优化实践" (xdnf.cn), section 2.4, with the KV-tile skip mask of its
section 2.3.  The tiled online-softmax method of its section 2.2 reaches this
same result up to rounding order, so this oracle is the plain definition: whole
rows at once, no tiling, no online merge.

For batch b, query head h, KV head g = h // (Hq / Hkv) and query row i:

    A(i) = { j : j < n_b, j <= pos(i), mask keeps tile (i // 128, j // 128) }
    s_j  = tau * sum_c q[i, c] * k_hat[j, c]            (tau = 1/sqrt(D) default)
    o_i  = sum_{j in A} exp(s_j - M) v_hat[j] / sum_{j in A} exp(s_j - M),
           M = max_{j in A} s_j;  o_i = 0 when A(i) is empty.

Prefill: pos(i) = i and rows i >= n_b are padding (A(i) empty).  Chunked
prefill (a chunk of Lq new rows whose keys are already appended to the cache):
pos(i) = n_b - Lq + i, the last Lq positions of the sequence (rows with
pos < 0 are padding); the tile mask is indexed by positions.  Decode: one
query row per head that attends to every cached key, so pos = n_b - 1 and the
mask has a single query-tile row per batch entry.

Pins (tests/test_oracle_attention.py): pure-Python brute force (``brute``) on
tiny shapes, rows of P summing to 1, uniform-V, constant-K (running mean /
mean over kept tiles / ragged mean), one-hot-K closed form, single key, GQA
with repeated query heads, Hq == Hkv reducing to MHA, key-permutation
invariance for decode.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ProcessPoolExecutor
import multiprocessing as mp

import numpy as np

TILE = 128


def _mask_for(mask, b, g):
    """The [nq][nk] tile mask of batch entry b and KV head g; a mask given as
    [nq][nk] is shared, [B][nq][nk] is per batch entry, [B][Hkv][nq][nk] per
    batch entry and KV head."""
    if mask is None:
        return None
    m = np.asarray(mask)
    if m.ndim == 4:
        return m[b, g]
    return m[b] if m.ndim == 3 else m


def _rows_one_head(q_rows, row_idx, k, v, n, mask_b, tau, causal):
    """Output rows for one (b, h): q_rows [R][D] fp64, row_idx [R] (query
    positions), k/v [cap][D] fp64.  Returns [R][D] fp64."""
    R, D = q_rows.shape
    out = np.zeros((R, D), dtype=np.float64)
    if n <= 0:
        return out
    kk, vv = k[:n], v[:n]
    j = np.arange(n)
    for r0 in range(0, R, 256):
        qi = q_rows[r0:r0 + 256]
        ii = row_idx[r0:r0 + 256]
        s = (qi @ kk.T) * tau                          # [r][n]
        allowed = np.ones(s.shape, dtype=bool)
        if causal:
            allowed &= j[None, :] <= ii[:, None]
            allowed &= (ii < n)[:, None]
        if mask_b is not None:
            qt = np.maximum(ii, 0) // TILE if causal else np.zeros_like(ii)
            allowed &= mask_b[qt[:, None], (j // TILE)[None, :]].astype(bool)
        s = np.where(allowed, s, -np.inf)
        m = s.max(axis=1)
        has = np.isfinite(m)
        m = np.where(has, m, 0.0)
        p = np.exp(s - m[:, None])                     # exp(-inf) = 0
        l = p.sum(axis=1)
        o = (p @ vv) / np.where(has, l, 1.0)[:, None]
        out[r0:r0 + 256] = np.where(has[:, None], o, 0.0)
    return out


# --- optional process pool over (b, h) pairs ---------------------------------
_G = {}


def _init_worker(payload):
    _G.update(payload)
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:
        pass


def _job(args):
    b, h, rows = args
    g = _G
    kvh = h // g["r"]
    if g["causal"]:
        q_rows = g["q"][b, h][rows].astype(np.float64)
    else:
        q_rows = g["q"][b, h][None, :].astype(np.float64)
    pos = np.asarray(rows) + int(g.get("qoff", np.zeros(b + 1, dtype=np.int64))[b])
    return _rows_one_head(q_rows, pos, g["k"][b, kvh], g["v"][b, kvh],
                          int(g["lens"][b]), _mask_for(g["mask"], b, kvh), g["tau"],
                          g["causal"])


def _run(jobs, payload, workers):
    if workers <= 1:
        _G.clear()
        _G.update(payload)
        return [_job(j) for j in jobs]
    ctx = mp.get_context("fork")
    with ProcessPoolExecutor(max_workers=workers, mp_context=ctx,
                             initializer=_init_worker, initargs=(payload,)) as ex:
        return list(ex.map(_job, jobs, chunksize=1))


def prefill(q, k_hat, v_hat, seq_lens, mask=None, scale=None, rows=None,
            heads=None, workers=1):
    """Causal prefill attention.

    q: fp16 [B][Hq][L][D]; k_hat, v_hat: dequantised fp64 [B][Hkv][cap][D];
    seq_lens: [B]; mask: None, [nq][nk], [B][nq][nk] or [B][Hkv][nq][nk]
    tile keep-mask (the last form one per KV head).
    rows: None (all L rows) or a 1-D array of query rows to evaluate.
    heads: None (all) or a list of (b, h) pairs.
    Returns fp64 [B][Hq][R][D] (R = L or len(rows)); heads not evaluated are 0.
    """
    B, Hq, L, D = q.shape
    Hkv = k_hat.shape[1]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    tau = (1.0 / math.sqrt(D)) if scale is None else float(scale)
    rows = np.arange(L) if rows is None else np.asarray(rows)
    heads = [(b, h) for b in range(B) for h in range(Hq)] if heads is None else heads
    payload = dict(q=q, k=k_hat, v=v_hat, lens=np.asarray(seq_lens), mask=mask,
                   tau=tau, r=Hq // Hkv, causal=True)
    res = _run([(b, h, rows) for b, h in heads], payload, workers)
    out = np.zeros((B, Hq, len(rows), D), dtype=np.float64)
    for (b, h), o in zip(heads, res):
        out[b, h] = o
    return out


def prefill_chunk(q, k_hat, v_hat, seq_lens, mask=None, scale=None, rows=None,
                  heads=None, workers=1):
    """Chunked prefill: q fp16 [B][Hq][Lq][D] holds the last Lq positions of
    each sequence, whose keys and values are already in the cache, so row i of
    batch b sits at position seq_lens[b] - Lq + i (bottom-right alignment);
    rows at negative positions are padding (zero).  mask: None, [nq][nk],
    [B][nq][nk] or [B][Hkv][nq][nk] over positions.  Returns fp64
    [B][Hq][R][D]."""
    B, Hq, Lq, D = q.shape
    Hkv = k_hat.shape[1]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    tau = (1.0 / math.sqrt(D)) if scale is None else float(scale)
    rows = np.arange(Lq) if rows is None else np.asarray(rows)
    heads = [(b, h) for b in range(B) for h in range(Hq)] if heads is None else heads
    lens = np.asarray(seq_lens, dtype=np.int64)
    payload = dict(q=q, k=k_hat, v=v_hat, lens=lens, mask=mask, tau=tau,
                   r=Hq // Hkv, causal=True, qoff=lens - Lq)
    res = _run([(b, h, rows) for b, h in heads], payload, workers)
    out = np.zeros((B, Hq, len(rows), D), dtype=np.float64)
    for (b, h), o in zip(heads, res):
        out[b, h] = o
    return out


def decode(q, k_hat, v_hat, seq_lens, mask=None, scale=None, heads=None,
           workers=1):
    """Single-token decode attention: q fp16 [B][Hq][D]; mask None or
    [B][nk] (one query-tile row per batch entry).  Returns fp64 [B][Hq][D]."""
    B, Hq, D = q.shape
    Hkv = k_hat.shape[1]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    tau = (1.0 / math.sqrt(D)) if scale is None else float(scale)
    heads = [(b, h) for b in range(B) for h in range(Hq)] if heads is None else heads
    m3 = None if mask is None else np.asarray(mask)[:, None, :]
    payload = dict(q=q, k=k_hat, v=v_hat, lens=np.asarray(seq_lens), mask=m3,
                   tau=tau, r=Hq // Hkv, causal=False)
    res = _run([(b, h, np.zeros(1, dtype=np.int64)) for b, h in heads], payload,
               workers)
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for (b, h), o in zip(heads, res):
        out[b, h] = o[0]
    return out


def probabilities(q_rows, k, tau):
    """Softmax rows over all given keys (fp64); used by the rows-sum-to-1 pin."""
    s = (np.asarray(q_rows, dtype=np.float64) @ np.asarray(k, dtype=np.float64).T) * tau
    s -= s.max(axis=1, keepdims=True)
    p = np.exp(s)
    return p / p.sum(axis=1, keepdims=True)


def default_workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))
