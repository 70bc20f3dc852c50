"""Brute-force attention in pure Python.  TEST INFRASTRUCTURE ONLY.

An explicit L x L score matrix with -inf for every excluded (row, key) pair,
``math.exp`` per entry and ``math.fsum`` for every sum; meant for tiny shapes
only.  It pins ``oracle.attention`` (same definition: the scaled dot-product
attention formula, section 3.1 of the Space Bunny inference-stack article, with
the causal / tile-mask / length rules of "分块稀疏注意力与KV Cache量化：长文本推理
显存优化实践", sections 2.2-2.3) through a different evaluation: no NumPy, no
vectorised masking, no max-subtraction shortcut.
"""
from __future__ import annotations

import math


def attention_rows(q, k, v, n, allowed, tau):
    """q: list of R query rows; k, v: lists of key/value rows; n: number of
    valid keys; allowed(i_row_index, j) -> bool.  Returns R output rows."""
    D = len(v[0]) if v else 0
    out = []
    for ri, qi in enumerate(q):
        scores = []
        for j in range(len(k)):
            if j < n and allowed(ri, j):
                scores.append(tau * math.fsum(a * b for a, b in zip(qi, k[j])))
            else:
                scores.append(-math.inf)
        finite = [s for s in scores if s != -math.inf]
        if not finite:
            out.append([0.0] * D)
            continue
        m = max(finite)
        w = [math.exp(s - m) if s != -math.inf else 0.0 for s in scores]
        l = math.fsum(w)
        out.append([math.fsum(w[j] * v[j][c] for j in range(len(k))) / l
                    for c in range(D)])
    return out


def prefill(q, k, v, seq_lens, Hq, Hkv, mask=None, tau=None, tile=128):
    """q[b][h][i][c], k/v[b][g][j][c] nested lists (or arrays); mask[qt][kt] or
    None.  Returns out[b][h][i][c]."""
    B = len(q)
    D = len(q[0][0][0])
    tau = 1.0 / math.sqrt(D) if tau is None else tau
    r = Hq // Hkv
    out = []
    for b in range(B):
        n = int(seq_lens[b])
        ob = []
        for h in range(Hq):
            g = h // r
            qs = [[float(x) for x in row] for row in q[b][h]]
            ks = [[float(x) for x in row] for row in k[b][g]]
            vs = [[float(x) for x in row] for row in v[b][g]]

            def allowed(i, j):
                if i >= n or j > i:
                    return False
                if mask is not None and not mask[i // tile][j // tile]:
                    return False
                return True
            ob.append(attention_rows(qs, ks, vs, n, allowed, tau))
        out.append(ob)
    return out


def prefill_chunk(q, k, v, seq_lens, Hq, Hkv, mask=None, tau=None, tile=128):
    """Chunk of Lq = len(q[b][h]) query rows at positions n_b - Lq + i (keys
    already in k/v); mask[qt][kt] over positions or None.  Returns
    out[b][h][i][c]."""
    B = len(q)
    D = len(q[0][0][0])
    tau = 1.0 / math.sqrt(D) if tau is None else tau
    r = Hq // Hkv
    out = []
    for b in range(B):
        n = int(seq_lens[b])
        ob = []
        for h in range(Hq):
            g = h // r
            qs = [[float(x) for x in row] for row in q[b][h]]
            ks = [[float(x) for x in row] for row in k[b][g]]
            vs = [[float(x) for x in row] for row in v[b][g]]
            off = n - len(qs)

            def allowed(i, j, off=off):
                p = off + i
                if p < 0 or j > p:
                    return False
                if mask is not None and not mask[p // tile][j // tile]:
                    return False
                return True
            ob.append(attention_rows(qs, ks, vs, n, allowed, tau))
        out.append(ob)
    return out


def decode(q, k, v, seq_lens, Hq, Hkv, mask=None, tau=None, tile=128):
    """q[b][h][c]; mask[b][kt] or None.  Returns out[b][h][c]."""
    B = len(q)
    D = len(q[0][0])
    tau = 1.0 / math.sqrt(D) if tau is None else tau
    r = Hq // Hkv
    out = []
    for b in range(B):
        n = int(seq_lens[b])
        ob = []
        for h in range(Hq):
            g = h // r
            qs = [[float(x) for x in q[b][h]]]
            ks = [[float(x) for x in row] for row in k[b][g]]
            vs = [[float(x) for x in row] for row in v[b][g]]

            def allowed(i, j):
                return mask is None or bool(mask[b][j // tile])
            ob.append(attention_rows(qs, ks, vs, n, allowed, tau)[0])
        out.append(ob)
    return out
