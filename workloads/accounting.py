"""Algorithmic work of one attention call: the bytes decode must move and the
flops prefill must do.  Used by the bench (roofline fractions) and by tests.

Counted work is algorithmic only: the KV codes, fp16 scales and u8 zero-points
of every permitted token read once per KV head, plus Q read and O written, for
decode; 4 * D flops (QK^T and PV, one multiply-add each per channel) for every
permitted (query head, query row, key) triple, for prefill.  Tiles skipped by
causality or by the mask, the masked half of diagonal tiles, re-reads from cache
and dequantisation instructions are not work.
"""
from __future__ import annotations

import numpy as np

GROUP = 32
TILE = 128


def token_bytes(D: int, bits: int) -> int:
    """Bytes of one token of one KV head in one cache (K or V): codes, fp16
    scales, u8 zeros."""
    G = D // GROUP
    return D * bits // 8 + 2 * G + G


def decode_kv_bytes(D: int, seq_lens, head_bits) -> int:
    per_tok = sum(2 * token_bytes(D, int(b)) for b in head_bits)
    return int(np.sum(np.asarray(seq_lens, dtype=np.int64))) * per_tok


def decode_bytes(B: int, Hq: int, D: int, seq_lens, head_bits) -> int:
    """KV bytes plus fp16 Q read and fp16 O written."""
    return decode_kv_bytes(D, seq_lens, head_bits) + 2 * B * Hq * D * 2


def causal_pairs(L: int, n: int | None = None, mask=None) -> int:
    """Number of (row, key) pairs with key <= row < n, key < n, whose 128x128
    tile the mask keeps.  Closed form for a dense mask: n(n+1)/2."""
    n = L if n is None else n
    if mask is None:
        return n * (n + 1) // 2
    mask = np.asarray(mask)
    total = 0
    nt = -(-n // TILE)
    for qt in range(nt):
        r0, r1 = qt * TILE, min(n, (qt + 1) * TILE)
        for kt in range(qt + 1):
            if not mask[qt, kt]:
                continue
            k0, k1 = kt * TILE, min(n, (kt + 1) * TILE)
            if kt < qt:
                total += (r1 - r0) * (k1 - k0)
            else:  # diagonal: keys k0..min(i, k1-1) for each row i
                for i in range(r0, r1):
                    total += min(i + 1, k1) - k0
    return total


def causal_pairs_fast(L: int, mask) -> int:
    """Same as causal_pairs for n = L a multiple of 128 (vectorised)."""
    mask = np.asarray(mask).astype(np.int64)
    nt = L // TILE
    off = np.tril(mask[:nt, :nt], k=-1).sum()
    diag = np.trace(mask[:nt, :nt])
    return int(off) * TILE * TILE + int(diag) * (TILE * (TILE + 1) // 2)


def prefill_flops(Hq: int, D: int, seq_lens, mask=None) -> int:
    total = 0
    for n in np.asarray(seq_lens):
        n = int(n)
        if mask is not None and n % TILE == 0:
            total += causal_pairs_fast(n, mask)
        else:
            total += causal_pairs(n, n, mask)
    return 4 * D * Hq * total


def maskgen_bytes(B: int, Hq: int, Hkv: int, D: int, L: int, head_bits) -> int:
    """Algorithmic bytes of the tile-mask generator over full-length sequences:
    fp16 Q read once, the K cache (codes, scales, zeros) read once, and the
    uint8 [B][Hkv][nt][nt] mask written once."""
    nt = -(-L // TILE)
    k_bytes = sum(token_bytes(D, int(b)) for b in head_bits) * L
    return B * (Hq * L * D * 2 + k_bytes + Hkv * nt * nt)


def score_matrix_bytes(n: int, elem_bytes: int = 2) -> int:
    """Bytes of a full n x n score matrix (what tiling never materialises)."""
    return n * n * elem_bytes


def kv_cache_bytes_dense(batch: int, seq_len: int, layers: int, hidden: int,
                         elem_bytes: int = 2) -> int:
    """2 * batch * seq_len * layers * hidden * bytes: a dense (MHA, fp16)
    whole-model KV cache."""
    return 2 * batch * seq_len * layers * hidden * elem_bytes
