"""Per-KV-head precision assignment from measured sensitivity.  TEST
INFRASTRUCTURE ONLY.

Source: section 2.4 of "分块稀疏注意力与KV Cache量化：长文本推理显存优化实践"
(xdnf.cn): every attention head gets a sensitivity score, and the sensitive
heads are stored at the higher precision while the others use fewer bits;
section 3.4 of the same page: keeping more heads at high precision lowers the
memory saving (from about 4x to about 2.5x).  The page does not define the
score.  Reading taken (one score per KV head, since a KV head's cache is what
is stored at one width):

    S_g = sum_b sum_{h : h // r = g} sum_d (O4[b, h, d] - O8[b, h, d])^2

where O_bits is the decode attention (oracle.attention.decode) of calibration
queries q[b][h] over keys and values 0 .. n_b - 1 of batch entry b, with every
head's K and V quantised at `bits` (oracle.quant), i.e. how far the head's
attention output moves when its cache drops from int8 to int4.  Assignment:
the n_high heads with the largest S get 8 bits (ties: the lower head index
first), the others 4.

Pins (tests/test_oracle_sensitivity.py): zero K/V give S = 0; a head with a
planted outlier channel ranks first; copies of a head score equally and tie to
the lower index; the composition against pure-Python brute-force attention;
assignment counts and extremes; the bytes-per-token saving for 0 .. Hkv
high-precision heads is monotone between the all-int4 and all-int8 figures.
"""
from __future__ import annotations

import numpy as np

from oracle import attention as oa
from oracle import quant as oq


def outputs(q, k, v, seq_lens, bits: int, scale=None, workers=1):
    """Decode outputs fp64 [B][Hq][D] with every head of K and V at `bits`."""
    B, Hkv, S, D = k.shape
    hb = [bits] * Hkv
    kh = oq.dequantized_all(oq.build_cache(k, hb, "token", cap=S))
    vh = oq.dequantized_all(oq.build_cache(v, hb, "channel", cap=S))
    return oa.decode(q, kh, vh, seq_lens, scale=scale, workers=workers)


def sensitivity(q, k, v, seq_lens, scale=None, workers=1) -> np.ndarray:
    """S_g for g < Hkv (fp64).  q fp16 [B][Hq][D]; k, v fp16 [B][Hkv][S][D]
    with S a multiple of 128."""
    Hq, Hkv = q.shape[1], k.shape[1]
    r = Hq // Hkv
    o8 = outputs(q, k, v, seq_lens, 8, scale, workers)
    o4 = outputs(q, k, v, seq_lens, 4, scale, workers)
    d2 = ((o4 - o8) ** 2).sum(axis=(0, 2))          # [Hq]
    return d2.reshape(Hkv, r).sum(axis=1)


def assign(scores, n_high: int) -> np.ndarray:
    """Bits per KV head: 8 for the n_high largest scores (ties: lower index)."""
    s = np.asarray(scores, dtype=np.float64)
    H = s.shape[0]
    if not 0 <= n_high <= H:
        raise ValueError("n_high must lie in [0, Hkv]")
    order = np.lexsort((np.arange(H), -s))            # by score descending, then index
    bits = np.full(H, 4, dtype=np.uint8)
    bits[order[:n_high]] = 8
    return bits


def saving(bits, D: int = 128) -> float:
    """fp16 bytes over quantised bytes per token, K and V together (codes plus
    an fp16 scale and a u8 zero-point per group of 32)."""
    G = D // 32
    q = sum(2 * (D * int(b) // 8 + 3 * G) for b in bits)
    return 2 * 2 * D * len(bits) / q
