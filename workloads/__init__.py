"""Seeded synthetic inputs for tiled attention over a grouped-quantized KV cache.

This module is shared by the tests, the bench and the oracle's callers.  It holds
no arithmetic of the method itself: it only draws fp16 tensors, context lengths,
per-head bit widths, outlier positions and KV-tile skip masks, in a fixed draw
order, from ``numpy.random.default_rng(seed)``.

Workloads (all head_dim 128, quantisation group 32 along head_dim):

* ``decode_4k``        - decode, B=1, Hq=8, Hkv=2, context 4096, int8 K/V.
* ``prefill_8k``       - causal prefill, B=1, Hq=32, Hkv=8, L=8192, int8 K/V.
* ``decode_ragged``    - decode, B=64, Hq=32, Hkv=8, lengths uniform in
                         [1024, 32768], int4 K/V.
* ``decode_128k_mixed``- decode, B=8, Hq=32, Hkv=8, context 131072, two seeded
                         KV heads int8 and six int4, 1% of K channels x8.
* ``prefill_128k_sparse`` - causal prefill, B=1, Hq=32, Hkv=8, L=131072,
                         int8, 128x128 KV-tile mask that drops a seeded 25% of
                         the off-diagonal tiles other than the first KV tile.

Draw order for one workload: structural choices (lengths, int8 heads, outlier
pairs, mask), then Q, then K, then V; each tensor is drawn as float32 standard
normal one (batch, head) slab at a time and rounded to fp16.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field
from typing import Optional, Tuple

import numpy as np

TILE = 128          # KV-tile edge of the skip mask and of the V block layout
GROUP = 32          # quantisation group along head_dim


@dataclass(frozen=True)
class Spec:
    """Shape and structure of one synthetic workload."""
    name: str
    kind: str                      # "decode" or "prefill"
    B: int
    Hq: int
    Hkv: int
    D: int = 128
    context: int = 0               # decode: fixed context; prefill: L
    ragged: Optional[Tuple[int, int]] = None   # decode lengths ~ U{lo..hi}
    bits: int = 8                  # default bits for every KV head
    n_int8_heads: int = 0          # mixed precision: this many heads int8, rest `bits`
    outlier_frac: float = 0.0      # fraction of (kv head, channel) pairs of K scaled
    outlier_scale: float = 1.0
    skip_frac: float = 0.0         # prefill: fraction of eligible KV tiles dropped
    seed: int = 0
    capacity: int = 0              # cache capacity (tokens); 0 = round up context

    @property
    def r(self) -> int:
        return self.Hq // self.Hkv

    @property
    def cap(self) -> int:
        if self.capacity:
            return self.capacity
        n = self.max_len
        return max(TILE, -(-n // TILE) * TILE)

    @property
    def max_len(self) -> int:
        if self.ragged is not None:
            return self.ragged[1]
        return self.context

    def replace(self, **kw) -> "Spec":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    "decode_4k": Spec("decode_4k", "decode", B=1, Hq=8, Hkv=2, context=4096,
                      bits=8, seed=1),
    "prefill_8k": Spec("prefill_8k", "prefill", B=1, Hq=32, Hkv=8, context=8192,
                       bits=8, seed=2),
    "decode_ragged": Spec("decode_ragged", "decode", B=64, Hq=32, Hkv=8,
                          ragged=(1024, 32768), bits=4, seed=3),
    "decode_128k_mixed": Spec("decode_128k_mixed", "decode", B=8, Hq=32, Hkv=8,
                              context=131072, bits=4, n_int8_heads=2,
                              outlier_frac=0.01, outlier_scale=8.0, seed=4),
    "prefill_128k_sparse": Spec("prefill_128k_sparse", "prefill", B=1, Hq=32,
                                Hkv=8, context=131072, bits=8, skip_frac=0.25,
                                seed=5),
}


@dataclass
class Structure:
    """Structural draws of a workload (everything except the tensors)."""
    seq_lens: np.ndarray                   # int32 [B]
    head_bits: np.ndarray                  # uint8 [Hkv]
    outliers: np.ndarray                   # int64 [n, 2] (kv head, channel)
    mask: Optional[np.ndarray] = None      # uint8 [nq_tiles, nk_tiles] or None


def _draw_structure(spec: Spec, rng: np.random.Generator) -> Structure:
    if spec.ragged is not None:
        lo, hi = spec.ragged
        lens = rng.integers(lo, hi, size=spec.B, endpoint=True).astype(np.int32)
    else:
        lens = np.full(spec.B, spec.context, dtype=np.int32)

    bits = np.full(spec.Hkv, spec.bits, dtype=np.uint8)
    if spec.n_int8_heads:
        hi8 = rng.choice(spec.Hkv, size=spec.n_int8_heads, replace=False)
        bits[np.sort(hi8)] = 8

    n_out = int(round(spec.outlier_frac * spec.Hkv * spec.D))
    if n_out:
        flat = rng.choice(spec.Hkv * spec.D, size=n_out, replace=False)
        flat = np.sort(flat)
        outliers = np.stack([flat // spec.D, flat % spec.D], axis=1).astype(np.int64)
    else:
        outliers = np.zeros((0, 2), dtype=np.int64)

    mask = None
    if spec.kind == "prefill" and spec.skip_frac > 0:
        mask = skip_mask(spec.context, spec.skip_frac, rng)
    return Structure(lens, bits, outliers, mask)


def skip_mask(L: int, skip_frac: float, rng: np.random.Generator) -> np.ndarray:
    """KV-tile keep mask for causal prefill of length L.

    Entry [qi, kj] = 1 keeps the 128x128 tile, 0 drops it.  The first KV tile
    (kj = 0) and the diagonal (kj = qi) are always kept; entries above the
    diagonal are 0.  Of the eligible tiles (1 <= kj < qi), exactly
    round(skip_frac * count) are dropped, picked by a seeded permutation of the
    eligible tiles listed row-major.
    """
    n = -(-L // TILE)
    m = np.tril(np.ones((n, n), dtype=np.uint8))
    qi, kj = np.nonzero(np.tril(np.ones((n, n), dtype=bool), k=-1))
    elig = kj >= 1
    qi, kj = qi[elig], kj[elig]
    n_skip = int(round(skip_frac * qi.size))
    pick = rng.permutation(qi.size)[:n_skip]
    m[qi[pick], kj[pick]] = 0
    return m


def _normal_f16(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(shape, dtype=np.float32).astype(np.float16)


@dataclass
class Inputs:
    spec: Spec
    structure: Structure
    q: np.ndarray       # fp16 decode [B][Hq][D]; prefill [B][Hq][L][D]
    k: np.ndarray       # fp16 [B][Hkv][cap][D], zero beyond seq_lens[b]
    v: np.ndarray       # fp16 [B][Hkv][cap][D], zero beyond seq_lens[b]


def make_inputs(spec: Spec, seed: Optional[int] = None) -> Inputs:
    """Draw one workload's inputs.  ``seed`` defaults to ``spec.seed``."""
    rng = np.random.default_rng(spec.seed if seed is None else seed)
    st = _draw_structure(spec, rng)
    B, Hq, Hkv, D, cap = spec.B, spec.Hq, spec.Hkv, spec.D, spec.cap

    if spec.kind == "decode":
        q = np.empty((B, Hq, D), dtype=np.float16)
        for b in range(B):
            for h in range(Hq):
                q[b, h] = _normal_f16(rng, (D,))
    else:
        L = spec.context
        q = np.empty((B, Hq, L, D), dtype=np.float16)
        for b in range(B):
            for h in range(Hq):
                q[b, h] = _normal_f16(rng, (L, D))

    out_scale = np.ones((Hkv, D), dtype=np.float32)
    for h, c in st.outliers:
        out_scale[h, c] = spec.outlier_scale

    k = np.zeros((B, Hkv, cap, D), dtype=np.float16)
    for b in range(B):
        n = int(st.seq_lens[b])
        for h in range(Hkv):
            x = rng.standard_normal((n, D), dtype=np.float32)
            if spec.outlier_frac:
                x *= out_scale[h][None, :]
            k[b, h, :n] = x.astype(np.float16)
    v = np.zeros((B, Hkv, cap, D), dtype=np.float16)
    for b in range(B):
        n = int(st.seq_lens[b])
        for h in range(Hkv):
            v[b, h, :n] = _normal_f16(rng, (n, D))
    return Inputs(spec, st, q, k, v)


def small(kind: str, B=1, Hq=4, Hkv=1, L=200, bits=8, ragged=None, seed=0,
          n_int8_heads=0, skip_frac=0.0, capacity=0, outlier_frac=0.0,
          outlier_scale=1.0) -> Spec:
    """A small spec for parity tests (sizes the oracle finishes in seconds)."""
    return Spec(f"small_{kind}", kind, B=B, Hq=Hq, Hkv=Hkv, context=L,
                ragged=ragged, bits=bits, n_int8_heads=n_int8_heads,
                skip_frac=skip_frac, seed=seed, capacity=capacity,
                outlier_frac=outlier_frac, outlier_scale=outlier_scale)
