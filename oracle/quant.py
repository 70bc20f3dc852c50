"""Grouped asymmetric KV quantisation, fp64 reference.  TEST INFRASTRUCTURE ONLY.

Source: "分块稀疏注意力与KV Cache量化：长文本推理显存优化实践" (xdnf.cn), section 2.4:
adjacent values along the channel dimension form small groups, and each group
keeps its own scale and zero-point; section 3.2 gives the group size, 32.  The
page fixes nothing else, so the readings below are this library's own (they are
listed with their reasons in the design notes):

1. A group is 32 consecutive head_dim channels of one token of one KV head.
2. Its range is extended to contain 0:  lo = min(0, min x), hi = max(0, max x).
3. With qmax = 2**bits - 1, the scale s is the smallest fp16 value with
   s * qmax >= hi - lo (the quotient (hi - lo)/qmax rounded toward +inf).
   A group with hi == lo (all zeros) gets s = +0, z = 0 and all codes 0.
4. The zero-point z = round-half-even(-lo / s) of the exact quotient (always in
   [0, qmax]); codes c = clamp(round-half-even(x / s) + z, 0, qmax).
5. The dequantised value is (c - z) * s; it is exact in fp32 (at most
   8 + 11 significant bits), and its fp16 form is the round-to-nearest-even of
   that exact value.
6. Unsigned codes; int4 codes are packed two per byte, the first of the pair in
   the low nibble.

Byte layouts of one cache (K or V) of shape B x Hkv x capacity x D, with
per-head bit widths bits[h] and RB(h) = D * bits[h] / 8 code bytes per token:

* codes of (b, h) start at  b * cap * sum_h RB(h)  +  cap * sum_{h' < h} RB(h').
* "token" layout (used for K): token t's RB(h) bytes sit at t * RB(h); within
  them channel c's code is byte c (int8) or nibble c % 2 of byte c // 2 (int4).
  scales fp16 [B][Hkv][cap][G], zeros u8 [B][Hkv][cap][G], G = D / 32.
* "channel" layout (used for V): tokens come in blocks of 32; block j of a
  head holds D rows of 32 * bits / 8 bytes; row d has token t's code for
  channel d at byte t % 32 (int8) or nibble (t % 32) % 2 of byte
  (t % 32) // 2 (int4).  scales fp16 [B][Hkv][G][cap], zeros u8 [B][Hkv][G][cap].
  The capacity is a multiple of 128 (the KV-tile size) in both layouts.

Pins (tests/test_oracle_quant.py): exact-rational re-derivation of s, z and c
per group (``oracle.exact``), a division-free brute-force nearest-code search,
the round-trip bound |x - x_hat| <= s/2, zeros map to exact zeros, grid points
round-trip exactly, s is the least fp16 >= (hi - lo)/qmax, byte layouts against
hand-written fixtures in tests/golden/.
"""
from __future__ import annotations

import numpy as np

GROUP = 32
BLOCK = 32      # tokens per block of the channel layout
CAP_MULTIPLE = 128


def _fp16_ceil_div(span: np.ndarray, qmax: int) -> np.ndarray:
    """Smallest fp16 s with s * qmax >= span (span >= 0 exact fp64 values).

    Start from the fp16 nearest to the fp64 quotient and step by fp16 ulps
    until the two exact conditions hold; the products s * qmax are exact in
    fp64 (11 + 8 significant bits).
    """
    s = (span / qmax).astype(np.float16)
    inf16 = np.float16(np.inf)
    for _ in range(4):
        low = s.astype(np.float64) * qmax < span
        if not low.any():
            break
        s = np.where(low, np.nextafter(s, inf16), s)
    for _ in range(4):
        prev = np.nextafter(s, np.float16(0))
        ok_prev = (prev.astype(np.float64) * qmax >= span) & (s > 0)
        if not ok_prev.any():
            break
        s = np.where(ok_prev, prev, s)
    return s


def quantize(x: np.ndarray, bits: int):
    """Quantise fp16 values ``x[..., D]`` group-wise along the last axis.

    Returns (codes uint8 [..., D] unpacked, scales fp16 [..., D/32],
    zeros uint8 [..., D/32]).  Section 2.4 of the block-sparse/KV-quantisation
    page; rounding readings 2-4 of the module header.
    """
    if bits not in (4, 8):
        raise ValueError("bits must be 4 or 8")
    x = np.asarray(x)
    if x.dtype != np.float16:
        raise TypeError("x must be fp16")
    D = x.shape[-1]
    if D % GROUP:
        raise ValueError("head_dim must be a multiple of 32")
    xg = x.astype(np.float64).reshape(*x.shape[:-1], D // GROUP, GROUP)
    if not np.isfinite(xg).all():
        raise ValueError("non-finite K/V values are outside the quantiser's domain")
    qmax = (1 << bits) - 1
    lo = np.minimum(xg.min(axis=-1), 0.0)
    hi = np.maximum(xg.max(axis=-1), 0.0)
    span = hi - lo                                   # exact: fp16 operands
    s16 = _fp16_ceil_div(span, qmax)
    s16 = np.where(span == 0, np.float16(0), s16)
    s = s16.astype(np.float64)
    safe = np.where(s > 0, s, 1.0)
    z = np.where(s > 0, np.rint(-lo / safe), 0.0)
    c = np.rint(xg / safe[..., None]) + z[..., None]
    c = np.clip(c, 0, qmax)
    c = np.where((s > 0)[..., None], c, 0.0)
    codes = c.astype(np.uint8).reshape(x.shape)
    return codes, s16, z.astype(np.uint8)


def dequantize(codes: np.ndarray, scales: np.ndarray, zeros: np.ndarray,
               dtype=np.float64) -> np.ndarray:
    """x_hat = (c - z) * s per element (reading 5).  ``dtype`` float64 gives the
    exact value, float32 the same value (exact), float16 its RNE rounding."""
    D = codes.shape[-1]
    cg = codes.astype(np.float64).reshape(*codes.shape[:-1], D // GROUP, GROUP)
    xh = (cg - zeros.astype(np.float64)[..., None]) * scales.astype(np.float64)[..., None]
    return xh.reshape(codes.shape).astype(dtype)


# ----------------------------------------------------------------------------
# byte layouts
# ----------------------------------------------------------------------------

def pack_nibbles(c: np.ndarray) -> np.ndarray:
    """Two 4-bit codes per byte along the last axis: element 2j in the low
    nibble, element 2j+1 in the high nibble (reading 6)."""
    if c.shape[-1] % 2:
        raise ValueError("odd length")
    c = c.astype(np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(b: np.ndarray) -> np.ndarray:
    out = np.empty(b.shape[:-1] + (b.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = b & 0x0F
    out[..., 1::2] = b >> 4
    return out


def row_bytes(D: int, bits: int) -> int:
    return D * bits // 8


def head_offsets(D: int, cap: int, head_bits) -> tuple[list[int], int]:
    """Byte offset of each head's code slab inside one batch entry, and the
    batch stride."""
    offs, acc = [], 0
    for b in head_bits:
        offs.append(acc)
        acc += cap * row_bytes(D, int(b))
    return offs, acc


class Cache:
    """A quantised K or V cache in the library's byte layout, built and read on
    the CPU.  Fields mirror the C descriptor: flat ``codes`` (uint8), ``scales``
    (fp16), ``zeros`` (uint8)."""

    def __init__(self, B: int, Hkv: int, D: int, cap: int, head_bits,
                 layout: str):
        if layout not in ("token", "channel"):
            raise ValueError(layout)
        if cap % CAP_MULTIPLE:
            raise ValueError("capacity must be a multiple of 128")
        self.B, self.Hkv, self.D, self.cap = B, Hkv, D, cap
        self.bits = [int(b) for b in head_bits]
        self.layout = layout
        self.G = D // GROUP
        self.offs, self.bstride = head_offsets(D, cap, self.bits)
        self.codes = np.zeros(B * self.bstride, dtype=np.uint8)
        self.scales = np.zeros((B, Hkv, self.G, cap) if layout == "channel"
                               else (B, Hkv, cap, self.G), dtype=np.float16)
        self.zeros = np.zeros(self.scales.shape, dtype=np.uint8)

    # -- code slab of one (b, h) as a [cap][D] array of unpacked codes ------
    def _slab(self, b: int, h: int) -> np.ndarray:
        n = self.cap * row_bytes(self.D, self.bits[h])
        o = b * self.bstride + self.offs[h]
        return self.codes[o:o + n]

    def write(self, b: int, h: int, start: int, codes: np.ndarray,
              scales: np.ndarray, zeros: np.ndarray) -> None:
        """Store unpacked codes [S][D], scales [S][G], zeros [S][G] for tokens
        start .. start+S-1 of (b, h)."""
        S = codes.shape[0]
        full = self.read_codes(b, h)
        full[start:start + S] = codes
        slab = self._slab(b, h)
        bits = self.bits[h]
        if self.layout == "token":
            rows = full if bits == 8 else pack_nibbles(full)
            slab[:] = rows.reshape(-1)
            self.scales[b, h, start:start + S] = scales
            self.zeros[b, h, start:start + S] = zeros
        else:
            nblk = self.cap // BLOCK
            blk = full.reshape(nblk, BLOCK, self.D).transpose(0, 2, 1)  # [j][d][t]
            rows = blk if bits == 8 else pack_nibbles(blk)
            slab[:] = np.ascontiguousarray(rows).reshape(-1)
            self.scales[b, h, :, start:start + S] = scales.T
            self.zeros[b, h, :, start:start + S] = zeros.T

    def read_codes(self, b: int, h: int) -> np.ndarray:
        """Unpacked codes [cap][D] of (b, h)."""
        slab = self._slab(b, h)
        bits = self.bits[h]
        if self.layout == "token":
            rows = slab.reshape(self.cap, row_bytes(self.D, bits))
            return rows.copy() if bits == 8 else unpack_nibbles(rows)
        nblk = self.cap // BLOCK
        rows = slab.reshape(nblk, self.D, BLOCK * bits // 8)
        blk = rows if bits == 8 else unpack_nibbles(rows)       # [j][d][t]
        return np.ascontiguousarray(blk.transpose(0, 2, 1)).reshape(self.cap, self.D)

    def read_meta(self, b: int, h: int):
        """(scales fp16 [cap][G], zeros u8 [cap][G]) of (b, h)."""
        if self.layout == "token":
            return self.scales[b, h].copy(), self.zeros[b, h].copy()
        return self.scales[b, h].T.copy(), self.zeros[b, h].T.copy()

    def dequantized(self, b: int, h: int, dtype=np.float64) -> np.ndarray:
        c = self.read_codes(b, h)
        s, z = self.read_meta(b, h)
        return dequantize(c, s, z, dtype)


def build_cache(x: np.ndarray, head_bits, layout: str, seq_lens=None,
                cap: int | None = None) -> Cache:
    """Quantise fp16 ``x`` [B][Hkv][S][D] (tokens 0..S-1) into a new cache.

    Tokens at or beyond ``seq_lens[b]`` are quantised too (they are zero in the
    generated inputs), exactly as a kernel call over tokens 0..S-1 would."""
    B, Hkv, S, D = x.shape
    cap = cap or S
    c = Cache(B, Hkv, D, cap, head_bits, layout)
    for b in range(B):
        for h in range(Hkv):
            codes, s, z = quantize(x[b, h], c.bits[h])
            c.write(b, h, 0, codes, s, z)
    return c


def dequantized_all(cache: Cache, dtype=np.float64) -> np.ndarray:
    """Dequantised values [B][Hkv][cap][D]."""
    out = np.empty((cache.B, cache.Hkv, cache.cap, cache.D), dtype=dtype)
    for b in range(cache.B):
        for h in range(cache.Hkv):
            out[b, h] = cache.dequantized(b, h, dtype)
    return out
