"""Python binding of libtaq.so: tiled causal attention over a grouped-quantized
KV cache on MI355X (gfx950).

This module only marshals arguments: every step of the computation runs in the
library's HIP kernels.  PyTorch provides device memory and the current stream.
There is no fallback: if ``libtaq.so`` is missing or the device is not gfx950,
calls raise.

Names follow the C ABI in ``include/taq.h``: ``kv_quantize``,
``kv_dequantize``, ``attn_decode``, ``attn_prefill``.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtaq.so")

LAYOUT_TOKEN = 0
LAYOUT_CHANNEL = 1

STATUS = {0: "OK", 1: "INVALID_ARGUMENT", 2: "UNSUPPORTED", 3: "MISALIGNED",
          4: "WORKSPACE_TOO_SMALL", 5: "HIP"}

EXPORTS = ("taq_last_error", "taq_abi_version", "taq_device_check",
           "taq_kv_codes_bytes", "taq_kv_meta_count", "taq_kv_quantize",
           "taq_kv_dequantize", "taq_attn_decode_workspace_bytes",
           "taq_attn_decode", "taq_attn_prefill", "taq_debug_set_arch_override",
           "taq_kv_append", "taq_attn_prefill_chunk", "taq_tile_mask_workspace_bytes",
           "taq_tile_mask_generate", "taq_attn_decode_two_pass",
           "taq_head_sensitivity_workspace_bytes", "taq_head_sensitivity",
           "taq_attn_prefill_chunk_workspace_bytes", "taq_kv_quantize_pair",
           "taq_attn_decode_noalloc", "taq_tile_mask_generate_chunk")


class TaqError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"taq {STATUS.get(status, status)}: {msg}")
        self.status = status
        self.status_name = STATUS.get(status, str(status))


class _Cache(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("group_size", ctypes.c_int32),
                ("capacity", ctypes.c_int32), ("layout", ctypes.c_int32),
                ("bits", ctypes.c_void_p), ("codes", ctypes.c_void_p),
                ("scales", ctypes.c_void_p), ("zeros", ctypes.c_void_p)]


class _Mask(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("tile", ctypes.c_int32),
                ("n_q_tiles", ctypes.c_int32), ("n_k_tiles", ctypes.c_int32),
                ("stride_b", ctypes.c_int64), ("stride_h", ctypes.c_int64)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libtaq.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m tiled_attention_quantized_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ, F = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                          ctypes.c_size_t, ctypes.c_float)
    CP, MP = ctypes.POINTER(_Cache), ctypes.POINTER(_Mask)
    sig = {
        "taq_last_error": (ctypes.c_char_p, []),
        "taq_abi_version": (ctypes.c_int, []),
        "taq_device_check": (ctypes.c_int, [ctypes.c_int]),
        "taq_kv_codes_bytes": (SZ, [CP]),
        "taq_kv_meta_count": (SZ, [CP]),
        "taq_kv_quantize": (ctypes.c_int, [CP, P, I32, I32, P]),
        "taq_kv_quantize_pair": (ctypes.c_int, [CP, CP, P, P, I32, I32, P]),
        "taq_kv_dequantize": (ctypes.c_int, [CP, I32, I32, P, P, P]),
        "taq_attn_decode_workspace_bytes": (SZ, [CP, I32, I32]),
        "taq_attn_decode": (ctypes.c_int, [CP, CP, P, I32, P, I32, MP, F, P, P, SZ, P]),
        "taq_attn_decode_two_pass": (ctypes.c_int, [CP, CP, P, I32, P, I32, MP, F, P, P, SZ, P]),
        "taq_attn_decode_noalloc": (ctypes.c_int, [CP, CP, P, I32, P, I32, MP, F, P, P]),
        "taq_attn_prefill": (ctypes.c_int, [CP, CP, P, I32, P, I32, MP, F, P, P]),
        "taq_debug_set_arch_override": (None, [ctypes.c_char_p]),
        "taq_kv_append": (ctypes.c_int, [CP, P, P, I32, P]),
        "taq_attn_prefill_chunk": (ctypes.c_int, [CP, CP, P, I32, I32, P, I32, MP, F, P, P, SZ,
                                                  P]),
        "taq_attn_prefill_chunk_workspace_bytes": (SZ, [CP, I32, I32, I32]),
        "taq_tile_mask_workspace_bytes": (SZ, [CP, I32]),
        "taq_head_sensitivity_workspace_bytes": (SZ, [I32, I32, I32, I32]),
        "taq_head_sensitivity": (ctypes.c_int, [P, P, P, I32, I32, I32, P, I32, F, I32, P, P, P,
                                                SZ, P]),
        "taq_tile_mask_generate": (ctypes.c_int, [CP, P, I32, P, I32, I32, P, P, SZ, P]),
        "taq_tile_mask_generate_chunk": (ctypes.c_int, [CP, P, I32, I32, P, I32, I32, P, P, SZ,
                                                         P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


def _check(status: int) -> None:
    if status != 0:
        raise TaqError(status, lib().taq_last_error().decode())


def _stream(device) -> int:
    import torch
    return torch.cuda.current_stream(device).cuda_stream


def _ptr(t) -> int:
    return 0 if t is None else int(t.data_ptr())


class KVCache:
    """A quantised K or V cache in device memory (torch tensors own the bytes).

    K caches use ``LAYOUT_TOKEN``, V caches ``LAYOUT_CHANNEL``."""

    def __init__(self, batch: int, num_kv_heads: int, head_dim: int, capacity: int,
                 bits: Sequence[int], layout: int, device="cuda"):
        import torch
        self.batch, self.num_kv_heads = int(batch), int(num_kv_heads)
        self.head_dim, self.capacity = int(head_dim), int(capacity)
        self.layout = int(layout)
        self.bits = np.ascontiguousarray(np.asarray(bits, dtype=np.uint8))
        if self.bits.shape != (self.num_kv_heads,):
            raise ValueError("bits must have one entry per KV head")
        d = self._desc(validate_only=True)
        nbytes = lib().taq_kv_codes_bytes(ctypes.byref(d))
        nmeta = lib().taq_kv_meta_count(ctypes.byref(d))
        if nbytes == 0 or nmeta == 0:
            raise TaqError(1, lib().taq_last_error().decode())
        self.codes = torch.zeros(nbytes, dtype=torch.uint8, device=device)
        self.scales = torch.zeros(nmeta, dtype=torch.int16, device=device)
        self.zeros = torch.zeros(nmeta, dtype=torch.uint8, device=device)

    def _desc(self, validate_only=False) -> _Cache:
        fake = 16  # a non-null, aligned placeholder used only to size the buffers
        return _Cache(self.batch, self.num_kv_heads, self.head_dim, 32, self.capacity,
                      self.layout, self.bits.ctypes.data,
                      fake if validate_only else _ptr(self.codes),
                      fake if validate_only else _ptr(self.scales),
                      fake if validate_only else _ptr(self.zeros))

    def desc(self) -> _Cache:
        return self._desc()

    @property
    def device(self):
        return self.codes.device


@dataclass
class TileMask:
    """KV-tile keep mask (device uint8 tensor) and its geometry."""
    data: "object"
    n_q_tiles: int
    n_k_tiles: int
    stride_b: int = 0
    stride_h: int = 0

    def desc(self) -> _Mask:
        return _Mask(_ptr(self.data), 128, self.n_q_tiles, self.n_k_tiles,
                     self.stride_b, self.stride_h)


def device_check(device: int = 0) -> None:
    _check(lib().taq_device_check(device))


def kv_quantize(cache: KVCache, x, start: int = 0) -> None:
    """Quantise fp16 x [B][Hkv][S][D] into tokens start .. start+S-1."""
    import torch
    if x.dtype != torch.float16 or not x.is_contiguous() or x.dim() != 4:
        raise ValueError("x must be a contiguous fp16 [B][Hkv][S][D] tensor")
    B, H, S, D = x.shape
    if (B, H, D) != (cache.batch, cache.num_kv_heads, cache.head_dim):
        raise ValueError("x shape does not match the cache")
    d = cache.desc()
    _check(lib().taq_kv_quantize(ctypes.byref(d), _ptr(x), start, S, _stream(x.device)))


def kv_quantize_pair(k: KVCache, v: KVCache, xk, xv, start: int = 0) -> None:
    """Quantise fp16 xk and xv [B][Hkv][S][D] into tokens start .. start+S-1 of
    the K and V caches in one launch (byte-identical to two kv_quantize calls)."""
    import torch
    for cache, x in ((k, xk), (v, xv)):
        if x.dtype != torch.float16 or not x.is_contiguous() or x.dim() != 4:
            raise ValueError("xk and xv must be contiguous fp16 [B][Hkv][S][D] tensors")
        B, H, S, D = x.shape
        if (B, H, D) != (cache.batch, cache.num_kv_heads, cache.head_dim):
            raise ValueError("x shape does not match its cache")
    if xk.shape[2] != xv.shape[2]:
        raise ValueError("xk and xv must hold the same number of tokens")
    kd, vd = k.desc(), v.desc()
    _check(lib().taq_kv_quantize_pair(ctypes.byref(kd), ctypes.byref(vd), _ptr(xk), _ptr(xv),
                                      start, xk.shape[2], _stream(xk.device)))


def kv_append(cache: KVCache, x, starts) -> None:
    """Quantise fp16 x [B][Hkv][S][D] into positions starts[b] .. starts[b]+S-1
    of each batch entry b; starts is a device int32 [B] tensor."""
    import torch
    if x.dtype != torch.float16 or not x.is_contiguous() or x.dim() != 4:
        raise ValueError("x must be a contiguous fp16 [B][Hkv][S][D] tensor")
    B, H, S, D = x.shape
    if (B, H, D) != (cache.batch, cache.num_kv_heads, cache.head_dim):
        raise ValueError("x shape does not match the cache")
    if starts.dtype != torch.int32 or starts.numel() != B or not starts.is_contiguous():
        raise ValueError("starts must be a contiguous int32 [B] tensor")
    d = cache.desc()
    _check(lib().taq_kv_append(ctypes.byref(d), _ptr(x), _ptr(starts), S, _stream(x.device)))


def kv_dequantize(cache: KVCache, start: int, count: int, f32: bool = True,
                  f16: bool = False):
    """Dequantised tokens [B][Hkv][count][D] as (fp32 or None, fp16 or None)."""
    import torch
    shp = (cache.batch, cache.num_kv_heads, count, cache.head_dim)
    o32 = torch.empty(shp, dtype=torch.float32, device=cache.device) if f32 else None
    o16 = torch.empty(shp, dtype=torch.float16, device=cache.device) if f16 else None
    d = cache.desc()
    _check(lib().taq_kv_dequantize(ctypes.byref(d), start, count, _ptr(o32), _ptr(o16),
                                   _stream(cache.device)))
    return o32, o16


def decode_workspace_bytes(k: KVCache, num_q_heads: int, max_seq_len: int) -> int:
    d = k.desc()
    return int(lib().taq_attn_decode_workspace_bytes(ctypes.byref(d), num_q_heads,
                                                      max_seq_len))


def attn_decode(k: KVCache, v: KVCache, q, seq_lens, max_seq_len: int,
                mask: Optional[TileMask] = None, softmax_scale: float = 0.0,
                out=None, workspace=None, two_pass: bool = False):
    """Decode attention; q fp16 [B][Hq][D], seq_lens int32 [B] on the device.
    two_pass=True runs the literal two-pass softmax (global maximum first)."""
    import torch
    B, Hq, D = q.shape
    if out is None:
        out = torch.empty_like(q)
    if workspace is None:
        nb = decode_workspace_bytes(k, Hq, max_seq_len)
        workspace = torch.empty(nb, dtype=torch.uint8, device=q.device)
    kd, vd = k.desc(), v.desc()
    md = mask.desc() if mask is not None else None
    fn = lib().taq_attn_decode_two_pass if two_pass else lib().taq_attn_decode
    _check(fn(ctypes.byref(kd), ctypes.byref(vd), _ptr(q), Hq, _ptr(seq_lens), max_seq_len,
              ctypes.byref(md) if md is not None else None, softmax_scale, _ptr(out),
              _ptr(workspace), workspace.numel() * workspace.element_size(),
              _stream(q.device)))
    return out


def attn_decode_noalloc(k: KVCache, v: KVCache, q, seq_lens, max_seq_len: int, out,
                        mask: Optional[TileMask] = None, softmax_scale: float = 0.0):
    """Decode attention with no workspace: the split partials go to the
    library's own fixed device scratch (TAQ_DECODE_SCRATCH_BYTES per GPU);
    nothing is allocated, so the caller passes the output tensor."""
    B, Hq, D = q.shape
    kd, vd = k.desc(), v.desc()
    md = mask.desc() if mask is not None else None
    _check(lib().taq_attn_decode_noalloc(ctypes.byref(kd), ctypes.byref(vd), _ptr(q), Hq,
                                         _ptr(seq_lens), max_seq_len,
                                         ctypes.byref(md) if md is not None else None,
                                         softmax_scale, _ptr(out), _stream(q.device)))
    return out


def attn_prefill(k: KVCache, v: KVCache, q, seq_lens, mask: Optional[TileMask] = None,
                 softmax_scale: float = 0.0, out=None):
    """Causal prefill; q fp16 [B][Hq][L][D] with L the padded length."""
    import torch
    B, Hq, L, D = q.shape
    if out is None:
        out = torch.empty_like(q)
    kd, vd = k.desc(), v.desc()
    md = mask.desc() if mask is not None else None
    _check(lib().taq_attn_prefill(ctypes.byref(kd), ctypes.byref(vd), _ptr(q), Hq,
                                  _ptr(seq_lens), L,
                                  ctypes.byref(md) if md is not None else None,
                                  softmax_scale, _ptr(out), _stream(q.device)))
    return out


def prefill_chunk_workspace_bytes(k: KVCache, num_q_heads: int, q_len: int,
                                  max_seq_len: int) -> int:
    d = k.desc()
    return int(lib().taq_attn_prefill_chunk_workspace_bytes(ctypes.byref(d), num_q_heads, q_len,
                                                            max_seq_len))


def attn_prefill_chunk(k: KVCache, v: KVCache, q, seq_lens, max_seq_len: int,
                       mask: Optional[TileMask] = None, softmax_scale: float = 0.0,
                       out=None, workspace="auto"):
    """Chunked prefill: q fp16 [B][Hq][Lq][D] holds the last Lq positions of each
    sequence (already appended to the cache); row i of batch b sits at
    position seq_lens[b] - Lq + i.  workspace: "auto" allocates the key-range
    split workspace the library asks for, None runs unsplit, or a device
    uint8 tensor."""
    import torch
    B, Hq, Lq, D = q.shape
    if out is None:
        out = torch.empty_like(q)
    if isinstance(workspace, str):
        nb = prefill_chunk_workspace_bytes(k, Hq, Lq, max_seq_len)
        workspace = torch.empty(nb, dtype=torch.uint8, device=q.device) if nb else None
    kd, vd = k.desc(), v.desc()
    md = mask.desc() if mask is not None else None
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().taq_attn_prefill_chunk(ctypes.byref(kd), ctypes.byref(vd), _ptr(q), Hq, Lq,
                                        _ptr(seq_lens), max_seq_len,
                                        ctypes.byref(md) if md is not None else None,
                                        softmax_scale, _ptr(out), _ptr(workspace), nbytes,
                                        _stream(q.device)))
    return out


def tile_mask_workspace_bytes(k: KVCache, max_seq_len: int) -> int:
    d = k.desc()
    return int(lib().taq_tile_mask_workspace_bytes(ctypes.byref(d), max_seq_len))


def tile_mask_generate(k: KVCache, q, seq_lens, skip_per_mille: int, out=None, workspace=None):
    """Training-free KV-tile mask from the queries and the quantised keys:
    returns a TileMask over a uint8 [B][Hkv][nt][nt] tensor (nt =
    ceil(L / 128) for q fp16 [B][Hq][L][D])."""
    import torch
    B, Hq, L, D = q.shape
    nt = (L + 127) // 128
    if q.dtype != torch.float16 or not q.is_contiguous() or q.dim() != 4:
        raise ValueError("q must be a contiguous fp16 [B][Hq][L][D] tensor")
    if out is None:
        out = torch.empty((B, k.num_kv_heads, nt, nt), dtype=torch.uint8, device=q.device)
    elif (out.dtype != torch.uint8 or not out.is_contiguous()
          or tuple(out.shape) != (B, k.num_kv_heads, nt, nt)):
        raise ValueError("out must be a contiguous uint8 [B][Hkv][nt][nt] tensor")
    if workspace is None:
        nb = tile_mask_workspace_bytes(k, L)
        workspace = torch.empty(max(nb, 1), dtype=torch.uint8, device=q.device)
    kd = k.desc()
    _check(lib().taq_tile_mask_generate(ctypes.byref(kd), _ptr(q), Hq, _ptr(seq_lens), L,
                                        int(skip_per_mille), _ptr(out), _ptr(workspace),
                                        workspace.numel() * workspace.element_size(),
                                        _stream(q.device)))
    return TileMask(out, nt, nt, stride_b=k.num_kv_heads * nt * nt, stride_h=nt * nt)


def tile_mask_generate_chunk(k: KVCache, q, seq_lens, max_seq_len: int, skip_per_mille: int,
                             out=None, workspace=None):
    """The KV-tile mask rows of one turn of a multi-turn prefill: q fp16
    [B][Hq][q_len][D] holds the last q_len positions of each sequence (whose
    keys are in `k`); returns a TileMask over uint8 [B][Hkv][nt][nt], nt =
    ceil(max_seq_len / 128), indexed by positions (for attn_prefill_chunk)."""
    import torch
    if q.dtype != torch.float16 or not q.is_contiguous() or q.dim() != 4:
        raise ValueError("q must be a contiguous fp16 [B][Hq][q_len][D] tensor")
    B, Hq, Lq, D = q.shape
    nt = (max_seq_len + 127) // 128
    if out is None:
        out = torch.empty((B, k.num_kv_heads, nt, nt), dtype=torch.uint8, device=q.device)
    elif (out.dtype != torch.uint8 or not out.is_contiguous()
          or tuple(out.shape) != (B, k.num_kv_heads, nt, nt)):
        raise ValueError("out must be a contiguous uint8 [B][Hkv][nt][nt] tensor")
    if workspace is None:
        nb = tile_mask_workspace_bytes(k, max_seq_len)
        workspace = torch.empty(max(nb, 1), dtype=torch.uint8, device=q.device)
    kd = k.desc()
    _check(lib().taq_tile_mask_generate_chunk(ctypes.byref(kd), _ptr(q), Hq, Lq, _ptr(seq_lens),
                                              max_seq_len, int(skip_per_mille), _ptr(out),
                                              _ptr(workspace),
                                              workspace.numel() * workspace.element_size(),
                                              _stream(q.device)))
    return TileMask(out, nt, nt, stride_b=k.num_kv_heads * nt * nt, stride_h=nt * nt)


def head_sensitivity(k, v, q, seq_lens, n_high: int, softmax_scale: float = 0.0,
                     workspace=None):
    """Per-KV-head sensitivity and precision: k, v fp16 [B][Hkv][S][D] (the
    calibration context), q fp16 [B][Hq][D].  Returns (scores float64 [Hkv],
    bits uint8 [Hkv]) as device tensors."""
    import torch
    for name, t, nd in (("k", k, 4), ("v", v, 4), ("q", q, 3)):
        if t.dtype != torch.float16 or not t.is_contiguous() or t.dim() != nd:
            raise ValueError(f"{name} must be a contiguous fp16 tensor of rank {nd}")
    B, Hkv, S, D = k.shape
    Hq = q.shape[1]
    if tuple(v.shape) != tuple(k.shape) or q.shape[0] != B or q.shape[2] != D:
        raise ValueError("k, v and q shapes do not match")
    scores = torch.empty(Hkv, dtype=torch.float64, device=k.device)
    bits = torch.empty(Hkv, dtype=torch.uint8, device=k.device)
    if workspace is None:
        nb = int(lib().taq_head_sensitivity_workspace_bytes(B, Hkv, Hq, S))
        workspace = torch.empty(max(nb, 1), dtype=torch.uint8, device=k.device)
    _check(lib().taq_head_sensitivity(_ptr(k), _ptr(v), _ptr(q), B, Hkv, Hq, _ptr(seq_lens), S,
                                      softmax_scale, int(n_high), _ptr(scores), _ptr(bits),
                                      _ptr(workspace),
                                      workspace.numel() * workspace.element_size(),
                                      _stream(k.device)))
    return scores, bits
