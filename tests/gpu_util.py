"""Helpers for the GPU parity tests: upload seeded inputs, run the library, and
build the oracle's side from the same fp16 inputs (the oracle never sees any
GPU output)."""
from __future__ import annotations

import sys

import numpy as np
import torch

import tiled_attention_quantized_amd as T
from oracle import quant as oq

TOL = 2e-3          # max-abs bound against the fp64 oracle (fp16 out, fp32 accumulation)


def require_gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    T.device_check(torch.cuda.current_device())


def note(msg: str) -> None:
    """Name the case before a GPU step (flushed, so it survives a crash)."""
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def gpu_cache(x: np.ndarray, bits, layout: int, cap: int) -> T.KVCache:
    """Allocate a cache and fill tokens 0..S-1 with kv_quantize on the GPU."""
    B, H, S, D = x.shape
    c = T.KVCache(B, H, D, cap, bits, layout)
    if S:
        xt = torch.from_numpy(np.ascontiguousarray(x)).cuda()
        T.kv_quantize(c, xt, 0)
    return c


def oracle_cache(x: np.ndarray, bits, layout: str, cap: int) -> oq.Cache:
    return oq.build_cache(x, bits, layout, cap=cap)


def assert_cache_equal(gc: T.KVCache, oc: oq.Cache) -> None:
    torch.cuda.synchronize()
    codes = gc.codes.cpu().numpy()
    scales = gc.scales.cpu().numpy().view(np.uint16).reshape(oc.scales.shape)
    zeros = gc.zeros.cpu().numpy().reshape(oc.zeros.shape)
    assert codes.shape == oc.codes.shape
    bad = np.nonzero(codes != oc.codes)[0]
    assert bad.size == 0, f"{bad.size} code bytes differ, first at {bad[:5]}"
    sb = oc.scales.view(np.uint16)
    assert np.array_equal(scales, sb), f"{int((scales != sb).sum())} scales differ"
    assert np.array_equal(zeros, oc.zeros), f"{int((zeros != oc.zeros).sum())} zeros differ"


def dequant_oracle(oc: oq.Cache, B, H) -> np.ndarray:
    return oq.dequantized_all(oc)


def max_abs(a, b) -> float:
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64)))) if np.size(a) else 0.0


def lens_tensor(lens) -> torch.Tensor:
    return torch.tensor(np.asarray(lens, dtype=np.int32), device="cuda")
