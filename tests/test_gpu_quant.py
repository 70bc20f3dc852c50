"""GPU parity of kv_quantize / kv_dequantize against the oracle: bit-exact codes,
scales, zero-points, int4 packing and dequantised values."""
import numpy as np
import pytest
import torch

import tiled_attention_quantized_amd as T
from oracle import quant as oq
from tests.gpu_util import (require_gpu, note, gpu_cache, oracle_cache, assert_cache_equal)

pytestmark = pytest.mark.gpu

LAYOUTS = [(T.LAYOUT_TOKEN, "token"), (T.LAYOUT_CHANNEL, "channel")]


def adversarial(rng, B, H, S, D):
    """fp16 values that stress rounding: ties on exact scales, zero groups,
    single non-zeros, subnormal ranges, x8 outliers, fp16 extremes."""
    x = rng.standard_normal((B, H, S, D)).astype(np.float32)
    g = x.reshape(B, H, S, D // 32, 32)
    kinds = rng.integers(0, 8, size=(B, H, S, D // 32))
    for idx in np.ndindex(*kinds.shape):
        k = kinds[idx]
        if k == 1:
            g[idx] = 0
        elif k == 2:
            v = g[idx][0]
            g[idx] = 0
            g[idx][rng.integers(32)] = v
        elif k == 3:
            g[idx] = rng.integers(-3, 4, 32) * 2.0 ** -24
        elif k == 4:
            g[idx][rng.integers(32)] *= 8
        elif k == 5:
            s = 2.0 ** rng.integers(-6, 2)
            g[idx] = rng.integers(-20, 40, 32) / 2.0 * s
        elif k == 6:
            g[idx] = rng.choice([65504.0, -65504.0, 1.0, 0.0, -2.0], 32)
    return g.reshape(B, H, S, D).astype(np.float16)


@pytest.mark.parametrize("layout,lname", LAYOUTS)
@pytest.mark.parametrize("bits", [(8,), (4,), (8, 4, 4)])
@pytest.mark.parametrize("D", [128, 64, 32])
def test_quantize_bit_exact(layout, lname, bits, D):
    require_gpu()
    rng = np.random.default_rng(100 + D + len(bits) + layout)
    B, H, cap = 2, len(bits), 384
    S = 300
    x = adversarial(rng, B, H, S, D)
    note(f"kv_quantize layout={lname} bits={bits} D={D} S={S}")
    gc = gpu_cache(x, bits, layout, cap)
    oc = oracle_cache(np.concatenate([x, np.zeros((B, H, cap - S, D), np.float16)], 2),
                      bits, lname, cap)
    assert_cache_equal(gc, oc)
    # dequantised values: fp32 exact, fp16 = RNE of exact
    o32, o16 = T.kv_dequantize(gc, 0, cap, f32=True, f16=True)
    want = oq.dequantized_all(oc)
    assert np.array_equal(o32.cpu().numpy().astype(np.float64), want)
    # The fp16 extremes among the adversarial groups dequantise to exact values
    # beyond fp16's finite range (from 65520 up): RNE gives +-inf there, on both
    # sides, and the bit patterns still have to match.
    with np.errstate(over="ignore"):
        w16 = want.astype(np.float16)
    assert np.array_equal(o16.cpu().numpy().view(np.uint16), w16.view(np.uint16))


@pytest.mark.parametrize("layout,lname", LAYOUTS)
@pytest.mark.parametrize("bits", [(4,), (8,)])
def test_partial_and_single_token_writes(layout, lname, bits):
    """Appending at odd offsets (shared int4 bytes in the channel layout) gives
    the same bytes as one whole write."""
    require_gpu()
    rng = np.random.default_rng(7)
    B, H, D, cap = 1, 1, 128, 256
    x = rng.standard_normal((B, H, cap, D)).astype(np.float16)
    note(f"kv_quantize partial layout={lname} bits={bits}")
    gc = T.KVCache(B, H, D, cap, bits, layout)
    xt = torch.from_numpy(x).cuda()
    for s0, s1 in ((0, 1), (1, 2), (2, 3), (3, 64), (64, 127), (127, 128), (128, 129),
                   (129, 255), (255, 256)):
        T.kv_quantize(gc, xt[:, :, s0:s1].contiguous(), s0)
    oc = oracle_cache(x, bits, lname, cap)
    assert_cache_equal(gc, oc)
    o32, _ = T.kv_dequantize(gc, 5, 100)
    assert np.array_equal(o32.cpu().numpy().astype(np.float64), oq.dequantized_all(oc)[:, :, 5:105])


def test_quantize_decode_workload_head_mix_outliers():
    """The long-context decode workload's K structure (2 int8 heads, 6 int4,
    1% of channels x8) on a short context."""
    require_gpu()
    import workloads as W
    spec = W.WORKLOADS["decode_128k_mixed"].replace(context=1024, B=2)
    inp = W.make_inputs(spec)
    bits = inp.structure.head_bits
    note("kv_quantize mixed heads with outliers")
    for layout, lname in LAYOUTS:
        gc = gpu_cache(inp.k, bits, layout, spec.cap)
        oc = oracle_cache(inp.k, bits, lname, spec.cap)
        assert_cache_equal(gc, oc)


@pytest.mark.parametrize("layouts", [(T.LAYOUT_TOKEN, T.LAYOUT_CHANNEL),
                                     (T.LAYOUT_CHANNEL, T.LAYOUT_CHANNEL),
                                     (T.LAYOUT_TOKEN, T.LAYOUT_TOKEN)])
def test_quantize_pair_equals_two_calls(layouts):
    """kv_quantize_pair (both caches in one launch) writes the bytes of two
    kv_quantize calls and of the oracle, over a range cut at odd positions,
    with different per-head bits for the two caches."""
    require_gpu()
    rng = np.random.default_rng(31 + layouts[0] * 2 + layouts[1])
    B, H, D, cap = 2, 3, 128, 384
    names = {T.LAYOUT_TOKEN: "token", T.LAYOUT_CHANNEL: "channel"}
    kb, vb = (8, 4, 4), (4, 8, 4)
    xk = adversarial(rng, B, H, cap, D)
    xv = adversarial(rng, B, H, cap, D)
    note(f"kv_quantize_pair layouts={layouts}")
    pk, pv = T.KVCache(B, H, D, cap, kb, layouts[0]), T.KVCache(B, H, D, cap, vb, layouts[1])
    sk, sv = T.KVCache(B, H, D, cap, kb, layouts[0]), T.KVCache(B, H, D, cap, vb, layouts[1])
    tk, tv = torch.from_numpy(xk).cuda(), torch.from_numpy(xv).cuda()
    for s0, s1 in ((0, 33), (33, 97), (97, 384)):
        ak, av = tk[:, :, s0:s1].contiguous(), tv[:, :, s0:s1].contiguous()
        T.kv_quantize_pair(pk, pv, ak, av, s0)
        T.kv_quantize(sk, ak, s0)
        T.kv_quantize(sv, av, s0)
    torch.cuda.synchronize()
    for a, b in ((pk, sk), (pv, sv)):
        assert torch.equal(a.codes, b.codes)
        assert torch.equal(a.scales, b.scales)
        assert torch.equal(a.zeros, b.zeros)
    assert_cache_equal(pk, oracle_cache(xk, kb, names[layouts[0]], cap))
    assert_cache_equal(pv, oracle_cache(xv, vb, names[layouts[1]], cap))
