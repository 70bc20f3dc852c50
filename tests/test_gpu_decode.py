"""GPU parity of attn_decode against the fp64 oracle (max-abs <= 2e-3), plus
edge cases and run-to-run determinism (every output of the full-size
workloads: test_gpu_full_size.py)."""
import numpy as np
import pytest
import torch

import tiled_attention_quantized_amd as T
import workloads as W
from oracle import attention as oa
from oracle import quant as oq
from tests.gpu_util import (TOL, require_gpu, note, gpu_cache, max_abs, lens_tensor)

pytestmark = pytest.mark.gpu


def run_decode(inp, mask=None, heads=None, workers=4, scale=None):
    spec, st = inp.spec, inp.structure
    bits = st.head_bits
    kc = gpu_cache(inp.k, bits, T.LAYOUT_TOKEN, spec.cap)
    vc = gpu_cache(inp.v, bits, T.LAYOUT_CHANNEL, spec.cap)
    q = torch.from_numpy(inp.q).cuda()
    lens = lens_tensor(st.seq_lens)
    tm = None
    if mask is not None:
        md = torch.from_numpy(np.ascontiguousarray(mask)).cuda()
        tm = T.TileMask(md, 1, mask.shape[-1], stride_b=mask.shape[-1] if mask.ndim == 2 else 0)
    out = T.attn_decode(kc, vc, q, lens, spec.max_len, mask=tm,
                        softmax_scale=0.0 if scale is None else scale)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    # oracle: quantise with the oracle's own quantiser, then exact attention
    okc = oq.build_cache(inp.k, bits, "token", cap=spec.cap)
    ovc = oq.build_cache(inp.v, bits, "channel", cap=spec.cap)
    want = oa.decode(inp.q, oq.dequantized_all(okc), oq.dequantized_all(ovc), st.seq_lens,
                     mask=mask, heads=heads, workers=workers, scale=scale)
    return got, want, (kc, vc, q, lens, tm)


@pytest.mark.parametrize("r", [1, 2, 4, 8])
@pytest.mark.parametrize("bits,n8", [(8, 0), (4, 0), (4, 1)])
def test_decode_small_ragged(r, bits, n8):
    require_gpu()
    Hkv = 2
    spec = W.small("decode", B=5, Hq=Hkv * r, Hkv=Hkv, ragged=(1, 700), bits=bits,
                   n_int8_heads=n8, seed=r * 10 + bits + n8)
    inp = W.make_inputs(spec)
    # force edge lengths into the batch
    inp.structure.seq_lens[:4] = [1, 31, 33, 128]
    for b in range(4):
        n = inp.structure.seq_lens[b]
        inp.k[b, :, n:] = 0
        inp.v[b, :, n:] = 0
    note(f"decode small r={r} bits={bits} n8={n8} lens={inp.structure.seq_lens.tolist()}")
    got, want, _ = run_decode(inp)
    err = max_abs(got, want)
    assert err <= TOL, err


@pytest.mark.parametrize("scale", [0.02, 0.25])
def test_decode_softmax_scale(scale):
    """A softmax scale other than 1/sqrt(d), int4 and int8 heads, ragged
    lengths, against the oracle at the same scale."""
    require_gpu()
    spec = W.small("decode", B=4, Hq=8, Hkv=2, ragged=(1, 900), bits=4, n_int8_heads=1, seed=43)
    inp = W.make_inputs(spec)
    note(f"decode softmax_scale={scale} lens={inp.structure.seq_lens.tolist()}")
    got, want, _ = run_decode(inp, scale=scale)
    err = max_abs(got, want)
    assert err <= TOL, err


@pytest.mark.parametrize("bits", [8, 4])
def test_decode_with_tile_mask(bits):
    require_gpu()
    spec = W.small("decode", B=3, Hq=8, Hkv=2, ragged=(300, 1000), bits=bits, seed=5)
    inp = W.make_inputs(spec)
    nk = spec.cap // 128
    rng = np.random.default_rng(1)
    mask = (rng.random((spec.B, nk)) < 0.6).astype(np.uint8)
    mask[:, 0] = 1
    mask[2, :] = 0          # batch entry 2 sees no key at all -> zeros
    note(f"decode masked bits={bits}")
    got, want, _ = run_decode(inp, mask=mask)
    assert max_abs(got, want) <= TOL
    assert not got[2].any()


@pytest.mark.parametrize("r", [1, 2, 4, 8])
def test_decode_multistep_waves_with_mask(r):
    """Shapes whose split uses 1024-token chunks (8 steps of 32 tokens per
    wave), so the step pipeline runs with its buffers in rotation: ragged odd
    lengths (a partial last step), a KV-tile mask that drops tiles inside a
    wave's range (steps skipped mid-range), int8 and int4 heads, every GQA
    ratio (r = 8 carries two row blocks of query heads per lane)."""
    require_gpu()
    spec = W.small("decode", B=16, Hq=8 * r, Hkv=8, ragged=(9001, 16383), bits=4,
                   n_int8_heads=2, seed=77 + r, capacity=16384)
    inp = W.make_inputs(spec)
    kc = T.KVCache(spec.B, spec.Hkv, spec.D, spec.cap, inp.structure.head_bits, T.LAYOUT_TOKEN)
    ws_bytes = T.decode_workspace_bytes(kc, spec.Hq, spec.max_len)
    del kc
    nchunk = ws_bytes // (spec.B * spec.Hq * (128 + 2) * 4)
    chunk = -(-spec.max_len // nchunk)
    assert chunk >= 1024, chunk          # several steps per wave
    nk = spec.cap // 128
    rng = np.random.default_rng(7)
    mask = (rng.random((spec.B, nk)) < 0.7).astype(np.uint8)
    mask[:, 0] = 1
    note(f"decode multi-step waves r={r}, chunk {chunk}, lens {inp.structure.seq_lens.tolist()}")
    got, want, _ = run_decode(inp, mask=mask, workers=8)
    err = max_abs(got, want)
    assert err <= TOL, err


def _decode_chunk(kc, hq, max_len, B):
    ws = T.decode_workspace_bytes(kc, hq, max_len)
    nchunk = ws // (B * hq * (128 + 2) * 4)
    return -(-max_len // nchunk)


def test_decode_split_count_and_key_permutation_invariance():
    """The same inputs decoded under two split geometries (a larger
    max_seq_len selects longer chunks), and with the tokens of every sequence
    permuted before quantisation (codes are per token, so the exact result is
    unchanged): each agrees with the oracle and with the others within the
    bar."""
    require_gpu()
    spec = W.small("decode", B=16, Hq=32, Hkv=8, ragged=(1500, 4000), bits=4,
                   n_int8_heads=3, seed=91, capacity=16384)
    inp = W.make_inputs(spec)
    st = inp.structure
    bits = st.head_bits
    kc = gpu_cache(inp.k, bits, T.LAYOUT_TOKEN, spec.cap)
    vc = gpu_cache(inp.v, bits, T.LAYOUT_CHANNEL, spec.cap)
    q = torch.from_numpy(inp.q).cuda()
    lens = lens_tensor(st.seq_lens)
    short, long_ = 4096, spec.cap
    c_short = _decode_chunk(kc, spec.Hq, short, spec.B)
    c_long = _decode_chunk(kc, spec.Hq, long_, spec.B)
    assert c_short != c_long, (c_short, c_long)
    note(f"decode split invariance: chunks {c_short} and {c_long}")
    a = T.attn_decode(kc, vc, q, lens, short).cpu().numpy().astype(np.float64)
    b = T.attn_decode(kc, vc, q, lens, long_).cpu().numpy().astype(np.float64)
    # permuted tokens within each sequence
    rng = np.random.default_rng(3)
    kp, vp = inp.k.copy(), inp.v.copy()
    for bb in range(spec.B):
        n = int(st.seq_lens[bb])
        perm = rng.permutation(n)
        kp[bb, :, :n] = inp.k[bb][:, perm]
        vp[bb, :, :n] = inp.v[bb][:, perm]
    del kc, vc
    kcp = gpu_cache(kp, bits, T.LAYOUT_TOKEN, spec.cap)
    vcp = gpu_cache(vp, bits, T.LAYOUT_CHANNEL, spec.cap)
    c = T.attn_decode(kcp, vcp, q, lens, short).cpu().numpy().astype(np.float64)
    okc = oq.build_cache(inp.k, bits, "token", cap=spec.cap)
    ovc = oq.build_cache(inp.v, bits, "channel", cap=spec.cap)
    want = oa.decode(inp.q, oq.dequantized_all(okc), oq.dequantized_all(ovc), st.seq_lens,
                     workers=8)
    for got in (a, b, c):
        assert max_abs(got, want) <= TOL
    assert max_abs(a, b) <= TOL
    assert max_abs(a, c) <= TOL


def test_decode_zero_length_and_uniform_v():
    require_gpu()
    spec = W.small("decode", B=3, Hq=4, Hkv=1, ragged=(1, 400), bits=8, seed=9)
    inp = W.make_inputs(spec)
    inp.structure.seq_lens[1] = 0
    inp.k[1] = 0
    inp.v[1] = 0
    # uniform V for batch 0: every key carries the same value row
    n0 = inp.structure.seq_lens[0]
    inp.v[0, :, :n0] = inp.v[0, :, :1]
    note("decode zero length + uniform V")
    got, want, _ = run_decode(inp)
    assert max_abs(got, want) <= TOL
    assert not got[1].any()
    vhat = oq.dequantize(*oq.quantize(inp.v[0, 0, :1], 8)).astype(np.float16).astype(np.float64)
    # output equals that value up to one fp16 ulp
    ulp = np.abs(np.spacing(vhat.astype(np.float16))).astype(np.float64)
    assert np.all(np.abs(got[0] - vhat) <= ulp + 1e-12)


def test_decode_deterministic():
    require_gpu()
    spec = W.small("decode", B=4, Hq=16, Hkv=4, ragged=(100, 3000), bits=4, seed=3)
    inp = W.make_inputs(spec)
    note("decode determinism")
    got, want, (kc, vc, q, lens, _) = run_decode(inp)
    for _ in range(3):
        again = T.attn_decode(kc, vc, q, lens, spec.max_len)
        torch.cuda.synchronize()
        assert np.array_equal(again.cpu().numpy().view(np.uint16),
                              got.astype(np.float16).view(np.uint16))


@pytest.mark.parametrize("bits,n8", [(4, 0), (4, 1), (8, 0)])
@pytest.mark.parametrize("kind", ["x12", "one_channel_20000"])
def test_decode_large_query_magnitudes(bits, n8, kind):
    """Queries far from unit scale: every channel x12 (group sums of the odd
    int4 pairs reach ~1e5, beyond fp16), or one channel at 20000 (near the
    fp16 range).  The scores take the zero-points off through per-row query
    sums, which must stay exact and finite for any fp16 query; outputs match
    the oracle within the bar."""
    require_gpu()
    spec = W.small("decode", B=2, Hq=8, Hkv=2, ragged=(300, 700), bits=bits,
                   n_int8_heads=n8, seed=47)
    inp = W.make_inputs(spec)
    q = inp.q.astype(np.float32)
    if kind == "x12":
        q *= 12
    else:
        q[:, :, 5] = 20000.0
    inp.q = q.astype(np.float16)
    assert np.isfinite(inp.q).all()
    note(f"decode large q {kind} bits={bits} n8={n8}")
    got, want, _ = run_decode(inp)
    assert np.isfinite(got).all()
    assert max_abs(got, want) <= TOL


def test_decode_error_scales_with_v_magnitude():
    """The 2e-3 bar is for unit-variance data.  V-hat enters the PV product as
    fp16, so its rounding error is relative: a V channel scaled by 2^4 keeps
    the same relative error, i.e. at most 16x the bar in absolute terms, while
    the other channels keep the bar."""
    require_gpu()
    spec = W.small("decode", B=2, Hq=8, Hkv=2, ragged=(600, 1000), bits=8, seed=41)
    inp = W.make_inputs(spec)
    inp.v[:, :, :, 40] = (inp.v[:, :, :, 40].astype(np.float32) * 16).astype(np.float16)
    note("decode with a V channel x16")
    got, want, _ = run_decode(inp)
    err = np.abs(got - want)
    assert err[:, :, 40].max() <= 16 * TOL
    others = np.delete(err, 40, axis=2)
    assert others.max() <= TOL
