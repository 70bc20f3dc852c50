"""GPU parity of the literal two-pass decode softmax (taq_attn_decode_two_pass:
exact maximum first, then weights against it with no rescaling) against the
fp64 oracle (max-abs <= 2e-3), and against the online-softmax decode it
cross-checks: ragged lengths, GQA ratios, mixed bits, masks with an empty
batch entry, wide score ranges where the online path rescales, and the
full-size long-context workload on sampled heads."""
import numpy as np
import pytest
import torch

import tiled_attention_quantized_amd as T
import workloads as W
from oracle import attention as oa
from oracle import quant as oq
from tests.gpu_util import TOL, require_gpu, note, gpu_cache, max_abs, lens_tensor

pytestmark = pytest.mark.gpu


def _run(inp, mask=None, scale=0.0):
    spec, st = inp.spec, inp.structure
    bits = st.head_bits
    kc = gpu_cache(inp.k, bits, T.LAYOUT_TOKEN, spec.cap)
    vc = gpu_cache(inp.v, bits, T.LAYOUT_CHANNEL, spec.cap)
    q = torch.from_numpy(inp.q).cuda()
    lens = lens_tensor(st.seq_lens)
    tm = None
    if mask is not None:
        md = torch.from_numpy(np.ascontiguousarray(mask)).cuda()
        tm = T.TileMask(md, 1, mask.shape[-1], stride_b=mask.shape[-1])
    two = T.attn_decode(kc, vc, q, lens, spec.max_len, mask=tm, softmax_scale=scale,
                        two_pass=True)
    one = T.attn_decode(kc, vc, q, lens, spec.max_len, mask=tm, softmax_scale=scale)
    torch.cuda.synchronize()
    okc = oq.build_cache(inp.k, bits, "token", cap=spec.cap)
    ovc = oq.build_cache(inp.v, bits, "channel", cap=spec.cap)
    want = oa.decode(inp.q, oq.dequantized_all(okc), oq.dequantized_all(ovc), st.seq_lens,
                     mask=mask, scale=None if scale == 0.0 else scale, workers=4)
    return (two.cpu().numpy().astype(np.float64), one.cpu().numpy().astype(np.float64), want,
            (kc, vc, q, lens, tm))


@pytest.mark.parametrize("r", [1, 2, 4, 8])
@pytest.mark.parametrize("bits,n8", [(8, 0), (4, 1)])
def test_two_pass_small_ragged(r, bits, n8):
    require_gpu()
    spec = W.small("decode", B=5, Hq=2 * r, Hkv=2, ragged=(1, 900), bits=bits, n_int8_heads=n8,
                   seed=300 + r * 10 + bits)
    inp = W.make_inputs(spec)
    inp.structure.seq_lens[:4] = [1, 31, 129, 640]
    for b in range(4):
        n = inp.structure.seq_lens[b]
        inp.k[b, :, n:] = 0
        inp.v[b, :, n:] = 0
    note(f"two-pass r={r} bits={bits} n8={n8} lens={inp.structure.seq_lens.tolist()}")
    two, one, want, _ = _run(inp)
    assert max_abs(two, want) <= TOL
    assert max_abs(two, one) <= TOL


def test_two_pass_mask_and_empty_entry():
    require_gpu()
    spec = W.small("decode", B=3, Hq=8, Hkv=2, ragged=(300, 1000), bits=4, seed=31)
    inp = W.make_inputs(spec)
    nk = spec.cap // 128
    mask = (np.random.default_rng(2).random((spec.B, nk)) < 0.5).astype(np.uint8)
    mask[:, 0] = 1
    mask[1, :] = 0                      # batch entry 1 sees no key: zeros
    note("two-pass masked")
    two, one, want, _ = _run(inp, mask=mask)
    assert max_abs(two, want) <= TOL
    assert not two[1].any()


def test_two_pass_wide_score_range():
    # scores spread over hundreds of log2 units: the online path moves its
    # running maximum and rescales many times, the two-pass path never does
    require_gpu()
    spec = W.small("decode", B=2, Hq=8, Hkv=2, ragged=(2000, 4000), bits=8, seed=33,
                   outlier_frac=0.05, outlier_scale=8.0)
    inp = W.make_inputs(spec)
    # ramp the keys along the sequence so later tokens carry larger scores
    for b in range(spec.B):
        n = int(inp.structure.seq_lens[b])
        ramp = np.linspace(0.25, 4.0, n, dtype=np.float32)[:, None]
        inp.k[b, :, :n] = (inp.k[b, :, :n].astype(np.float32) * ramp).astype(np.float16)
    note("two-pass wide score range")
    two, one, want, _ = _run(inp, scale=0.5)
    assert max_abs(two, want) <= TOL
    assert max_abs(one, want) <= TOL


def test_two_pass_deterministic():
    require_gpu()
    spec = W.small("decode", B=4, Hq=16, Hkv=4, ragged=(100, 3000), bits=4, seed=35)
    inp = W.make_inputs(spec)
    note("two-pass determinism")
    two, _, _, (kc, vc, q, lens, _) = _run(inp)
    for _ in range(3):
        again = T.attn_decode(kc, vc, q, lens, spec.max_len, two_pass=True)
        torch.cuda.synchronize()
        assert np.array_equal(again.cpu().numpy().view(np.uint16),
                              two.astype(np.float16).view(np.uint16))


def test_two_pass_long_context_sampled():
    """The 128K mixed-precision workload in the benchmarked launch
    configuration: two-pass and online agree everywhere, and sampled heads
    match the oracle."""
    require_gpu()
    spec = W.WORKLOADS["decode_128k_mixed"]
    inp = W.make_inputs(spec)
    st = inp.structure
    bits = st.head_bits
    note("two-pass decode_128k_mixed")
    kc = gpu_cache(inp.k, bits, T.LAYOUT_TOKEN, spec.cap)
    vc = gpu_cache(inp.v, bits, T.LAYOUT_CHANNEL, spec.cap)
    q = torch.from_numpy(inp.q).cuda()
    lens = lens_tensor(st.seq_lens)
    two = T.attn_decode(kc, vc, q, lens, spec.max_len, two_pass=True)
    one = T.attn_decode(kc, vc, q, lens, spec.max_len)
    torch.cuda.synchronize()
    two = two.cpu().numpy().astype(np.float64)
    one = one.cpu().numpy().astype(np.float64)
    del kc, vc
    assert max_abs(two, one) <= TOL
    rng = np.random.default_rng(7)
    heads = sorted({(int(b), int(h)) for b, h in zip(rng.integers(0, spec.B, 6),
                                                     rng.integers(0, spec.Hq, 6))})
    for b, h in heads:
        g = h // spec.r
        n = int(st.seq_lens[b])
        kh = oq.dequantize(*oq.quantize(inp.k[b, g, :n], int(bits[g])))
        vh = oq.dequantize(*oq.quantize(inp.v[b, g, :n], int(bits[g])))
        want = oa.decode(inp.q[b:b + 1, h:h + 1], kh[None, None], vh[None, None], [n])[0, 0]
        assert max_abs(two[b, h], want) <= TOL, (b, h)


@pytest.mark.parametrize("r", [1, 8])
def test_two_pass_multistep_waves_with_mask(r):
    """1024-token split chunks (8 steps per wave) through both passes: ragged
    odd lengths, tiles dropped inside a wave's range, int8 and int4 heads."""
    require_gpu()
    spec = W.small("decode", B=16, Hq=8 * r, Hkv=8, ragged=(9001, 16383), bits=4,
                   n_int8_heads=2, seed=700 + r, capacity=16384)
    inp = W.make_inputs(spec)
    nk = spec.cap // 128
    rng = np.random.default_rng(11)
    mask = (rng.random((spec.B, nk)) < 0.7).astype(np.uint8)
    mask[:, 0] = 1
    note(f"two-pass multi-step r={r}")
    two, one, want, _ = _run(inp, mask=mask)
    assert max_abs(two, want) <= TOL
    assert max_abs(one, want) <= TOL
    assert max_abs(two, one) <= TOL
