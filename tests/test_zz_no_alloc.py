"""The allocation-free decode entry point (taq_attn_decode_noalloc) against
taq_attn_decode with a caller workspace: two calls in a row on the library's
fixed device scratch, the second with smaller shapes, each bitwise equal to
the workspace call with the same arguments and within 2e-3 of the fp64
oracle."""
import numpy as np
import pytest
import torch

import tiled_attention_quantized_amd as T
import workloads as W
from oracle import attention as oa
from oracle import quant as oq
from tests.gpu_util import TOL, require_gpu, note, gpu_cache, lens_tensor, max_abs

pytestmark = pytest.mark.gpu


def _case(spec):
    inp = W.make_inputs(spec)
    st = inp.structure
    kc = gpu_cache(inp.k, st.head_bits, T.LAYOUT_TOKEN, spec.cap)
    vc = gpu_cache(inp.v, st.head_bits, T.LAYOUT_CHANNEL, spec.cap)
    q = torch.from_numpy(inp.q).cuda()
    lens = lens_tensor(st.seq_lens)
    okc = oq.build_cache(inp.k, st.head_bits, "token", cap=spec.cap)
    ovc = oq.build_cache(inp.v, st.head_bits, "channel", cap=spec.cap)
    want = oa.decode(inp.q, oq.dequantized_all(okc), oq.dequantized_all(ovc), st.seq_lens)
    return inp, kc, vc, q, lens, want


def test_noalloc_decode_equals_workspace_decode_twice():
    require_gpu()
    big = W.small("decode", B=3, Hq=16, Hkv=4, ragged=(900, 5000), bits=4, n_int8_heads=1,
                  seed=71)
    small = W.small("decode", B=1, Hq=8, Hkv=2, ragged=(100, 700), bits=8, seed=72)
    for spec in (big, small):
        inp, kc, vc, q, lens, want = _case(spec)
        note(f"noalloc decode B={spec.B} Hq={spec.Hq} Hkv={spec.Hkv} lens={inp.structure.seq_lens.tolist()}")
        out_na = torch.empty_like(q)
        T.attn_decode_noalloc(kc, vc, q, lens, spec.max_len, out=out_na)
        out_ws = T.attn_decode(kc, vc, q, lens, spec.max_len)
        torch.cuda.synchronize()
        a = out_na.cpu().numpy()
        b = out_ws.cpu().numpy()
        assert np.array_equal(a.view(np.uint16), b.view(np.uint16))
        assert max_abs(a.astype(np.float64), want) <= TOL
