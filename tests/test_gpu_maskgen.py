"""GPU parity of the training-free tile-mask generator (taq_tile_mask_generate,
and taq_tile_mask_generate_chunk for one turn of a multi-turn prefill)
against the oracle's generator: the masks are compared byte for byte (the
decision is taken in the same fp64 arithmetic on both sides), over ragged and
empty sequences, mixed int4/int8 heads, several GQA ratios, every skip level
from dense to first-plus-diagonal, and the largest supported length (2048
tiles, the longest sort); then a generated mask drives the prefill kernel and
the output is checked against the oracle's attention under the oracle's mask."""
import numpy as np
import pytest
import torch

import tiled_attention_quantized_amd as T
import workloads as W
from oracle import attention as oa
from oracle import maskgen as omg
from oracle import quant as oq
from tests.gpu_util import TOL, require_gpu, note, gpu_cache, max_abs, lens_tensor

pytestmark = pytest.mark.gpu


def _case(B, Hq, Hkv, L, lens, bits=4, n_int8=1, seed=0, cap=0):
    spec = W.small("prefill", B=B, Hq=Hq, Hkv=Hkv, L=L, bits=bits, n_int8_heads=n_int8,
                   seed=seed, capacity=cap)
    inp = W.make_inputs(spec)
    hb = inp.structure.head_bits
    kc = gpu_cache(inp.k, hb, T.LAYOUT_TOKEN, spec.cap)
    k_hat = oq.dequantized_all(oq.build_cache(inp.k, hb, "token", cap=spec.cap))
    return spec, inp, kc, k_hat, np.asarray(lens, dtype=np.int32)


def _gpu_mask(kc, q, lens, spm):
    tm = T.tile_mask_generate(kc, torch.from_numpy(q).cuda(), lens_tensor(lens), spm)
    torch.cuda.synchronize()
    return tm, tm.data.cpu().numpy()


def _assert_mask_equal(got, want):
    assert got.shape == want.shape
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{len(bad)} tiles differ, first at {bad[:4].tolist()}"


@pytest.mark.parametrize("r", [1, 4, 8])
@pytest.mark.parametrize("spm", [0, 250, 600, 1000])
def test_mask_equals_oracle_small(r, spm):
    require_gpu()
    Hkv = 2 if r < 8 else 1
    lens = [1000, 333, 0, 129][: 4 if r < 8 else 3]
    spec, inp, kc, k_hat, lens = _case(len(lens), Hkv * r, Hkv, 1000, lens,
                                       n_int8=1 if Hkv == 2 else 0, seed=r * 7 + spm)
    note(f"maskgen r={r} spm={spm} lens={lens.tolist()}")
    _, got = _gpu_mask(kc, inp.q, lens, spm)
    want = omg.generate(inp.q, k_hat, lens, spm)
    _assert_mask_equal(got, want)


def test_mask_equals_oracle_8k_heads():
    require_gpu()
    # the 8K prefill shape (Hq 32, Hkv 8) with two ragged sequences
    lens = [8192, 5000]
    spec, inp, kc, k_hat, lens = _case(2, 32, 8, 8192, lens, bits=8, n_int8=0, seed=91)
    note(f"maskgen 8k lens={lens.tolist()}")
    _, got = _gpu_mask(kc, inp.q, lens, 250)
    _assert_mask_equal(got, omg.generate(inp.q, k_hat, lens, 250))


def test_mask_equals_oracle_longest_supported():
    require_gpu()
    # 262144 positions = 2048 tiles per side: the largest sort (2047 candidates)
    L = 262144
    lens = [L - 77]
    spec, inp, kc, k_hat, lens = _case(1, 2, 1, L, lens, bits=4, n_int8=0, seed=93)
    note("maskgen 2048 tiles")
    _, got = _gpu_mask(kc, inp.q, lens, 500)
    want = omg.generate(inp.q, k_hat, lens, 500)
    _assert_mask_equal(got, want)
    # structure: per-row kept counts follow the cap exactly
    nt = 2048
    kept = got[0, 0].sum(axis=1).astype(np.int64)
    i = np.arange(nt)
    expect = np.where(i == 0, 1, 2 + np.maximum(i - 1, 0) - (np.maximum(i - 1, 0) * 500) // 1000)
    assert np.array_equal(kept, expect)


@pytest.mark.parametrize("r", [2, 4])
def test_generated_mask_drives_prefill(r):
    require_gpu()
    Hkv = 2
    L = 1000
    lens = [1000, 700]
    spec, inp, kc, k_hat, lens = _case(2, Hkv * r, Hkv, L, lens, seed=101 + r)
    hb = inp.structure.head_bits
    vc = gpu_cache(inp.v, hb, T.LAYOUT_CHANNEL, spec.cap)
    note(f"maskgen->prefill r={r}")
    q = torch.from_numpy(inp.q).cuda()
    lt = lens_tensor(lens)
    tm = T.tile_mask_generate(kc, q, lt, 500)
    out = T.attn_prefill(kc, vc, q, lt, mask=tm)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    mask = omg.generate(inp.q, k_hat, lens, 500)
    assert np.array_equal(tm.data.cpu().numpy(), mask)
    v_hat = oq.dequantized_all(oq.build_cache(inp.v, hb, "channel", cap=spec.cap))
    want = oa.prefill(inp.q, k_hat, v_hat, lens, mask=mask, workers=4)
    err = max_abs(got, want)
    assert err <= TOL, err
    # and the mask did drop tiles that matter: dense attention differs
    dense = oa.prefill(inp.q, k_hat, v_hat, lens, mask=None, rows=np.arange(896, 1000),
                       heads=[(0, 0)])
    assert max_abs(dense[0, 0], want[0, 0, 896:1000]) > 1e-2


# ---- per-turn masks (taq_tile_mask_generate_chunk) ---------------------------

@pytest.mark.parametrize("r,Lq,spm", [(1, 1, 500), (4, 100, 250), (4, 300, 600), (8, 1000, 250),
                                      (2, 1000, 1000), (4, 0, 250)])
def test_chunk_mask_equals_oracle(r, Lq, spm):
    """Mask rows of one turn (the last Lq positions of ragged, empty and
    short sequences; turns longer than a sequence carry padding rows) equal
    the oracle's byte for byte."""
    require_gpu()
    Hkv = 2 if r < 8 else 1
    lens = [1000, 333, 0, 129][: 4 if r < 8 else 3]
    spec, inp, kc, k_hat, lens = _case(len(lens), Hkv * r, Hkv, 1000, lens,
                                       n_int8=1 if Hkv == 2 else 0, seed=r * 11 + Lq)
    qc = np.ascontiguousarray(inp.q[:, :, :Lq])      # the turn's queries (any fp16 data)
    note(f"maskgen turn r={r} Lq={Lq} spm={spm} lens={lens.tolist()}")
    tm = T.tile_mask_generate_chunk(kc, torch.from_numpy(qc).cuda(), lens_tensor(lens), 1000, spm)
    torch.cuda.synchronize()
    got = tm.data.cpu().numpy()
    want = omg.generate_chunk(qc, k_hat, lens, spm, 1000)
    _assert_mask_equal(got, want)


@pytest.mark.parametrize("r,Lq", [(4, 300), (2, 700)])
def test_chunk_mask_drives_chunked_prefill(r, Lq):
    """A turn's generated mask drives taq_attn_prefill_chunk (key range split
    over workgroups) within the bar of the oracle's chunked prefill under the
    oracle's mask, and the mask drops tiles that change the result."""
    require_gpu()
    Hkv = 2
    L = 1200
    lens = [1200, 900]
    spec, inp, kc, k_hat, lens = _case(2, Hkv * r, Hkv, L, lens, seed=201 + r)
    hb = inp.structure.head_bits
    vc = gpu_cache(inp.v, hb, T.LAYOUT_CHANNEL, spec.cap)
    # the turn: the last Lq positions' queries of each sequence
    qc = np.zeros((2, Hkv * r, Lq, 128), dtype=np.float16)
    for b, n in enumerate(lens):
        lo = n - Lq
        qc[b, :, max(0, -lo):] = inp.q[b, :, max(lo, 0):n]
    note(f"maskgen turn -> chunked prefill r={r} Lq={Lq}")
    q = torch.from_numpy(qc).cuda()
    lt = lens_tensor(lens)
    tm = T.tile_mask_generate_chunk(kc, q, lt, L, 600)
    out = T.attn_prefill_chunk(kc, vc, q, lt, L, mask=tm)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    mask = omg.generate_chunk(qc, k_hat, lens, 600, L)
    assert np.array_equal(tm.data.cpu().numpy(), mask)
    v_hat = oq.dequantized_all(oq.build_cache(inp.v, hb, "channel", cap=spec.cap))
    want = oa.prefill_chunk(qc, k_hat, v_hat, lens, mask=mask, workers=4)
    err = max_abs(got, want)
    assert err <= TOL, err
    dense = oa.prefill_chunk(qc, k_hat, v_hat, lens, mask=None, workers=4)
    assert max_abs(dense, want) > 1e-2
