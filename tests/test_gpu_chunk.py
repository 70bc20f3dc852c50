"""GPU parity of quantise-on-append (taq_kv_append) and chunked prefill
(taq_attn_prefill_chunk) against the oracle: appended bytes equal the
oracle's quantiser written at the same per-batch positions (odd int4 starts,
positions past the capacity skipped); chunk outputs within max-abs 2e-3 of
the fp64 oracle for ragged lengths, padding rows, masks whose tiles the chunk
straddles and several GQA ratios; and a two-turn run (prefill, append,
chunk) equals the same rows of one prefill over the whole sequence."""
import numpy as np
import pytest
import torch

import tiled_attention_quantized_amd as T
import workloads as W
from oracle import attention as oa
from oracle import quant as oq
from tests.gpu_util import (TOL, require_gpu, note, gpu_cache, assert_cache_equal, max_abs,
                            lens_tensor)

pytestmark = pytest.mark.gpu


def _mask_tensor(mask):
    """[nq][nk] (shared) or [B][nq][nk] (per batch entry) keep-mask."""
    md = torch.from_numpy(np.ascontiguousarray(mask)).cuda()
    sb = mask.shape[-2] * mask.shape[-1] if mask.ndim == 3 else 0
    return T.TileMask(md, mask.shape[-2], mask.shape[-1], stride_b=sb)


@pytest.mark.parametrize("layout", ["token", "channel"])
def test_kv_append_bytes(layout):
    require_gpu()
    spec = W.small("prefill", B=4, Hq=2, Hkv=2, L=256, bits=4, n_int8_heads=1, seed=71)
    inp = W.make_inputs(spec)            # k: history over all 256 positions
    new = W.make_inputs(W.small("prefill", B=4, Hq=2, Hkv=2, L=50, bits=4, seed=72)).k[:, :, :50]
    bits = inp.structure.head_bits
    starts = np.array([0, 37, 131, 230], dtype=np.int32)   # 230 + 50 runs past 256
    lay = T.LAYOUT_TOKEN if layout == "token" else T.LAYOUT_CHANNEL
    note(f"kv_append layout={layout} bits={bits.tolist()} starts={starts.tolist()}")
    gc = gpu_cache(inp.k, bits, lay, spec.cap)
    T.kv_append(gc, torch.from_numpy(np.ascontiguousarray(new)).cuda(), lens_tensor(starts))
    oc = oq.build_cache(inp.k, bits, layout, cap=spec.cap)
    S = new.shape[2]
    for b in range(spec.B):
        n_ok = min(S, spec.cap - int(starts[b]))
        for h in range(spec.Hkv):
            codes, s, z = oq.quantize(new[b, h, :n_ok], int(bits[h]))
            oc.write(b, h, int(starts[b]), codes, s, z)
    assert_cache_equal(gc, oc)


def _chunk_case(r, Lq, lens, cap, mask=None, seed=0, bits=8, n_int8=0, workspace="auto",
                also_unsplit=False):
    Hkv = 2 if r < 8 else 1
    Hq = Hkv * r
    B = len(lens)
    kv = W.make_inputs(W.small("prefill", B=B, Hq=Hq, Hkv=Hkv, L=cap, bits=bits,
                               n_int8_heads=n_int8, seed=seed))
    q = W.make_inputs(W.small("prefill", B=B, Hq=Hq, Hkv=Hkv, L=Lq, bits=bits,
                              seed=seed + 1000)).q
    hb = kv.structure.head_bits
    kc = gpu_cache(kv.k, hb, T.LAYOUT_TOKEN, cap)
    vc = gpu_cache(kv.v, hb, T.LAYOUT_CHANNEL, cap)
    tm = _mask_tensor(mask) if mask is not None else None
    out = T.attn_prefill_chunk(kc, vc, torch.from_numpy(q).cuda(), lens_tensor(lens), cap,
                               mask=tm, workspace=workspace)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    if also_unsplit:
        one = T.attn_prefill_chunk(kc, vc, torch.from_numpy(q).cuda(), lens_tensor(lens), cap,
                                   mask=tm, workspace=None)
        torch.cuda.synchronize()
        got = (got, one.cpu().numpy().astype(np.float64))
    okc = oq.build_cache(kv.k, hb, "token", cap=cap)
    ovc = oq.build_cache(kv.v, hb, "channel", cap=cap)
    want = oa.prefill_chunk(q, oq.dequantized_all(okc), oq.dequantized_all(ovc), lens,
                            mask=mask, workers=4)
    return got, want


@pytest.mark.parametrize("r", [1, 4, 8])
@pytest.mark.parametrize("Lq", [1, 40, 130])
def test_chunk_small(r, Lq):
    require_gpu()
    lens = np.array([384, 300, 25, 129], dtype=np.int32)   # 25 < Lq: padding rows
    note(f"chunk r={r} Lq={Lq} lens={lens.tolist()}")
    got, want = _chunk_case(r, Lq, lens, 384, seed=10 * r + Lq)
    err = max_abs(got, want)
    assert err <= TOL, err
    n_pad = max(0, Lq - 25)
    assert not got[2, :, :n_pad].any()


@pytest.mark.parametrize("r", [2, 4])
def test_chunk_with_mask_straddling_tiles(r):
    require_gpu()
    # chunk positions 260..299 and 90..129 cross query-tile boundaries at
    # offsets that are not multiples of 32
    lens = np.array([300, 130, 384], dtype=np.int32)
    mask = np.tril(np.ones((3, 3), np.uint8))
    mask[2, 1] = 0
    mask[1, 0] = 0
    note(f"chunk masked r={r} lens={lens.tolist()}")
    got, want = _chunk_case(r, 40, lens, 384, mask=mask, seed=300 + r, bits=4, n_int8=1)
    err = max_abs(got, want)
    assert err <= TOL, err


def test_two_turns_equal_one_prefill():
    require_gpu()
    B, Hq, Hkv, cap, Lq = 3, 8, 2, 512, 96
    n1 = np.array([300, 17, 416], dtype=np.int32)      # first-turn lengths
    full = W.make_inputs(W.small("prefill", B=B, Hq=Hq, Hkv=Hkv, L=cap, bits=4,
                                 n_int8_heads=1, seed=501))
    hb = full.structure.head_bits
    note(f"two turns n1={n1.tolist()} Lq={Lq}")
    # turn 1: the first n1[b] tokens of each sequence (the rest of the cache
    # is written by turn 2 or stays unused)
    kc = gpu_cache(full.k, hb, T.LAYOUT_TOKEN, cap)
    vc = gpu_cache(full.v, hb, T.LAYOUT_CHANNEL, cap)
    # turn 2: append Lq new tokens at n1[b] (new values, not the ones above)
    newk = W.make_inputs(W.small("prefill", B=B, Hq=Hq, Hkv=Hkv, L=Lq, bits=4, seed=502)).k[:, :, :Lq]
    newv = W.make_inputs(W.small("prefill", B=B, Hq=Hq, Hkv=Hkv, L=Lq, bits=4, seed=503)).k[:, :, :Lq]
    T.kv_append(kc, torch.from_numpy(np.ascontiguousarray(newk)).cuda(), lens_tensor(n1))
    T.kv_append(vc, torch.from_numpy(np.ascontiguousarray(newv)).cuda(), lens_tensor(n1))
    n2 = n1 + Lq
    qfull = full.q                                     # [B][Hq][cap][D]
    qchunk = np.stack([qfull[b, :, n1[b]:n1[b] + Lq] for b in range(B)])
    out = T.attn_prefill_chunk(kc, vc, torch.from_numpy(np.ascontiguousarray(qchunk)).cuda(),
                               lens_tensor(n2), cap)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    # oracle: one prefill over the whole sequences (history + appended chunk)
    kall, vall = full.k.copy(), full.v.copy()
    for b in range(B):
        kall[b, :, n1[b]:n1[b] + Lq] = newk[b]
        vall[b, :, n1[b]:n1[b] + Lq] = newv[b]
    okc = oq.build_cache(kall, hb, "token", cap=cap)
    ovc = oq.build_cache(vall, hb, "channel", cap=cap)
    want_full = oa.prefill(qfull, oq.dequantized_all(okc), oq.dequantized_all(ovc), n2, workers=4)
    want = np.stack([want_full[b, :, n1[b]:n1[b] + Lq] for b in range(B)])
    err = max_abs(got, want)
    assert err <= TOL, err


def test_chunk_long_history_sampled_rows():
    require_gpu()
    # 8192 cached tokens of history + a 512-row chunk, GQA 32/8, int8
    B, Hq, Hkv, Lq = 1, 32, 8, 512
    cap = 8192 + 512
    lens = np.array([cap], dtype=np.int32)
    kv = W.make_inputs(W.small("prefill", B=B, Hq=Hq, Hkv=Hkv, L=cap, bits=8, seed=601))
    q = W.make_inputs(W.small("prefill", B=B, Hq=Hq, Hkv=Hkv, L=Lq, bits=8, seed=602)).q
    hb = kv.structure.head_bits
    note("chunk long history 8192 + 512")
    kc = gpu_cache(kv.k, hb, T.LAYOUT_TOKEN, cap)
    vc = gpu_cache(kv.v, hb, T.LAYOUT_CHANNEL, cap)
    out = T.attn_prefill_chunk(kc, vc, torch.from_numpy(q).cuda(), lens_tensor(lens), cap)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    rng = np.random.default_rng(603)
    rows = np.unique(np.concatenate([[0, 31, 32, 255, 511], rng.integers(0, Lq, 19)]))
    heads = [(0, int(h)) for h in rng.choice(Hq, 6, replace=False)]
    okc = oq.build_cache(kv.k, hb, "token", cap=cap)
    ovc = oq.build_cache(kv.v, hb, "channel", cap=cap)
    want = oa.prefill_chunk(q, oq.dequantized_all(okc), oq.dequantized_all(ovc), lens,
                            rows=rows, heads=heads, workers=8)
    err = max(max_abs(got[0, h][rows], want[0, h]) for _, h in heads)
    assert err <= TOL, err


@pytest.mark.parametrize("r", [1, 4, 8])
def test_chunk_key_range_split(r):
    """Short chunks over a long history split each query block's key range
    over several workgroups (partials merged in split order): ragged lengths,
    a sequence shorter than the chunk (padding rows, empty splits) and a mask,
    against the oracle and against the unsplit kernel."""
    require_gpu()
    cap, Lq = 2048, 100
    lens = np.array([2048, 1500, 60, 700], dtype=np.int32)
    Hkv = 2 if r < 8 else 1
    kd = T.KVCache(4, Hkv, 128, cap, [8] * Hkv, T.LAYOUT_TOKEN)
    assert T.prefill_chunk_workspace_bytes(kd, Hkv * r, Lq, cap) > 0     # the split is taken
    nt = cap // 128
    mask = np.tril(np.ones((4, nt, nt), np.uint8))
    mask[0, 15, 3:9] = 0
    mask[1, 11, 1:4] = 0
    note(f"chunk split r={r} lens={lens.tolist()}")
    (got, one), want = _chunk_case(r, Lq, lens, cap, mask=mask, seed=500 + r, also_unsplit=True)
    assert max_abs(got, want) <= TOL
    assert max_abs(got, one) <= TOL
    assert not got[2, :, :Lq - 60].any()          # rows at negative positions


@pytest.mark.parametrize("bits,n8", [(4, 0), (4, 1)])
def test_chunk_key_range_split_int4_and_mixed(bits, n8):
    """The split path over int4 and mixed int4/int8 heads (r = 2), with a
    one-row chunk and a chunk longer than one query block."""
    require_gpu()
    cap = 4096
    lens = np.array([4096, 3000, 77], dtype=np.int32)
    for Lq in (1, 300):
        note(f"chunk split bits={bits} n8={n8} Lq={Lq}")
        (got, one), want = _chunk_case(2, Lq, lens, cap, seed=520 + Lq + n8, bits=bits,
                                       n_int8=n8, also_unsplit=True)
        assert max_abs(got, want) <= TOL
        assert max_abs(got, one) <= TOL


def test_chunk_zero_length_entry():
    """An empty batch entry in a chunk over a long history, through the
    key-range split (its partials carry a zero normaliser into the merge) and
    without it: its rows are all zero, the live entries match the oracle."""
    require_gpu()
    cap, Lq = 2048, 100
    lens = np.array([2048, 0, 700], dtype=np.int32)
    kd = T.KVCache(3, 2, 128, cap, [8, 8], T.LAYOUT_TOKEN)
    assert T.prefill_chunk_workspace_bytes(kd, 8, Lq, cap) > 0     # the split is taken
    note(f"chunk zero-length entry lens={lens.tolist()}")
    (got, one), want = _chunk_case(4, Lq, lens, cap, seed=560, bits=4, n_int8=1,
                                   also_unsplit=True)
    assert max_abs(got, want) <= TOL
    assert max_abs(got, one) <= TOL
    assert not got[1].any() and not one[1].any()
