"""GPU parity of attn_prefill against the fp64 oracle (max-abs <= 2e-3): small
shapes checked everywhere (ragged lengths, several tiles and a ragged tail,
masks, GQA ratios, mixed bits), invariants and determinism (the full-size
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


def gpu_run(inp, mask=None, lens=None, scale=0.0):
    spec, st = inp.spec, inp.structure
    bits = st.head_bits
    kc = gpu_cache(inp.k, bits, T.LAYOUT_TOKEN, spec.cap)
    vc = gpu_cache(inp.v, bits, T.LAYOUT_CHANNEL, spec.cap)
    q = torch.from_numpy(inp.q).cuda()
    lt = lens_tensor(st.seq_lens if lens is None else lens)
    tm = None
    if mask is not None:
        md = torch.from_numpy(np.ascontiguousarray(mask)).cuda()
        tm = T.TileMask(md, mask.shape[-2], mask.shape[-1],
                        stride_b=mask.shape[-2] * mask.shape[-1] if mask.ndim == 3 else 0)
    out = T.attn_prefill(kc, vc, q, lt, mask=tm, softmax_scale=scale)
    torch.cuda.synchronize()
    return out, (kc, vc, q, lt, tm)


def gpu_run_np(inp, mask=None, lens=None, scale=0.0):
    out, ctx = gpu_run(inp, mask=mask, lens=lens, scale=scale)
    return out.cpu().numpy().astype(np.float64), ctx


def oracle_run(inp, mask=None, lens=None, rows=None, heads=None, workers=4, scale=None):
    spec, st = inp.spec, inp.structure
    bits = st.head_bits
    okc = oq.build_cache(inp.k, bits, "token", cap=spec.cap)
    ovc = oq.build_cache(inp.v, bits, "channel", cap=spec.cap)
    return oa.prefill(inp.q, oq.dequantized_all(okc), oq.dequantized_all(ovc),
                      st.seq_lens if lens is None else lens, mask=mask, rows=rows,
                      heads=heads, workers=workers, scale=scale)


@pytest.mark.parametrize("r", [1, 2, 4, 8])
@pytest.mark.parametrize("L", [1, 77, 200, 513])
def test_prefill_small_dense(r, L):
    require_gpu()
    Hkv = 2 if r < 8 else 1
    spec = W.small("prefill", B=2, Hq=Hkv * r, Hkv=Hkv, L=L, bits=8, seed=r + L)
    inp = W.make_inputs(spec)
    lens = np.array([L, max(1, L // 2 + 3) if L > 1 else 1], dtype=np.int32)
    note(f"prefill dense r={r} L={L} lens={lens.tolist()}")
    got, _ = gpu_run_np(inp, lens=lens)
    want = oracle_run(inp, lens=lens)
    err = max_abs(got, want)
    assert err <= TOL, err
    # rows at or beyond the sequence length are zero
    assert not got[1, :, lens[1]:].any()


@pytest.mark.parametrize("scale", [0.02, 0.25])
def test_prefill_softmax_scale(scale):
    """A softmax scale other than 1/sqrt(d), int4 and int8 heads, against the
    oracle at the same scale.  The K-hat tiles are staged in fp16, so the
    score error is proportional to the scores: at or below 1/sqrt(d) the bar
    holds, above it (0.25 makes the scores ~2.8x the default's) the error
    may grow in proportion (measured 2.9e-3 at 0.25)."""
    require_gpu()
    spec = W.small("prefill", B=2, Hq=8, Hkv=2, L=300, bits=4, n_int8_heads=1, seed=41)
    inp = W.make_inputs(spec)
    lens = np.array([300, 170], dtype=np.int32)
    note(f"prefill softmax_scale={scale} lens={lens.tolist()}")
    got, _ = gpu_run_np(inp, lens=lens, scale=scale)
    want = oracle_run(inp, lens=lens, scale=scale)
    err = max_abs(got, want)
    growth = max(1.0, scale * np.sqrt(spec.D))
    note(f"max-abs {err:.3e} (bar {TOL * growth:.2e})")
    assert err <= TOL * growth, err


@pytest.mark.parametrize("r", [1, 4])
def test_prefill_zero_length_entry(r):
    """An empty batch entry between two live ones (mixed int4/int8 heads): no
    key is visible to any of its rows, so they are all zero; the live entries
    match the oracle."""
    require_gpu()
    Hkv = 2
    spec = W.small("prefill", B=3, Hq=Hkv * r, Hkv=Hkv, L=200, bits=4, n_int8_heads=1,
                   seed=90 + r)
    inp = W.make_inputs(spec)
    lens = np.array([200, 0, 77], dtype=np.int32)
    note(f"prefill zero-length entry r={r} lens={lens.tolist()}")
    got, _ = gpu_run_np(inp, lens=lens)
    want = oracle_run(inp, lens=lens)
    assert max_abs(got, want) <= TOL
    assert not got[1].any()
    assert not got[2, :, 77:].any()


@pytest.mark.parametrize("bits,n8", [(4, 0), (4, 1), (8, 1)])
def test_prefill_bits(bits, n8):
    require_gpu()
    spec = W.small("prefill", B=1, Hq=8, Hkv=2, L=384, bits=bits, n_int8_heads=n8, seed=3)
    inp = W.make_inputs(spec)
    note(f"prefill bits={bits} n8={n8}")
    got, _ = gpu_run_np(inp)
    want = oracle_run(inp)
    assert max_abs(got, want) <= TOL


@pytest.mark.parametrize("r", [4, 1])
def test_prefill_masked(r):
    require_gpu()
    L = 640
    spec = W.small("prefill", B=2, Hq=2 * r, Hkv=2, L=L, bits=8, seed=11)
    inp = W.make_inputs(spec)
    rng = np.random.default_rng(4)
    nt = 5
    mask = np.stack([W.skip_mask(L, 0.4, rng) for _ in range(2)])
    mask[1, 3, 3] = 0      # a dropped diagonal: rows 384..511 of batch 1 see keys in kept tiles only
    mask[1, 4, :] = 0      # query tile 4 of batch 1 sees nothing -> zeros
    assert mask.shape == (2, nt, nt)
    note(f"prefill masked r={r}")
    got, _ = gpu_run_np(inp, mask=mask)
    want = oracle_run(inp, mask=mask)
    assert max_abs(got, want) <= TOL
    assert not got[1, :, 512:].any()


@pytest.mark.parametrize("masked", [False, True])
def test_prefill_batched_ragged_every_output(masked):
    """Three entries of different lengths (3000, 2049, 700: ragged tails inside
    a 64-key tile and a 128-row mask tile), int4 and int8 heads, GQA 4, with
    and without a per-entry block mask (40% of the eligible tiles dropped):
    every output against the oracle."""
    require_gpu()
    L = 3000
    spec = W.small("prefill", B=3, Hq=8, Hkv=2, L=L, bits=4, n_int8_heads=1, seed=47)
    inp = W.make_inputs(spec)
    lens = np.array([3000, 2049, 700], dtype=np.int32)
    mask = None
    if masked:
        rng = np.random.default_rng(48)
        mask = np.stack([W.skip_mask(L, 0.4, rng) for _ in range(3)])
    note(f"prefill batched ragged lens={lens.tolist()} masked={masked}")
    got, _ = gpu_run_np(inp, mask=mask, lens=lens)
    want = oracle_run(inp, mask=mask, lens=lens)
    err = max_abs(got, want)
    note(f"max-abs {err:.3e}")
    assert err <= TOL, err
    assert not got[1, :, 2049:].any() and not got[2, :, 700:].any()


@pytest.mark.parametrize("r", [4, 1])
def test_prefill_mask_long_dropped_runs(r):
    """A mask whose kept tiles are far apart: the query tiles of the second
    half keep only tile 0, the diagonal and tiles next to the boundaries of
    64-key-tile windows (mask tiles 31, 32, 63, 64, ...), so the tile walk
    crosses windows with no kept tile at all, and rows of one wave can fall on
    both sides of a query-tile boundary with different keep bits (r = 1: 256-row
    query blocks).  Two entries, the second shorter (ragged tail in a dropped
    run).  Sampled rows of every head against the oracle."""
    require_gpu()
    L = 16384
    nt = L // 128
    spec = W.small("prefill", B=2, Hq=2 * r, Hkv=2, L=L, bits=8, seed=31 + r)
    inp = W.make_inputs(spec)
    lens = np.array([L, L - 200], dtype=np.int32)
    mask = np.tril(np.ones((nt, nt), dtype=np.uint8))
    for qi in range(nt // 2, nt):
        keep = {0, qi} | {k for k in (31, 32, 63, 64, 95, 96) if k <= qi}
        if qi % 3 == 0:
            keep.add(qi - 1)        # neighbour rows of a wave differ in this tile
        mask[qi, :] = 0
        mask[qi, sorted(keep)] = 1
    masks = np.stack([mask, mask])
    rows = np.unique(np.concatenate([np.arange(0, 130), np.arange(L // 2 - 130, L // 2 + 130),
                                     np.linspace(L // 2, L - 1, 64).round().astype(int),
                                     np.arange(L - 300, L)]))
    note(f"prefill mask long dropped runs r={r} rows={rows.size}")
    got, _ = gpu_run_np(inp, mask=masks, lens=lens)
    want = oracle_run(inp, mask=masks, lens=lens, rows=rows, workers=8)
    err = max_abs(got[:, :, rows], want)
    assert err <= TOL, err
    assert not got[1, :, lens[1]:].any()


def _planted_inputs(r, q_scale, seed, low_start=0, n_high=0):
    """Prefill inputs (L = 900, two KV heads) with queries scaled by q_scale.
    The first low_start keys of each KV head are set to -40 times the unit
    mean-query direction of the head (every row's first tile then scores far
    below its later keys, so the running maximum has to move), and n_high
    keys late in the sequence to +40 times it (scores far above the rest)."""
    L = 900
    spec = W.small("prefill", B=1, Hq=2 * r, Hkv=2, L=L, bits=8, seed=seed)
    inp = W.make_inputs(spec)
    q = inp.q.astype(np.float32) * q_scale
    k = inp.k.astype(np.float32)
    rng = np.random.default_rng(seed)
    for g in range(2):
        qd = q[0, g * r:(g + 1) * r].mean(axis=(0, 1))
        qd /= np.linalg.norm(qd) + 1e-6
        k[0, g, :low_start] = -40.0 * qd
        for pos in rng.choice(np.arange(500, L), size=n_high, replace=False):
            k[0, g, pos] = 40.0 * qd
    inp.q = q.astype(np.float16)
    inp.k = k.astype(np.float16)
    nt = (L + 127) // 128
    mask = np.tril(np.ones((nt, nt), dtype=np.uint8))
    mask[5, 1:5] = 0         # rows of query tile 5 see only tile 0 and their own tile
    return inp, mask


@pytest.mark.parametrize("r", [4, 1])
def test_prefill_rescale_path(r):
    """Unit-scale queries whose first tile (keys set against the query
    direction) scores more than 15 (log2 units) below later keys: the kernel
    starts the running maximum at the first tile's row maximum, so its rare
    branch (re-form the tile's scores, move the maximum, rescale the
    accumulator and normaliser) runs for those rows.  The first tile's keys
    end with weights ~2^-15 or less, so their larger K-hat rounding does not
    reach the outputs.  Against the oracle within the bar."""
    require_gpu()
    inp, mask = _planted_inputs(r, 1.0, seed=61 + r, low_start=64)
    okc = oq.build_cache(inp.k, inp.structure.head_bits, "token", cap=inp.spec.cap)
    kh = oq.dequantized_all(okc)[0]
    qs = inp.q[0].astype(np.float64)
    jumps = 0
    for h in range(2 * r):
        s = qs[h] @ kh[h // r, :900].T / np.sqrt(128) / np.log(2)    # log2 units
        s = np.where(np.tril(np.ones((900, 900), dtype=bool)), s, -np.inf)
        first = s[:, :64].max(axis=1)
        jumps += int(((s.max(axis=1) - first) > 15)[64:].sum())
    assert jumps > 0                    # the rare branch is taken somewhere
    note(f"prefill rescale path r={r} rows={jumps}")
    got, _ = gpu_run_np(inp, mask=mask)
    want = oracle_run(inp, mask=mask)
    assert np.isfinite(got).all()
    assert max_abs(got, want) <= TOL


def test_prefill_large_scores_error_scales():
    """Queries x10 (scores up to ~70 in log2 units) and a dozen planted keys:
    K-hat enters the QK product as fp16, so the score error grows with the
    score magnitude; the bar is for unit-scale queries, and ten times the
    queries stay within ten times the bar (the output and V-hat rounding do
    not grow).  Outputs stay finite through many rescales."""
    require_gpu()
    inp, mask = _planted_inputs(4, 10.0, seed=65, n_high=12)
    note("prefill large scores")
    got, _ = gpu_run_np(inp, mask=mask)
    want = oracle_run(inp, mask=mask)
    assert np.isfinite(got).all()
    assert max_abs(got, want) <= 10 * TOL


def test_prefill_uniform_v_and_determinism():
    require_gpu()
    spec = W.small("prefill", B=1, Hq=4, Hkv=1, L=300, bits=8, seed=21)
    inp = W.make_inputs(spec)
    inp.v[0, 0, :300] = inp.v[0, 0, :1]
    note("prefill uniform V")
    got, (kc, vc, q, lt, tm) = gpu_run_np(inp)
    vhat = oq.dequantize(*oq.quantize(inp.v[0, 0, :1], 8)).astype(np.float16)
    ulp = np.abs(np.spacing(vhat)).astype(np.float64)
    assert np.all(np.abs(got[0] - vhat.astype(np.float64)) <= ulp + 1e-12)
    for _ in range(2):
        again = T.attn_prefill(kc, vc, q, lt)
        torch.cuda.synchronize()
        assert np.array_equal(again.cpu().numpy().view(np.uint16),
                              got.astype(np.float16).view(np.uint16))
