"""GPU parity of the per-KV-head sensitivity scores and precision assignment
(taq_head_sensitivity) against the oracle.  The scores are sums of squared
differences of two fp16 decode outputs, so they are compared within a relative
bound; the assignment is then checked where it is unique (heads whose oracle
scores are separated by more than that bound) and checked for validity where
it is not (a near-tie may go either way)."""
import numpy as np
import pytest
import torch

import tiled_attention_quantized_amd as T
import workloads as W
from oracle import sensitivity as sens
from tests.gpu_util import require_gpu, note, lens_tensor

pytestmark = pytest.mark.gpu

REL = 0.05      # relative bound on a score (two fp16 outputs, fp32 weights in each)


def _case(B, Hq, Hkv, S, lens, seed, outlier_heads=(), scale=0.0, v_outliers=True):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, 128), dtype=np.float32).astype(np.float16)
    k = np.zeros((B, Hkv, S, 128), np.float16)
    v = np.zeros((B, Hkv, S, 128), np.float16)
    for b in range(B):
        n = int(lens[b])
        k[b, :, :n] = rng.standard_normal((Hkv, n, 128), dtype=np.float32).astype(np.float16)
        v[b, :, :n] = rng.standard_normal((Hkv, n, 128), dtype=np.float32).astype(np.float16)
    for i, g in enumerate(outlier_heads):
        # one channel of K and of V scaled up: its group's int4 step grows with it
        f = 8.0 * (i + 2)
        k[:, g, :, 3 + i] = (k[:, g, :, 3 + i].astype(np.float32) * f).astype(np.float16)
        if v_outliers:
            v[:, g, :, 40 + i] = (v[:, g, :, 40 + i].astype(np.float32) * f).astype(np.float16)
    return q, k, v


def _check(q, k, v, lens, n_high, scale=0.0):
    Hkv = k.shape[1]
    scores, bits = T.head_sensitivity(torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(),
                                      torch.from_numpy(q).cuda(), lens_tensor(lens), n_high,
                                      softmax_scale=scale)
    torch.cuda.synchronize()
    got_s = scores.cpu().numpy()
    got_b = bits.cpu().numpy()
    want_s = sens.sensitivity(q, k, v, lens, scale=None if scale == 0.0 else scale, workers=4)
    tol = REL * want_s + 1e-12
    assert np.all(np.abs(got_s - want_s) <= tol), (got_s, want_s)
    assert int((got_b == 8).sum()) == n_high and set(np.unique(got_b)) <= {4, 8}
    # validity: every int8 head scores at least every int4 head, up to the bound
    hi, lo = np.nonzero(got_b == 8)[0], np.nonzero(got_b == 4)[0]
    for a in hi:
        for c in lo:
            assert want_s[a] + tol[a] + tol[c] >= want_s[c], (a, c, want_s)
    # uniqueness: where the oracle's choice is separated by more than the bound
    want_b = sens.assign(want_s, n_high)
    srt = np.sort(want_s)[::-1]
    if 0 < n_high < Hkv and srt[n_high - 1] - srt[n_high] > 2 * REL * srt[n_high - 1]:
        assert np.array_equal(got_b, want_b)
    return got_s, got_b, want_s


@pytest.mark.parametrize("r", [1, 4, 8])
def test_scores_and_assignment_small(r):
    require_gpu()
    Hkv = 4
    lens = np.array([700, 333, 1], dtype=np.int32)
    q, k, v = _case(3, Hkv * r, Hkv, 768, lens, seed=400 + r, outlier_heads=(2,))
    note(f"head sensitivity r={r}")
    got_s, got_b, want_s = _check(q, k, v, lens, 1)
    assert list(got_b) == [4, 4, 8, 4]          # the planted head is clearly the most sensitive


def test_budget_sweep_and_extremes():
    require_gpu()
    Hkv = 8
    lens = np.array([2048, 1500], dtype=np.int32)
    q, k, v = _case(2, 32, Hkv, 2048, lens, seed=410, outlier_heads=(5, 1, 6))
    note("head sensitivity budget sweep")
    for n_high in (0, 2, 3, 4, 8):
        _, got_b, want_s = _check(q, k, v, lens, n_high)
        if n_high == 0:
            assert (got_b == 4).all()
        if n_high == 8:
            assert (got_b == 8).all()
        if n_high == 3:
            assert sorted(np.nonzero(got_b == 8)[0].tolist()) == [1, 5, 6]


def test_zero_heads_and_ties():
    require_gpu()
    Hkv = 4
    lens = np.array([512, 512], dtype=np.int32)
    q, k, v = _case(2, 8, Hkv, 512, lens, seed=420)
    k[:, 1] = 0
    v[:, 1] = 0
    k[:, 3] = k[:, 2]                  # head 3 copies head 2, with the same queries
    v[:, 3] = v[:, 2]
    q[:, 6:8] = q[:, 4:6]
    note("head sensitivity zeros and ties")
    got_s, got_b, _ = _check(q, k, v, lens, 2)
    assert got_s[1] == 0.0
    assert got_s[2] == got_s[3]        # same bytes in, same reduction order


def test_mixed_cache_from_the_assignment_decodes():
    """The assigned bits build a mixed-precision cache that the decode kernel
    reads, closing the loop of the method."""
    require_gpu()
    from oracle import attention as oa
    from oracle import quant as oq
    from tests.gpu_util import TOL, gpu_cache, max_abs
    Hkv = 4
    lens = np.array([900, 640], dtype=np.int32)
    # outliers in K only: V stays unit-variance, where the 2e-3 output bar applies
    q, k, v = _case(2, 16, Hkv, 1024, lens, seed=430, outlier_heads=(0, 3), v_outliers=False)
    _, bits = T.head_sensitivity(torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(),
                                 torch.from_numpy(q).cuda(), lens_tensor(lens), 2)
    hb = bits.cpu().numpy()
    assert sorted(np.nonzero(hb == 8)[0].tolist()) == [0, 3]
    note(f"mixed cache from assigned bits {hb.tolist()}")
    kc = gpu_cache(k, hb, T.LAYOUT_TOKEN, 1024)
    vc = gpu_cache(v, hb, T.LAYOUT_CHANNEL, 1024)
    out = T.attn_decode(kc, vc, torch.from_numpy(q).cuda(), lens_tensor(lens), 1024)
    torch.cuda.synchronize()
    kh = oq.dequantized_all(oq.build_cache(k, hb, "token", cap=1024))
    vh = oq.dequantized_all(oq.build_cache(v, hb, "channel", cap=1024))
    want = oa.decode(q, kh, vh, lens)
    assert max_abs(out.cpu().numpy().astype(np.float64), want) <= TOL
