"""Pins of the oracle's per-head sensitivity score and precision assignment."""
import numpy as np
import pytest

from oracle import brute
from oracle import quant as oq
from oracle import sensitivity as sens


def _inputs(rng, B=2, Hq=4, Hkv=2, S=256, D=32):
    q = rng.standard_normal((B, Hq, D)).astype(np.float16)
    k = rng.standard_normal((B, Hkv, S, D)).astype(np.float16)
    v = rng.standard_normal((B, Hkv, S, D)).astype(np.float16)
    return q, k, v


def test_zero_head_has_zero_score():
    rng = np.random.default_rng(0)
    q, k, v = _inputs(rng)
    k[:, 1] = 0
    v[:, 1] = 0
    s = sens.sensitivity(q, k, v, [256, 200])
    assert s[1] == 0.0 and s[0] > 0.0


def test_planted_outlier_head_ranks_first():
    rng = np.random.default_rng(1)
    q, k, v = _inputs(rng, B=2, Hq=8, Hkv=4)
    # one channel x32 in K of head 2 and in V: its group's int4 step grows 32x
    k[:, 2, :, 5] = (k[:, 2, :, 5].astype(np.float32) * 32).astype(np.float16)
    v[:, 2, :, 7] = (v[:, 2, :, 7].astype(np.float32) * 32).astype(np.float16)
    s = sens.sensitivity(q, k, v, [256, 256])
    assert int(np.argmax(s)) == 2
    assert list(sens.assign(s, 1)) == [4, 4, 8, 4]


def test_copies_score_equally_and_tie_to_lower_index():
    rng = np.random.default_rng(2)
    q, k, v = _inputs(rng, B=1, Hq=4, Hkv=2)
    k[:, 1] = k[:, 0]
    v[:, 1] = v[:, 0]
    q[:, 2:] = q[:, :2]
    s = sens.sensitivity(q, k, v, [256])
    assert s[0] == s[1]
    assert list(sens.assign(s, 1)) == [8, 4]


def test_matches_brute_force_attention():
    rng = np.random.default_rng(3)
    B, Hq, Hkv, S, D = 2, 4, 2, 128, 8
    q = rng.standard_normal((B, Hq, D)).astype(np.float16)
    k = rng.standard_normal((B, Hkv, S, D)).astype(np.float16)
    v = rng.standard_normal((B, Hkv, S, D)).astype(np.float16)
    # D = 8 is below one quantisation group: pad to 32 channels with zeros
    pad = lambda x: np.concatenate([x, np.zeros(x.shape[:-1] + (24,), np.float16)], axis=-1)
    q, k, v = pad(q), pad(k), pad(v)
    lens = [128, 77]
    want = np.zeros(Hkv)
    outs = {}
    for bits in (8, 4):
        kh = oq.dequantized_all(oq.build_cache(k, [bits] * Hkv, "token", cap=S))
        vh = oq.dequantized_all(oq.build_cache(v, [bits] * Hkv, "channel", cap=S))
        outs[bits] = np.array(brute.decode(q.astype(np.float64), kh, vh, lens, Hq, Hkv))
    for h in range(Hq):
        want[h // 2] += ((outs[4][:, h] - outs[8][:, h]) ** 2).sum()
    np.testing.assert_allclose(sens.sensitivity(q, k, v, lens), want, rtol=1e-10, atol=0)


def test_assign_counts_and_extremes():
    s = np.array([0.3, 0.1, 0.3, 0.5, 0.0])
    assert list(sens.assign(s, 0)) == [4] * 5
    assert list(sens.assign(s, 5)) == [8] * 5
    assert list(sens.assign(s, 2)) == [8, 4, 4, 8, 4]       # 0.5, then the first 0.3
    assert list(sens.assign(s, 3)) == [8, 4, 8, 8, 4]
    with pytest.raises(ValueError):
        sens.assign(s, 6)


def test_saving_falls_as_heads_move_to_int8():
    vals = [sens.saving([8] * n + [4] * (8 - n)) for n in range(9)]
    assert vals == sorted(vals, reverse=True)
    # 512 fp16 bytes per token-head against 152 (int4) / 280 (int8)
    assert vals[0] == pytest.approx(512 / 152) and vals[8] == pytest.approx(512 / 280)
