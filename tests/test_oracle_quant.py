"""Pins of the oracle's quantiser and cache layouts (CPU only).

The vectorised fp64 quantiser in ``oracle.quant`` is checked against things
that do not share its arithmetic: hand-derived golden groups, an exact-rational
re-derivation, a division-free nearest-code search, closed-form bounds and
hand-written byte layouts.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import quant, exact

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _group(values, fill=0.0):
    x = np.full(32, fill, dtype=np.float16)
    x[:len(values)] = np.asarray(values, dtype=np.float16)
    return x


def _adversarial_groups(rng, n):
    """Groups that stress rounding: exact ties, all zeros, one non-zero, tiny
    (subnormal) ranges, x8 outliers, all-positive / all-negative groups, fp16
    extremes, and values sitting on quantisation grid points."""
    out = []
    for i in range(n):
        kind = i % 9
        if kind == 0:
            x = rng.standard_normal(32).astype(np.float16)
        elif kind == 1:
            x = np.zeros(32, np.float16)
        elif kind == 2:
            x = np.zeros(32, np.float16)
            x[rng.integers(32)] = np.float16(rng.standard_normal())
        elif kind == 3:
            x = (rng.integers(-3, 4, 32) * 2.0 ** -24).astype(np.float16)
        elif kind == 4:
            x = rng.standard_normal(32).astype(np.float32)
            x[rng.integers(32)] *= 8
            x = x.astype(np.float16)
        elif kind == 5:
            x = np.abs(rng.standard_normal(32)).astype(np.float16)
        elif kind == 6:
            x = -np.abs(rng.standard_normal(32)).astype(np.float16)
        elif kind == 7:
            x = rng.choice(np.array([65504.0, -65504.0, 1.0, 0.0, -2.0]), 32).astype(np.float16)
        else:
            # grid points of an exactly representable scale, with half-steps
            s = 2.0 ** rng.integers(-6, 2)
            k = rng.integers(-20, 40, 32) / 2.0
            x = (k * s).astype(np.float16)
        out.append(x)
    return np.stack(out)


@pytest.mark.parametrize("bits", [8, 4])
def test_golden_groups(bits):
    with open(os.path.join(GOLDEN, "quant_groups.json")) as f:
        cases = [c for c in json.load(f)["cases"] if c["bits"] == bits]
    assert cases
    for c in cases:
        x = _group(c["x"])
        codes, s, z = quant.quantize(x[None], bits)
        exp_codes = list(c["codes"]) + [c["fill_code"]] * (32 - len(c["codes"]))
        assert codes[0].tolist() == exp_codes, c["name"]
        assert int(s.view(np.uint16)[0, 0]) == int(c["scale_bits"], 16), c["name"]
        assert int(z[0, 0]) == c["zero"], c["name"]


@pytest.mark.parametrize("bits", [8, 4])
def test_matches_exact_rational(bits):
    rng = np.random.default_rng(11 + bits)
    xs = _adversarial_groups(rng, 360)
    codes, s, z = quant.quantize(xs, bits)
    for i in range(xs.shape[0]):
        ce, se, ze = exact.quantize_group_exact(xs[i], bits)
        assert codes[i].tolist() == ce, i
        assert Fraction(float(s[i, 0])) == se, i
        assert int(z[i, 0]) == ze, i


@pytest.mark.parametrize("bits", [8, 4])
def test_codes_are_nearest_grid_points(bits):
    """Division-free brute force: every code is the nearest representable
    level (c - z) s in [0, qmax], ties to even (c - z)."""
    rng = np.random.default_rng(23 + bits)
    xs = _adversarial_groups(rng, 72)
    codes, s, z = quant.quantize(xs, bits)
    for i in range(xs.shape[0]):
        si = Fraction(float(s[i, 0]))
        if si == 0:
            assert not codes[i].any()
            continue
        lo = min(min(Fraction(float(v)) for v in xs[i]), Fraction(0))
        assert int(z[i, 0]) == exact.nearest_zero_search(lo, si, bits)
        for j in range(32):
            want = exact.nearest_code_search(Fraction(float(xs[i, j])), si,
                                             int(z[i, 0]), bits)
            assert int(codes[i, j]) == want, (i, j)


@pytest.mark.parametrize("bits", [8, 4])
def test_scale_is_least_fp16_above_range(bits):
    rng = np.random.default_rng(5)
    xs = rng.standard_normal((4000, 32)).astype(np.float16)
    _, s, _ = quant.quantize(xs, bits)
    qmax = (1 << bits) - 1
    x64 = xs.astype(np.float64)
    span = np.maximum(x64.max(1), 0) - np.minimum(x64.min(1), 0)
    s64 = s[:, 0].astype(np.float64)
    assert np.all(s64 * qmax >= span)
    pred = np.nextafter(s[:, 0], np.float16(0)).astype(np.float64)
    assert np.all(pred * qmax < span)


@pytest.mark.parametrize("bits", [8, 4])
def test_round_trip_bounds_and_invariants(bits):
    rng = np.random.default_rng(7 + bits)
    xs = np.concatenate([rng.standard_normal((3000, 128)).astype(np.float16),
                         _adversarial_groups(rng, 400).reshape(100, 128)])
    codes, s, z = quant.quantize(xs, bits)
    qmax = (1 << bits) - 1
    assert codes.max() <= qmax
    assert np.all(z <= qmax)
    xh = quant.dequantize(codes, s, z)
    err = np.abs(xs.astype(np.float64) - xh).reshape(-1, 4, 32)
    half = s.astype(np.float64)[..., None] / 2
    assert np.all(err <= half)
    # x == 0 dequantises to exactly 0
    zero = xs == 0
    assert np.all(xh[zero] == 0)
    # all-non-negative groups have z == 0
    g = xs.astype(np.float64).reshape(-1, 4, 32)
    nonneg = (g >= 0).all(-1)
    assert np.all(z[nonneg] == 0)
    # fp32 dequantisation is exact
    assert np.array_equal(quant.dequantize(codes, s, z, np.float32).astype(np.float64), xh)


def test_grid_points_round_trip_exactly():
    rng = np.random.default_rng(3)
    for bits in (4, 8):
        _, s, z = quant.quantize(rng.standard_normal((50, 32)).astype(np.float16), bits)
        qmax = (1 << bits) - 1
        for i in range(50):
            si, zi = float(s[i, 0]), int(z[i, 0])
            c = rng.integers(0, qmax + 1, 32)
            c[0], c[1] = 0, qmax  # keep the group's range equal to this grid
            pts = ((c - zi) * si)
            x = pts.astype(np.float16)
            if not np.array_equal(x.astype(np.float64), pts):
                continue  # level not representable in fp16
            c2, s2, z2 = quant.quantize(x[None], bits)
            xh = quant.dequantize(c2, s2, z2)[0]
            assert np.array_equal(xh, pts)


def test_fp16_dequant_is_rne_of_exact():
    rng = np.random.default_rng(9)
    xs = rng.standard_normal((500, 128)).astype(np.float16)
    codes, s, z = quant.quantize(xs, 8)
    exact64 = quant.dequantize(codes, s, z)
    h = quant.dequantize(codes, s, z, np.float16)
    # RNE: nearest fp16, and on exact ties the even mantissa
    up = np.nextafter(h, np.float16(np.inf)).astype(np.float64)
    dn = np.nextafter(h, np.float16(-np.inf)).astype(np.float64)
    hv = h.astype(np.float64)
    d = np.abs(hv - exact64)
    assert np.all(d <= np.abs(up - exact64))
    assert np.all(d <= np.abs(dn - exact64))


def test_rejects_bad_input():
    with pytest.raises(ValueError):
        quant.quantize(np.zeros((1, 32), np.float16), 3)
    with pytest.raises(ValueError):
        quant.quantize(np.zeros((1, 31), np.float16), 8)
    with pytest.raises(ValueError):
        quant.quantize(np.array([[np.inf] + [0] * 31], np.float16), 8)


# ---------------------------------------------------------------------------
# byte layouts, hand-written expectations
# ---------------------------------------------------------------------------

def test_nibble_packing_low_nibble_first():
    c = np.array(list(range(16)) + list(range(15, -1, -1)), dtype=np.uint8)
    b = quant.pack_nibbles(c)
    assert b.tolist() == [0x10, 0x32, 0x54, 0x76, 0x98, 0xBA, 0xDC, 0xFE,
                          0xEF, 0xCD, 0xAB, 0x89, 0x67, 0x45, 0x23, 0x01]
    assert np.array_equal(quant.unpack_nibbles(b), c)


def test_token_layout_mixed_heads():
    # B=2, Hkv=2, bits [8, 4], D=32, cap=128: row bytes 32 and 16;
    # head offsets 0 and 128*32; batch stride 128*(32+16) = 6144.
    cache = quant.Cache(2, 2, 32, 128, [8, 4], "token")
    assert cache.offs == [0, 4096] and cache.bstride == 6144
    codes8 = np.arange(32, dtype=np.uint8)[None].repeat(3, 0) + np.arange(3, dtype=np.uint8)[:, None]
    cache.write(1, 0, 5, codes8, np.ones((3, 1), np.float16), np.zeros((3, 1), np.uint8))
    base = 6144 + 5 * 32
    assert cache.codes[base:base + 32].tolist() == list(range(32))
    assert cache.codes[base + 32:base + 64].tolist() == list(range(1, 33))
    codes4 = np.full((1, 32), 3, dtype=np.uint8)
    codes4[0, 1] = 12
    cache.write(0, 1, 2, codes4, np.ones((1, 1), np.float16), np.zeros((1, 1), np.uint8))
    base = 4096 + 2 * 16
    assert cache.codes[base] == (3 | (12 << 4))
    assert cache.codes[base + 1] == 0x33
    assert cache.scales.shape == (2, 2, 128, 1)


def test_channel_layout_int8_and_int4():
    cache = quant.Cache(1, 2, 32, 256, [8, 4], "channel")
    # head 0 int8: token t, channel d at block t//32 (32*32 bytes each),
    # byte d*32 + t%32
    codes = np.zeros((256, 32), np.uint8)
    codes[130, 7] = 201      # block 4, row 7, byte 2
    codes[3, 31] = 17        # block 0, row 31, byte 3
    cache.write(0, 0, 0, codes, np.ones((256, 1), np.float16), np.zeros((256, 1), np.uint8))
    slab0 = cache.codes[:256 * 32]
    assert slab0[4 * 1024 + 7 * 32 + 2] == 201
    assert slab0[0 * 1024 + 31 * 32 + 3] == 17
    assert int(np.count_nonzero(slab0)) == 2
    # head 1 int4: block t//32 of 32*16 bytes, byte d*16 + (t%32)//2,
    # low nibble for even t
    codes = np.zeros((256, 32), np.uint8)
    codes[4, 2] = 9
    codes[5, 2] = 6
    codes[129, 0] = 15       # block 4, row 0, byte 0, high nibble
    cache.write(0, 1, 0, codes, np.ones((256, 1), np.float16), np.zeros((256, 1), np.uint8))
    slab1 = cache.codes[256 * 32:]
    assert slab1[0 * 512 + 2 * 16 + 2] == (9 | (6 << 4))
    assert slab1[4 * 512 + 0 * 16 + 0] == (15 << 4)
    assert cache.scales.shape == (1, 2, 1, 256)
    assert np.array_equal(cache.read_codes(0, 1), codes)


def test_partial_writes_keep_other_tokens():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((1, 1, 256, 64)).astype(np.float16)
    for layout in ("token", "channel"):
        for bits in (4, 8):
            whole = quant.build_cache(x, [bits], layout)
            part = quant.Cache(1, 1, 64, 256, [bits], layout)
            for s0, s1 in ((0, 3), (3, 130), (130, 131), (131, 256)):
                c, s, z = quant.quantize(x[0, 0, s0:s1], bits)
                part.write(0, 0, s0, c, s, z)
            assert np.array_equal(whole.codes, part.codes)
            assert np.array_equal(whole.scales.view(np.uint16), part.scales.view(np.uint16))
            assert np.array_equal(whole.zeros, part.zeros)
