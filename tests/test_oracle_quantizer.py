"""Pins of the oracle's fp16 rounding and group quantizer (CPU only).

The quantizer follows TriAxialKV key design 3 (asymmetric groups of G = 32 with a
scale and a zero point).  Each pin checks the oracle against something other than
itself: numpy's float16 conversion, brute-force nearest codes, the error bound
|x - x_hat| <= s/2, closed forms and hand-derived worked examples."""
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "quantizer_examples.txt")


def _np_f16_bits(x):
    return int(np.array([x], np.float16).view(np.uint16)[0])


def _canon(bits):
    return 0 if bits == 0x8000 else bits


def _library_down_up(x):
    """Largest fp16 <= x and smallest fp16 >= x via numpy's float16 (a library routine)."""
    h = np.float16(x)
    lo = h if float(h) <= float(x) else np.nextafter(h, np.float16(-np.inf))
    hi = h if float(h) >= float(x) else np.nextafter(h, np.float16(np.inf))
    return _canon(_np_f16_bits(lo)), _canon(_np_f16_bits(hi))


def _sample_floats(n, seed):
    r = np.random.default_rng(seed)
    e = r.uniform(-30, 16, n)                       # spans fp16 subnormals to 65504
    x = (r.choice([-1.0, 1.0], n) * 2.0 ** e).astype(np.float32)
    x = x[np.abs(x) <= 65504]
    exact = np.array([0.0, 1.0, -1.0, 65504.0, -65504.0, 2.0 ** -24, -2.0 ** -24, 2.0 ** -14,
                      6.097555e-5, 0.1, -0.1, 1.0009765625, 1e-9, -1e-9, 2.0 ** -25], np.float32)
    return np.concatenate([exact, x])


def test_f16_directed_rounding_matches_numpy(orc):
    for x in _sample_floats(4000, 1):
        down, up = _library_down_up(x)
        assert orc.f16_down(x) == down, (x, orc.f16_down(x), down)
        assert orc.f16_up(x) == up, (x, orc.f16_up(x), up)
        assert orc.f16_nearest(x) == _canon(_np_f16_bits(x)), x


def test_f16_value_matches_numpy(orc):
    bits = np.arange(0, 65536, 7, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    for b, r in zip(bits.tolist(), ref.tolist()):
        v = orc.f16_value(b)
        assert (np.isnan(v) and np.isnan(r)) or v == r


def _groups(seed):
    r = np.random.default_rng(seed)
    out = []
    for i in range(300):
        kind = i % 6
        if kind == 0:
            x = r.standard_normal(32)
        elif kind == 1:
            x = r.standard_normal(32) * 10.0 + 100.0      # |min| >> range
        elif kind == 2:
            x = r.uniform(-1e-3, 1e-3, 32)               # fp16 subnormal scales
        elif kind == 3:
            x = r.standard_normal(32); x[r.integers(32)] *= 30.0   # outlier
        elif kind == 4:
            x = np.round(r.standard_normal(32) * 4) / 4  # many ties on the grid
        else:
            x = r.uniform(-60000, 60000, 32)
        out.append(x.astype(np.float32))
    return out


@pytest.mark.parametrize("bits", [2, 4])
def test_quantizer_error_bound_and_brute_force(orc, bits):
    """|x - x_hat| <= s/2 (+ fp32 noise); each code is a nearest grid level."""
    L = (1 << bits) - 1
    for x in _groups(10 + bits):
        codes, sb, zb = orc.quantize(x, bits)
        s, z = orc.f16_value(sb), orc.f16_value(zb)
        xd = x.astype(np.float64)
        assert z <= xd.min() and (s == 0 or z + L * s >= xd.max() - 2 ** -18 * (xd.max() - z + s))
        assert codes.max() <= L
        xh = z + codes * s
        eps = 2.0 ** -18 * (np.abs(xd - z) + s)
        assert np.all(np.abs(xd - xh) <= s / 2 + eps)
        levels = z + np.arange(L + 1) * s
        dist = np.abs(xd[:, None] - levels[None, :])
        best = dist.min(axis=1)
        assert np.all(dist[np.arange(32), codes] <= best + eps)


@pytest.mark.parametrize("bits", [2, 4])
def test_quantizer_extremes_and_idempotence(orc, bits):
    L = (1 << bits) - 1
    for x in _groups(20 + bits):
        codes, sb, zb = orc.quantize(x, bits)
        s, z = orc.f16_value(sb), orc.f16_value(zb)
        if s == 0:
            continue
        assert codes[np.argmax(x)] == L or abs(x.max() - (z + (L - 1) * s)) <= s / 2 * (1 + 1e-6)
        if x.min() - z < s / 2 * (1 - 1e-6):
            assert codes[np.argmin(x)] == 0
        xh = (np.float32(z) + codes.astype(np.float32) * np.float32(s)).astype(np.float32)
        # re-quantize x_hat with the same (s, z) grid: same codes
        t = np.rint((xh.astype(np.float64) - z) / s).clip(0, L).astype(np.uint8)
        assert np.array_equal(t, codes)


def test_quantizer_constant_groups(orc):
    for v in [0.0, -0.0, 1.0, -2.5, 0.75, 65504.0, -65504.0]:       # fp16-exact values
        for bits in (2, 4):
            codes, sb, zb = orc.quantize(np.full(32, v, np.float32), bits)
            assert sb == 0 and not codes.any() and orc.f16_value(zb) == v and zb != 0x8000


def _parse_golden():
    rows = []
    for line in open(GOLDEN):
        if not line.strip() or line.startswith("#"):
            continue
        head, vals, codes = [p.strip() for p in line.split("|")]
        name, bits, s, z = head.split()
        if vals == "range32":
            x = np.arange(32, dtype=np.float32)
        elif vals.startswith("const"):
            x = np.full(32, np.float32(vals.split()[1]), np.float32)
        else:
            x = np.tile(np.array(vals.split()[1:], np.float32), 8)
        if codes.endswith("*32"):
            c = np.full(32, int(codes[:-3]), np.uint8)
        elif codes.startswith("repeat"):
            c = np.tile(np.array(codes.split()[1:], np.uint8), 8)
        else:
            c = np.array(codes.split(), np.uint8)
        rows.append((name, int(bits), int(s, 16), int(z, 16), x, c))
    return rows


def test_quantizer_golden_examples(orc):
    rows = _parse_golden()
    assert len(rows) == 4
    for name, bits, s, z, x, c in rows:
        codes, sb, zb = orc.quantize(x, bits)
        assert (sb, zb) == (s, z), name
        assert np.array_equal(codes, c), name


# ---------------------------------------------------------------- INT2 key scales ----
# INT2 key groups (one channel over 32 tokens) round their scale up once more, to the
# next fp16 value whose two lowest mantissa bits are zero (at most 9 significant bits),
# so that c s (c = 0..3) is an fp16 value and the decode forms its key operand exactly
# with one fused multiply-add.

def _candidates4():
    """Every finite fp16 value whose two lowest mantissa bits are zero, ascending
    (numpy's float16 decoding of the bit patterns)."""
    bits = np.arange(0, 0x10000, 4, dtype=np.uint32).astype(np.uint16)
    vals = bits.view(np.float16).astype(np.float64)
    vals = vals[np.isfinite(vals)]
    return np.unique(vals)


def test_f16_up4_is_the_next_value_with_two_zero_low_bits(orc):
    cand = _candidates4()
    for x in _sample_floats(4000, 5):
        if x > cand[-1]:  # (above 65408 the next such value is past fp16's range)
            continue
        want = cand[np.searchsorted(cand, float(x), side="left")]
        got = orc.f16_value(orc.f16_up4(x))
        assert got == want, (x, got, want)
        assert orc.f16_up4(x) & 3 == 0 and orc.f16_up4(x) != 0x8000


def test_quantize_k2_is_the_quantizer_with_the_coarser_scale(orc):
    """Same zero as the plain quantizer; scale = the next value with two zero low bits at
    or above the plain scale; codes nearest on that grid; |x - x_hat| <= s/2."""
    cand = _candidates4()
    for x in _groups(31):
        codes, sb, zb = orc.quantize_k2(x)
        _, sb0, zb0 = orc.quantize(x, 2)
        assert zb == zb0
        s0 = orc.f16_value(sb0)
        s, z = orc.f16_value(sb), orc.f16_value(zb)
        assert s == cand[np.searchsorted(cand, s0, side="left")], (s, s0)
        assert sb & 3 == 0 and s0 <= s <= s0 * (1 + 2.0 ** -8) + 2.0 ** -22
        xd = x.astype(np.float64)
        if s == 0:
            assert not codes.any()
            continue
        assert codes.max() <= 3
        eps = 2.0 ** -18 * (np.abs(xd - z) + s)
        assert np.all(np.abs(xd - (z + codes * s)) <= s / 2 + eps)
        levels = z + np.arange(4) * s
        dist = np.abs(xd[:, None] - levels[None, :])
        assert np.all(dist[np.arange(32), codes] <= dist.min(axis=1) + eps)


def test_int2_key_operand_is_exact_for_every_such_scale():
    """For every fp16 scale with two zero low mantissa bits in [2^-7, 32752): c s 2^-9
    (c = 0..3) and s times 2, 1/2, 1/8, 1/32 are fp16 values (numpy float16 round trip),
    which is what makes the decode's fma(off + 2^-9 c, s, -off s) exact."""
    cand = _candidates4()
    s = cand[(cand >= 2.0 ** -7) & (cand < 32752.0)]
    for c in range(4):
        v = c * s * 2.0 ** -9
        assert np.array_equal(v.astype(np.float16).astype(np.float64), v), c
    for off in (2.0, 0.5, 0.125, 0.03125):
        v = off * s
        assert np.array_equal(v.astype(np.float16).astype(np.float64), v), off
