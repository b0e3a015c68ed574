"""Pins of the oracle's FP8 anchors (OCP e4m3 codes with a power-of-two scale per token
and KV head; HyQuant names FP8 anchors as the smaller form of its FP16 ones).  Values
and rounding against torch's float8_e4m3fn (a library routine), the scale rule by its
bounds, and decode attention over an FP8-anchor cache against scipy attention over
torch-decoded anchors (CPU only)."""
import math

import numpy as np
import torch
from scipy.special import logsumexp, softmax

import synth


def _torch_codes(y):
    """torch's round-to-nearest-even fp32 -> e4m3 codes, with -0 taken as +0."""
    c = torch.as_tensor(np.asarray(y, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
    c[c == 0x80] = 0
    return c


def _torch_values(codes):
    return torch.as_tensor(np.asarray(codes, np.uint8)).view(torch.float8_e4m3fn).double().numpy()


def test_e4m3_values_match_torch(orc):
    ref = _torch_values(np.arange(256, dtype=np.uint8))
    got = np.array([orc.e4m3_value(c) for c in range(256)])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert orc.e4m3_value(0x7E) == 448.0 and orc.e4m3_value(0x01) == 2.0 ** -9


def test_nearest_matches_torch_rounding(orc):
    r = np.random.default_rng(1)
    mags = np.exp(r.uniform(math.log(2.0 ** -12), math.log(448.0), 3000))
    ys = np.concatenate([mags, -mags[:500], [0.0, -0.0, 448.0, -448.0, 2.0 ** -10, 2.0 ** -11]])
    # every midpoint between consecutive finite magnitudes: exact ties, to the even code
    vals = np.array([orc.e4m3_value(c) for c in range(0x7F)])
    mids = (vals[:-1] + vals[1:]) / 2
    ys = np.concatenate([ys, mids, -mids]).astype(np.float32)
    got = np.array([orc.e4m3_nearest(float(y)) for y in ys], np.uint8)
    assert np.array_equal(got, _torch_codes(ys))
    tie = np.array([orc.e4m3_nearest(float(m)) for m in mids])
    assert np.all(tie % 2 == 0)


def test_row_scale_is_the_smallest_power_of_two(orc):
    r = np.random.default_rng(2)
    rows = [r.standard_normal(128) * 2.0 ** r.integers(-30, 16) for _ in range(200)]
    edge = np.zeros(128)
    edge[5] = 448.0 * 2.0 ** -3                       # max exactly 448 * 2^e
    rows += [np.zeros(128), np.full(128, 1e-12), edge, np.full(128, -65504.0)]
    for x in rows:
        x = np.float32(x)
        codes, sbits = orc.fp8_row(x)
        s = float(np.uint16(sbits).view(np.float16))
        e = int(round(math.log2(s)))
        assert s == 2.0 ** e and e >= -24
        amax = float(np.abs(x.astype(np.float64)).max())
        assert amax <= 448.0 * s and (e == -24 or amax > 448.0 * s / 2)
        assert np.array_equal(codes, _torch_codes(x.astype(np.float64) / s))
        xh = _torch_values(codes) * s
        mag = np.maximum(np.abs(x.astype(np.float64)), 2.0 ** -300)
        spacing = np.maximum(2.0 ** (np.floor(np.log2(mag)) - 3), 2.0 ** -9 * s)
        assert np.all(np.abs(xh - x) <= spacing / 2 + 1e-300)
    codes, _ = orc.fp8_row(np.float32(edge))
    assert codes[5] == 0x7E


def test_fp8_anchor_cache_attention(orc):
    """An FP8-anchor cache: each token's K and V rows are e4m3 codes times a power of
    two; decode attention over it equals scipy attention over the torch-decoded rows."""
    T, g, heads = 53, 4, 2
    r = np.random.default_rng(3)
    k = r.standard_normal((T, heads, 128)).astype(np.float32)
    k[:, :, 7] *= 30.0
    v = r.standard_normal((T, heads, 128)).astype(np.float32)
    npg = -(-T // 16)
    c = orc.Cache(heads, 0, 0, npg, anchor_fp8=True)
    assert c.pool_bytes(orc.FP16).shape[0] == npg * heads * 4160
    c.append(k, v, orc.F32, heads * 128, 128, rows16=np.arange(T), slots16=np.arange(T))
    tables = np.arange(npg, dtype=np.int32)[None]

    def dec(rows):
        out = np.zeros(rows.shape)
        for t in range(rows.shape[0]):
            amax = np.abs(rows[t].astype(np.float64)).max()
            e = -24
            while amax > 448.0 * 2.0 ** e:
                e += 1
            out[t] = _torch_values(_torch_codes(rows[t].astype(np.float64) / 2.0 ** e)) * 2.0 ** e
        return out

    q = r.standard_normal((1, g * heads, 128)).astype(np.float32)
    for h in range(heads):
        rng = synth.ranges_array([(0, h, orc.FP16, 0, T)])
        out, lse = c.attend(q, 1, g * heads, heads, tables, orc.PAGES, rng)
        kd, vd = dec(k[:, h]), dec(v[:, h])
        x = q[0, h * g:(h + 1) * g].astype(np.float64) @ kd.T / math.sqrt(128)
        rows = slice(h * g, (h + 1) * g)
        assert np.allclose(out[0, rows], softmax(x, axis=-1) @ vd, rtol=0, atol=1e-12)
        assert np.allclose(lse[0, rows], logsumexp(x, axis=-1), atol=1e-12)
        for t in (0, 17, T - 1):
            kk, vv = c.token(t // 16, t % 16, h)
            assert np.array_equal(kk, kd[t]) and np.array_equal(vv, vd[t])
