"""Pins of the oracle's prefill attention with an INT8 prefix (HyQuant Algorithm 2):
full-precision limits equal scipy's causal attention, an exactly representable INT8
prefix equals it too, the quantizer's closed-form properties, causality, and the
vertical lines' exclusion from K's tile maximum (CPU only)."""
import math

import numpy as np
from scipy.special import softmax

from oracle import oracle


def _textbook(q, k, v, n):
    """Causal softmax(q k^T / sqrt(d)) v per query head in fp64 (GQA: head j reads j // g)."""
    batch, n_max, hq, _ = q.shape
    hkv = k.shape[2]
    g = hq // hkv
    out = np.zeros(q.shape)
    for b in range(batch):
        for j in range(hq):
            qq = q[b, : n[b], j].astype(np.float64)
            kk = k[b, : n[b], j // g].astype(np.float64)
            x = qq @ kk.T / math.sqrt(128)
            x[np.triu_indices(n[b], 1)] = -np.inf
            out[b, : n[b], j] = softmax(x, axis=1) @ v[b, : n[b], j // g].astype(np.float64)
    return out


def _data(seed, batch=2, n=150, hq=4, hkv=2):
    r = np.random.default_rng(seed)
    q = r.standard_normal((batch, n, hq, 128)).astype(np.float32)
    k = r.standard_normal((batch, n, hkv, 128)).astype(np.float32)
    v = r.standard_normal((batch, n, hkv, 128)).astype(np.float32)
    return q, k, v


def test_full_precision_limits_are_textbook_causal_attention():
    q, k, v = _data(1)
    n = [150, 97]
    ref = _textbook(q, k, v, n)
    wide, *_ = oracle.prefill_attend(q, k, v, n, None, window=150)          # every key in the window
    assert np.allclose(wide, ref, rtol=1e-12, atol=1e-12)
    allvl = np.ones((2, 2, 150), np.uint8)                                  # every key a vertical line
    vl, *_ = oracle.prefill_attend(q, k, v, n, allvl, window=0)
    assert np.allclose(vl, ref, rtol=1e-12, atol=1e-12)
    assert not wide[1, 97:].any()


def test_exactly_representable_int8_prefix_is_exact():
    """Inputs s * integer with |integer| <= 127 reaching 127 in every tile: codes and
    scales are exact, so the all-INT8 result (window 0, no vertical line) is exact."""
    r = np.random.default_rng(2)
    batch, n, hq, hkv = 1, 192, 4, 2
    def ints(shape):
        x = r.integers(-127, 128, shape)
        x[:, ::64, ...] = 127                                               # every 64-row tile reaches 127
        return x
    sq, sk = 2.0 ** -6, 2.0 ** -5
    qi, ki = ints((batch, n, hq, 128)), ints((batch, n, hkv, 128))
    q, k = (qi * sq).astype(np.float32), (ki * sk).astype(np.float32)
    v = r.standard_normal((batch, n, hkv, 128)).astype(np.float32)
    out, qc, qs, kc, ks = oracle.prefill_attend(q, k, v, [n], None, window=0)
    assert np.array_equal(qc, qi) and np.array_equal(kc, ki)
    assert np.all(qs == np.float32(127 * sq / 127)) and np.all(ks == np.float32(sk))
    assert np.allclose(out, _textbook(q, k, v, [n]), rtol=1e-12, atol=1e-12)


def test_quantizer_properties_and_vertical_lines_leave_the_tile_maximum():
    q, k, v = _data(3, batch=1, n=130)
    cls = np.zeros((1, 2, 130), np.uint8)
    k2 = k.copy()
    k2[0, 10, 0] *= 1000.0                                                  # a huge key...
    cls[0, 0, 10] = 1                                                       # ...that is a vertical line
    _, qc, qs, kc, ks = oracle.prefill_attend(q, k2, v, [130], cls, window=16)
    _, _, _, kc0, ks0 = oracle.prefill_attend(q, k, v, [130], cls, window=16)
    assert np.array_equal(ks, ks0)                                          # its tile's scale unchanged
    for x, c, s, axis in ((q, qc, qs, 2), (k, kc, ks0, 2)):
        for h in range(x.shape[2]):
            for tile in range(3):
                rows = slice(64 * tile, min(64 * tile + 64, 130))
                sc = float(s[0, h, tile])
                xt = x[0, rows, h].astype(np.float64)
                if h == 0 and x is k and tile == 0:
                    xt = np.delete(xt, 10, axis=0)
                    ct = np.delete(c[0, rows, h], 10, axis=0)
                else:
                    ct = c[0, rows, h]
                assert sc == np.float32(np.float32(np.abs(xt).max()) / np.float32(127))
                assert np.abs(ct).max() == 127 and np.abs(ct).max() <= 127
                assert np.all(np.abs(xt - sc * ct) <= sc / 2 * (1 + 1e-5))


def test_causality():
    q, k, v = _data(4, batch=1, n=120)
    cls = np.zeros((1, 2, 120), np.uint8)
    cls[0, :, ::17] = 1
    out, *_ = oracle.prefill_attend(q, k, v, [120], cls, window=32)
    k2, v2 = k.copy(), v.copy()
    k2[0, 80:] += 5.0
    v2[0, 80:] -= 3.0
    out2, *_ = oracle.prefill_attend(q, k2, v2, [120], cls, window=32)
    assert np.array_equal(out[0, :64], out2[0, :64])                        # same tiles, earlier keys
    assert not np.allclose(out[0, 80:], out2[0, 80:])


def test_window_edge_and_lines_on_an_exact_grid():
    """Which keys each row reads through INT8, pinned exactly.  Q and K sit on INT8 grids
    (integers times a power of two, 127 reached in every tile), except that a random
    half of the K entries carry +1/4 of a step: INT8 reads such an entry as the grid
    value, full precision reads it as it is.  One vertical line is far larger than
    the tile maximum (left out of K's scale, else the grid would change).  Row t must
    read key p exactly iff p is a line of its head or p > t - W; the expected rows are
    plain causal softmax attention with that key set written out per row."""
    r = np.random.default_rng(9)
    batch, n, hq, hkv, w = 1, 192, 4, 2, 16
    g = hq // hkv
    sq, sk = 2.0 ** -6, 2.0 ** -5
    qi = r.integers(-126, 127, (batch, n, hq, 128))
    ki = r.integers(-126, 127, (batch, n, hkv, 128))
    qi[:, ::64, :, 0] = 127
    ki[:, ::64, :, 0] = 127
    off = (r.random((batch, n, hkv, 128)) < 0.5) * 0.25
    off[:, ::64, :, 0] = 0.0
    cls = np.zeros((batch, hkv, n), np.uint8)
    cls[0, 0, 5::13] = 1
    cls[0, 1, 3::7] = 1
    ki_line = ki.copy().astype(np.float64)
    big = 70                                             # a line of head 0 in tile 1, channel 3
    assert cls[0, 0, big] == 1
    ki_line[0, big, 0, 3] = 400.0
    q = (qi * sq).astype(np.float32)
    k_exact = ((ki_line + off) * sk).astype(np.float32)
    k_grid = (ki * sk).astype(np.float64)
    v = r.standard_normal((batch, n, hkv, 128)).astype(np.float32)
    out, qc, _, kc, ks = oracle.prefill_attend(q, k_exact, v, [n], cls, window=w)
    assert np.all(ks == np.float32(sk))                  # the big line left every scale alone
    lines_free = cls[0].T == 0                           # [n, hkv]
    assert np.array_equal(kc[0][lines_free], ki[0][lines_free])
    want = np.zeros((n, hq, 128))
    for t in range(n):
        p = np.arange(t + 1)
        for j in range(hq):
            h = j // g
            exact = (cls[0, h, p] == 1) | (p > t - w)
            keys = np.where(exact[:, None], k_exact[0, p, h].astype(np.float64), k_grid[0, p, h])
            x = keys @ q[0, t, j].astype(np.float64) / np.sqrt(128.0)
            e = np.exp(x - x.max())
            want[t, j] = (e / e.sum()) @ v[0, p, h].astype(np.float64)
    assert np.allclose(out[0], want, rtol=1e-12, atol=1e-12)


def test_rows_entry_matches_the_full_computation():
    """The sampled-rows entry (used at sizes the full oracle cannot finish) gives the
    full computation's rows, codes and scales."""
    q, k, v = _data(5, batch=2, n=150)
    cls = np.zeros((2, 2, 150), np.uint8)
    cls[:, :, 3::11] = 1
    full, qc, qs, kc, ks = oracle.prefill_attend(q, k, v, [150, 97], cls, window=24)
    rows = [(0, 0), (0, 63), (0, 64), (0, 149), (1, 50), (1, 96)]
    part, qc2, qs2, kc2, ks2 = oracle.prefill_attend_rows(q, k, v, [150, 97], cls, 24, rows)
    for i, (b, t) in enumerate(rows):
        assert np.array_equal(part[i], full[b, t])
    assert all(np.array_equal(x, y) for x, y in ((qc, qc2), (qs, qs2), (kc, kc2), (ks, ks2)))
