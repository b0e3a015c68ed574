"""Pins of the oracle's prefill attention with an INT8 prefix (HyQuant, core method's
fused operator and Algorithm 2: the query as given, the quantized prefix's keys and
values both through per-tile INT8, vertical lines and the window in full precision):
full-precision limits equal causal softmax attention written out in numpy; K and V
on exact INT8 grids with an unquantized query give that attention exactly; the
quantizer's closed-form properties for K and V; causality; and, on exact grids with
quarter-step offsets, which keys and which values each row reads through INT8 (CPU
only)."""
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


def _grid(r, shape, lo=-127, hi=128):
    """Integers in [lo, hi) with 127 in every 64-row tile of every head (column 0)."""
    x = r.integers(lo, hi, shape)
    x[:, ::64, :, 0] = 127
    return x


def test_exact_int8_prefix_with_a_plain_query_is_textbook_attention():
    """K and V are integers times a power of two reaching 127 in every tile, the query is
    a plain N(0, 1) sample: codes and scales are exact, K-hat = K and V-hat = V, so the
    all-INT8 result (window 0, no vertical line) is textbook attention with the query as
    given (a quantized query would not be)."""
    r = np.random.default_rng(2)
    batch, n, hq, hkv = 1, 192, 4, 2
    sk, sv = 2.0 ** -5, 2.0 ** -7
    ki, vi = _grid(r, (batch, n, hkv, 128)), _grid(r, (batch, n, hkv, 128))
    k, v = (ki * sk).astype(np.float32), (vi * sv).astype(np.float32)
    q = r.standard_normal((batch, n, hq, 128)).astype(np.float32)
    out, kc, ks, vc, vs = oracle.prefill_attend(q, k, v, [n], None, window=0)
    assert np.array_equal(kc, ki) and np.array_equal(vc, vi)
    assert np.all(ks == np.float32(sk)) and np.all(vs == np.float32(sv))
    assert np.allclose(out, _textbook(q, k, v, [n]), rtol=1e-12, atol=1e-12)
    # the same query on an INT8 grid of its own gives another result: q is not rounded
    qg = (np.rint(q / np.abs(q).max() * 127) * (np.abs(q).max() / 127)).astype(np.float32)
    out_g, *_ = oracle.prefill_attend(qg, k, v, [n], None, window=0)
    assert not np.allclose(out_g, out, rtol=1e-6, atol=1e-6)


def test_quantizer_properties_and_vertical_lines_leave_the_tile_maximum():
    q, k, v = _data(3, batch=1, n=130)
    cls = np.zeros((1, 2, 130), np.uint8)
    k2, v2 = k.copy(), v.copy()
    k2[0, 10, 0] *= 1000.0                                                  # a huge key and value...
    v2[0, 10, 0] *= 1000.0
    cls[0, 0, 10] = 1                                                       # ...of a vertical line
    _, kc, ks, vc, vs = oracle.prefill_attend(q, k2, v2, [130], cls, window=16)
    _, kc0, ks0, vc0, vs0 = oracle.prefill_attend(q, k, v, [130], cls, window=16)
    assert np.array_equal(ks, ks0) and np.array_equal(vs, vs0)             # its tiles' scales unchanged
    for x, c, s in ((k, kc0, ks0), (v, vc0, vs0)):
        for h in range(x.shape[2]):
            for tile in range(3):
                rows = slice(64 * tile, min(64 * tile + 64, 130))
                sc = float(s[0, h, tile])
                xt = x[0, rows, h].astype(np.float64)
                ct = c[0, rows, h]
                if h == 0 and tile == 0:
                    xt, ct = np.delete(xt, 10, axis=0), np.delete(ct, 10, axis=0)
                assert sc == np.float32(np.float32(np.abs(xt).max()) / np.float32(127))
                assert np.abs(ct).max() == 127
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


def test_window_edge_lines_and_values_on_an_exact_grid():
    """Which keys and which values each row reads through INT8, pinned exactly.  K and V
    sit on INT8 grids (integers times a power of two, 127 reached in every tile), except
    that a random half of their entries carry +1/4 of a step: INT8 reads such an entry as
    the grid value, full precision reads it as it is.  One vertical line of head 0 is far
    larger than the tile maximum in K and in V (left out of both scales, else the grids
    would change).  Row t must read key and value p exactly iff p is a line of its head
    or p > t - W, and the query always as given; the expected rows are causal softmax
    attention with that key and value set written out per row.  A value read past its
    quantization, an off-by-one at the window edge or a line read through INT8 fails
    it."""
    r = np.random.default_rng(9)
    batch, n, hq, hkv, w = 1, 192, 4, 2, 16
    g = hq // hkv
    sk, sv = 2.0 ** -5, 2.0 ** -6
    ki, vi = _grid(r, (batch, n, hkv, 128), -126, 127), _grid(r, (batch, n, hkv, 128), -126, 127)
    offk = (r.random((batch, n, hkv, 128)) < 0.5) * 0.25
    offv = (r.random((batch, n, hkv, 128)) < 0.5) * 0.25
    offk[:, ::64, :, 0] = offv[:, ::64, :, 0] = 0.0
    cls = np.zeros((batch, hkv, n), np.uint8)
    cls[0, 0, 5::13] = 1
    cls[0, 1, 3::7] = 1
    big = 70                                             # a line of head 0 in tile 1, channel 3
    assert cls[0, 0, big] == 1
    ki_line, vi_line = ki.astype(np.float64), vi.astype(np.float64)
    ki_line[0, big, 0, 3] = 400.0
    vi_line[0, big, 0, 3] = -500.0
    q = r.standard_normal((batch, n, hq, 128)).astype(np.float32)
    k_exact = ((ki_line + offk) * sk).astype(np.float32)
    v_exact = ((vi_line + offv) * sv).astype(np.float32)
    k_grid, v_grid = ki * sk, vi * sv
    out, kc, ks, vc, vs = oracle.prefill_attend(q, k_exact, v_exact, [n], cls, window=w)
    assert np.all(ks == np.float32(sk)) and np.all(vs == np.float32(sv))   # the big line left every scale alone
    lines_free = cls[0].T == 0                           # [n, hkv]
    assert np.array_equal(kc[0][lines_free], ki[0][lines_free])
    assert np.array_equal(vc[0][lines_free], vi[0][lines_free])
    want = np.zeros((n, hq, 128))
    for t in range(n):
        p = np.arange(t + 1)
        for j in range(hq):
            h = j // g
            exact = ((cls[0, h, p] == 1) | (p > t - w))[:, None]
            keys = np.where(exact, k_exact[0, p, h].astype(np.float64), k_grid[0, p, h])
            vals = np.where(exact, v_exact[0, p, h].astype(np.float64), v_grid[0, p, h])
            x = keys @ q[0, t, j].astype(np.float64) / np.sqrt(128.0)
            e = np.exp(x - x.max())
            want[t, j] = (e / e.sum()) @ vals
    assert np.allclose(out[0], want, rtol=1e-12, atol=1e-12)


def test_rows_entry_matches_the_full_computation():
    """The sampled-rows entry (used at sizes the full oracle cannot finish) gives the
    full computation's rows, codes and scales."""
    q, k, v = _data(5, batch=2, n=150)
    cls = np.zeros((2, 2, 150), np.uint8)
    cls[:, :, 3::11] = 1
    full, *codes = oracle.prefill_attend(q, k, v, [150, 97], cls, window=24)
    rows = [(0, 0), (0, 63), (0, 64), (0, 149), (1, 50), (1, 96)]
    part, *codes2 = oracle.prefill_attend_rows(q, k, v, [150, 97], cls, 24, rows)
    for i, (b, t) in enumerate(rows):
        assert np.array_equal(part[i], full[b, t])
    assert all(np.array_equal(x, y) for x, y in zip(codes, codes2))
