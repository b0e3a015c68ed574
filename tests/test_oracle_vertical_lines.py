"""Pins of the oracle's vertical-line selection and FREEZE routing (CPU only).

Followed: HyQuant Algorithm 1 (the last W = 128 tokens are the window; a tail-query
proxy, the mean of the tail queries, scores the non-window prefix through the GQA group;
the top rho = 5 % become vertical lines) and Algorithm 4 (FREEZE: vertical lines and
window stay full precision, the rest of the prefix is quantized).  Pinned by planted
answers, invariances, ties and the count rule, not by recomputing the scores."""
import numpy as np
import pytest

from oracle import oracle


def _data(seed, batch=2, n=600, hkv=2, g=4, tail=16):
    r = np.random.default_rng(seed)
    k = r.standard_normal((batch, n, hkv, 128)).astype(np.float32)
    q = r.standard_normal((batch, tail, hkv * g, 128)).astype(np.float32)
    return k, q


def test_planted_vertical_lines_are_found_and_window_is_kept_apart():
    """Tail queries all equal to v: keys planted along v in the prefix are the vertical
    lines; an even larger key inside the window stays a window token."""
    r = np.random.default_rng(1)
    n, W, hkv, g = 800, 128, 2, 4
    k = r.standard_normal((1, n, hkv, 128)).astype(np.float32)
    v = r.standard_normal(128).astype(np.float32)
    q = np.broadcast_to(v, (1, 8, hkv * g, 128)).copy()
    n_vl = int(np.floor(0.05 * (n - W) + 0.5))                  # 34
    planted = np.sort(r.choice(n - W, n_vl, replace=False))
    for h in range(hkv):
        k[0, planted, h] = 20.0 * v / np.linalg.norm(v) ** 2 * 64 + k[0, planted, h] * 0.01
        k[0, n - 5, h] = 1000.0 * v                              # in the window
    s, cls, cnt = oracle.select_vl(k, q, [n], [8], window=W, rho=0.05)
    assert cnt.tolist() == [[n_vl, n_vl]]
    # identical tail queries: the proxy of a group is g v, so score = g (v . k)
    for h in range(hkv):
        want = g * (k[0, :, h].astype(np.float64) @ v.astype(np.float64))
        assert np.allclose(s[0, h, :n], want, rtol=1e-12, atol=1e-9)
    for h in range(hkv):
        assert np.array_equal(np.flatnonzero(cls[0, h] == 1), planted)
        assert np.all(cls[0, h, n - W:] == 2) and cls[0, h, n - 5] == 2
        assert np.all(cls[0, h, : n - W][np.setdiff1d(np.arange(n - W), planted)] == 0)


def test_selection_follows_a_permutation_of_the_prefix():
    k, q = _data(2)
    n, W = k.shape[1], 128
    _, cls, _ = oracle.select_vl(k, q, [n, n], [16, 16], window=W)
    perm = np.random.default_rng(3).permutation(n - W)
    k2 = k.copy()
    k2[:, : n - W] = k[:, perm]
    _, cls2, _ = oracle.select_vl(k2, q, [n, n], [16, 16], window=W)
    assert np.array_equal(cls2[:, :, : n - W], cls[:, :, perm])
    assert np.array_equal(cls2[:, :, n - W:], cls[:, :, n - W:])


def test_positive_scaling_keeps_and_negation_flips_the_selection():
    k, q = _data(4)
    n = k.shape[1]
    s1, c1, _ = oracle.select_vl(k, q, [n, n], [16, 16])
    _, c2, _ = oracle.select_vl(k, q * 3.0, [n, n], [16, 16])
    _, c3, _ = oracle.select_vl(k, -q, [n, n], [16, 16])
    assert np.array_equal(c1, c2)
    assert not np.any((c1 == 1) & (c3 == 1))                    # top and bottom 5 % are disjoint
    for b in range(2):                                          # every pick outranks every non-pick
        for h in range(2):
            pre = s1[b, h, : n - 128]
            sel = c1[b, h, : n - 128] == 1
            assert pre[sel].min() > pre[~sel].max()


def test_group_sum_and_tail_mean():
    """u sums the g heads of a group and averages the tail: heads that cancel leave all
    scores 0 (ties go to the lowest indices); repeating the tail changes nothing."""
    k, q = _data(5, batch=1)
    q[:, :, 1] = -q[:, :, 0]
    q[:, :, 2] = -q[:, :, 3]
    q[:, :, 5] = -q[:, :, 4]
    q[:, :, 6] = -q[:, :, 7]
    n = k.shape[1]
    s, cls, cnt = oracle.select_vl(k, q, [n], [16])
    assert np.all(s == 0.0)
    m = int(cnt[0, 0])
    assert np.array_equal(np.flatnonzero(cls[0, 0] == 1), np.arange(m))
    k2, q2 = _data(6, batch=1, tail=8)
    _, c_a, _ = oracle.select_vl(k2, q2, [n], [8])
    _, c_b, _ = oracle.select_vl(k2, np.concatenate([q2, q2], axis=1), [n], [16])
    assert np.array_equal(c_a, c_b)


def test_ties_and_counts():
    r = np.random.default_rng(7)
    n, W = 300, 128
    k = r.standard_normal((1, n, 1, 128)).astype(np.float32)
    q = r.standard_normal((1, 4, 1, 128)).astype(np.float32)
    k[0, [40, 10, 90, 70], 0] = k[0, 5, 0] * 0 + 50.0 * q[0].mean(axis=0)[0]  # four equal top scores
    _, cls, cnt = oracle.select_vl(k, q, [n], [4], window=W, rho=0.02)    # n_vl = round(3.44) = 3
    assert cnt[0, 0] == 3
    assert np.flatnonzero(cls[0, 0] == 1).tolist() == [10, 40, 70]
    for n_pre, rho, want in [(10, 0.05, 1), (30, 0.05, 2), (50, 0.05, 3), (172, 0.05, 9), (40, 0.0, 0), (40, 1.0, 40)]:
        _, c, m = oracle.select_vl(k, q, [n_pre + W], [4], window=W, rho=rho)
        assert m[0, 0] == want and int((c == 1).sum()) == want
    _, c, m = oracle.select_vl(k, q, [100], [4], window=W)         # shorter than the window
    assert m[0, 0] == 0 and np.all(c[0, 0, :100] == 2) and np.all(c[0, 0, 100:] == 0)
    with pytest.raises(RuntimeError):
        oracle.select_vl(k, q, [n + 1], [4])                          # beyond max_tokens
