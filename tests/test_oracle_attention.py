"""Pins of the oracle's decode attention and log-sum-exp merge (CPU only).

Definitions followed: softmax(q k^T / sqrt(d)) v with d = 128 and online-softmax state
(m, l, acc) merged by log-sum-exp (HyQuant background and Algorithm 3; TriAxialKV key
design 4); GQA query head j reads KV head j // g (HyQuant background, GQA); a sentinel
dead slot contributes nothing (IntentKV, layout-preserving eviction).  Pins compare
with scipy's softmax / logsumexp, closed forms and invariances."""
import math

import numpy as np
import pytest
from scipy.special import logsumexp, softmax

import synth


def _fp16_cache(orc, seed, T, heads=1, kv_std=1.0):
    r = np.random.default_rng(seed)
    k = (r.standard_normal((T, heads, 128)) * kv_std).astype(np.float32)
    v = r.standard_normal((T, heads, 128)).astype(np.float32)
    c = orc.Cache(heads, 0, 0, -(-T // 16))
    c.append(k, v, orc.F32, heads * 128, 128, rows16=np.arange(T), slots16=np.arange(T))
    tables = np.arange(-(-T // 16), dtype=np.int32)[None]
    return c, k, v, tables


def _textbook(q, k, v):
    """softmax(q k^T / sqrt(d)) v with scipy, in fp64."""
    x = (q.astype(np.float64) @ k.astype(np.float64).T) / math.sqrt(128)
    return softmax(x, axis=-1) @ v.astype(np.float64), logsumexp(x, axis=-1)


def test_fp16_cache_is_textbook_attention(orc):
    T, g = 77, 4
    c, k, v, tables = _fp16_cache(orc, 0, T)
    q = np.random.default_rng(1).standard_normal((1, g, 128)).astype(np.float32)
    rng = synth.ranges_array([(0, 0, orc.FP16, 0, T)])
    out, lse = c.attend(q, 1, g, 1, tables, orc.PAGES, rng)
    k16 = k[:, 0].astype(np.float16).astype(np.float64)
    v16 = v[:, 0].astype(np.float16).astype(np.float64)
    ro, rl = _textbook(q[0], k16, v16)
    assert np.allclose(out[0], ro, rtol=0, atol=1e-13) and np.allclose(lse[0], rl, atol=1e-12)


def _quant_cache(orc, seed, n_units=10, heads=1):
    """Mixed INT2 / INT4 cache of one table, shuffled 32-token units."""
    r = np.random.default_rng(seed)
    u = r.permutation(np.array([0] * (n_units - 3) + [1] * 3, np.uint8))
    flags = np.repeat(u, 32)
    flags[-5:] = 1
    T = flags.shape[0]
    k = r.standard_normal((T, heads, 128)).astype(np.float32)
    k[:, :, 3] *= 10
    v = r.standard_normal((T, heads, 128)).astype(np.float32)
    cls = orc.route(flags)[0]
    n2 = int((cls == 0).sum()) // 16
    n4 = -(-int((cls == 1).sum()) // 16) + 1
    alloc = synth.PageAllocator((n2, n4, 0), heads, 1, T // 16 + 2, seed)
    lists = synth.AppendLists()
    alloc.place(0, cls, np.arange(T), lists)
    c = orc.Cache(heads, n2, n4, 0)
    c.append(k, v, orc.F32, heads * 128, 128, **lists.arrays())
    return c, alloc, k, v


def _dequantized(orc, c, alloc, head=0):
    ks, vs = [], []
    for e in range(int(alloc.n_entries[0])):
        for off in range(alloc.fill[0][e]):
            kk, vv = c.token(int(alloc.tables[0, e]), off, head)
            ks.append(kk)
            vs.append(vv)
    return np.array(ks), np.array(vs)


def test_quantized_attention_brute_force(orc):
    c, alloc, _, _ = _quant_cache(orc, 3)
    g = 4
    q = np.random.default_rng(4).standard_normal((1, g, 128)).astype(np.float32)
    rng = synth.ranges_array(alloc.ranges(0, [0]))
    out, lse = c.attend(q, 1, g, 1, alloc.tables, orc.PAGES, rng)
    kd, vd = _dequantized(orc, c, alloc)
    ro, rl = _textbook(q[0], kd, vd)
    assert np.allclose(out[0], ro, atol=1e-13) and np.allclose(lse[0], rl, atol=1e-12)


def test_single_token_and_uniform_weights(orc):
    c, alloc, _, _ = _quant_cache(orc, 5)
    kd, vd = _dequantized(orc, c, alloc)
    g = 2
    q = np.random.default_rng(6).standard_normal((1, g, 128)).astype(np.float32)
    one = synth.ranges_array([(0, 0, orc.INT2 if alloc.tables[0, 0] < c.n_pages[0] else orc.INT4, 0, 1)])
    out, lse = c.attend(q, 1, g, 1, alloc.tables, orc.PAGES, one)
    assert np.array_equal(out[0, 0], vd[0]) and np.allclose(out[0, 1], vd[0], atol=0)
    assert np.allclose(lse[0], q[0].astype(np.float64) @ kd[0] / math.sqrt(128), atol=1e-12)
    rng = synth.ranges_array(alloc.ranges(0, [0]))
    out, lse = c.attend(np.zeros((1, g, 128), np.float32), 1, g, 1, alloc.tables, orc.PAGES, rng)
    assert np.allclose(out[0, 0], vd.mean(0), atol=1e-13)
    assert np.allclose(lse[0], math.log(len(vd)), atol=1e-12)


def _split(rng_items, pieces):
    """Cut every range into `pieces` parts (INT2 parts on 32-token boundaries)."""
    out = []
    for (t, h, c, b, e) in rng_items:
        unit = 32 if c == 0 else 1
        n = (e - b) // unit
        cuts = sorted(set([0, n] + [round(n * i / pieces) for i in range(1, pieces)]))
        for a, z in zip(cuts[:-1], cuts[1:]):
            out.append((t, h, c, b + a * unit, min(e, b + z * unit) if z < n else e))
    return out


@pytest.mark.parametrize("pieces", [1, 2, 4, 7, 64])
def test_split_merge_invariance(orc, pieces):
    c, alloc, _, _ = _quant_cache(orc, 8, n_units=12, heads=2)
    hq, hkv = 8, 2
    q = np.random.default_rng(9).standard_normal((1, hq, 128)).astype(np.float32)
    full = synth.ranges_array(alloc.ranges(0, [0, 1]))
    ref, ref_lse = c.attend(q, 1, hq, hkv, alloc.tables, orc.PAGES, full)
    items = _split(alloc.ranges(0, [0]), pieces) + _split(alloc.ranges(0, [1]), pieces)
    parts = synth.ranges_array(items)
    po, pl = c.attend_ranges(q, 1, hq, hkv, alloc.tables, orc.PAGES, parts)
    n0 = sum(1 for it in items if it[1] == 0)
    out, lse = orc.merge(po, pl, np.array([0, n0, len(items)], np.int32), 1, hq, hkv)
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-14) and np.allclose(lse, ref_lse, atol=1e-12)


def test_reorder_permutation_invariance(orc):
    c, alloc, _, _ = _quant_cache(orc, 11, n_units=16)
    g = 4
    q = np.random.default_rng(12).standard_normal((1, g, 128)).astype(np.float32)
    before = synth.ranges_array(alloc.ranges(0, [0]))
    ref, ref_lse = c.attend(q, 1, g, 1, alloc.tables, orc.PAGES, before)
    tab = alloc.tables.copy()
    counts = c.reorder(tab, alloc.n_entries)
    after = synth.ranges_array(synth.class_ordered_ranges(0, [0], alloc.tokens[0]))
    assert counts[0, 0] * 16 == alloc.tokens[0, 0]
    out, lse = c.attend(q, 1, g, 1, tab, orc.PAGES, after)
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-14) and np.allclose(lse, ref_lse, atol=1e-12)


def test_gqa_and_table_mapping(orc):
    """Table t serves request t // (hkv / H) and KV heads of its group; query head j
    reads KV head j // g."""
    r = np.random.default_rng(13)
    B, hq, hkv, H, T = 2, 8, 4, 2, 40
    tpr = hkv // H
    k = r.standard_normal((B * tpr * T, H, 128)).astype(np.float32)
    v = r.standard_normal((B * tpr * T, H, 128)).astype(np.float32)
    q = r.standard_normal((B, hq, 128)).astype(np.float32)
    pages = -(-T // 16)
    c = orc.Cache(H, 0, 0, B * tpr * pages)
    rows = np.arange(B * tpr * T)
    slots = (rows // T) * pages * 16 + rows % T
    c.append(k, v, orc.F32, H * 128, 128, rows16=rows, slots16=slots)
    tables = np.arange(B * tpr * pages, dtype=np.int32).reshape(B * tpr, pages)
    items = [(t, h, orc.FP16, 0, T) for t in range(B * tpr) for h in range(H)]
    out, lse = c.attend(q, B, hq, hkv, tables, orc.PAGES, synth.ranges_array(items))
    g = hq // hkv
    for b in range(B):
        for j in range(hq):
            kvh = j // g
            t, h = b * tpr + kvh // H, kvh % H
            kk = k[t * T:(t + 1) * T, h].astype(np.float16).astype(np.float64)
            vv = v[t * T:(t + 1) * T, h].astype(np.float16).astype(np.float64)
            ro, rl = _textbook(q[b, j:j + 1], kk, vv)
            assert np.allclose(out[b, j], ro[0], atol=1e-13) and abs(lse[b, j] - rl[0]) < 1e-12


def test_dead_slots_equal_dropped_tokens(orc):
    """Slot-map entries redirected to the sentinel contribute exactly nothing."""
    r = np.random.default_rng(14)
    T, g = 200, 4
    k = r.standard_normal((T + 1, 1, 128)).astype(np.float32)
    v = r.standard_normal((T + 1, 1, 128)).astype(np.float32)
    k[0], v[0] = -1e4, 0.0
    pages = -(-T // 16) + 1
    c = orc.Cache(1, 0, pages, 0, sentinel_slot=0)
    slots = np.arange(16, 16 + T)
    c.append(k, v, orc.F32, 128, 128, rows4=np.concatenate([[0], 1 + np.arange(T)]),
             slots4=np.concatenate([[0], slots]))
    q = r.standard_normal((1, g, 128)).astype(np.float32)
    dead = np.sort(r.choice(T, 40, replace=False))
    live = np.setdiff1d(np.arange(T), dead)
    tab = slots.astype(np.int32).copy()
    tab[dead] = 0
    out, lse = c.attend(q, 1, g, 1, tab[None], orc.SLOTS, synth.ranges_array([(0, 0, 1, 0, T)]))
    tab2 = np.full(T, -1, np.int32)
    tab2[:len(live)] = slots[live]
    ref, rl = c.attend(q, 1, g, 1, tab2[None], orc.SLOTS, synth.ranges_array([(0, 0, 1, 0, len(live))]))
    assert np.allclose(out, ref, rtol=1e-13, atol=1e-15) and np.allclose(lse, rl, atol=1e-13)
    tab[:] = 0                                                # every entry dead
    out, lse = c.attend(q, 1, g, 1, tab[None], orc.SLOTS, synth.ranges_array([(0, 0, 1, 0, T)]))
    assert not out.any() and np.all(np.isneginf(lse))


def test_slot_compaction_keeps_attention_and_order(orc):
    """Compacting a two-head slot table (live entries first, in order) and reading each
    head's live count leaves every head's attention as it was: the dead entries carry
    no weight.  Counts, order and the all-dead / empty-prefix cases checked directly."""
    r = np.random.default_rng(16)
    T, g, H = 300, 4, 2
    k = r.standard_normal((T + 1, H, 128)).astype(np.float32)
    v = r.standard_normal((T + 1, H, 128)).astype(np.float32)
    k[0], v[0] = -1e4, 0.0
    c = orc.Cache(H, 0, -(-T // 16) + 1, 0, sentinel_slot=0)
    slots = 16 + r.permutation(T)                      # scattered slots
    c.append(k, v, orc.F32, H * 128, 128, rows4=np.concatenate([[0], 1 + np.arange(T)]),
             slots4=np.concatenate([[0], slots]))
    q = r.standard_normal((1, g * H, 128)).astype(np.float32)
    tabs = np.full((3, T), 7, np.int32)                # table 1: all dead; table 2: empty prefixes
    tabs[0] = slots
    tabs[0, np.sort(r.choice(T, 61, replace=False))] = 0
    tabs[1] = 0
    n_entries = np.array([T, 40, 0], np.int32)
    head_tokens = np.array([[T, 173], [40, 9], [0, 0]], np.int32)
    orig = tabs.copy()
    live = c.compact_slots(tabs, n_entries, head_tokens)
    for t in range(3):
        n = n_entries[t]
        keep = orig[t, :n][orig[t, :n] != 0]
        assert np.array_equal(tabs[t, :len(keep)], keep) and np.all(tabs[t, len(keep):n] == 0)
        assert np.array_equal(tabs[t, n:], orig[t, n:])  # past n_entries: untouched
        for h in range(H):
            assert live[t, h] == int((orig[t, :head_tokens[t, h]] != 0).sum())
    # attention of table 0 (both heads: one request, hkv = 2)
    before = synth.ranges_array([(0, h, 1, 0, int(head_tokens[0, h])) for h in range(H)])
    after = synth.ranges_array([(0, h, 1, 0, int(live[0, h])) for h in range(H)])
    o0, l0 = c.attend(q, 1, g * H, H, np.ascontiguousarray(orig[:1]), orc.SLOTS, before)
    o1, l1 = c.attend(q, 1, g * H, H, np.ascontiguousarray(tabs[:1]), orc.SLOTS, after)
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1) and np.isfinite(l0).all()
    assert live[1].tolist() == [0, 0] and live[2].tolist() == [0, 0]
    with pytest.raises(RuntimeError):                   # a prefix longer than the table
        c.compact_slots(orig.copy(), n_entries, np.array([[T + 1, 0], [0, 0], [0, 0]], np.int32))


def test_merge_closed_form(orc):
    r = np.random.default_rng(15)
    g, S = 3, 5
    po = r.standard_normal((S, g, 128))
    pl = r.standard_normal((S, g)) * 3
    pl[2, 1] = -np.inf
    out, lse = orc.merge(po, pl, np.array([0, S], np.int32), 1, g, 1)
    w = softmax(pl, axis=0)
    assert np.allclose(lse[0], logsumexp(pl, axis=0), atol=1e-13)
    assert np.allclose(out[0], np.einsum("sg,sgc->gc", w, po), atol=1e-13)
    two, lse2 = orc.merge(np.stack([po[0], po[0]]), np.stack([pl[0], pl[0]]),
                          np.array([0, 2], np.int32), 1, g, 1)
    assert np.allclose(two[0], po[0], atol=1e-14) and np.allclose(lse2[0], pl[0] + math.log(2), atol=1e-13)
    empty, lse3 = orc.merge(po[:0], pl[:0], np.array([0, 0], np.int32), 1, g, 1)
    assert not empty.any() and np.all(np.isneginf(lse3))
