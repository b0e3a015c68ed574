"""Pins of the oracle's write path: routing, byte layout and page-table reorder (CPU).

Routing follows TriAxialKV key design 3 (INT2 tokens form G = 32 groups; the residual
tail of fewer than 32 goes to INT4 per-token).  The reorder follows key design 4,
phase 1 (every request's INT2 page pointers move ahead of its INT4 pointers).  The
layout pins compare against byte patterns derived by hand in
tests/golden/layout_examples.txt."""
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "layout_examples.txt")


def _golden():
    rows = {}
    for line in open(GOLDEN):
        if not line.strip() or line.startswith("#"):
            continue
        key, val = [p.strip() for p in line.split(" = ", 1)]
        parts = val.split()
        if parts[-1].startswith("x"):
            parts = parts[:-1] * int(parts[-1][1:])
        rows[key] = bytes(int(b, 16) for b in parts)
    return rows


def test_route_closed_form(orc):
    r = np.random.default_rng(3)
    for n in [0, 1, 31, 32, 33, 64, 95, 1000, 4097]:
        flags = r.choice([0, 0, 0, 1, 2], n).astype(np.uint8)
        cls, n2g, n4, n16 = orc.route(flags)
        w2 = int((flags == 0).sum())
        assert n2g == w2 // 32
        assert n16 == int((flags == 2).sum())
        assert n4 == int((flags == 1).sum()) + w2 % 32
        idx2 = np.flatnonzero(flags == 0)
        assert np.all(cls[idx2[: 32 * n2g]] == 0) and np.all(cls[idx2[32 * n2g:]] == 1)
        assert np.all(cls[flags == 1] == 1) and np.all(cls[flags == 2] == 2)


def test_int4_layout_golden(orc):
    g = _golden()
    c = orc.Cache(1, 0, 2, 0)
    k = np.zeros((1, 128), np.float32)
    v = np.zeros((1, 128), np.float32)
    k[0] = np.arange(128) % 16
    v[0] = 15 - np.arange(128) % 16
    c.append(k, v, orc.F32, 128, 128, rows4=[0], slots4=[1 * 16 + 3])   # page 1, offset 3
    blk = c.pool_bytes(orc.INT4)[2560:5120]
    assert not c.pool_bytes(orc.INT4)[:2560].any()
    assert bytes(blk[192:256]) == g["int4 token_off=3 kcodes@192"]
    assert bytes(blk[1472:1536]) == g["int4 token_off=3 vcodes@1472"]
    assert bytes(blk[1072:1088]) == g["int4 token_off=3 kmeta@1072"]
    for off in (2316, 2380, 2444, 2508):
        assert bytes(blk[off:off + 4]) == g["int4 token_off=3 vmeta@2316,2380,2444,2508"]
    written = np.zeros(2560, bool)
    written[192:256] = written[1472:1536] = written[1072:1088] = True
    for off in (2316, 2380, 2444, 2508):
        written[off:off + 4] = True
    assert not blk[~written].any(), "bytes of other tokens must stay untouched"


def test_int2_layout_golden(orc):
    g = _golden()
    c = orc.Cache(1, 4, 0, 0)
    t = np.arange(32)[:, None]
    ch = np.arange(128)[None, :]
    k = ((t + ch) % 4).astype(np.float32)
    v = np.broadcast_to(ch % 4, (32, 128)).astype(np.float32).copy()
    c.append(k, v, orc.F32, 128, 128, rows2=np.arange(32), pages2=[2])
    pool = c.pool_bytes(orc.INT2)
    assert not pool[:2 * 1536].any()
    even, odd = pool[2 * 1536:3 * 1536], pool[3 * 1536:4 * 1536]
    for tt in range(32):
        blk = even if tt < 16 else odd
        off = tt % 16
        assert bytes(blk[off * 32:off * 32 + 32]) == g[f"int2 token_t%4={tt % 4} krow"]
        assert bytes(blk[768 + off * 32:768 + off * 32 + 32]) == g["int2 vrow"]
        for gi in range(4):
            m = 1280 + gi * 64 + off * 2
            assert bytes(blk[m:m + 2]) == g["int2 vscale"] and bytes(blk[m + 32:m + 34]) == g["int2 vzero"]
    for page in (even, odd):
        assert bytes(page[512:640]) == g["int2 kscales"] and bytes(page[640:768]) == g["int2 kzeros"]


def test_int2_v_meta_runs_golden(orc):
    """INT2 V metadata: per group the 16 tokens' scales, then their 16 zeros."""
    g = _golden()
    c = orc.Cache(1, 4, 0, 0)
    t = np.arange(32)[:, None]
    ch = np.arange(128)[None, :]
    k = np.zeros((32, 128), np.float32)
    v = ((ch % 4) * (t + 1)).astype(np.float32)
    c.append(k, v, orc.F32, 128, 128, rows2=np.arange(32), pages2=[0])
    pool = c.pool_bytes(orc.INT2)
    for page, key in ((pool[:1536], "int2 vscale run even"), (pool[1536:3072], "int2 vscale run odd")):
        for gi in range(4):
            m = 1280 + gi * 64
            assert bytes(page[m:m + 32]) == g[key], (key, gi)
            assert not page[m + 32:m + 64].any()
        for off in range(16):
            assert bytes(page[768 + off * 32:768 + off * 32 + 32]) == g["int2 vrow"]


def test_fp16_layout_golden(orc):
    g = _golden()
    c = orc.Cache(1, 0, 0, 1)
    k = (np.arange(128) / 2).astype(np.float32)[None]
    c.append(k, k, orc.F32, 128, 128, rows16=[0], slots16=[5])
    blk = c.pool_bytes(orc.FP16)
    assert bytes(blk[1286:1288]) == g["fp16 token_off=5 k[3]@1286"]
    assert np.array_equal(blk[5 * 256:6 * 256].view(np.float16), k[0].astype(np.float16))
    assert np.array_equal(blk[4096 + 5 * 256:4096 + 6 * 256].view(np.float16), k[0].astype(np.float16))


def test_heads_are_head_major_blocks(orc):
    """Head h of a page lives in block h; a different head's block is not touched."""
    c = orc.Cache(3, 0, 1, 0)
    r = np.random.default_rng(0)
    k = r.standard_normal((1, 3, 128)).astype(np.float32)
    v = r.standard_normal((1, 3, 128)).astype(np.float32)
    c.append(k, v, orc.F32, 3 * 128, 128, rows4=[0], slots4=[7])
    for h in range(3):
        kh, vh = c.token(0, 7, h)
        single = orc.Cache(1, 0, 1, 0)
        single.append(k[:, h], v[:, h], orc.F32, 128, 128, rows4=[0], slots4=[7])
        ks, vs = single.token(0, 7, 0)
        assert np.array_equal(kh, ks) and np.array_equal(vh, vs)


def test_bf16_source_is_widened_exactly(orc):
    r = np.random.default_rng(1)
    x = r.standard_normal((2, 128)).astype(np.float32)
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)                    # truncated bf16
    widened = (bits.astype(np.uint32) << 16).view(np.float32)
    a, b = orc.Cache(1, 0, 1, 0), orc.Cache(1, 0, 1, 0)
    a.append(bits, bits, orc.BF16, 128, 128, rows4=[0, 1], slots4=[0, 1])
    b.append(widened, widened, orc.F32, 128, 128, rows4=[0, 1], slots4=[0, 1])
    assert np.array_equal(a.pool_bytes(orc.INT4), b.pool_bytes(orc.INT4))


@pytest.mark.parametrize("bits_cls", ["int4", "int2"])
def test_dequantized_tokens_within_bound(orc, bits_cls):
    """Every dequantized value is within half a quantization step of its source."""
    r = np.random.default_rng(7)
    k = r.standard_normal((32, 2, 128)).astype(np.float32)
    k[:, :, 5] *= 10
    v = r.standard_normal((32, 2, 128)).astype(np.float32)
    if bits_cls == "int4":
        c = orc.Cache(2, 0, 2, 0)
        c.append(k, v, orc.F32, 256, 128, rows4=np.arange(32), slots4=np.arange(32))
        L = 15
    else:
        c = orc.Cache(2, 2, 0, 0)
        c.append(k, v, orc.F32, 256, 128, rows2=np.arange(32), pages2=[0])
        L = 3
    for t in range(32):
        for h in range(2):
            kh, vh = c.token(t // 16, t % 16, h)
            for ref, got, per_channel in ((k, kh, bits_cls == "int2"), (v, vh, False)):
                x = ref[t, h].astype(np.float64)
                if per_channel:
                    col = ref[:, h].astype(np.float64)
                    step = (col.max(0) - col.min(0)) / L
                else:
                    grp = x.reshape(4, 32)
                    step = np.repeat((grp.max(1) - grp.min(1)) / L, 32)
                assert np.all(np.abs(x - got) <= step / 2 * 1.01 + 1e-6)


def _mixed_table(orc, seed, n_units=12):
    """A one-table INT2/INT4 cache in shuffled 32-token units plus its source rows."""
    import synth
    r = np.random.default_rng(seed)
    u = r.permutation(np.array([0] * (n_units * 2 // 3) + [1] * (n_units - n_units * 2 // 3), np.uint8))
    flags = np.repeat(u, 32)
    T = flags.shape[0]
    k = r.standard_normal((T, 1, 128)).astype(np.float32)
    v = r.standard_normal((T, 1, 128)).astype(np.float32)
    n2 = int((flags == 0).sum()) // 16
    n4 = -(-int((flags == 1).sum()) // 16)
    alloc = synth.PageAllocator((n2, n4, 0), 1, 1, T // 16, seed)
    lists = synth.AppendLists()
    alloc.place(0, orc.route(flags)[0], np.arange(T), lists)
    c = orc.Cache(1, n2, n4, 0)
    c.append(k, v, orc.F32, 128, 128, **lists.arrays())
    return c, alloc, k, v


def test_reorder_is_stable_partition(orc):
    for seed in range(5):
        c, alloc, _, _ = _mixed_table(orc, seed)
        before = alloc.tables.copy()
        tab = alloc.tables.copy()
        counts = c.reorder(tab, alloc.n_entries)
        n = int(alloc.n_entries[0])
        assert sorted(tab[0, :n].tolist()) == sorted(before[0, :n].tolist())   # permutation
        n2 = c.n_pages[0]
        cls = np.where(tab[0, :n] < n2, 0, 1)
        assert np.all(np.diff(cls) >= 0)                                         # partition
        for k_ in (0, 1):                                                         # stable
            sel = before[0, :n][np.where(before[0, :n] < n2, 0, 1) == k_]
            assert np.array_equal(tab[0, :n][cls == k_], sel)
        p = tab[0, :counts[0, 0]]
        assert np.all(p[0::2] % 2 == 0) and np.all(p[1::2] == p[0::2] + 1)      # aligned pairs
        assert counts[0].tolist() == [int((cls == 0).sum()), int((cls == 1).sum()), 0]


def test_reorder_rejects_broken_pairs(orc):
    c, alloc, _, _ = _mixed_table(orc, 1)
    tab = alloc.tables.copy()
    i2 = np.flatnonzero(tab[0] < c.n_pages[0])
    tab[0, i2[0]], tab[0, i2[1]] = tab[0, i2[1]], tab[0, i2[0]]   # swap the pair's pages
    with pytest.raises(RuntimeError):
        c.reorder(tab, alloc.n_entries)
