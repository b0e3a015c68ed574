"""CPU tests of the C ABI: the library loads, exports every declared symbol, and its
host-side logic (routing, split planning, ahead-of-time split counts, argument
validation) behaves as include/kvq.h states.  No device work is enqueued here."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def kvq():
    from mixed_precision_quantized_amd import kvq
    return kvq


def _declared():
    text = open(os.path.join(ROOT, "include", "kvq.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w\s\*]*?\b(kvq_\w+)\s*\(", text, flags=re.M)))


def test_every_declared_symbol_is_exported(kvq):
    names = _declared()
    assert len(names) >= 11, names
    lib = kvq.raw_library()
    for n in names:
        assert hasattr(lib, n), f"{n} declared in kvq.h but not exported"
    assert set(names) == set(kvq.EXPORTED)


def test_block_bytes(kvq):
    # INT2, INT4, FP16 and an FP8 anchor block (e4m3 K and V rows of 16 tokens plus 16
    # fp16 scales each: 2 * (2048 + 32)); unknown classes 0
    assert [kvq.block_bytes(c) for c in (0, 1, 2, 3, 4)] == [1536, 2560, 8192, 4160, 0]


def test_route_matches_oracle_and_closed_form(kvq, orc):
    r = np.random.default_rng(5)
    for n in (0, 1, 31, 32, 33, 100, 5000):
        flags = r.choice([0, 0, 1, 2], n).astype(np.uint8)
        got = kvq.route_tokens(flags)
        ref = orc.route(flags)
        assert np.array_equal(got[0], ref[0]) and got[1:] == ref[1:]
        assert got[1] == int((flags == 0).sum()) // 32


def test_route_rejects_bad_flags(kvq):
    with pytest.raises(kvq.KvqError):
        kvq.route_tokens(np.array([0, 3], np.uint8))


def _ranges(items, kvq):
    return np.array(items, dtype=kvq.SPLIT_DTYPE)


def test_plan_splits_cover_ranges_exactly(kvq):
    r = np.random.default_rng(6)
    for trial in range(20):
        batch, hkv, H = 3, 4, 2
        items = []
        for t in range(batch * hkv // H):
            for h in range(H):
                n2 = int(r.integers(0, 8)) * 32
                n4 = int(r.integers(0, 300))
                if n2:
                    items.append((t, h, 0, 0, n2))
                if n4:
                    items.append((t, h, 1, n2, n2 + n4))
        rng = _ranges(items, kvq)
        kw = [dict(target_bytes=int(r.integers(1000, 50000))), dict(tokens_per_split=[64, 17, 5])][trial % 2]
        splits, off = kvq.plan_splits(rng, batch, hkv, H, **kw)
        # every range covered exactly once, pieces in order, INT2 pieces on 32-token edges
        for (t, h, c, b, e) in items:
            mine = splits[(splits[:, 0] == t) & (splits[:, 1] == h) & (splits[:, 2] == c)]
            assert mine[0, 3] == b and mine[-1, 4] == e
            assert np.all(mine[1:, 3] == mine[:-1, 4]) and np.all(mine[:, 4] > mine[:, 3])
            if c == 0:
                assert np.all(mine[:, 3] % 32 == 0) and np.all(mine[:, 4] % 32 == 0)
        # offsets: non-decreasing, partials of (b, kvh) contiguous
        assert off[0] == 0 and off[-1] == len(splits) and np.all(np.diff(off) >= 0)
        tpr = hkv // H
        for pair in range(batch * hkv):
            b, kvh = divmod(pair, hkv)
            rows = splits[off[pair]:off[pair + 1]]
            assert np.all(rows[:, 0] == b * tpr + kvh // H) and np.all(rows[:, 1] == kvh % H)


def test_plan_splits_tokens_per_split_and_aot(kvq):
    rng = _ranges([(0, 0, 0, 0, 192), (0, 0, 1, 192, 256)], kvq)
    s, off = kvq.plan_splits(rng, 1, 1, 1, tokens_per_split=[64, 64, 64])
    assert s.tolist() == [[0, 0, 0, 0, 64], [0, 0, 0, 64, 128], [0, 0, 0, 128, 192], [0, 0, 1, 192, 256]]
    assert off.tolist() == [0, 4]
    s, _ = kvq.plan_splits(rng, 1, 1, 1, splits_per_head=np.array([8], np.int32))
    assert len(s) == 8 or len(s) == 7
    budgets = (0.1 + 0.9 * np.arange(8) / 7).astype(np.float32)
    c = kvq.aot_split_counts(budgets, 64, 2048).reshape(64, 8)
    assert np.all(c == c[0]) and np.all(np.diff(c[0]) >= 0) and c[0, 0] >= 1
    assert abs(int(c[0].sum()) - 32) <= 4                         # 2048 work groups / 64 requests
    assert np.array_equal(kvq.aot_split_counts(budgets, 64, 2048),
                          kvq.aot_split_counts(budgets, 64, 2048))  # independent of lengths


def test_plan_splits_rejects_unsorted_and_misaligned(kvq):
    with pytest.raises(kvq.KvqError):
        kvq.plan_splits(_ranges([(1, 0, 1, 0, 5), (0, 0, 1, 0, 5)], kvq), 2, 1, 1)
    with pytest.raises(kvq.KvqError):
        kvq.plan_splits(_ranges([(0, 0, 0, 0, 40)], kvq), 1, 1, 1)


def _cache_struct(kvq, head_dim=128, page=16, heads=1, n=(2, 2, 0)):
    c = kvq._CacheC()
    c.head_dim, c.page_size, c.heads_per_page = head_dim, page, heads
    for i in range(3):
        c.n_pages[i] = n[i]
        c.pool[i] = 0x1000 if n[i] else 0          # never dereferenced: calls fail validation
    c.sentinel_slot = -1
    return c


def test_validation_fails_before_any_launch(kvq):
    lib = kvq.raw_library()
    fake = ctypes.c_void_p(0x1000)
    cases = [
        (_cache_struct(kvq, head_dim=64), 1, 8, 8, 1, -2),     # head_dim 64: unsupported
        (_cache_struct(kvq, page=32), 1, 8, 8, 1, -2),         # page size 32: unsupported
        (_cache_struct(kvq), 1, 8, 3, 1, -1),                  # hq % hkv != 0
        (_cache_struct(kvq), 1, 8, 8, 3, -1),                  # n_tables != batch*hkv/H
        (_cache_struct(kvq), 1, 8 * 17, 8, 8, -2),             # g = 17 > 16
        (_cache_struct(kvq, n=(3, 2, 0)), 1, 8, 8, 8, -1),     # odd INT2 pool
    ]
    for c, batch, hq, hkv, n_tables, want in cases:
        st = lib.kvq_decode_attn(ctypes.byref(c), fake, 0, batch, hq, hkv, fake, n_tables, 4, 0, fake, 1,
                                 fake, fake, None, None)
        assert st == want, (st, want, kvq.raw_library().kvq_last_error())
    c = _cache_struct(kvq)
    assert lib.kvq_quantize_append(ctypes.byref(c), fake, fake, 7, 1, 128, 128, 0, None, None, 0, None,
                                   None, 0, None, None, None, None) == -1       # bad dtype
    assert lib.kvq_quantize_append(ctypes.byref(c), fake, fake, 0, 1, 128, 128, 3, None, None, 0, None,
                                   None, 0, None, None, None, None) == -1       # NULL list
    assert lib.kvq_reorder_pages(ctypes.byref(c), fake, 1, 32769, fake, None, None, None) == -2
    assert lib.kvq_lse_merge(fake, fake, 1, fake, 1, 8, 3, fake, 0, None, None) == -1
    assert lib.kvq_lse_merge(fake, fake, 1, fake, 1, 8, 8, fake, 9, None, None) == -1
    assert b"dtype" in lib.kvq_last_error()
    for st in (0, -1, -2, -3, -4, -5, 7):
        assert kvq.status_string(st)


def test_plan_splits_class_cost_shares_a_head_count(kvq):
    """A head's count is shared by tokens x class cost, largest remainders first."""
    rng = _ranges([(0, 0, 0, 0, 640), (0, 0, 1, 640, 960)], kvq)   # 640 INT2 + 320 INT4 tokens
    sph = np.array([9], np.int32)
    s, _ = kvq.plan_splits(rng, 1, 1, 1, splits_per_head=sph, class_cost=[1.0, 1.0, 1.0])
    assert [int((s[:, 2] == c).sum()) for c in (0, 1)] == [6, 3]     # 1 + 7*2/3, 1 + 7/3 -> 5.67, 3.33
    s, _ = kvq.plan_splits(rng, 1, 1, 1, splits_per_head=sph, class_cost=[1.0, 2.0, 1.0])
    assert [int((s[:, 2] == c).sum()) for c in (0, 1)] == [5, 4]     # 1 + 3.5, 1 + 3.5 -> 4.5, 4.5
    with pytest.raises(kvq.KvqError):
        kvq.plan_splits(rng, 1, 1, 1, splits_per_head=sph, class_cost=[1.0, 0.0, 1.0])


def test_plan_splits_per_kernel(kvq):
    """Per (table, head): the INT2 / INT4 ranges share int_splits by tokens x cost and
    the FP16 ranges share fp16_splits by tokens, each at least one piece per range;
    every range covered exactly once; with no FP16 range it is kvq_plan_splits."""
    items = [(0, 0, 1, 0, 6000), (0, 0, 2, 6000, 6320), (0, 0, 2, 6336, 6400),       # INT4, VL, window
             (0, 1, 0, 0, 640), (0, 1, 1, 640, 960), (0, 1, 2, 960, 1000)]
    rng = _ranges(items, kvq)
    s, off = kvq.plan_splits_per_kernel(rng, 1, 2, 2, np.array([5, 9], np.int32), np.array([3, 2], np.int32),
                                        class_cost=[1.0, 1.0, 1.0])
    count = lambda h, c: int(((s[:, 1] == h) & (s[:, 2] == c)).sum())  # noqa: E731
    assert count(0, 1) == 5 and count(0, 2) == 3          # 320 + 64 FP16 tokens: 1 + 2 * 320 / 384 -> 2 + 1
    assert [len(s[(s[:, 1] == 0) & (s[:, 3] >= 6000) & (s[:, 4] <= 6320)]),
            len(s[(s[:, 1] == 0) & (s[:, 3] >= 6336)])] == [2, 1]
    assert count(1, 0) == 6 and count(1, 1) == 3 and count(1, 2) == 2   # 640 / 320 INT2 / INT4; one FP16 range
    for (t, h, c, b, e) in items:
        mine = s[(s[:, 1] == h) & (s[:, 2] == c) & (s[:, 3] >= b) & (s[:, 4] <= e)]
        assert mine[0, 3] == b and mine[-1, 4] == e and np.all(mine[1:, 3] == mine[:-1, 4])
    assert off.tolist() == [0, 8, 8 + 11]
    no16 = _ranges([it for it in items if it[2] != 2], kvq)
    a, oa = kvq.plan_splits_per_kernel(no16, 1, 2, 2, np.array([5, 9], np.int32), np.array([3, 2], np.int32))
    b, ob = kvq.plan_splits(no16, 1, 2, 2, splits_per_head=np.array([5, 9], np.int32))
    assert np.array_equal(a, b) and np.array_equal(oa, ob)
    with pytest.raises(kvq.KvqError):
        kvq.plan_splits_per_kernel(_ranges([(0, 0, 0, 0, 40)], kvq), 1, 1, 1, [1], [1])


def test_balanced_split_counts_minimal_cap(kvq):
    """Counts fit the work groups, and no smaller cap on one piece's work would."""
    r = np.random.default_rng(8)
    work = r.integers(300, 120000, 512).astype(np.int64)
    work[::37] = 0
    total = 3072
    out = kvq.balanced_split_counts(work, total)
    assert out.sum() <= total and np.array_equal(out == 0, work == 0)
    live = work > 0
    cap = int(np.max(-(-work[live] // out[live])))          # the longest piece
    assert int(np.sum(-(-work[live] // (cap - 1)))) > total  # one less does not fit
    same = kvq.balanced_split_counts(np.full(128, 4096, np.int64), 3072)
    assert np.all(same == 24)
    few = kvq.balanced_split_counts(np.array([5, 0, 7, 9], np.int64), 2)   # more entries than groups
    assert few.tolist() == [1, 0, 1, 1]
    with pytest.raises(kvq.KvqError):
        kvq.balanced_split_counts(np.array([3, -1], np.int64), 4)


def test_plan_balanced_counts_follow_cost_weighted_work(kvq):
    """kvq_plan_balanced: a head's split count is the balanced count of its tokens x class
    cost (in 1/256 token units), its pieces are kvq_plan_splits' pieces for that count,
    equal heads get equal counts, and the default INT4 weight is 0.82 only for 4 < g <= 8."""
    rng = np.random.default_rng(11)
    batch, hkv, hpp = 4, 2, 2
    items = []
    for t in range(batch * hkv // hpp):
        for h in range(hpp):
            n2 = 32 * int(rng.integers(0, 200))
            n4 = int(rng.integers(0, 5000))
            if n2:
                items.append((t, h, 0, 0, n2))
            if n4:
                items.append((t, h, 1, n2, n2 + n4))
    ranges = _ranges(items, kvq)
    r = np.asarray(ranges).view(np.int32).reshape(-1, 5)
    for g, w4 in ((4, 1.0), (8, 0.82), (16, 1.0)):
        total = 40
        splits, offsets, sph = kvq.plan_balanced(ranges, batch, hkv, hpp, g, total)
        work = np.zeros(batch * hkv, np.int64)
        for t, h, c, b, e in r:
            work[t * hpp + h] += int(round(256.0 * (e - b) * (1.0 if c == 0 else w4)))
        assert np.array_equal(sph, kvq.balanced_split_counts(work, total))
        ref, ref_off = kvq.plan_splits(ranges, batch, hkv, hpp, splits_per_head=sph,
                                       class_cost=[1.0, w4, 6.0])
        assert np.array_equal(splits, ref) and np.array_equal(offsets, ref_off)
    # equal heads: equal counts, the same plan as a fixed count per head
    eq = _ranges([(t, h, 0, 0, 4096) for t in range(4) for h in range(2)], kvq)
    splits, offsets, sph = kvq.plan_balanced(eq, 4, 2, 2, 4, 64)
    ref, ref_off = kvq.plan_splits(eq, 4, 2, 2, splits_per_head=np.full(8, 8, np.int32))
    assert np.all(sph == 8) and np.array_equal(splits, ref) and np.array_equal(offsets, ref_off)
    # a long head gets more splits than a short one, in proportion
    two = _ranges([(0, 0, 1, 0, 30000), (0, 1, 1, 0, 10000)], kvq)
    _, _, sph = kvq.plan_balanced(two, 1, 2, 2, 4, 8)
    assert sph.tolist() == [6, 2]
    for bad in ((0, 8), (4, 0)):
        with pytest.raises(kvq.KvqError):
            kvq.plan_balanced(two, 1, 2, 2, *bad)


def test_wave_timeline_only_in_the_profiling_build(kvq):
    """The production library records no timeline: kvq_wave_timeline says UNSUPPORTED
    (no device call is made); the profiling build exports the same symbols."""
    with pytest.raises(kvq.KvqError) as e:
        kvq.wave_timeline(None)
    assert e.value.status == -2  # KVQ_ERR_UNSUPPORTED
    path = os.path.join(ROOT, "mixed_precision_quantized_amd", "libkvq_timeline.so")
    if os.path.exists(path):
        lib = ctypes.CDLL(path)
        for n in kvq.EXPORTED:
            assert hasattr(lib, n), n


def test_prefill_workspace_and_validation(kvq):
    """The prefill scratch size follows its region list (V^T and V-hat^T fp16, fp16 keep
    mask, line positions, per-tile line counts, gathered K and V^T, K codes as bf16,
    each 256-byte aligned); the entry points reject g outside {1, 2, 4, 8, 16}, n_max off
    64 and a short scratch before touching any pointer."""
    lib = kvq.raw_library()
    up = lambda x: (x + 255) // 256 * 256  # noqa: E731
    for batch, n_max, hkv in ((1, 64, 1), (2, 1024, 8), (3, 192, 2)):
        bh = batch * hkv
        want = 0
        for size in (bh * 128 * n_max * 2, bh * 128 * n_max * 2, bh * n_max * 2, bh * n_max * 4,
                     bh * (n_max // 64) * 4, bh * n_max * 128 * 2, bh * 128 * n_max * 2, bh * n_max * 128 * 2):
            want = up(want + size)
        assert lib.kvq_prefill_workspace_bytes(batch, n_max, hkv) == want
    assert lib.kvq_prefill_workspace_bytes(1, 100, 1) == 0
    assert lib.kvq_prefill_workspace_bytes(0, 64, 1) == 0
    fake = ctypes.c_void_p(0x1000)
    need = lib.kvq_prefill_workspace_bytes(1, 128, 2)

    def attn(hq=4, hkv=2, n_max=128, nbytes=need, dtype=1, out=fake):
        return lib.kvq_prefill_attn(fake, fake, dtype, 1, n_max, hq, hkv, fake, None, 16, fake, fake, nbytes, out,
                                    None, None)

    def prepare(hkv=2, n_max=128, nbytes=need, dtype=1, v=fake):
        return lib.kvq_prefill_prepare(fake, v, dtype, 1, n_max, hkv, fake, None, fake, fake, fake, fake, fake,
                                       nbytes, None, None)
    assert attn(hq=6, hkv=2) == -2              # g = 3
    assert attn(hq=64, hkv=2) == -2             # g = 32
    assert attn(hq=6, hkv=4) == -1              # hq % hkv != 0
    for call in (attn, prepare):
        assert call(n_max=100) == -1            # not a multiple of 64
        assert call(dtype=0) == -2              # fp32 inputs
        assert call(nbytes=need - 1) == -3      # scratch too small
        assert b"workspace" in lib.kvq_last_error()
    assert attn(out=None) == -1 and prepare(v=None) == -1
    odd = ctypes.c_void_p(0x1008)                     # 8-byte aligned only
    assert lib.kvq_prefill_attn(odd, fake, 1, 1, 128, 4, 2, fake, None, 16, fake, fake, need, fake, None,
                                None) == -1
    assert lib.kvq_prefill_prepare(fake, fake, 1, 1, 128, 2, fake, None, fake, fake, fake, fake,
                                   ctypes.c_void_p(0x1010), need, None, None) == -1   # workspace off 256
    assert b"aligned" in lib.kvq_last_error()


def test_plan_workers_shares_by_cost_and_caps(kvq):
    """Shared-window plan: a head's workers are shared among its ranges by tokens x cost
    (largest remainders, one at least each), an FP16 range gets one, no range more than
    its windows; every worker carries its group's range; groups are numbered in order."""
    r = _ranges([(0, 0, 0, 0, 640), (0, 0, 1, 640, 1000), (0, 0, 2, 1008, 1100), (0, 1, 1, 0, 96),
                 (1, 0, 1, 16, 17)], kvq)
    workers, groups, n_groups, offsets = kvq.plan_workers(r, 2, 2, 2, np.array([10, 50, 4, 4], np.int32))
    assert n_groups == 5
    # head (0, 0): 10 = 1 FP16 + 9 shared 640 : 360 -> 5 INT2, 4 INT4 (remainders .48 / .52)
    counts = np.bincount(groups, minlength=n_groups).tolist()
    assert counts == [5, 4, 1, 3, 1]          # (0, 1): 3 windows cap 50; (1, 0): one window
    for gi in range(n_groups):
        rows = workers[groups == gi]
        assert (rows == rows[0]).all()
    assert [tuple(workers[groups == gi][0]) for gi in range(n_groups)] == [tuple(x) for x in np.asarray(r).view(np.int32).reshape(-1, 5)]
    assert offsets.tolist() == [0, 10, 13, 14, 14]
    with pytest.raises(kvq.KvqError):
        kvq.plan_workers(r, 2, 2, 2, np.array([-1, 1, 1, 1], np.int32))
