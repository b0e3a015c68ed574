"""GPU parity: the HIP path (through the C ABI) against the CPU oracle, element by element.

Bars: packed codes, scales, zeros and reordered tables bit-exact; attention outputs
within 2e-3 by the per-row metric max_c |o - o_ref| / max_c |o_ref| on fp32 outputs
(the tolerance the target states), bf16 outputs within 2e-3 + 2^-8.  Sizes span
several pages, splits and ragged tails; the full-size Qwen3-8B-shaped workload is
checked on sampled requests."""
import numpy as np
import pytest
import torch

import synth
from harness import DeviceRun, OracleRun, row_metric

pytestmark = pytest.mark.gpu
TOL = 2e-3


def _say(*a):
    print("[gpu-parity]", *a, flush=True)


def _pools_equal(gpu, orc):
    for cls in range(3):
        g = gpu.cache.pool_bytes(cls).cpu().numpy()
        o = orc.cache.pool_bytes(cls)
        if not np.array_equal(g, o):
            bad = np.flatnonzero(g != o)
            raise AssertionError(f"class {cls}: {bad.size} bytes differ, first at {bad[:8]}")


def _check_case(name, make, plan_kw, reorder=True, out_dtype=torch.float32, compact=False, anchor_fp8=False):
    _say(name, plan_kw, "compacted" if compact else "", "fp8 anchors" if anchor_fp8 else "")
    wg, wo = make(), make()
    gpu = DeviceRun(wg, reorder=reorder, compact=compact, anchor_fp8=anchor_fp8)
    orc = OracleRun(wo, reorder=reorder, compact=compact, anchor_fp8=anchor_fp8)
    torch.cuda.synchronize()
    assert int(gpu.err.item()) == 0, f"device error bits {int(gpu.err.item())}"
    _pools_equal(gpu, orc)
    if compact:
        assert np.array_equal(gpu.tables.cpu().numpy(), orc.tables)
        assert np.array_equal(gpu.live_tokens.cpu().numpy(), orc.live_tokens)
    if wg.kind == synth.PAGES:
        assert np.array_equal(gpu.tables.cpu().numpy(), orc.tables)
        if reorder:
            assert np.array_equal(gpu.class_counts.cpu().numpy(), orc.class_counts)
    ref, ref_lse = orc.attend()
    splits, offsets = gpu.plan(**plan_kw)
    out, lse, _, _ = gpu.decode(splits, offsets, out_dtype=out_dtype)
    assert int(gpu.err.item()) == 0, f"device error bits {int(gpu.err.item())}"
    got = out.float().cpu().numpy()
    err = row_metric(ref, got)
    tol = TOL if out_dtype == torch.float32 else TOL + 2.0 ** -8
    _say(f"  {name}: {splits.shape[0]} splits, row error {err:.2e}")
    assert err <= tol, f"{name}: row error {err:.3e} > {tol}"
    fin = np.isfinite(ref_lse)
    assert np.array_equal(fin, np.isfinite(lse.cpu().numpy()))
    assert np.allclose(lse.cpu().numpy()[fin], ref_lse[fin], atol=1e-3, rtol=1e-4)
    return gpu, orc


def test_tiny_four_splits():
    _check_case("tiny", lambda: synth.tiny(), dict(tokens_per_split=[64, 64, 64]))


@pytest.mark.parametrize("plan", [dict(target_bytes=1 << 16), dict(target_bytes=1 << 20),
                                  dict(tokens_per_split=[32, 7, 7])])
def test_qwen3_8b_small(plan):
    _check_case("qwen3_8b 2x2048", lambda: synth.qwen3_8b(batch=2, n_tokens=2048), plan)


def test_qwen3_8b_bf16_output():
    _check_case("qwen3_8b bf16 out", lambda: synth.qwen3_8b(batch=1, n_tokens=1024),
                dict(target_bytes=1 << 16), out_dtype=torch.bfloat16)


def _scaled(q_factor=1.0, k_factor=1.0, channels=None):
    """The small Qwen3-8B-shaped case with its bf16 queries (all channels, or the given
    ones) and keys scaled."""
    def make():
        w = synth.qwen3_8b(batch=2, n_tokens=2048)
        q = w.q.float()
        if channels is None:
            q *= q_factor
        else:
            q[..., channels] *= q_factor
        w.q = q.to(torch.bfloat16)
        w.k = (w.k.float() * k_factor).to(torch.bfloat16)
        return w
    return make


@pytest.mark.parametrize("case", ["beyond_fp16", "outlier_channels", "below_fp16_normal"])
def test_query_magnitudes(case):
    """Queries are staged as fp16 after a power-of-two scaling per row: queries beyond
    fp16's range (every channel x 1e5), four outlier channels x 3e4 beside ordinary ones,
    and queries in fp16's subnormal range (x 2^-16, keys x 2^10 so that the logits still
    matter) all stay within the bar."""
    make = {"beyond_fp16": _scaled(1e5),
            "outlier_channels": _scaled(3e4, channels=[3, 40, 77, 120]),
            "below_fp16_normal": _scaled(2.0 ** -16, 2.0 ** 10)}[case]
    _check_case(f"q {case}", make, dict(target_bytes=1 << 16))


def test_qwen3_8b_unreordered_table():
    """Mixed-class page order without the phase-1 reorder: many short pure ranges."""
    _check_case("qwen3_8b no reorder", lambda: synth.qwen3_8b(batch=1, n_tokens=1024),
                dict(target_bytes=1 << 16), reorder=False)


def test_hybrid_anchor_small():
    _check_case("hybrid 2x4096", lambda: synth.hybrid_anchor(batch=2, n_tokens=4096),
                dict(target_bytes=1 << 17))


def test_hybrid_anchor_fp8_small():
    """FP8 anchors (e4m3 codes, a power-of-two scale per token and head): anchor blocks
    bit-exact with the oracle, decode within the bar over the dequantized anchors."""
    _check_case("hybrid fp8 2x4096", lambda: synth.hybrid_anchor(batch=2, n_tokens=4096),
                dict(target_bytes=1 << 17), anchor_fp8=True)


def test_ragged_dead_small():
    def plan_for(w):
        from mixed_precision_quantized_amd import kvq
        return dict(splits_per_head=kvq.aot_split_counts(w.head_budget, w.batch, 64))
    make = lambda: synth.ragged_dead(batch=4, lo=512, hi=4096)  # noqa: E731
    _check_case("ragged 4", make, plan_for(make()))


@pytest.mark.parametrize("plan", ["aot", "tokens"])
def test_ragged_dead_small_compacted(plan):
    """The same ragged slot maps compacted ahead of time (dead entries dropped, each
    head reading its live count): tables and counts bit-exact, attention within TOL."""
    from mixed_precision_quantized_amd import kvq
    make = lambda: synth.ragged_dead(batch=4, lo=512, hi=4096)  # noqa: E731
    w = make()
    if plan == "aot":
        kw = dict(splits_per_head=kvq.aot_split_counts(w.head_budget, w.batch, 64))
    else:
        kw = dict(tokens_per_split=[512, 512, 512])
    _check_case("ragged 4", make, kw, compact=True)


def test_slot_compaction_edges():
    """Compaction alone on crafted tables: several 256-entry batches and a ragged tail,
    an all-dead table, empty prefixes, no dead entry; a prefix longer than its table is
    reported and leaves that table untouched."""
    from mixed_precision_quantized_amd import kvq
    from oracle import oracle
    r = np.random.default_rng(3)
    H, sentinel, me = 2, 16, 1000
    n = np.array([1000, 37, 64, 0, 300, 5], np.int32)
    tabs = (32 + r.integers(0, 5000, (len(n), me))).astype(np.int32)
    for t, frac in enumerate([0.2, 1.0, 0.5, 0.0, 0.0, 0.6]):
        dead = r.random(me) < frac
        tabs[t, dead] = sentinel
    ht = np.array([[1000, 517], [37, 0], [64, 63], [0, 0], [300, 300], [1, 5]], np.int32)
    cache = kvq.Cache(H, (0, 400, 0), "cuda", sentinel_slot=sentinel)
    ocache = oracle.Cache(H, 0, 400, 0, sentinel_slot=sentinel)
    for bad in (False, True):
        h2 = ht.copy()
        if bad:
            h2[4, 1] = 301  # beyond n_entries of table 4
        dt = torch.as_tensor(tabs, device="cuda").contiguous()
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        live = kvq.compact_slots(cache, dt, torch.as_tensor(n, device="cuda"),
                                 torch.as_tensor(h2, device="cuda").contiguous(), dev_err=err)
        torch.cuda.synchronize()
        got, got_live = dt.cpu().numpy(), live.cpu().numpy()
        if not bad:
            ot = tabs.copy()
            ol = ocache.compact_slots(ot, n, h2)
            assert int(err.item()) == 0
            assert np.array_equal(got, ot) and np.array_equal(got_live, ol)
        else:
            assert int(err.item()) == kvq.DEVERR_RANGE
            assert np.array_equal(got[4], tabs[4])   # the bad table is left as it was
            good = [0, 1, 2, 3, 5]
            ot = np.ascontiguousarray(tabs[good])
            ol = ocache.compact_slots(ot, n[good], np.ascontiguousarray(ht[good]))
            assert np.array_equal(got[good], ot) and np.array_equal(got_live[good], ol)


def test_g8_and_g1_heads():
    """g = 8 (Qwen3-VL-32B GQA ratio) and g = 1 (MHA) on the same cache layout."""
    for hq in (64, 8):
        def make(hq=hq):
            w = synth.qwen3_8b(batch=1, n_tokens=1024)
            w.hq = hq
            w.q = synth._bf16(synth.randn((1, hq, 128), 2, 77))
            return w
        _check_case(f"g={hq // 8}", make, dict(target_bytes=1 << 16))


def _with_ratio(w, g, seed):
    """The workload with g query heads per KV head (bf16 queries of the new shape)."""
    w.hq = g * w.hkv
    w.q = synth._bf16(synth.randn((w.batch, w.hq, 128), seed, 78))
    return w


@pytest.mark.parametrize("g", [2, 16])
def test_gqa_ratios_every_kernel(g):
    """g = 2 and g = 16 through every decode kernel: INT2 / INT4 pages (LDS-staged, two
    waves per split at g = 16), FP16 anchor pages (register-staged, four query tiles at
    g = 16) and slot maps with dead entries (LDS-staged INT4 at g = 2, register-staged
    for every split at g = 16)."""
    _check_case(f"qwen3_8b g={g}", lambda: _with_ratio(synth.qwen3_8b(batch=1, n_tokens=1024), g, 5),
                dict(target_bytes=1 << 16))
    _check_case(f"hybrid g={g}", lambda: _with_ratio(synth.hybrid_anchor(batch=1, n_tokens=4096), g, 6),
                dict(target_bytes=1 << 16))

    def make():
        return _with_ratio(synth.ragged_dead(batch=2, lo=256, hi=1024), g, 7)
    from mixed_precision_quantized_amd import kvq
    _check_case(f"ragged g={g}", make,
                dict(splits_per_head=kvq.aot_split_counts(make().head_budget, 2, 64)))


def test_split_count_invariance_on_gpu():
    """Different split plans of the same cache agree to the parity tolerance (fp16 operand
    roundings depend on each split's running maximum, so agreement is not bitwise)."""
    wg = synth.qwen3_8b(batch=1, n_tokens=2048)
    gpu = DeviceRun(wg)
    outs = []
    for kw in (dict(target_bytes=1 << 30), dict(target_bytes=1 << 16), dict(tokens_per_split=[32, 1, 1])):
        s, o = gpu.plan(**kw)
        outs.append(gpu.decode(s, o)[0].cpu().numpy())
        _say("split plan", kw, s.shape[0])
    for o in outs[1:]:
        assert row_metric(outs[0], o) < TOL


def test_edge_cases_empty_dead_single():
    """Empty split, all-dead split, single-token split, and a (b, head) with no split."""
    wg = synth.ragged_dead(batch=2, lo=64, hi=128)
    gpu = DeviceRun(wg)
    w = gpu.w
    sentinel = w.sentinel_slot
    tab = gpu.tables.cpu().numpy()
    tab[0, :5] = sentinel                                     # first 5 entries of table 0 dead
    live = int(np.flatnonzero(tab[0, 5:] != sentinel)[0]) + 5
    gpu.tables.copy_(torch.as_tensor(tab))
    splits = np.array([[0, 0, 1, 0, 0],                       # empty
                       [0, 0, 1, 0, 5],                       # all dead
                       [0, 0, 1, live, live + 1],             # one live token
                       [0, 1, 1, live, live + 3]], np.int32)  # head 1 of the group
    offsets = np.zeros(w.batch * w.hkv + 1, np.int32)
    offsets[1:] = 3
    offsets[2:] = 4
    out, lse, po, pl = gpu.decode(splits, offsets)
    po, pl = po.cpu().numpy(), pl.cpu().numpy()
    assert int(gpu.err.item()) == 0
    assert not po[0].any() and np.all(np.isneginf(pl[0]))
    assert not po[1].any() and np.all(np.isneginf(pl[1]))
    orc = OracleRun(synth.ragged_dead(batch=2, lo=64, hi=128))
    o_tab = orc.tables.copy()
    o_tab[0, :5] = sentinel
    ref, ref_lse = orc.cache.attend_ranges(orc.q, w.batch, w.hq, w.hkv, o_tab, orc.kind,
                                           synth.ranges_array([tuple(r) for r in splits]))
    assert row_metric(ref[2], po[2]) <= TOL and row_metric(ref[3], po[3]) <= TOL
    assert np.allclose(pl[2:], ref_lse[2:], atol=1e-4)
    o = out.cpu().numpy()
    assert not o[1].any()                                     # request 1 has no split at all
    assert np.all(np.isneginf(lse.cpu().numpy()[1]))


def test_bad_device_data_is_reported_not_faulted():
    """Out-of-range split / page ids set dev_err bits; the kernels stay in bounds."""
    wg = synth.tiny()
    gpu = DeviceRun(wg)
    splits = np.array([[5, 0, 1, 0, 16],        # table out of range
                       [0, 0, 0, 0, 10],        # INT2 range not on 32-token pairs
                       [0, 0, 1, 0, 1 << 20]], np.int32)   # past the table
    offsets = np.array([0, 3], np.int32)
    out, lse, po, pl = gpu.decode(splits, offsets)
    assert int(gpu.err.item()) & 8
    assert not po.cpu().numpy().any() and np.all(np.isneginf(pl.cpu().numpy()))
    gpu.err.zero_()
    tab = gpu.tables.clone()
    gpu.tables[0, 0] = 10 ** 6                   # page id outside every pool
    out, lse, po, pl = gpu.decode(*gpu.plan(tokens_per_split=[64, 64, 64]))
    assert int(gpu.err.item()) & 1
    gpu.tables.copy_(tab)


def _resident_plan(gpu, ragged_plan="aot"):
    """The benchmark's plan: one split per resident work group of the decode kernel,
    shared among heads by budget (Tangram AOT) for ragged workloads, or (ragged_plan
    "tokens") by balanced split counts over the tokens each head reads."""
    w = gpu.w
    per_cu, n_cu = gpu.kvq.decode_occupancy(w.g, gpu.kvq.TABLE_SLOTS if w.kind == synth.SLOTS else 0)
    if w.kind == synth.PAGES and w.n_pages[2]:  # one round of each of the two kernels
        per16, _ = gpu.kvq.decode_fp16_occupancy(w.g, gpu.cache.anchor_fp8)
        heads = w.batch * w.hkv
        return gpu.kvq.plan_splits_per_kernel(gpu.ranges, w.batch, w.hkv, w.heads_per_page,
                                              max(1, per_cu * n_cu // heads), max(1, per16 * n_cu // heads))
    if w.head_tokens is not None and ragged_plan == "tokens":
        read = w.head_tokens if gpu.live_tokens is None else gpu.live_tokens.cpu().numpy()
        return gpu.plan(splits_per_head=gpu.kvq.balanced_split_counts(read, per_cu * n_cu))
    if w.head_budget is not None:
        return gpu.plan(splits_per_head=gpu.kvq.aot_split_counts(w.head_budget, w.batch, per_cu * n_cu))
    splits, offsets, _ = gpu.kvq.plan_balanced(gpu.ranges, w.batch, w.hkv, w.heads_per_page, w.g, per_cu * n_cu)
    return splits, offsets


def _full_size_sampled(name, make, requests, compact=False, ragged_plan="aot"):
    """Full-size workload with the benchmark's plan on the GPU; the oracle recomputes
    the sampled requests from the same seeded sources (slot maps: uncompacted)."""
    _say(f"full-size {name}: generating on the GPU" + (" (compacted slot maps)" if compact else "")
         + f", {ragged_plan} plan")
    w = make()
    gpu = DeviceRun(w, compact=compact)
    splits, offsets = _resident_plan(gpu, ragged_plan)
    out, lse, _, _ = gpu.decode(splits, offsets)
    assert int(gpu.err.item()) == 0
    _say(f"  {w.note}; {splits.shape[0]} splits decoded; oracle on requests {requests}")
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    del gpu, w
    ref, ref_lse = OracleRun(synth.subset(make(), requests)).attend()
    err = row_metric(ref, out[requests])
    _say(f"  sampled row error {err:.2e}")
    assert err <= TOL
    assert np.allclose(lse[requests], ref_lse, rtol=0, atol=1e-3)


def _full_size_full(name, make, compact=False, ragged_plan="aot"):
    """A full-size workload on both sides, each from its own seeded copy, with the
    benchmark's plan on the GPU: every pool byte, the tables (and class counts or live
    counts) bit-exact, and every request's rows against the oracle."""
    _say(f"full-size {name}: generating on the GPU" + (" (compacted slot maps)" if compact else "")
         + f", {ragged_plan} plan, compared in full")
    gpu = DeviceRun(make(), compact=compact)
    orc = OracleRun(make(), compact=compact)
    torch.cuda.synchronize()
    assert int(gpu.err.item()) == 0
    _pools_equal(gpu, orc)
    assert np.array_equal(gpu.tables.cpu().numpy(), orc.tables)
    if gpu.w.kind == synth.PAGES:
        assert np.array_equal(gpu.class_counts.cpu().numpy(), orc.class_counts)
    if compact:
        assert np.array_equal(gpu.live_tokens.cpu().numpy(), orc.live_tokens)
    _say(f"  {gpu.w.note}; pools (every byte) and tables bit-exact")
    splits, offsets = _resident_plan(gpu, ragged_plan)
    out, lse, _, _ = gpu.decode(splits, offsets)
    assert int(gpu.err.item()) == 0
    ref, ref_lse = orc.attend(n_threads=16)
    err = row_metric(ref, out.cpu().numpy())
    _say(f"  {splits.shape[0]} splits decoded; row error over all {gpu.w.batch} requests {err:.2e}")
    assert err <= TOL
    assert np.allclose(lse.cpu().numpy(), ref_lse, rtol=0, atol=1e-3)


def test_full_size_hybrid_anchor():
    """FP16 anchors at full size (32 requests x 8 heads x 65536 tokens, INT4 prefix and
    FP16 vertical-line / staging / window segments; two launches, INT4 and FP16) against
    the oracle in full: every pool byte, the reordered tables and class counts, and the
    rows of all 32 requests."""
    _full_size_full("hybrid_anchor", lambda: synth.hybrid_anchor(device="cuda"))


def test_full_size_ragged_dead_sampled():
    """Ragged slot maps with 20 % dead slots at full size (64 requests, 4K-128K tokens),
    budget-proportional split counts; a short and a long request sampled."""
    lens = synth.ragged_lengths()
    pick = sorted({int(np.argmin(lens)), int(np.argmax(lens))})
    _full_size_sampled("ragged_dead", lambda: synth.ragged_dead(device="cuda"), pick)


def test_full_size_ragged_dead_compacted_sampled():
    """The same full-size ragged workload with its slot maps compacted (the benchmark's
    default for slot maps), sampled requests against the uncompacted oracle."""
    lens = synth.ragged_lengths()
    pick = sorted({int(np.argmin(lens)), int(np.argmax(lens))})
    _full_size_sampled("ragged_dead", lambda: synth.ragged_dead(device="cuda"), pick, compact=True)


def test_full_size_ragged_dead_balanced():
    """The full-size ragged workload (64 requests, 4K-128K tokens, 20 % dead slots),
    compacted, under balanced split counts over the tokens each head reads (the
    benchmark's plan), against the oracle in full: every pool byte, the compacted slot
    maps and live counts, and the rows of all 64 requests."""
    _full_size_full("ragged_dead", lambda: synth.ragged_dead(device="cuda"), compact=True, ragged_plan="tokens")


def test_qwen3_vl_agentic_small():
    """g = 8 (Qwen3-VL-32B GQA ratio) over tagged multi-turn contexts appended in
    4096-token calls (an INT4 residual per call), full oracle comparison."""
    make = lambda: synth.qwen3_vl_agentic(batch=2, lo=9000, hi=12000, chunk=4096)  # noqa: E731
    _check_case("qwen3_vl_agentic 2 x ~10K", make, dict(splits_per_head=np.full(16, 5, np.int32)))


def test_full_size_qwen3_vl_agentic():
    """The agentic workload at full size (8 requests of 64K-128K tokens, g = 8, flags from
    each side's own tags and widths) with the resident-wave plan, against the oracle in
    full: every pool byte, the reordered tables and class counts, all 8 requests' rows."""
    _say("full-size qwen3_vl_agentic: generating on the GPU")
    gpu = DeviceRun(synth.qwen3_vl_agentic(device="cuda"))
    orc = OracleRun(synth.qwen3_vl_agentic(device="cuda"))
    torch.cuda.synchronize()
    assert int(gpu.err.item()) == 0
    assert all(np.array_equal(x, y) for x, y in zip(gpu.flags, orc.flags))
    _pools_equal(gpu, orc)
    assert np.array_equal(gpu.tables.cpu().numpy(), orc.tables)
    assert np.array_equal(gpu.class_counts.cpu().numpy(), orc.class_counts)
    _say(f"  {gpu.w.note}; flags, pools (every byte), tables and class counts bit-exact")
    splits, offsets = _resident_plan(gpu)
    out, lse, _, _ = gpu.decode(splits, offsets)
    assert int(gpu.err.item()) == 0
    ref, ref_lse = orc.attend(n_threads=16)
    err = row_metric(ref, out.cpu().numpy())
    _say(f"  {splits.shape[0]} splits decoded; row error over all 8 requests {err:.2e}")
    assert err <= TOL
    assert np.allclose(lse.cpu().numpy(), ref_lse, rtol=0, atol=1e-3)


def test_full_size_qwen3_8b():
    """The benchmark's workload (16 x 32768 tokens, 8 KV heads, g = 4) and split plan
    against the oracle in full: every pool byte, the reordered tables and their class
    counts bit-exact, and the attention rows of all 16 requests within the bar."""
    _say("full-size qwen3_8b: generating on the GPU")
    gpu = DeviceRun(synth.qwen3_8b(device="cuda"))
    orc = OracleRun(synth.qwen3_8b(device="cuda"))
    torch.cuda.synchronize()
    assert int(gpu.err.item()) == 0
    _pools_equal(gpu, orc)
    assert np.array_equal(gpu.tables.cpu().numpy(), orc.tables)
    assert np.array_equal(gpu.class_counts.cpu().numpy(), orc.class_counts)
    _say("  pools (every byte), tables and class counts bit-exact")
    splits, offsets = _resident_plan(gpu)
    out, lse, _, _ = gpu.decode(splits, offsets)
    assert int(gpu.err.item()) == 0
    ref, ref_lse = orc.attend(n_threads=16)
    err = row_metric(ref, out.cpu().numpy())
    _say(f"  {splits.shape[0]} splits decoded; row error over all 16 requests {err:.2e}")
    assert err <= TOL
    assert np.allclose(lse.cpu().numpy(), ref_lse, rtol=0, atol=1e-3)


def test_graph_replay_matches_eager():
    """Decode + merge captured as one HIP graph (as the benchmark replays it): three
    replays, each after eager launches and a synchronization, equal the eager result
    bit for bit and the oracle within the tolerance."""
    w = synth.qwen3_8b(batch=2, n_tokens=2048)
    gpu = DeviceRun(w, reorder=True)
    orc = OracleRun(synth.qwen3_8b(batch=2, n_tokens=2048), reorder=True)
    ref, _ = orc.attend()
    kvq = gpu.kvq
    splits, offsets = gpu.plan(target_bytes=1 << 16)
    n = splits.shape[0]
    sp = torch.as_tensor(splits, device="cuda").contiguous()
    off = torch.as_tensor(offsets, device="cuda")
    part_o = torch.empty((n, w.g, 128), dtype=torch.float32, device="cuda")
    part_lse = torch.empty((n, w.g), dtype=torch.float32, device="cuda")
    out = torch.empty((w.batch, w.hq, 128), dtype=torch.float32, device="cuda")
    stream = torch.cuda.Stream()

    def bind():
        d = kvq.bind_decode_attn(gpu.cache, gpu.q, w.hkv, gpu.tables, kvq.TABLE_PAGES, sp, part_o, part_lse,
                                 dev_err=gpu.err, stream=stream)
        m = kvq.bind_lse_merge(part_o, part_lse, n, off, w.batch, w.hq, w.hkv, out, stream=stream)
        return lambda: (d(), m())

    run = bind()
    with torch.cuda.stream(stream):
        run()
    torch.cuda.synchronize()
    eager = out.clone()
    assert row_metric(ref, eager.cpu().numpy()) <= TOL
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        run()
    torch.cuda.synchronize()
    for r in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {r} differs from the eager result"
        with torch.cuda.stream(stream):
            run()
        torch.cuda.synchronize()
    assert int(gpu.err.item()) == 0


@pytest.mark.parametrize("fp8", [False, True])
def test_slot_map_anchors(fp8):
    """Anchor tokens reached through a slot map (one head-group table holding 2 KV heads,
    slots shuffled over the anchor pages, sentinel entries among them), FP16 and FP8
    anchors: the anchor blocks bit-exact with the oracle, both heads' splits within the
    bar."""
    from mixed_precision_quantized_amd import kvq
    from oracle import oracle
    H, g, T, n_pages = 2, 4, 150, 12
    hkv, hq = H, H * g
    sentinel = n_pages * 16 - 1
    _say("slot-map anchors", "fp8" if fp8 else "fp16")
    r = np.random.default_rng(21)
    k = r.standard_normal((T, H, 128)).astype(np.float32)
    k[:, :, 9] *= 20.0
    v = r.standard_normal((T, H, 128)).astype(np.float32)
    slots = r.permutation(sentinel)[:T].astype(np.int32)
    cache = kvq.Cache(H, (0, 0, n_pages), "cuda", sentinel_slot=sentinel, anchor_fp8=fp8)
    ocache = oracle.Cache(H, 0, 0, n_pages, sentinel_slot=sentinel, anchor_fp8=fp8)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    kvq.quantize_append(cache, torch.as_tensor(k, device="cuda"), torch.as_tensor(v, device="cuda"),
                        rows16=torch.arange(T, dtype=torch.int32, device="cuda"),
                        slots16=torch.as_tensor(slots, device="cuda"), dev_err=err)
    ocache.append(k, v, oracle.F32, H * 128, 128, rows16=np.arange(T, dtype=np.int32), slots16=slots)
    ocache.append(np.zeros((1, H, 128), np.float32), np.zeros((1, H, 128), np.float32), oracle.F32, H * 128, 128,
                  rows16=np.zeros(1, np.int32), slots16=np.array([sentinel], np.int32))
    kvq.quantize_append(cache, torch.zeros((1, H, 128), device="cuda"), torch.zeros((1, H, 128), device="cuda"),
                        rows16=torch.zeros(1, dtype=torch.int32, device="cuda"),
                        slots16=torch.full((1,), sentinel, dtype=torch.int32, device="cuda"), dev_err=err)
    entries = list(slots)
    for at in sorted(r.choice(T, 6, replace=False), reverse=True):
        entries.insert(int(at), sentinel)                     # dead entries among the live ones
    table = np.array([entries], np.int32)
    L = table.shape[1]
    splits = np.array([[0, 0, 2, 0, L], [0, 1, 2, 0, L], [0, 0, 2, 7, 61]], np.int32)
    q = r.standard_normal((1, hq, 128)).astype(np.float32)
    part_o = torch.empty((3, g, 128), dtype=torch.float32, device="cuda")
    part_lse = torch.empty((3, g), dtype=torch.float32, device="cuda")
    kvq.decode_attn(cache, torch.as_tensor(q, device="cuda"), hkv, torch.as_tensor(table, device="cuda"),
                    kvq.TABLE_SLOTS, torch.as_tensor(splits, device="cuda"), part_o, part_lse, dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    assert np.array_equal(cache.pool_bytes(2).cpu().numpy(), ocache.pool_bytes(2))
    ref, ref_lse = ocache.attend_ranges(q, 1, hq, hkv, table, oracle.SLOTS,
                                        synth.ranges_array([tuple(s) for s in splits]))
    got = part_o.cpu().numpy()
    e = max(row_metric(ref[i], got[i]) for i in range(3))
    _say(f"  slot-map anchors ({'fp8' if fp8 else 'fp16'}): row error {e:.2e}")
    assert e <= TOL
    assert np.allclose(part_lse.cpu().numpy(), ref_lse, atol=1e-3, rtol=1e-4)


def test_reorder_at_the_entry_limit():
    """kvq_reorder_pages at its limit of 32,768 entries per table (a 128 KB LDS stage):
    tables of 32,768, 32,767, 1 and 0 entries mixing INT2 page pairs, INT4 and FP16
    pages, bit-exact with the oracle's stable partition and class counts; one entry
    more is rejected before any launch."""
    from mixed_precision_quantized_amd import kvq
    from oracle import oracle
    limit = 32768
    rng = np.random.default_rng(41)
    n2, n4, n16 = 2 * 6000, 9000, 3000
    tabs = np.full((4, limit), -1, np.int32)
    fill = [limit, limit - 1, 1, 0]
    for t, n in enumerate(fill):
        row = []
        while len(row) < n:
            kind = rng.integers(0, 3) if n - len(row) >= 2 else rng.integers(1, 3)
            if kind == 0:  # an INT2 page pair, its two pages one after the other
                p = 2 * int(rng.integers(0, n2 // 2))
                row += [p, p + 1]
            elif kind == 1:
                row.append(n2 + int(rng.integers(0, n4)))
            else:
                row.append(n2 + n4 + int(rng.integers(0, n16)))
        tabs[t, :n] = row
    n_entries = np.array(fill, np.int32)
    orc_tabs = tabs.copy()
    orc_counts = oracle.Cache(1, n2, n4, n16).reorder(orc_tabs, n_entries)
    cache = kvq.Cache(1, (n2, n4, n16), "cuda")
    g_tabs = torch.as_tensor(tabs, device="cuda").contiguous()
    g_n = torch.as_tensor(n_entries, device="cuda")
    counts = torch.zeros((4, 3), dtype=torch.int32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    kvq.reorder_pages(cache, g_tabs, g_n, counts, dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    assert np.array_equal(g_tabs.cpu().numpy(), orc_tabs)
    assert np.array_equal(counts.cpu().numpy(), orc_counts)
    _say(f"reorder at {limit} entries per table: tables and counts bit-exact {orc_counts[0].tolist()}")
    wide = torch.full((1, limit + 1), n2, dtype=torch.int32, device="cuda")
    with pytest.raises(kvq.KvqError):
        kvq.reorder_pages(cache, wide, torch.ones(1, dtype=torch.int32, device="cuda"), dev_err=err)


def test_reorder_and_decode_past_131072_tokens():
    """A request of 163,840 tokens (a 128K prompt plus 32K generated tokens; 10,240
    table entries, past the 8,192 a 64 KB LDS stage holds): the reordered table and its
    class counts bit-exact with the oracle, the decode within the bar."""
    make = lambda: synth.qwen3_8b(batch=1, n_tokens=163840)  # noqa: E731
    gpu, orc = _check_case("qwen3_8b 1 x 163840", make, dict(splits_per_head=np.full(8, 24, np.int32)))
    assert int(gpu.w.alloc.n_entries[0]) == 10240
