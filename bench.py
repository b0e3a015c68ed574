#!/usr/bin/env python3
"""Decode-attention benchmark on one MI355X.

Default workload (the metric's): Qwen3-8B-shaped decode step over a mixed INT2 / INT4
paged KV cache: batch 16, Hq 32 / Hkv 8 (g = 4), d 128, 32768 tokens per request (70 %
INT2 / 30 % INT4 in shuffled 32-token units, INT2-first reorder), 16-token pages, bf16
q and output, 36 layers each with its own pools (17.4 GB in total, so no layer is
served from the 256 MB Infinity Cache).  A step = split-K decode + log-sum-exp merge
for every layer.  Inputs are resident in HBM before timing starts.

--workload also times the other synthetic workloads (agentic g = 8, FP16 anchors,
ragged slot maps with dead slots) with the same columns, on fewer layers by default.

Prints ONE JSON line: effective KV GB/s of the whole step (algorithmic bytes: packed
codes + fp16 scale/zero of every live token-head, 4 B per table entry, q and the
output), us per step, the roofline of the decode kernel and the CPU oracle's rate on a
bounded sample of the same workload."""
import argparse
import functools
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)
sys.path.insert(1, os.path.join(ROOT, "tests"))

HBM_PEAK_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_qwen3_8b_traffic.md")
PREFILL_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "prefill_llama8b_16k_traffic.md")
PREFILL_SOURCES = ("kvq_prefill.hip", "kvq_internal.h")
CPU_SECONDS = 10.0  # lower bound on the timed oracle work

# name: (metric suffix, default layers, description)
WORKLOADS = {
    "qwen3_8b": ("Qwen3-8B shape @32K", 36,
                 "Qwen3-8B-shaped decode: batch 16, Hq 32 / Hkv 8, d 128, 32768 tokens per request, "
                 "70% INT2 / 30% INT4, 16-token pages"),
    "qwen3_vl_agentic": ("Qwen3-VL-32B agentic shape @64K-128K", 8,
                         "Qwen3-VL-32B-shaped agentic decode: batch 8, Hq 64 / Hkv 8, d 128, "
                         "65536-131072 tokens per request, tri-axis tags at 2.6 bits, 8192-token appends"),
    "hybrid_anchor": ("Llama-3.1-8B hybrid FP16-anchor shape @64K", 4,
                      "Llama-3.1-8B-shaped hybrid decode: batch 32, Hq 32 / Hkv 8, one table per "
                      "(request, head), 65536 tokens: INT4 prefix + FP16 vertical lines, staging, window"),
    "ragged_dead": ("ragged head-group slot maps with dead slots", 8,
                    "ragged decode: batch 64, Hq 32 / Hkv 8, lengths 4K-128K, per-head budgets "
                    "0.1-1.0, 2-head slot-map tables, 20% dead slots, INT4"),
}


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def effective_bytes(w, q_bytes_per_elem=2, out_bytes_per_elem=2, anchor_fp8=False):
    """Algorithmic bytes of one layer: live token-heads x (96 / 160 / 512 B; FP8 anchors
    260 B = 2 x (128 codes + 2 B scale)), 4 B per table entry, q and output; and the
    decode kernel's share (without the output)."""
    import numpy as np
    import synth
    per_tok = np.array([96, 160, 260 if anchor_fp8 else 512], np.int64)
    if w.kind == synth.PAGES:
        kv = int((w.alloc.tokens * per_tok).sum()) * w.heads_per_page
        tables = int(w.alloc.n_entries.sum()) * 4
    else:  # slot maps: each head reads its first head_tokens entries; dead ones move nothing
        live = 0
        for t in range(w.n_tables):
            dead = np.asarray(w.dead_entries[t])
            for h in range(w.heads_per_page):
                n = int(w.head_tokens[t, h])
                live += n - int((dead < n).sum())
        kv = live * int(per_tok[synth.INT4])
        tables = int(w.head_tokens.sum()) * 4
    q = w.batch * w.hq * 128 * q_bytes_per_elem
    return kv + tables + q + w.batch * w.hq * 128 * out_bytes_per_elem, kv + tables + q


def kernel_source_sha(files=("kvq_decode.hip", "kvq_internal.h")):
    """Hash of a kernel's source code (comments and layout ignored)."""
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "mixed_precision_quantized_amd", "csrc", f)) as fh:
            text = re.sub(r"/\*.*?\*/", " ", fh.read(), flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(path=None, files=("kvq_decode.hip", "kvq_internal.h")):
    """HBM bytes per launch from a committed rocprofv3 PMC summary (its line starting
    'bench-traffic:'), if it was taken on the current kernel source; else None."""
    try:
        with open(path or TRAFFIC_FILE) as f:
            for line in f:
                if line.startswith("bench-traffic:"):
                    t = json.loads(line.split(":", 1)[1])
                    break
            else:
                return None
    except (OSError, ValueError):
        return None
    if t.get("kernel_sha") != kernel_source_sha(files):
        return None
    return t.get("bytes_per_launch")


def resident_plan(gpu, kvq, synth, splits_per_head=0, class_cost=None, ragged_plan="aot"):
    """One work group per split, as many splits as the decode kernel keeps resident at
    once (a second, partial round would leave most of the chip idle); with FP16 pages,
    one round of each of the two kernels (kvq_plan_splits_per_kernel).  Ragged slot maps
    share the count among heads in proportion to their budgets (Tangram AOT), or, with
    ragged_plan="tokens", so that no piece holds more tokens than it must for the count
    to fit (balanced split counts over the tokens each head reads).  Page tables without
    FP16 pages get counts balanced over each head's tokens x class cost
    (kvq_plan_balanced)."""
    import numpy as np
    w = gpu.w
    kind = kvq.TABLE_SLOTS if w.kind == synth.SLOTS else kvq.TABLE_PAGES
    per_cu, n_cu = kvq.decode_occupancy(w.g, kind)
    if not splits_per_head and w.kind == synth.PAGES and w.n_pages[2]:
        # FP16 pages: the INT2 / INT4 splits and the FP16 splits run in two kernels; each
        # kernel gets one resident round of its own
        per16, _ = kvq.decode_fp16_occupancy(w.g, gpu.cache.anchor_fp8)
        heads = w.batch * w.hkv
        splits, offsets = kvq.plan_splits_per_kernel(gpu.ranges, w.batch, w.hkv, w.heads_per_page,
                                                     max(1, per_cu * n_cu // heads), max(1, per16 * n_cu // heads),
                                                     class_cost)
        return splits, offsets, per_cu, n_cu
    if splits_per_head:
        sph = np.full(w.batch * w.hkv, splits_per_head, np.int32)
    elif w.head_tokens is not None and ragged_plan == "tokens":
        read = w.head_tokens if getattr(gpu, "live_tokens", None) is None else gpu.live_tokens.cpu().numpy()
        sph = kvq.balanced_split_counts(read, per_cu * n_cu)  # no piece longer than needed to fit
    elif w.head_budget is not None:
        sph = kvq.aot_split_counts(w.head_budget, w.batch, per_cu * n_cu)
    else:
        # page tables: counts by each head's tokens x class cost, so that long requests
        # get more splits and one resident round ends together
        splits, offsets, _ = kvq.plan_balanced(gpu.ranges, w.batch, w.hkv, w.heads_per_page, w.g, per_cu * n_cu,
                                               class_cost)
        return splits, offsets, per_cu, n_cu
    splits, offsets = gpu.plan(splits_per_head=sph, class_cost=class_cost)
    return splits, offsets, per_cu, n_cu


def cpu_info():
    """(CPU model name, processors online, processors this process may run on)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        allowed = len(os.sched_getaffinity(0))
    except AttributeError:
        allowed = os.cpu_count() or 1
    return model, os.cpu_count() or 1, allowed


def cpu_baseline(cpu_sample, w0, args, make):
    """The oracle's decode timed on the host: whole passes over a sample of the layer
    for at least CPU_SECONDS, on all the cores this process may use (at most 16, the
    host share of one GPU) and on one thread over a smaller sample."""
    import synth
    from harness import OracleRun

    def leg(sample, n_threads):
        orc = OracleRun(sample, anchor_fp8=args.anchor_fp8)
        reps, t = 0, time.perf_counter()
        while True:
            orc.attend(n_threads=n_threads)
            reps += 1
            dt = time.perf_counter() - t
            if dt >= CPU_SECONDS:
                break
        nbytes, _ = effective_bytes(sample, anchor_fp8=args.anchor_fp8)
        return round(nbytes * reps / dt / 1e9, 3), reps, dt

    model, online, allowed = cpu_info()
    n_threads = min(16, allowed)
    multi, reps, dt = leg(cpu_sample, n_threads)
    one_req = list(range(max(1, cpu_sample.batch // 8)))
    single, reps1, dt1 = leg(synth.subset(make(device="cuda", layer=0), one_req, device="cpu"), 1)
    log(f"cpu oracle {multi} GB/s on {n_threads} threads ({dt:.1f} s), {single} GB/s on 1 thread ({dt1:.1f} s); "
        f"{model}, {online} processors online, {allowed} allowed")
    return {
        "value": multi,
        "unit": "GB/s",
        "cores": n_threads,
        "kind": "oracle",
        "sample": f"{cpu_sample.batch} of {w0.batch} requests of one layer (all {w0.hkv} KV heads, "
                  f"g = {w0.g}), fp64 two-pass softmax, {reps} passes in {dt:.1f} s",
        "single_thread": {"value": single, "unit": "GB/s", "cores": 1,
                          "sample": f"{len(one_req)} of {w0.batch} requests of one layer, {reps1} passes in "
                                    f"{dt1:.1f} s"},
        "cpu_model": model,
        "nproc": online,
        "affinity": allowed,
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", choices=sorted(WORKLOADS) + ["vl_select", "prefill"], default="qwen3_8b",
                    help="a decode workload; vl_select: vertical-line selection + FREEZE routing at the "
                         "hybrid-anchor prefill shape; prefill: INT8-prefix prefill attention")
    ap.add_argument("--prefill-tokens", type=int, default=16384, help="prompt length of the prefill workload")
    ap.add_argument("--anchor-fp8", action="store_true",
                    help="decode workloads: anchors (the FP16 class) stored as e4m3 codes with a power-of-two scale")
    ap.add_argument("--ordered-pages", action="store_true",
                    help="qwen3_8b: physical pages handed out in id order instead of shuffled")
    ap.add_argument("--layers", type=int, default=0, help="0 = the workload's default")
    ap.add_argument("--splits-per-head", type=int, default=0,
                    help="splits per (request, KV head); 0 = as many as the decode kernel keeps resident")
    ap.add_argument("--class-cost", default=None,
                    help="per-token decode cost INT2,INT4,FP16 for sharing splits (default: the library's)")
    ap.add_argument("--ragged-plan", choices=("aot", "tokens"), default="tokens",
                    help="split counts of ragged slot maps: balanced by the tokens each head reads, or by budget (Tangram AOT)")
    ap.add_argument("--cpu-requests", type=int, default=16, help="requests in the CPU-oracle sample")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run plain 1 GiB device copies (reference for HBM byte counters)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-compact", action="store_true",
                    help="slot maps: decode the tables as they are instead of dropping dead entries ahead of time")
    ap.add_argument("--eager", action="store_true",
                    help="launch every kernel from Python instead of replaying a captured HIP graph")
    ap.add_argument("--decode", choices=("static", "shared"), default="static",
                    help="page-table decode: fixed splits (kvq_decode_attn), or the resident workers of each "
                         "(request, head) range sharing its windows (kvq_decode_attn_shared)")
    ap.add_argument("--timeline", action="store_true",
                    help="profiling: run the profiling build libkvq_timeline.so and print a per-wave timeline "
                         "summary of the fixed-split decode (graph replays) instead of the result line")
    ap.add_argument("--timeline-samples", type=int, default=5, help="launches summarized by --timeline")
    args = ap.parse_args()
    if args.timeline:
        # before the binding is imported: it loads the library named here (another
        # profiling build of the same sources may be named by KVQ_LIBRARY)
        os.environ.setdefault("KVQ_LIBRARY", os.path.join(ROOT, "mixed_precision_quantized_amd", "libkvq_timeline.so"))
        if args.decode != "static" or args.eager:
            sys.exit("--timeline records the fixed-split decode replayed as a graph")
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(requests and KV heads shard with no exchange; see the design notes)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    from harness import DeviceRun
    from mixed_precision_quantized_amd import kvq

    if args.workload == "vl_select":
        return bench_vl(args)
    if args.workload == "prefill":
        return bench_prefill(args)
    suffix, default_layers, description = WORKLOADS[args.workload]
    make = getattr(synth, args.workload)
    if args.ordered_pages:
        if args.workload != "qwen3_8b":
            sys.exit("--ordered-pages applies to the qwen3_8b workload only")
        make = functools.partial(make, ordered_pages=True)
    layers = args.layers or default_layers
    base_make = make

    def make(**kw):  # page tables get room for one decode step's INT4 tail page per table
        w = base_make(**kw)
        return synth.reserve_tail(w, synth.PAGE) if w.kind == synth.PAGES else w
    dev = "cuda"
    torch.cuda.set_device(0)
    t0 = time.time()

    # Layer 0 is built, placed, quantized and reordered through the library; every other
    # layer gets its own pools holding its own K / V with the same placement, so the
    # reordered tables, ranges and plan serve all layers.
    gpu = DeviceRun(make(device=dev, layer=0), compact=not args.no_compact)
    w0 = gpu.w
    eff_layer, decode_bytes = effective_bytes(w0, anchor_fp8=args.anchor_fp8)
    log(f"workload: {w0.note}; effective bytes per layer {eff_layer}")
    cpu_sample = None
    if args.timeline and (w0.kind != synth.PAGES or w0.n_pages[2]):
        sys.exit("--timeline records the page-table decode of INT2 / INT4 splits (no slot maps, no FP16 pages)")
    if not args.no_cpu_baseline and not args.timeline and w0.kind == synth.PAGES:
        req = list(range(min(args.cpu_requests, w0.batch)))
        cpu_sample = synth.subset(make(device=dev, layer=0), req, device="cpu")
    lists = {n: torch.as_tensor(a, device=dev) for n, a in gpu.lists.arrays().items()}
    lists = {n: (a if len(a) else None) for n, a in lists.items()}
    sent = synth.sentinel_lists(w0).arrays() if w0.kind == synth.SLOTS and w0.sentinel_slot >= 0 else None
    caches, qs = [gpu.cache], [gpu.q]
    w0.k = w0.v = gpu.k = gpu.v = None
    for L in range(1, layers):
        w = make(device=dev, layer=L)
        cache = kvq.Cache(w0.heads_per_page, w0.n_pages, dev, sentinel_slot=w0.sentinel_slot,
                          anchor_fp8=args.anchor_fp8)
        if sent is not None:
            kvq.quantize_append(cache, w.k, w.v, rows4=torch.as_tensor(sent["rows4"], device=dev),
                                slots4=torch.as_tensor(sent["slots4"], device=dev), dev_err=gpu.err)
        kvq.quantize_append(cache, w.k, w.v, dev_err=gpu.err, **lists)
        caches.append(cache)
        qs.append(w.q.contiguous())
        del w
    # One decode step's tail append per layer: a new token per table, placed INT4 at the
    # table's tail (the reordered table's last INT4 page where it has room, else a fresh
    # page) and written by kvq_quantize_append.  The decode's ranges stay those of the
    # prefix: the append is timed beside the step, not inside it.
    tail_app = []
    if w0.kind == synth.PAGES:
        tl = synth.AppendLists()
        tabs = gpu.tables.cpu().numpy()
        for t in range(w0.n_tables):
            n = int(w0.alloc.n_entries[t])
            w0.alloc.append_tail(t, int(tabs[t, n - 1]) if n else None, [t], tl)
        ta = tl.arrays()
        r4, s4 = (torch.as_tensor(ta[x], device=dev) for x in ("rows4", "slots4"))
        for L in range(layers):
            tk, tv, _ = synth.tail_rows(w0, L, 1, device=dev)
            tail_app.append((tk, tv))
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    cost = None if args.class_cost is None else [float(x) for x in args.class_cost.split(",")]
    g = w0.g
    kind = kvq.TABLE_SLOTS if w0.kind == synth.SLOTS else kvq.TABLE_PAGES
    shared = args.decode == "shared"
    if shared and (kind != kvq.TABLE_PAGES or g > 8):
        sys.exit("--decode shared: page tables and g <= 8 only")
    if shared:
        per_cu, n_cu = kvq.decode_occupancy(g, kind)
        wph = args.splits_per_head or max(1, per_cu * n_cu // (w0.batch * w0.hkv))
        splits, groups, n_groups, offsets = gpu.plan_workers(wph, cost)
        grp = torch.as_tensor(groups, device=dev).contiguous()
        work = kvq.decode_work(n_groups, dev)
    else:
        splits, offsets, per_cu, n_cu = resident_plan(gpu, kvq, synth, args.splits_per_head, cost, args.ragged_plan)
    n_splits = splits.shape[0]
    sp = torch.as_tensor(splits, device=dev).contiguous()
    off = torch.as_tensor(offsets, device=dev)
    part_o = torch.empty((n_splits, g, 128), dtype=torch.float32, device=dev)
    part_lse = torch.empty((n_splits, g), dtype=torch.float32, device=dev)
    outs = [torch.empty((w0.batch, w0.hq, 128), dtype=torch.bfloat16, device=dev) for _ in range(layers)]
    torch.cuda.synchronize()
    assert int(gpu.err.item()) == 0, f"device error bits {int(gpu.err.item())}"
    log(f"setup {time.time() - t0:.1f}s: {layers} layers, {n_splits} splits per layer "
        f"({per_cu} resident per CU x {n_cu} CUs), "
        f"pools {sum(sum(p.numel() for p in c.pools) for c in caches) / 2**30:.1f} GiB")

    # Every launch goes to `stream`: torch's current stream when eager, a side stream
    # (default priority) for graph capture; events recorded on it bracket the kernels.
    stream = torch.cuda.current_stream() if args.eager else torch.cuda.Stream()

    def bound(st):
        if shared:
            d = [kvq.bind_decode_attn_shared(caches[L], qs[L], w0.hkv, gpu.tables, kind, sp, grp, n_groups, work,
                                             part_o, part_lse, dev_err=gpu.err, stream=st) for L in range(layers)]
        else:
            d = [kvq.bind_decode_attn(caches[L], qs[L], w0.hkv, gpu.tables, kind, sp, part_o, part_lse, stream=st)
                 for L in range(layers)]
        m = [kvq.bind_lse_merge(part_o, part_lse, n_splits, off, w0.batch, w0.hq, w0.hkv, outs[L], stream=st)
             for L in range(layers)]
        return d, m

    dec, mrg = bound(stream)
    app = [kvq.bind_quantize_append(caches[L], tk, tv, rows4=r4, slots4=s4, dev_err=gpu.err, stream=stream)
           for L, (tk, tv) in enumerate(tail_app)]

    def appends():
        for a in app:
            a()

    def step():
        for L in range(layers):
            dec[L]()
            mrg[L]()

    def decodes():
        for L in range(layers):
            dec[L]()

    if args.copy_calibration:
        # Known-size references for the HBM byte counters: 1 GiB read + 1 GiB written,
        # once as bytes and once as float32 (torch picks a different copy kernel for each).
        for dt in (torch.uint8, torch.float32):
            src = torch.ones((1 << 30) // torch.empty((), dtype=dt).element_size(), dtype=dt, device=dev)
            dst = torch.empty_like(src)
            torch.cuda.synchronize()
            dst.copy_(src)
            torch.cuda.synchronize()
            del src, dst
        log("copy calibration: two 1 GiB device-to-device copies (uint8, float32)")

    with torch.cuda.stream(stream):
        step()  # first launches (code objects load) outside any capture
    torch.cuda.synchronize()
    run_step, run_decodes, run_appends = step, decodes, (appends if app else None)
    if app:
        with torch.cuda.stream(stream):
            appends()  # first launch outside any capture
        torch.cuda.synchronize()
    if not args.eager:
        # The step as one HIP graph (the 2 x layers launches, no allocation, no memset),
        # and the decode launches alone for the kernel's own duration.  Each replay of
        # the step is checked against the eager outputs, with eager work in between.
        ref = torch.stack([o.float() for o in outs])
        g_step, g_dec = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_step, stream=stream):
            step()
        with torch.cuda.graph(g_dec, stream=stream):
            decodes()
        g_app = None
        if app:
            g_app = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g_app, stream=stream):
                appends()
        torch.cuda.synchronize()
        for _ in range(3):
            for o in outs:
                o.zero_()
            g_step.replay()
            torch.cuda.synchronize()
            got = torch.stack([o.float() for o in outs])
            if shared:  # the windows a worker takes vary: the same sums in another order
                dif = (got - ref).abs().amax(-1) / ref.abs().amax(-1).clamp_min(1e-30)
                assert float(dif.max()) <= 2.0 ** -7, "graph replay differs from eager"
            else:
                assert torch.equal(got, ref), "graph replay differs from eager"
            if shared:
                assert not work.any().item(), "work counters not reset"
            with torch.cuda.stream(stream):
                step()
            torch.cuda.synchronize()
        assert int(gpu.err.item()) == 0
        run_step, run_decodes = g_step.replay, g_dec.replay
        run_appends = g_app.replay if g_app is not None else None
        log("step captured as a HIP graph of the decode + merge launches; 3 replays equal to eager"
            + (" (to bf16 rounding: shared windows sum in another order)" if shared else ""))

    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            run_step()
    torch.cuda.synchronize()
    if args.timeline:
        return wave_timeline(args, kvq, run_decodes, stream, splits, layers, description)

    def timed(fn, reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            e0.record(stream)
            for _ in range(reps):
                fn()
            e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / reps  # seconds per rep

    # The timed steps: K steps back to back between two events, nothing in between.
    ms_step = timed(run_step, args.steps) * 1e3
    # The dominant kernel alone: the layers' decode launches back to back, K times;
    # the average launch duration is the span over the number of launches.
    us_decode = timed(run_decodes, args.steps) * 1e6 / layers
    achieved = decode_bytes / (us_decode * 1e-6) / 1e9
    us_append = timed(run_appends, args.steps) * 1e6 / layers if run_appends else None
    if us_append is not None:
        log(f"decode-time tail append {us_append:.1f} us per layer ({w0.n_tables} tokens, one per table)")
    log(f"step {ms_step * 1000:.1f} us ({ms_step * 1000 / layers:.1f} us per layer)")
    log(f"decode kernel {us_decode:.1f} us per launch ({layers} x {args.steps} back-to-back launches), "
        f"{achieved:.0f} GB/s algorithmic")
    assert int(gpu.err.item()) == 0

    gbs = eff_layer * layers / (ms_step * 1e-3) / 1e9
    default = args.workload == "qwen3_8b"
    if w0.kind == synth.SLOTS:
        description += (", slot maps as given (dead entries decoded and masked)" if args.no_compact
                        else ", slot maps compacted ahead of time (dead entries dropped)")
        description += f", {args.ragged_plan} split counts"
    result = {
        "metric": "decode-attn effective KV GB/s (% HBM peak) + µs/step, " + suffix,
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "us_per_step": round(ms_step * 1000, 1),
        "us_per_layer": round(ms_step * 1000 / layers, 2),
        "append_us_per_layer": None if us_append is None else round(us_append, 2),
        "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u2/u4 codes, fp16 scale/zero" + ((", fp8 anchors" if args.anchor_fp8 else ", fp16 anchors")
                                                   if w0.n_pages[2] else "") + ", fp32 math",
        "data": "synthetic",
        "config": {
            "workload": description + (" (FP8 anchors)" if args.anchor_fp8 else "")
            + (" (pages in id order)" if args.ordered_pages else "") + f", {layers} layers",
            "batch": w0.batch, "hq": w0.hq, "hkv": w0.hkv, "layers": layers, "splits_per_layer": n_splits,
            "decode": "shared windows (kvq_decode_attn_shared)" if shared else "fixed splits (kvq_decode_attn)",
            "effective_bytes_per_layer": eff_layer,
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "decode",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic() if default else None,
            "bytes_per_launch": decode_bytes,
            "us_per_launch": round(us_decode, 2),
        },
        "cpu_baseline": None,
    }

    if cpu_sample is not None:
        result["cpu_baseline"] = cpu_baseline(cpu_sample, w0, args, make)
    print(json.dumps(result), flush=True)


def wave_timeline(args, kvq, run_decodes, stream, splits, layers, description):
    """Per-wave timeline of the decode kernel (profiling build): after three back-to-back
    replays of the layers' decode launches the buffer holds the last launch; repeated
    --timeline-samples times.  Prints one JSON line of per-launch summaries."""
    import numpy as np
    import torch
    n = splits.shape[0]
    buf = torch.zeros((n, 8), dtype=torch.int64, device="cuda")
    kvq.wave_timeline(buf)
    cls = np.asarray(splits).view(np.int32).reshape(n, 5)[:, 2]
    samples = []
    for _ in range(args.timeline_samples):
        buf.zero_()
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            for _ in range(3):
                run_decodes()
        torch.cuda.synchronize()
        r = buf.cpu().numpy().astype(np.int64)
        assert (r[:, 2] > 0).all(), "a split recorded no end"
        t0 = r[:, 0].min()
        st, fw, en = ((r[:, k] - t0) / 100.0 for k in (0, 1, 2))  # us (100 MHz)
        mhz = (r[:, 4] - r[:, 3]) / np.maximum(r[:, 2] - r[:, 0], 1) * 100.0
        xcc = r[:, 5] & 0xF
        hw = r[:, 6]
        cu = xcc * 4096 + ((hw >> 13) & 7) * 32 + ((hw >> 12) & 1) * 16 + ((hw >> 8) & 15)
        per_cu = [float(np.mean(en[cu == c])) for c in np.unique(cu)]
        per_xcd = [float(np.mean(en[xcc == x])) for x in range(8) if (xcc == x).any()]
        rate = r[:, 7] / np.maximum(en - fw, 1e-3)
        samples.append({
            "span_us": round(float(en.max()), 1),
            "start_max_us": round(float(st.max()), 2),
            "first_window_us": {"median": round(float(np.median(fw)), 1), "p90": round(float(np.percentile(fw, 90)), 1)},
            "end_us": {q: round(float(np.percentile(en, p)), 1) for q, p in (("p50", 50), ("p90", 90), ("p99", 99))},
            "mean_wave_us": round(float(np.mean(en - st)), 1),
            "end_median_per_xcd_us": [round(float(np.median(en[xcc == x])), 1) for x in range(8) if (xcc == x).any()],
            "clock_mhz_median_per_xcd": [round(float(np.median(mhz[xcc == x]))) for x in range(8) if (xcc == x).any()],
            "max_cu_mean_end_us": round(max(per_cu), 1),
            "max_xcd_mean_end_us": round(max(per_xcd), 1),
            "windows_per_us_median": {c: round(float(np.median(rate[cls == k])), 3)
                                      for c, k in (("int2", 0), ("int4", 1)) if (cls == k).any()},
        })
        log(f"timeline: span {samples[-1]['span_us']} us, median end {samples[-1]['end_us']['p50']} us, "
            f"mean wave {samples[-1]['mean_wave_us']} us")
    kvq.wave_timeline(None)
    print(json.dumps({"kind": "wave_timeline", "workload": description + f", {layers} layers",
                      "splits": n, "launch": "the last of three back-to-back replays of the layers' decode launches",
                      "samples": samples}), flush=True)


def bench_vl(args):
    """Vertical-line selection + FREEZE routing (one kvq_select_vertical_lines call: proxy,
    scores, selection) on the hybrid-anchor prefill shape: 32 requests x 65536 tokens,
    Hq 32 / Hkv 8, 64 bf16 tail queries, bf16 keys resident in HBM.  Algorithmic bytes per
    call: the keys and tail queries read once, per token-head a 4-byte score written and
    read back and a 1-byte class written."""
    import numpy as np
    import torch

    import synth
    from mixed_precision_quantized_amd import kvq

    dev = "cuda"
    torch.cuda.set_device(0)
    w = synth.vl_prefill(device=dev)
    batch, mt, hkv = w.k.shape[:3]
    hq = w.q_tail.shape[2]
    nt = torch.as_tensor(w.n_tokens, device=dev)
    ntl = torch.as_tensor(w.n_tail, device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    stream = torch.cuda.Stream()
    out = kvq.select_vertical_lines(w.k, w.q_tail, nt, ntl, dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    log(f"vl_select: {w.note}; {int(out[3].sum())} vertical lines")
    call = lambda: kvq.select_vertical_lines(w.k, w.q_tail, nt, ntl, out=out, dev_err=err,  # noqa: E731
                                             stream=stream)
    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        e0.record(stream)
        for _ in range(args.steps):
            call()
        e1.record(stream)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    sec = e0.elapsed_time(e1) * 1e-3 / args.steps
    token_heads = int(w.n_tokens.astype(np.int64).sum()) * hkv
    nbytes = w.k.numel() * w.k.element_size() + w.q_tail.numel() * w.q_tail.element_size() + 9 * token_heads
    gbs = nbytes / sec / 1e9
    log(f"vl_select: {sec * 1e6:.1f} us per call, {gbs:.0f} GB/s algorithmic")
    result = {
        "metric": "vertical-line selection + FREEZE routing GB/s (HyQuant Alg. 1, 4), hybrid-anchor prefill shape",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(sec * 1e3, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16 keys and queries, fp32 scores", "data": "synthetic",
        "config": {"workload": f"vertical-line selection: {w.note}, window 128, rho 0.05",
                   "batch": batch, "max_tokens": mt, "hkv": hkv, "hq": hq, "bytes_per_call": nbytes},
        "roofline": {"bound": "hbm", "kernel": "vl_select (proxy, scores, selection)", "achieved": round(gbs, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        from oracle import oracle
        req = [0, 1]
        k = w.k[req].float().cpu().numpy()
        q = w.q_tail[req].float().cpu().numpy()
        reps, t = 0, time.perf_counter()
        while True:
            oracle.select_vl(k, q, w.n_tokens[req], w.n_tail[req])
            reps += 1
            dt = time.perf_counter() - t
            if dt >= CPU_SECONDS:
                break
        sample = k.nbytes // 2 + q.nbytes // 2 + 9 * int(w.n_tokens[req].astype(np.int64).sum()) * hkv
        result["cpu_baseline"] = {"value": round(sample * reps / dt / 1e9, 3), "unit": "GB/s", "cores": 1,
                                  "kind": "oracle",
                                  "sample": f"2 of {batch} requests (bf16-sized bytes), fp64 scores and a "
                                            f"sort per head, one thread, {reps} passes in {dt:.1f} s"}
        log(f"cpu oracle {result['cpu_baseline']['value']} GB/s on 1 thread ({dt:.1f} s)")
    print(json.dumps(result), flush=True)


def bench_prefill(args):
    """INT8-prefix prefill attention (HyQuant: the core method's fused operator, Algorithm
    2) at the Llama-3.1-8B shape: one request of --prefill-tokens positions, Hq 32 / Hkv
    8, bf16, 5 % vertical lines, a 128-token window.  Algorithmic work per call: the
    causal Q K^T and P V products, 2 x 2 x 128 x n (n + 1) / 2 x Hq operations, all on
    bf16 / fp16 matrix cores (the query is never quantized, so no product is INT8 x
    INT8), against the dense bf16 MFMA peak."""
    import numpy as np
    import torch

    import synth
    from mixed_precision_quantized_amd import kvq

    dev = "cuda"
    torch.cuda.set_device(0)
    n, hq, hkv = args.prefill_tokens, 32, 8
    q, k, v, lens, cls = synth.prefill_qkv(seed=8, batch=1, n_max=n, hq=hq, hkv=hkv, device=dev)
    nt = torch.as_tensor(lens, device=dev)
    cd = torch.as_tensor(cls, device=dev).contiguous()
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    ws = kvq.prefill_workspace(1, n, hq, hkv, dev)
    stream = torch.cuda.Stream()
    prepare = lambda: kvq.prefill_prepare(k, v, nt, cd, ws, err, stream)  # noqa: E731
    attend = lambda: kvq.prefill_attend(q, k, nt, cd, 128, ws, err, stream)  # noqa: E731
    # Kernel durations fall over the first ~15 calls (2.3 -> 1.76 ms for the attention at
    # 16K), so the warm-up is at least 20 calls.
    warm = max(20, args.warmup)
    with torch.cuda.stream(stream):
        for _ in range(warm):
            prepare()
            attend()
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    steps = max(1, args.steps // 4)

    def timed(fns):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            e0.record(stream)
            for _ in range(steps):
                for f in fns:
                    f()
            e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / steps

    sec = timed((prepare, attend))      # the whole path: codes, scratch, attention
    sec_attn = timed((attend,))         # the attention kernel alone
    flops = 2 * 2 * 128 * n * (n + 1) / 2 * hq
    peak = 2500.0  # dense bf16 / fp16 MFMA, TFLOP/s
    tflops = flops / sec / 1e12
    attn_tflops = flops / sec_attn / 1e12
    log(f"prefill: {n} tokens, Hq {hq} / Hkv {hkv}: {sec * 1e3:.3f} ms per call ({tflops:.1f} TFLOP/s); "
        f"attention kernel {sec_attn * 1e3:.3f} ms ({attn_tflops:.1f} TFLOP/s)")
    result = {
        "metric": "INT8-prefix prefill attention TFLOP/s (HyQuant fused operator, Alg. 2), Llama-3.1-8B shape",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": steps, "warmup": args.warmup,
        "ms_per_step": round(sec * 1e3, 3), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16 Q K^T (INT8 K codes as exact bf16), fp16 P V, fp32 softmax", "warmup_calls": warm, "data": "synthetic",
        "config": {"workload": f"prefill attention: 1 request x {n} tokens, Hq {hq} / Hkv {hkv}, 5% vertical lines, "
                               "window 128", "tokens": n, "hq": hq, "hkv": hkv, "flops_per_call": flops},
        "roofline": {"bound": "mfma", "kernel": "pf_attn_kernel", "achieved": round(attn_tflops, 2),
                     "peak": round(peak, 1), "unit": "TFLOP/s", "frac": round(attn_tflops / peak, 4),
                     "traffic": (measured_traffic(PREFILL_TRAFFIC_FILE, PREFILL_SOURCES)
                                 if n == 16384 else None), "kernel_ms": round(sec_attn * 1e3, 4)},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        from oracle import oracle
        m = 1024  # a prompt prefix the fp64 oracle finishes in seconds
        qq, kk, vv = (x[:, :m].float().cpu().numpy() for x in (q, k, v))
        cc = np.ascontiguousarray(cls[:, :, :m])
        reps, t = 0, time.perf_counter()
        while True:
            oracle.prefill_attend(qq, kk, vv, [m], cc, 128)
            reps += 1
            dt = time.perf_counter() - t
            if dt >= CPU_SECONDS:
                break
        f = 2 * 2 * 128 * m * (m + 1) / 2 * hq
        result["cpu_baseline"] = {"value": round(f * reps / dt / 1e12, 6), "unit": "TFLOP/s", "cores": 1,
                                  "kind": "oracle", "sample": f"the first {m} positions, fp64, one thread, "
                                                              f"{reps} passes in {dt:.1f} s"}
        log(f"cpu oracle {result['cpu_baseline']['value']} TFLOP/s on 1 thread ({dt:.1f} s)")
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
