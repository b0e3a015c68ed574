#!/usr/bin/env python3
"""Decode-attention benchmark on one MI355X.

Workload: Qwen3-8B-shaped decode step over a mixed INT2 / INT4 paged KV cache: batch
16, Hq 32 / Hkv 8 (g = 4), d 128, 32768 tokens per request (70 % INT2 / 30 % INT4 in
shuffled 32-token units, INT2-first reorder), 16-token pages, bf16 q and output,
36 layers each with its own pools (17.4 GB in total, so no layer is served from the
256 MB Infinity Cache).  A step = split-K decode + log-sum-exp merge for all 36
layers.  Inputs are resident in HBM before timing starts.

Prints ONE JSON line: effective KV GB/s of the whole step (algorithmic bytes: packed
codes + fp16 scale/zero of every live token-head, 4 B per page-table entry, q and the
output), us per step, the roofline of the decode kernel and the CPU oracle's rate on a
bounded sample of the same workload."""
import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode-attn effective KV GB/s (% HBM peak) + µs/step, Qwen3-8B shape @32K"
HBM_PEAK_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_qwen3_8b_traffic.md")
CPU_SECONDS = 10.0  # lower bound on the timed oracle work


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def effective_bytes(w, q_bytes_per_elem=2, out_bytes_per_elem=2):
    """Algorithmic bytes of one layer: live token-heads x (96 / 160 / 512 B), 4 B per
    page-table entry, q and output."""
    H = w.heads_per_page
    kv = int((w.alloc.tokens[:, 0] * 96 + w.alloc.tokens[:, 1] * 160 + w.alloc.tokens[:, 2] * 512).sum()) * H
    tables = int(w.alloc.n_entries.sum()) * 4
    qo = w.batch * w.hq * 128 * (q_bytes_per_elem + out_bytes_per_elem)
    return kv + tables + qo, kv


def kernel_source_sha():
    """Hash of the decode kernel's source code (comments and layout ignored)."""
    h = hashlib.sha256()
    for f in ("kvq_decode.hip", "kvq_internal.h"):
        with open(os.path.join(ROOT, "mixed_precision_quantized_amd", "csrc", f)) as fh:
            text = re.sub(r"/\*.*?\*/", " ", fh.read(), flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per decode launch from the committed rocprofv3 PMC summary (its line
    starting 'bench-traffic:'), if it was taken on the current kernel source; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            for line in f:
                if line.startswith("bench-traffic:"):
                    t = json.loads(line.split(":", 1)[1])
                    break
            else:
                return None
    except (OSError, ValueError):
        return None
    if t.get("kernel_sha") != kernel_source_sha():
        return None
    return t.get("bytes_per_launch")


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--layers", type=int, default=36)
    ap.add_argument("--splits-per-head", type=int, default=0,
                    help="splits per (request, KV head); 0 = as many as the decode kernel keeps resident")
    ap.add_argument("--cpu-requests", type=int, default=16, help="requests in the CPU-oracle sample")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain 1 GiB device copy (reference for HBM byte counters)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(requests and KV heads shard with no exchange; see the design notes)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    from mixed_precision_quantized_amd import kvq

    dev = "cuda"
    torch.cuda.set_device(0)
    t0 = time.time()
    w0 = synth.qwen3_8b(device=dev, layer=0)
    lists = synth.place_all(w0, lambda f: kvq.route_tokens(f)[0])
    dl = {n: torch.as_tensor(a, device=dev) for n, a in lists.arrays().items()}
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    tables = torch.as_tensor(w0.alloc.tables, device=dev).contiguous()
    n_entries = torch.as_tensor(w0.alloc.n_entries, device=dev)
    counts = torch.zeros((w0.n_tables, 3), dtype=torch.int32, device=dev)
    eff_layer, kv_layer = effective_bytes(w0)
    log(f"workload: {w0.note}; effective bytes per layer {eff_layer}")

    cpu_sample = None
    if not args.no_cpu_baseline:
        cpu_sample = synth.subset(w0, list(range(args.cpu_requests)), device="cpu")

    caches, qs = [], []
    for L in range(args.layers):
        w = w0 if L == 0 else synth.qwen3_8b(device=dev, layer=L)
        cache = kvq.Cache(w0.heads_per_page, w0.n_pages, dev)
        kvq.quantize_append(cache, w.k, w.v, rows4=dl["rows4"], slots4=dl["slots4"], rows2=dl["rows2"],
                            pages2=dl["pages2"], dev_err=err)
        caches.append(cache)
        qs.append(w.q.contiguous())
        w.k = w.v = None
        del w
    torch.cuda.synchronize()
    w0.k = w0.v = None
    torch.cuda.empty_cache()
    kvq.reorder_pages(caches[0], tables, n_entries, counts, dev_err=err)
    items = []
    for t in range(w0.n_tables):
        items += w0.alloc.ranges_after_partition(t, list(range(w0.heads_per_page)))
    ranges = synth.ranges_array(items)
    # One wave per split; fill every resident slot of the chip once (a second, partial
    # round of waves would leave most of the chip idle at the end).
    per_cu, n_cu = kvq.decode_occupancy(w0.g)
    sph = args.splits_per_head or max(1, (per_cu * n_cu) // (w0.batch * w0.hkv))
    splits, offsets = kvq.plan_splits(ranges, w0.batch, w0.hkv, w0.heads_per_page,
                                      splits_per_head=np.full(w0.batch * w0.hkv, sph, np.int32))
    n_splits = splits.shape[0]
    sp = torch.as_tensor(splits, device=dev).contiguous()
    off = torch.as_tensor(offsets, device=dev)
    g = w0.g
    part_o = torch.empty((n_splits, g, 128), dtype=torch.float32, device=dev)
    part_lse = torch.empty((n_splits, g), dtype=torch.float32, device=dev)
    outs = [torch.empty((w0.batch, w0.hq, 128), dtype=torch.bfloat16, device=dev) for _ in range(args.layers)]
    dec = [kvq.bind_decode_attn(caches[L], qs[L], w0.hkv, tables, kvq.TABLE_PAGES, sp, part_o, part_lse)
           for L in range(args.layers)]
    mrg = [kvq.bind_lse_merge(part_o, part_lse, n_splits, off, w0.batch, w0.hq, w0.hkv, outs[L])
           for L in range(args.layers)]
    torch.cuda.synchronize()
    assert int(err.item()) == 0, f"device error bits {int(err.item())}"
    log(f"setup {time.time() - t0:.1f}s: {args.layers} layers, {n_splits} splits per layer "
        f"({sph} per head; {per_cu} resident per CU x {n_cu} CUs), "
        f"pools {sum(sum(p.numel() for p in c.pools) for c in caches) / 2**30:.1f} GiB")

    def step():
        for L in range(args.layers):
            dec[L]()
            mrg[L]()

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

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # Every launch goes to torch's current stream (the bound calls pass it), so events
    # recorded there bracket exactly the kernels.  Inside the timed steps each decode
    # launch is bracketed too, for the roofline of the dominant kernel.
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps * args.layers)]
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    i = 0
    for _ in range(args.steps):
        for L in range(args.layers):
            ev[i][0].record(stream)
            dec[L]()
            ev[i][1].record(stream)
            mrg[L]()
            i += 1
    e1.record(stream)
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / args.steps
    us_decode = sum(a.elapsed_time(b) for a, b in ev) * 1000 / len(ev)
    log(f"step {ms_step * 1000:.1f} us ({ms_step * 1000 / args.layers:.1f} us per layer)")
    decode_bytes = kv_layer + int(w0.alloc.n_entries.sum()) * 4 + w0.batch * w0.hq * 128 * 2
    achieved = decode_bytes / (us_decode * 1e-6) / 1e9
    log(f"decode kernel {us_decode:.1f} us per launch, {achieved:.0f} GB/s algorithmic")
    assert int(err.item()) == 0

    gbs = eff_layer * args.layers / (ms_step * 1e-3) / 1e9
    result = {
        "metric": METRIC,
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "us_per_step": round(ms_step * 1000, 1),
        "us_per_layer": round(ms_step * 1000 / args.layers, 2),
        "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u2/u4 codes, fp16 scale/zero, fp32 math",
        "data": "synthetic",
        "config": {
            "workload": "Qwen3-8B-shaped decode: batch 16, Hq 32 / Hkv 8, d 128, 32768 tokens per "
                        "request, 70% INT2 / 30% INT4, 16-token pages, 36 layers",
            "batch": w0.batch, "context": 32768, "layers": args.layers, "splits_per_layer": n_splits,
            "effective_bytes_per_layer": eff_layer,
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "decode",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(),
            "bytes_per_launch": decode_bytes,
            "us_per_launch": round(us_decode, 2),
        },
        "cpu_baseline": None,
    }

    if cpu_sample is not None:
        sys.path.insert(0, os.path.join(ROOT, "tests"))
        from harness import OracleRun
        try:
            n_threads = min(16, len(os.sched_getaffinity(0)))
        except AttributeError:
            n_threads = min(16, os.cpu_count() or 1)
        orc = OracleRun(cpu_sample)
        reps, t = 0, time.perf_counter()
        while True:  # whole passes over the sample until CPU_SECONDS have gone by
            orc.attend(n_threads=n_threads)
            reps += 1
            dt = time.perf_counter() - t
            if dt >= CPU_SECONDS:
                break
        sample_bytes, _ = effective_bytes(cpu_sample)
        result["cpu_baseline"] = {
            "value": round(sample_bytes * reps / dt / 1e9, 3),
            "unit": "GB/s",
            "cores": n_threads,
            "kind": "oracle",
            "sample": f"{args.cpu_requests} of 16 requests of one layer (all 8 KV heads, g = 4, "
                      f"32768 tokens each), fp64 two-pass softmax, {reps} passes in {dt:.1f} s",
        }
        log(f"cpu oracle {result['cpu_baseline']['value']} GB/s on {n_threads} threads ({dt:.1f} s)")
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
