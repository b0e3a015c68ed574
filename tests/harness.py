"""Builders that run one synthetic workload through the GPU library or through the CPU
oracle.  The two builders never share anything but the seeded workload itself
(synth): DeviceRun routes with the library's router and only calls the binding;
OracleRun routes with the oracle's router and only calls the oracle.  Build each side
from its own Workload object (same constructor, same seed) because placement is
stateful."""
from __future__ import annotations

import numpy as np
import torch

import synth


def row_metric(ref: np.ndarray, got: np.ndarray) -> float:
    """max over rows of max_c |ref - got| / max_c |ref| (rows: all but the last axis)."""
    ref = ref.reshape(-1, ref.shape[-1]).astype(np.float64)
    got = got.reshape(-1, got.shape[-1]).astype(np.float64)
    den = np.abs(ref).max(axis=1)
    num = np.abs(ref - got).max(axis=1)
    ok = den > 0
    worst = float((num[ok] / den[ok]).max()) if ok.any() else 0.0
    if (~ok).any():
        worst = max(worst, float(num[~ok].max()))
    return worst


def _table_ranges(w, tables):
    """Token ranges of every (table, head), sorted by (table, head), from a side's own
    tables (as its reorder left them, or as placed) and the fill the caller gave each
    page."""
    items = []
    for t in range(w.n_tables):
        n = int(w.alloc.n_entries[t])
        items += w.alloc.ranges_in_order(t, tables[t, :n], list(range(w.heads_per_page)))
    items.sort(key=lambda it: (it[0], it[1]))
    return synth.ranges_array(items)


def library_flags(kvq, w):
    """Routing flags per request of a tagged workload, made by the library: tri-axis
    tags (kvq_tag_tokens), tokens per tag over the batch (kvq_count_tags), greedy widths
    (kvq_allocate_bits), flags (kvq_tag_flags)."""
    ev = {name: getattr(kvq, "EV_" + name.upper()) for name in synth._STREAM_EVENTS}
    memo = {}

    def tags_of(st):
        if id(st) not in memo:
            memo[id(st)] = kvq.tag_tokens(st.tokens, {t: ev[e] for t, e in st.markers.items()})[0]
        return memo[id(st)]
    counts = np.zeros(kvq.N_TAGS, np.int64)
    for st in w.count_streams:
        kvq.count_tags(tags_of(st), counts)
    bits, _ = kvq.allocate_bits(w.distortion[0], w.distortion[1], counts, w.budget_bits)
    return [kvq.tag_flags(tags_of(st), bits) for st in w.streams]


def oracle_flags(w):
    """The same flags made by the oracle's plain-Python tagger and width allocation."""
    from oracle import tags as ot
    memo = {}

    def tags_of(st):
        if id(st) not in memo:
            names, _ = ot.tag_tokens(st.tokens.tolist(), st.markers)
            memo[id(st)] = [ot.tag_index(*x) for x in names]
        return memo[id(st)]
    counts = [0] * (len(ot.TEMPORAL) * len(ot.MODAL) * len(ot.SEMANTIC))
    for st in w.count_streams:
        for k in tags_of(st):
            counts[k] += 1
    bits, _ = ot.allocate_bits(list(w.distortion[0]), list(w.distortion[1]), counts, w.budget_bits)
    return [np.array([0 if bits[k] == 2 else 1 for k in tags_of(st)], np.uint8) for st in w.streams]


class DeviceRun:
    """Route (library), place, quantize + append, reorder and decode on the GPU."""

    def __init__(self, w: synth.Workload, device="cuda", reorder=True, compact=False, anchor_fp8=False):
        from mixed_precision_quantized_amd import kvq
        self.kvq, self.w, self.device = kvq, w, device
        self.flags = library_flags(kvq, w) if w.streams is not None else None
        self.lists = synth.place_all(w, lambda f: kvq.route_tokens(f)[0], self.flags)
        self.cache = kvq.Cache(w.heads_per_page, w.n_pages, device, sentinel_slot=w.sentinel_slot,
                               anchor_fp8=anchor_fp8)
        self.err = torch.zeros(1, dtype=torch.int32, device=device)
        self.k = w.k.to(device)
        self.v = w.v.to(device)
        self.q = w.q.to(device).contiguous()
        a = {n: torch.as_tensor(x, device=device) for n, x in self.lists.arrays().items()}
        if w.kind == synth.SLOTS and w.sentinel_slot >= 0:
            s = synth.sentinel_lists(w).arrays()
            kvq.quantize_append(self.cache, self.k, self.v,
                                rows4=torch.as_tensor(s["rows4"], device=device),
                                slots4=torch.as_tensor(s["slots4"], device=device), dev_err=self.err)
        kvq.quantize_append(self.cache, self.k, self.v,
                            rows4=a["rows4"] if len(a["rows4"]) else None,
                            slots4=a["slots4"] if len(a["slots4"]) else None,
                            rows2=a["rows2"] if len(a["rows2"]) else None,
                            pages2=a["pages2"] if len(a["pages2"]) else None,
                            rows16=a["rows16"] if len(a["rows16"]) else None,
                            slots16=a["slots16"] if len(a["slots16"]) else None, dev_err=self.err)
        if w.kind == synth.PAGES:
            self.tables = torch.as_tensor(w.alloc.tables, device=device).contiguous()
            self.n_entries = torch.as_tensor(w.alloc.n_entries, device=device)
            self.class_counts = torch.zeros((w.n_tables, 3), dtype=torch.int32, device=device)
            self.reordered = reorder
            if reorder:
                kvq.reorder_pages(self.cache, self.tables, self.n_entries, self.class_counts,
                                  dev_err=self.err)
            self.ranges = _table_ranges(w, self.tables.cpu().numpy())
        else:
            self.tables = torch.as_tensor(synth.slot_tables(w), device=device).contiguous()
            self.reordered = False
            self.live_tokens = None
            if compact:  # dead entries dropped ahead of time; heads read their live counts
                self.live_tokens = kvq.compact_slots(
                    self.cache, self.tables, torch.as_tensor(synth.slot_entry_counts(w), device=device),
                    torch.as_tensor(w.head_tokens, device=device).contiguous(), dev_err=self.err)
                self.ranges = synth.slot_ranges(w, self.live_tokens.cpu().numpy())
            else:
                self.ranges = synth.slot_ranges(w)

    def append_tail(self, k, v, q=None):
        """One decode step's new tokens (k, v: n_new rows per table, rows t * n_new + i):
        placed as INT4 at each table's tail (the table as this side's reorder left it),
        written by kvq_quantize_append; the tables gain the pages the tail opened and
        the ranges are taken again from them.  q, if given, is the step's query."""
        w, kvq, dev = self.w, self.kvq, self.device
        n_new = k.shape[0] // w.n_tables
        tabs = self.tables.cpu().numpy()
        lists = synth.AppendLists()
        for t in range(w.n_tables):
            n = int(w.alloc.n_entries[t])
            pushed = w.alloc.append_tail(t, int(tabs[t, n - 1]) if n else None,
                                         np.arange(t * n_new, (t + 1) * n_new), lists)
            tabs[t, n:n + len(pushed)] = pushed
        a = lists.arrays()
        kvq.quantize_append(self.cache, k.to(dev), v.to(dev), rows4=torch.as_tensor(a["rows4"], device=dev),
                            slots4=torch.as_tensor(a["slots4"], device=dev), dev_err=self.err)
        self.tables.copy_(torch.as_tensor(tabs))
        self.ranges = _table_ranges(w, tabs)
        if q is not None:
            self.q = q.to(dev).contiguous()
        return a

    def plan(self, **kw):
        w = self.w
        return self.kvq.plan_splits(self.ranges, w.batch, w.hkv, w.heads_per_page, **kw)

    def plan_workers(self, workers_per_head, class_cost=None):
        w = self.w
        wph = np.broadcast_to(np.asarray(workers_per_head, np.int32), (w.n_tables * w.heads_per_page,))
        return self.kvq.plan_workers(self.ranges, w.batch, w.hkv, w.heads_per_page, wph, class_cost)

    def decode_shared(self, workers, groups, n_groups, offsets, out_dtype=torch.float32, work=None):
        """Shared-window decode + merge; returns (out, lse, part_o, part_lse, work)."""
        w, kvq = self.w, self.kvq
        n = workers.shape[0]
        wk = torch.as_tensor(workers, device=self.device).contiguous()
        gr = torch.as_tensor(groups, device=self.device).contiguous()
        off = torch.as_tensor(offsets, device=self.device)
        if work is None:
            work = kvq.decode_work(n_groups, self.device)
        part_o = torch.empty((max(n, 1), w.g, 128), dtype=torch.float32, device=self.device)
        part_lse = torch.empty((max(n, 1), w.g), dtype=torch.float32, device=self.device)
        out = torch.empty((w.batch, w.hq, 128), dtype=out_dtype, device=self.device)
        out_lse = torch.empty((w.batch, w.hq), dtype=torch.float32, device=self.device)
        kvq.decode_attn_shared(self.cache, self.q, w.hkv, self.tables, kvq.TABLE_PAGES, wk, gr, n_groups, work,
                               part_o, part_lse, dev_err=self.err)
        kvq.lse_merge(part_o, part_lse, n, off, w.batch, w.hq, w.hkv, out, out_lse)
        torch.cuda.synchronize()
        return out, out_lse, part_o[:n], part_lse[:n], work

    def decode(self, splits: np.ndarray, offsets: np.ndarray, out_dtype=torch.float32):
        w, kvq = self.w, self.kvq
        g = w.g
        n = splits.shape[0]
        sp = torch.as_tensor(splits, device=self.device).contiguous()
        off = torch.as_tensor(offsets, device=self.device)
        part_o = torch.empty((max(n, 1), g, 128), dtype=torch.float32, device=self.device)
        part_lse = torch.empty((max(n, 1), g), dtype=torch.float32, device=self.device)
        out = torch.empty((w.batch, w.hq, 128), dtype=out_dtype, device=self.device)
        out_lse = torch.empty((w.batch, w.hq), dtype=torch.float32, device=self.device)
        kvq.decode_attn(self.cache, self.q, w.hkv, self.tables,
                        kvq.TABLE_SLOTS if w.kind == synth.SLOTS else kvq.TABLE_PAGES,
                        sp, part_o, part_lse, dev_err=self.err)
        kvq.lse_merge(part_o, part_lse, n, off, w.batch, w.hq, w.hkv, out, out_lse)
        torch.cuda.synchronize()
        return out, out_lse, part_o[:n], part_lse[:n]


class OracleRun:
    """Route (oracle), place, quantize + append and reorder on the CPU oracle."""

    def __init__(self, w: synth.Workload, reorder=True, compact=False, anchor_fp8=False):
        from oracle import oracle
        self.orc, self.w = oracle, w
        self.flags = oracle_flags(w) if w.streams is not None else None
        self.lists = synth.place_all(w, lambda f: oracle.route(f)[0], self.flags)
        self.cache = oracle.Cache(w.heads_per_page, *w.n_pages, sentinel_slot=w.sentinel_slot,
                                  anchor_fp8=anchor_fp8)
        k, v, dt = _host_rows(w)
        self.k, self.v, self.dtype = k, v, dt
        row_stride = w.heads_per_page * 128
        if w.kind == synth.SLOTS and w.sentinel_slot >= 0:
            self.cache.append(k, v, dt, row_stride, 128, **synth.sentinel_lists(w).arrays())
        self.cache.append(k, v, dt, row_stride, 128, **self.lists.arrays())
        self.q = w.q.float().cpu().numpy()
        if w.kind == synth.PAGES:
            self.tables = w.alloc.tables.copy()
            self.class_counts = None
            self.ranges_before = _table_ranges(w, self.tables)
            if reorder:
                self.class_counts = self.cache.reorder(self.tables, w.alloc.n_entries)
            self.ranges = _table_ranges(w, self.tables)
            self.kind = oracle.PAGES
        else:
            self.tables = synth.slot_tables(w)
            self.kind = oracle.SLOTS
            self.class_counts = None
            self.live_tokens = None
            if compact:
                self.live_tokens = self.cache.compact_slots(self.tables, synth.slot_entry_counts(w),
                                                            w.head_tokens.astype(np.int32))
                self.ranges = synth.slot_ranges(w, self.live_tokens)
            else:
                self.ranges = synth.slot_ranges(w)

    def append_tail(self, k, v, q=None):
        """The same decode step on the oracle: its own tail placement on its own
        tables, its own append."""
        w = self.w
        n_new = k.shape[0] // w.n_tables
        lists = synth.AppendLists()
        for t in range(w.n_tables):
            n = int(w.alloc.n_entries[t])
            pushed = w.alloc.append_tail(t, int(self.tables[t, n - 1]) if n else None,
                                         np.arange(t * n_new, (t + 1) * n_new), lists)
            self.tables[t, n:n + len(pushed)] = pushed
        a = lists.arrays()
        kh, vh, dt = _host_pair(k, v)
        self.cache.append(kh, vh, dt, w.heads_per_page * 128, 128, rows4=a["rows4"], slots4=a["slots4"])
        self.ranges = _table_ranges(w, self.tables)
        if q is not None:
            self.q = q.float().cpu().numpy()
        return a

    def attend(self, n_threads=8):
        w = self.w
        return self.cache.attend(self.q, w.batch, w.hq, w.hkv, self.tables, self.kind, self.ranges,
                                 n_threads=n_threads)


def _host_rows(w):
    """Source rows as host numpy arrays plus the oracle dtype code (bf16 as uint16 bits)."""
    return _host_pair(w.k, w.v)


def _host_pair(k, v):
    if k.dtype == torch.bfloat16:
        kh = k.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
        vh = v.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
        return kh, vh, 1
    return k.float().cpu().contiguous().numpy(), v.float().cpu().contiguous().numpy(), 0
