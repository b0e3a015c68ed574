"""Seeded synthetic workloads for decode attention over a mixed-precision KV cache.

Shared by the tests, the benchmark and the smoke check, for both the GPU path and
the CPU oracle.  This module holds none of the method's arithmetic: no
quantization, no routing, no reorder, no attention and no merge.  It draws random
numbers, fixes shapes, and does the caller-side page bookkeeping a serving system
does around the cache (handing out physical pages and slots, recording which table
entry holds which tokens).

Workload shapes follow the pages' settings: TriAxialKV (mixed INT2/INT4 with G = 32
groups; Qwen3-8B and Qwen3-VL shapes), HyQuant (INT4 prefix plus FP16 anchors:
vertical-line tokens, a staging buffer and a W = 128 window) and Tangram/IntentKV
(ragged per-head budgets, head-group page tables, sentinel dead slots).  Values are
synthetic: no dataset, suite or model weight is involved.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional

import numpy as np
import torch

INT2, INT4, FP16 = 0, 1, 2          # precision classes (flags use the same numbers)
PAGE = 16
GROUP = 32
HEAD_DIM = 128
PAGES, SLOTS = 0, 1

RANGE_DTYPE = np.dtype([("table", "<i4"), ("head", "<i4"), ("cls", "<i4"),
                        ("tok_begin", "<i4"), ("tok_end", "<i4")])


# ----------------------------------------------------------------------------
# random streams
# ----------------------------------------------------------------------------

def np_rng(seed: int, *stream: int) -> np.random.Generator:
    """Independent numpy stream for (seed, stream ids)."""
    return np.random.default_rng([int(seed) & 0xFFFFFFFF, *[int(s) & 0xFFFFFFFF for s in stream]])


def torch_gen(seed: int, *stream: int, device="cpu") -> torch.Generator:
    """Independent torch stream for (seed, stream ids) on a device."""
    s = int(np_rng(seed, 0x7A11, *stream).integers(0, 2**62))
    g = torch.Generator(device=device)
    g.manual_seed(s)
    return g


def randn(shape, seed, *stream, device="cpu", std=1.0) -> torch.Tensor:
    t = torch.randn(shape, generator=torch_gen(seed, *stream, device=device),
                    device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t


# ----------------------------------------------------------------------------
# caller-side page bookkeeping
# ----------------------------------------------------------------------------

@dataclasses.dataclass
class AppendLists:
    """Destination lists of one append call (rows index the k / v row space)."""
    rows4: List[int] = dataclasses.field(default_factory=list)
    slots4: List[int] = dataclasses.field(default_factory=list)
    rows2: List[int] = dataclasses.field(default_factory=list)
    pages2: List[int] = dataclasses.field(default_factory=list)
    rows16: List[int] = dataclasses.field(default_factory=list)
    slots16: List[int] = dataclasses.field(default_factory=list)

    def arrays(self):
        a = lambda x: np.asarray(x, dtype=np.int32)  # noqa: E731
        return dict(rows4=a(self.rows4), slots4=a(self.slots4), rows2=a(self.rows2),
                    pages2=a(self.pages2), rows16=a(self.rows16), slots16=a(self.slots16))


class PageAllocator:
    """Hands out physical pages from shuffled free lists and records every table.

    Page ids use one id space: INT2 [0, n2), INT4 [n2, n2+n4), FP16 after.  INT2
    pages are handed out as aligned pairs (even, even+1): one 32-token group."""

    def __init__(self, n_pages, heads_per_page, n_tables, max_entries, seed, reserve_int4=0, ordered=False):
        self.n_pages = tuple(int(n) for n in n_pages)
        self.heads_per_page = heads_per_page
        r = np_rng(seed, 0xA110C)
        n2, n4, n16 = self.n_pages
        assert n2 % 2 == 0
        self.free2 = list((r.permutation(n2 // 2) * 2).astype(np.int64))
        ids4 = np.arange(n2 + reserve_int4, n2 + n4)
        self.free4 = list(r.permutation(ids4))
        self.free16 = list(r.permutation(np.arange(n2 + n4, n2 + n4 + n16)))
        if ordered:  # pages handed out in increasing id order (pop() takes the last)
            self.free2.sort(reverse=True)
            self.free4.sort(reverse=True)
            self.free16.sort(reverse=True)
        self.reserved4 = list(range(n2, n2 + reserve_int4))
        self.ordered = ordered
        self.max_entries = max_entries
        self.tables = np.full((n_tables, max_entries), -1, dtype=np.int32)
        self.n_entries = np.zeros(n_tables, dtype=np.int32)
        self.fill = [[] for _ in range(n_tables)]          # tokens per entry
        self.entry_cls = [[] for _ in range(n_tables)]
        self.open = [dict() for _ in range(n_tables)]      # cls -> entry index of open page
        self.tokens = np.zeros((n_tables, 3), dtype=np.int64)

    def _push(self, t, page, cls, fill):
        e = int(self.n_entries[t])
        assert e < self.max_entries, "table capacity exceeded"
        self.tables[t, e] = page
        self.n_entries[t] += 1
        self.fill[t].append(fill)
        self.entry_cls[t].append(cls)
        return e

    def place(self, t, classes, rows, lists: AppendLists, new_page=False):
        """Give every token of one append call (classes already routed) a place.

        classes / rows: per token, in position order.  new_page: start a fresh
        page for the first INT4 / FP16 token (a new buffer segment)."""
        classes = np.asarray(classes)
        rows = np.asarray(rows)
        if new_page:
            self.open[t].pop(INT4, None)
            self.open[t].pop(FP16, None)
        in_group = 0
        for c, row in zip(classes.tolist(), rows.tolist()):
            if c == INT2:
                if in_group == 0:
                    p = int(self.free2.pop())
                    self._push(t, p, INT2, 16)
                    self._push(t, p + 1, INT2, 16)
                    lists.pages2.append(p)
                lists.rows2.append(row)
                in_group = (in_group + 1) % GROUP
                self.tokens[t, INT2] += 1
            else:
                e = self.open[t].get(c)
                if e is None or self.fill[t][e] == PAGE:
                    p = int((self.free4 if c == INT4 else self.free16).pop())
                    e = self._push(t, p, c, 0)
                    self.open[t][c] = e
                slot = int(self.tables[t, e]) * PAGE + self.fill[t][e]
                self.fill[t][e] += 1
                self.tokens[t, c] += 1
                if c == INT4:
                    lists.rows4.append(row)
                    lists.slots4.append(slot)
                else:
                    lists.rows16.append(row)
                    lists.slots16.append(slot)
        assert in_group == 0, "INT2 tokens of an append call must fill whole groups"

    def ranges(self, t, heads):
        """Token ranges of table t in its current entry order (one class per range)."""
        out = []
        start = None
        cls_run = None
        for e, (c, f) in enumerate(zip(self.entry_cls[t], self.fill[t])):
            if start is not None and c == cls_run and prev_full:
                end = e * PAGE + f
            else:
                if start is not None:
                    out.append((cls_run, start, end))
                start, cls_run, end = e * PAGE, c, e * PAGE + f
            prev_full = f == PAGE
        if start is not None:
            out.append((cls_run, start, end))
        return [(t, h, c, b, e) for h in heads for (c, b, e) in out if e > b]


    def append_tail(self, t, last_page, rows, lists: AppendLists):
        """Place decode-time tokens of table t as INT4 at the table's tail: into its
        last entry while that is an INT4 page with room (last_page: the page id the
        caller's table ends with now, e.g. as a reorder left it), then into fresh INT4
        pages pushed at the end of the table.  Returns the page ids pushed, in order."""
        n2, n4, _ = self.n_pages
        e = None
        if last_page is not None and n2 <= last_page < n2 + n4:
            e = int(np.flatnonzero(self.tables[t, :self.n_entries[t]] == last_page)[0])
        pushed = []
        for row in np.asarray(rows).tolist():
            if e is None or self.fill[t][e] == PAGE:
                p = int(self.free4.pop())
                e = self._push(t, p, INT4, 0)
                pushed.append(p)
            lists.rows4.append(row)
            lists.slots4.append(int(self.tables[t, e]) * PAGE + self.fill[t][e])
            self.fill[t][e] += 1
            self.tokens[t, INT4] += 1
        return pushed

    def ranges_in_order(self, t, pages, heads):
        """Token ranges of table t when its entries hold `pages` (page ids, e.g. the
        table as a reorder left it): the caller's record of where its tokens sit, from
        the fill it gave each page and the class of each page id."""
        fill_of = {int(self.tables[t, e]): f for e, f in enumerate(self.fill[t])}
        n2, n4, _ = self.n_pages
        saved = (self.entry_cls[t], self.fill[t])
        pages = [int(p) for p in pages]
        self.entry_cls[t] = [INT2 if p < n2 else INT4 if p < n2 + n4 else FP16 for p in pages]
        self.fill[t] = [fill_of[p] for p in pages]
        try:
            return self.ranges(t, heads)
        finally:
            self.entry_cls[t], self.fill[t] = saved


def ranges_array(items) -> np.ndarray:
    return np.array(list(items), dtype=RANGE_DTYPE).reshape(-1)


def class_ordered_ranges(t, heads, tokens_per_class):
    """Ranges of a table whose entries are grouped INT2, INT4, FP16 (in that order)
    and whose only partially filled page per class is the last one of the class."""
    out, page0 = [], 0
    for c in (INT2, INT4, FP16):
        n = int(tokens_per_class[c])
        if n:
            out.append((c, page0 * PAGE, page0 * PAGE + n))
        page0 += -(-n // PAGE)
    return [(t, h, c, b, e) for h in heads for (c, b, e) in out]


# ----------------------------------------------------------------------------
# workloads
# ----------------------------------------------------------------------------

@dataclasses.dataclass
class Workload:
    name: str
    seed: int
    batch: int
    hq: int
    hkv: int
    heads_per_page: int
    kind: int                       # PAGES or SLOTS
    src_dtype: torch.dtype          # dtype of K / V source rows
    q_dtype: torch.dtype
    k: torch.Tensor                 # [R, heads_per_page, 128]
    v: torch.Tensor
    q: torch.Tensor                 # [batch, hq, 128]
    n_pages: tuple                  # pages per class
    alloc: PageAllocator
    calls: list                     # per append call: (table, flags np.uint8, rows np.int32, new_page)
    sentinel_slot: int = -1
    dead_entries: Optional[list] = None  # per table: entry indices redirected to the sentinel
    head_tokens: Optional[np.ndarray] = None  # [n_tables, heads_per_page] tokens read per head
    head_budget: Optional[np.ndarray] = None  # [hkv] retained fraction per KV head (ragged tables)
    call_spans: Optional[list] = None         # per call with flags None: its token span (c0, c1) in the request
    streams: Optional[list] = None            # per request (table): AgenticStream whose tags give the flags
    count_streams: Optional[list] = None      # the streams whose aggregate tag counts fix the widths
    distortion: Optional[tuple] = None        # (d2, d4) per tag
    budget_bits: float = 0.0
    note: str = ""

    @property
    def n_tables(self):
        return self.alloc.tables.shape[0]

    @property
    def g(self):
        return self.hq // self.hkv


def _bf16(t):
    return t.to(torch.bfloat16)


def _unit_flags(n_tokens, frac_int2, rng):
    """Per-token flags from 32-token units, INT2 units a fraction of all, shuffled."""
    units = n_tokens // GROUP
    n2 = int(round(frac_int2 * units))
    u = np.array([INT2] * n2 + [INT4] * (units - n2), dtype=np.uint8)
    rng.shuffle(u)
    return np.repeat(u, GROUP)


def tiny(seed=0, device="cpu"):
    """Tiny decode step: batch 1, Hq 4 / Hkv 1, 256 tokens = 6 INT2 groups + 64 INT4
    tokens in shuffled 32-token units; fp32 K, V, q ~ N(0,1); four K outlier
    channels x10."""
    B, hq, hkv, T = 1, 4, 1, 256
    rng = np_rng(seed, 1)
    k = randn((T, 1, HEAD_DIM), seed, 2, device=device)
    v = randn((T, 1, HEAD_DIM), seed, 3, device=device)
    out_ch = torch.as_tensor(np.sort(rng.choice(HEAD_DIM, 4, replace=False)), device=device)
    k[:, :, out_ch] *= 10.0
    q = randn((B, hq, HEAD_DIM), seed, 4, device=device)
    flags = np.repeat(rng.permutation(np.array([INT2] * 6 + [INT4] * 2, np.uint8)), GROUP)
    n_pages = (12, 4, 0)
    alloc = PageAllocator(n_pages, 1, 1, 16, seed)
    return Workload("tiny", seed, B, hq, hkv, 1, PAGES, torch.float32, torch.float32, k, v, q,
                    n_pages, alloc, [(0, flags, np.arange(T, dtype=np.int32), False)])


def qwen3_8b(seed=2, batch=16, n_tokens=32768, device="cpu", frac_int2=0.7, layer=0, ordered_pages=False):
    """Qwen3-8B-shaped decode: Hq 32 / Hkv 8 (g = 4), d 128, one page table per request
    holding all 8 KV heads, 16-token pages.  Per request 70 % INT2 / 30 % INT4 tokens in
    shuffled runs of 32; bf16 K, V ~ N(0,1) with 1 % of K channels (10 of 1024 head
    channels) x8; bf16 q."""
    hq, hkv, H = 32, 8, 8
    assert n_tokens % GROUP == 0
    rng = np_rng(seed, 11, layer)
    flags = [_unit_flags(n_tokens, frac_int2, np_rng(seed, 12, t)) for t in range(batch)]
    n2 = sum(int((f == INT2).sum()) for f in flags) // PAGE
    n4 = sum(-(-int((f == INT4).sum()) // PAGE) for f in flags)
    k = randn((batch * n_tokens, H, HEAD_DIM), seed, 13, layer, device=device)
    v = randn((batch * n_tokens, H, HEAD_DIM), seed, 14, layer, device=device)
    n_out = max(1, round(0.01 * H * HEAD_DIM))
    hc = rng.choice(H * HEAD_DIM, n_out, replace=False)
    kf = k.view(batch * n_tokens, H * HEAD_DIM)
    kf[:, torch.as_tensor(np.sort(hc), device=device)] *= 8.0
    k, v = _bf16(k), _bf16(v)
    q = _bf16(randn((batch, hq, HEAD_DIM), seed, 15, layer, device=device))
    max_entries = n_tokens // PAGE
    alloc = PageAllocator((n2, n4, 0), H, batch, max_entries, seed, ordered=ordered_pages)
    calls = [(t, flags[t], np.arange(t * n_tokens, (t + 1) * n_tokens, dtype=np.int32), False)
             for t in range(batch)]
    return Workload("qwen3_8b", seed, batch, hq, hkv, H, PAGES, torch.bfloat16, torch.bfloat16,
                    k, v, q, (n2, n4, 0), alloc, calls,
                    note=f"{batch}x{n_tokens} tokens, {frac_int2:.0%} INT2 units")


# Tag axes of the agentic workload (TriAxialKV key design 1): temporal (turns from the
# end: current, one before, two before, older), modal (text, image), semantic role
# (inst, user, assistant, reasoning, tool_call, obs, delim).  Tag index =
# (temporal * N_MODAL + modal) * N_SEMANTIC + semantic.  The tags themselves are read
# from the token streams by the library and by the oracle, each with its own code.
N_TEMPORAL, N_MODAL, N_SEMANTIC = 4, 2, 7
N_TAGS = N_TEMPORAL * N_MODAL * N_SEMANTIC
# Synthetic distortion table (input data of the width allocation, in place of the
# offline calibration the page describes): per-axis 2-bit weights, semantic axis
# dominant and its first value (inst) highest; the 4-bit distortion is 1/25 of it.
_D_SEM = np.array([8.0, 4.0, 2.0, 1.5, 1.0, 0.7, 0.5])
_D_MOD = np.array([1.0, 0.6])
_D_TMP = np.array([4.0, 2.0, 1.3, 1.0])


def agentic_distortion():
    """(d2, d4) float64 [N_TAGS] in tag-index order."""
    d2 = (_D_TMP[:, None, None] * _D_MOD[None, :, None] * _D_SEM[None, None, :]).reshape(-1)
    return d2, d2 / 25.0


@dataclasses.dataclass
class AgenticStream:
    """One request's context as template token ids: tokens int32 [n], markers {token id:
    event name}, and the rows of tokens generated inside image spans (K, V there carry
    twice the variance)."""
    tokens: np.ndarray
    markers: dict
    image: np.ndarray        # bool [n]


def agentic_conversation(length, rng, vocab=900) -> AgenticStream:
    """A seeded multi-turn agent context of exactly `length` tokens: a system prompt
    (tool specifications), then 12-40 turns of near-equal share, each a user message
    (an image span in 30 % of them), an assistant reply with a think span (70 %) and 0-2
    tool calls each answered by an observation (20 % with an image), text in runs of
    geometric length; boundary tokens are ids vocab .. vocab + 10.  Truncated at
    `length` (a span cut there stays open)."""
    markers = {vocab + i: e for i, e in enumerate(_STREAM_EVENTS)}
    mid = {e: vocab + i for i, e in enumerate(_STREAM_EVENTS)}
    toks, img = [], []

    def mark(name):
        toks.append(np.array([mid[name]], np.int32))
        img.append(np.zeros(1, bool))

    def text(n, image=False):
        n = max(1, int(n))
        toks.append(rng.integers(0, vocab, n).astype(np.int32))
        img.append(np.full(n, image))

    def span(name, n, image=False):
        mark(name + "_begin")
        text(n, image)
        mark(name + "_end")

    n_turns = int(rng.integers(12, 41))
    share = length / (n_turns + 0.5)
    mark("system"); text(0.5 * share); mark("end")
    for _ in range(n_turns):
        mark("user"); text(rng.geometric(1.0 / (0.18 * share)))
        if rng.random() < 0.3:
            span("image", rng.geometric(1.0 / (0.15 * share)), image=True)
        mark("end")
        mark("assistant")
        if rng.random() < 0.7:
            span("think", rng.geometric(1.0 / (0.2 * share)))
        text(rng.geometric(1.0 / (0.15 * share)))
        for _ in range(int(rng.integers(0, 3))):
            span("tool_call", rng.geometric(1.0 / (0.07 * share)))
            mark("end")
            mark("observation"); text(rng.geometric(1.0 / (0.1 * share)))
            if rng.random() < 0.2:
                span("image", rng.geometric(1.0 / (0.1 * share)), image=True)
            mark("end")
            mark("assistant"); text(rng.geometric(1.0 / (0.05 * share)))
        mark("end")
    tokens, image = np.concatenate(toks), np.concatenate(img)
    while tokens.shape[0] < length:  # a long tail of the last reply
        tokens = np.concatenate([tokens, rng.integers(0, vocab, length - tokens.shape[0]).astype(np.int32)])
        image = np.concatenate([image, np.zeros(length - image.shape[0], bool)])
    return AgenticStream(tokens[:length], markers, image[:length])


def qwen3_vl_agentic(seed=3, batch=8, lo=65536, hi=131072, device="cpu", chunk=8192,
                     budget_bits=2.6, layer=0):
    """Qwen3-VL-32B-shaped agentic decode: Hq 64 / Hkv 8 (g = 8), d 128, one page table
    per request holding all 8 KV heads, contexts uniform in [lo, hi].  Each request is a
    synthetic agent conversation (agentic_conversation) whose tri-axis tags, widths at
    `budget_bits` (one tag -> width map for the batch, from its aggregate tag counts and
    the agentic_distortion table) and routing flags are made by the side that runs it;
    tokens are appended in `chunk`-token calls, so every call leaves its own INT4
    residual.  bf16 K, V ~ N(0,1), N(0, 2) (variance) on image-span tokens; bf16 q.  Pool
    sizes are upper bounds (every token INT2, or every token INT4)."""
    hq, hkv, H = 64, 8, 8
    rng = np_rng(seed, 31)
    lens = rng.integers(lo, hi + 1, batch)
    streams = [agentic_conversation(int(n), np_rng(seed, 32, b)) for b, n in enumerate(lens)]
    rows_total = int(lens.sum())
    k = randn((rows_total, H, HEAD_DIM), seed, 33, layer, device=device)
    v = randn((rows_total, H, HEAD_DIM), seed, 34, layer, device=device)
    calls, spans, n2, n4, row = [], [], 0, 0, 0
    image_rows = []
    for b, st in enumerate(streams):
        n = int(lens[b])
        image_rows.append(row + np.nonzero(st.image)[0])
        for c0 in range(0, n, chunk):
            c1 = min(n, c0 + chunk)
            calls.append((b, None, np.arange(row + c0, row + c1, dtype=np.int32), False))
            spans.append((c0, c1))
            n2 += 2 * ((c1 - c0) // GROUP)
            n4 += -(-(c1 - c0) // PAGE)
        row += n
    img = torch.as_tensor(np.concatenate(image_rows), device=device, dtype=torch.long)
    k[img] *= math.sqrt(2.0)
    v[img] *= math.sqrt(2.0)
    k, v = _bf16(k), _bf16(v)
    q = _bf16(randn((batch, hq, HEAD_DIM), seed, 35, layer, device=device))
    max_entries = -(-int(hi) // PAGE) + -(-int(hi) // chunk)  # every call may end on a partial INT4 page
    alloc = PageAllocator((n2, n4, 0), H, batch, max_entries, seed)
    return Workload("qwen3_vl_agentic", seed, batch, hq, hkv, H, PAGES, torch.bfloat16, torch.bfloat16,
                    k, v, q, (n2, n4, 0), alloc, calls, call_spans=spans, streams=streams,
                    count_streams=streams, distortion=agentic_distortion(), budget_bits=budget_bits,
                    note=f"{batch} requests of {int(lens.min())}..{int(lens.max())} tokens, "
                         f"tri-axis tags at {budget_bits} bits, {chunk}-token appends")


def hybrid_anchor(seed=4, batch=32, n_tokens=65536, device="cpu", window=128, staging=64,
                  vl_ratio=0.05, layer=0, vl_positions=None):
    """Hybrid FP16-anchor decode (Llama-3.1-8B shape): Hq 32 / Hkv 8, one table per
    (request, KV head).  Per head: an INT4 prefix, FP16 vertical-line tokens (top 5 %
    of the non-window prefix by a Zipf(1.1) column mass over randomly permuted ranks,
    or the given vl_positions[table]: sorted positions in the non-window prefix), a
    64-token FP16 staging buffer and a W = 128 FP16 window; each anchor segment starts
    on its own page.  bf16 K, V ~ N(0,1); table t holds rows t * n_tokens + position."""
    hq, hkv, H = 32, 8, 1
    n_tables = batch * hkv
    frozen = n_tokens - staging               # tokens present at the freeze point
    nonwin = frozen - window
    n_vl = int(round(vl_ratio * nonwin))
    n_q = nonwin - n_vl
    k = _bf16(randn((n_tables * n_tokens, 1, HEAD_DIM), seed, 41, layer, device=device))
    v = _bf16(randn((n_tables * n_tokens, 1, HEAD_DIM), seed, 42, layer, device=device))
    q = _bf16(randn((batch, hq, HEAD_DIM), seed, 43, layer, device=device))
    pg = lambda n: -(-n // PAGE)  # noqa: E731
    n4 = n_tables * pg(n_q)
    n16 = n_tables * (pg(n_vl) + pg(staging) + pg(window))
    max_entries = pg(n_q) + pg(n_vl) + pg(staging) + pg(window)
    alloc = PageAllocator((0, n4, n16), H, n_tables, max_entries, seed)
    calls = []
    ranks_mass = np.arange(1, nonwin + 1, dtype=np.float64) ** -1.1   # Zipf(1.1) by rank
    for t in range(n_tables):
        if vl_positions is None:
            r = np_rng(seed, 44, t)
            rank_of_pos = r.permutation(nonwin)            # random rank per position
            mass = ranks_mass[rank_of_pos]
            vl = np.sort(np.argsort(-mass, kind="stable")[:n_vl])
        else:
            vl = np.asarray(vl_positions[t], np.int64)
            assert vl.shape == (n_vl,) and np.all(np.diff(vl) > 0) and vl[0] >= 0 and vl[-1] < nonwin
        is_vl = np.zeros(nonwin, bool)
        is_vl[vl] = True
        base = t * n_tokens
        pos = np.arange(nonwin)
        rows_q = (base + pos[~is_vl]).astype(np.int32)
        rows_vl = (base + pos[is_vl]).astype(np.int32)
        rows_win = (base + nonwin + np.arange(window)).astype(np.int32)
        rows_stage = (base + frozen + np.arange(staging)).astype(np.int32)
        calls.append((t, np.full(n_q, INT4, np.uint8), rows_q, False))
        calls.append((t, np.full(n_vl, FP16, np.uint8), rows_vl, True))
        calls.append((t, np.full(staging, FP16, np.uint8), rows_stage, True))
        calls.append((t, np.full(window, FP16, np.uint8), rows_win, True))
    return Workload("hybrid_anchor", seed, batch, hq, hkv, H, PAGES, torch.bfloat16,
                    torch.bfloat16, k, v, q, (0, n4, n16), alloc, calls,
                    note=f"per head {n_q} INT4 + {n_vl} VL + {staging} staging + {window} window")


def ragged_lengths(seed=5, batch=64, lo=4096, hi=131072):
    """Context lengths of the ragged workload: log-uniform in [lo, hi]."""
    rng = np_rng(seed, 51)
    return np.round(np.exp(rng.uniform(math.log(lo), math.log(hi), batch))).astype(np.int64)


def ragged_dead(seed=5, batch=64, lo=4096, hi=131072, device="cpu", dead_frac=0.2, layer=0):
    """Ragged per-head budgets with sentinel dead slots: Hq 32 / Hkv 8, context lengths
    log-uniform in [lo, hi]; per-KV-head retained fraction r_h = 0.1 + 0.9 h / 7; heads
    in 4 groups of 2 with one slot-map table per (request, group) of length
    ceil(max r_h * len); each head reads its first ceil(r_h * len) entries; slots are
    handed out in shuffled 16-slot pages; 20 % of each table's entries point at the
    sentinel dead slot.  INT4 per-token."""
    hq, hkv, H = 32, 8, 2
    groups = hkv // H
    lens = ragged_lengths(seed, batch, lo, hi)  # structure is the same in every layer
    r_h = 0.1 + 0.9 * np.arange(hkv) / (hkv - 1)
    n_tables = batch * groups
    head_tokens = np.zeros((n_tables, H), np.int32)
    tlen = np.zeros(n_tables, np.int64)
    for b in range(batch):
        for gr in range(groups):
            t = b * groups + gr
            for h in range(H):
                head_tokens[t, h] = int(math.ceil(r_h[gr * H + h] * lens[b]))
            tlen[t] = head_tokens[t].max()
    pg = lambda n: -(-int(n) // PAGE)  # noqa: E731
    n4 = 1 + sum(pg(n) for n in tlen)       # page 0 of the INT4 pool holds the sentinel
    max_entries = int(tlen.max())
    rows_total = int(tlen.sum()) + 1
    k = randn((rows_total, H, HEAD_DIM), seed, 52, layer, device=device)
    v = randn((rows_total, H, HEAD_DIM), seed, 53, layer, device=device)
    k[0] = -1.0e4                            # sentinel row: K = -1e4, V = 0
    v[0] = 0.0
    k, v = _bf16(k), _bf16(v)
    q = _bf16(randn((batch, hq, HEAD_DIM), seed, 54, layer, device=device))
    alloc = PageAllocator((0, n4, 0), H, n_tables, max_entries, seed, reserve_int4=1)
    calls, dead, row = [], [], 1
    for t in range(n_tables):
        n = int(tlen[t])
        calls.append((t, np.full(n, INT4, np.uint8), np.arange(row, row + n, dtype=np.int32), True))
        row += n
        dead.append(np.sort(np_rng(seed, 55, t).choice(n, int(round(dead_frac * n)), replace=False)))
    sentinel = alloc.reserved4[0] * PAGE
    return Workload("ragged_dead", seed, batch, hq, hkv, H, SLOTS, torch.bfloat16, torch.bfloat16,
                    k, v, q, (0, n4, 0), alloc, calls, sentinel_slot=sentinel, dead_entries=dead,
                    head_tokens=head_tokens, head_budget=r_h.astype(np.float32),
                    note=f"lengths {int(lens.min())}..{int(lens.max())}, {dead_frac:.0%} dead")


def subset(w: Workload, requests, device="cpu") -> Workload:
    """The same workload restricted to some requests (tables of those requests, their
    source rows and queries), with a fresh allocator sized for them.  Entry structure
    per table is unchanged; physical page ids differ."""
    if w.kind == SLOTS:
        return _subset_slots(w, requests, device)
    tpr = w.hkv // w.heads_per_page
    tabs = [b * tpr + i for b in requests for i in range(tpr)]
    rows, calls, new_calls, spans = [], [], [], []
    for i, (t, flags, r, new_page) in enumerate(w.calls):
        if t in tabs:
            calls.append((tabs.index(t), flags, r, new_page))
            spans.append(w.call_spans[i] if w.call_spans else None)
    all_rows = np.unique(np.concatenate([c[2] for c in calls]))
    remap = {int(r): i for i, r in enumerate(all_rows.tolist())}
    for (t, flags, r, new_page) in calls:
        new_calls.append((t, flags, np.array([remap[int(x)] for x in r.tolist()], np.int32), new_page))
    idx = torch.as_tensor(all_rows, device=w.k.device, dtype=torch.long)
    k = w.k.index_select(0, idx).to(device)
    v = w.v.index_select(0, idx).to(device)
    q = w.q[torch.as_tensor(list(requests), device=w.q.device)].to(device)
    # Pool sizes: upper bounds from the flags alone (whatever the routing decides).
    n2 = n4 = n16 = 0
    for (_, flags, rws, _) in new_calls:
        if flags is None:  # flags made by the running side: any split of the call's tokens
            n2 += 2 * (len(rws) // GROUP)
            n4 += -(-len(rws) // PAGE) + 1
            continue
        c0, c1, c2 = (int((flags == c).sum()) for c in (INT2, INT4, FP16))
        n2 += 2 * (c0 // GROUP)
        n4 += -(-(c0 + c1) // PAGE) + 1
        n16 += -(-c2 // PAGE) + 1
    n_pages = (n2, n4, n16)
    alloc = PageAllocator(n_pages, w.heads_per_page, len(tabs), w.alloc.max_entries, w.seed + 1000)
    extra = {}
    if w.streams is not None:  # the widths stay those of the whole batch
        extra = dict(call_spans=spans, streams=[w.streams[b] for b in requests], count_streams=w.count_streams)
    return dataclasses.replace(w, batch=len(requests), k=k, v=v, q=q, n_pages=n_pages, alloc=alloc,
                               calls=new_calls, note=w.note + f" (requests {list(requests)})", **extra)


def _subset_slots(w: Workload, requests, device="cpu") -> Workload:
    """subset() for slot-map workloads: row 0 (the sentinel row) is kept as row 0."""
    tpr = w.hkv // w.heads_per_page
    tabs = [b * tpr + i for b in requests for i in range(tpr)]
    calls = [(tabs.index(t), f, r, n) for (t, f, r, n) in w.calls if t in tabs]
    all_rows = np.unique(np.concatenate([np.array([0], np.int32)] + [c[2] for c in calls]))
    remap = np.zeros(int(all_rows.max()) + 1, np.int64)
    remap[all_rows] = np.arange(len(all_rows))
    new_calls = [(t, f, remap[r].astype(np.int32), n) for (t, f, r, n) in calls]
    idx = torch.as_tensor(all_rows, device=w.k.device, dtype=torch.long)
    k = w.k.index_select(0, idx).to(device)
    v = w.v.index_select(0, idx).to(device)
    q = w.q[torch.as_tensor(list(requests), device=w.q.device)].to(device)
    n4 = 1 + sum(-(-len(c[1]) // PAGE) for c in new_calls)
    alloc = PageAllocator((0, n4, 0), w.heads_per_page, len(tabs), w.alloc.max_entries, w.seed + 1000,
                          reserve_int4=1)
    return dataclasses.replace(w, batch=len(requests), k=k, v=v, q=q, n_pages=(0, n4, 0), alloc=alloc,
                               calls=new_calls, sentinel_slot=alloc.reserved4[0] * PAGE,
                               dead_entries=[w.dead_entries[t] for t in tabs],
                               head_tokens=w.head_tokens[tabs].copy(),
                               note=w.note + f" (requests {list(requests)})")


def reserve_tail(w: Workload, tail_tokens) -> Workload:
    """The same page-table workload with room for `tail_tokens` decode-time tokens per
    table: INT4 pool and table width grown by the pages they may open (a fresh
    allocator, so placement is redone from the start by whoever runs it)."""
    assert w.kind == PAGES
    extra = -(-int(tail_tokens) // PAGE)
    n2, n4, n16 = w.n_pages
    n_pages = (n2, n4 + extra * w.n_tables, n16)
    alloc = PageAllocator(n_pages, w.heads_per_page, w.n_tables, w.alloc.max_entries + extra, w.seed,
                          ordered=w.alloc.ordered)
    return dataclasses.replace(w, n_pages=n_pages, alloc=alloc)


def tail_rows(w: Workload, step, n_new, device="cpu"):
    """Source rows of one decode step: `n_new` new tokens per table (rows t * n_new + i,
    all heads of the table) and the step's query.  K, V ~ N(0,1) and q ~ N(0,1) in the
    workload's dtypes, seeded by the step."""
    rows = w.n_tables * n_new
    k = randn((rows, w.heads_per_page, HEAD_DIM), w.seed, 91, step, device=device).to(w.src_dtype)
    v = randn((rows, w.heads_per_page, HEAD_DIM), w.seed, 92, step, device=device).to(w.src_dtype)
    q = randn((w.batch, w.hq, HEAD_DIM), w.seed, 93, step, device=device).to(w.q_dtype)
    return k, v, q


# ----------------------------------------------------------------------------
# turning a routed workload into append lists, tables and ranges
# ----------------------------------------------------------------------------

def place_all(w: Workload, route_fn, flags=None):
    """Route every append call with route_fn(flags) -> classes and give each token a
    place.  A call without flags of its own takes them from flags[table] (the routing
    flags the running side made for the request, e.g. from its tags) over its span.
    Returns the append lists of the whole workload (one list set)."""
    lists = AppendLists()
    for i, (t, f, rows, new_page) in enumerate(w.calls):
        if f is None:
            c0, c1 = w.call_spans[i]
            f = np.ascontiguousarray(flags[t][c0:c1], np.uint8)
        classes = route_fn(f)
        w.alloc.place(t, classes, rows, lists, new_page=new_page)
    return lists


def slot_tables(w: Workload):
    """Slot-map tables of a slot-mode workload after placement: entry e of table t
    holds its token's slot, or the sentinel slot if the entry is dead."""
    assert w.kind == SLOTS
    nt, me = w.alloc.tables.shape
    out = np.full((nt, me), -1, np.int32)
    for t in range(nt):
        pages = w.alloc.tables[t, : w.alloc.n_entries[t]]
        n = int(sum(w.alloc.fill[t]))
        e = np.arange(n)
        out[t, :n] = pages[e // PAGE] * PAGE + e % PAGE
        out[t, w.dead_entries[t]] = w.sentinel_slot
    return out


def slot_entry_counts(w: Workload):
    """Entries per slot-map table (the longest head prefix of the table)."""
    assert w.kind == SLOTS
    return np.array([int(sum(w.alloc.fill[t])) for t in range(w.n_tables)], np.int32)


def slot_ranges(w: Workload, head_tokens=None):
    """One INT4 range [0, n) per (table, head); n = the workload's head_tokens, or the
    given per-(table, head) counts (the live counts of compacted tables)."""
    ht = w.head_tokens if head_tokens is None else np.asarray(head_tokens)
    items = []
    for t in range(w.n_tables):
        for h in range(w.heads_per_page):
            items.append((t, h, INT4, 0, int(ht[t, h])))
    return ranges_array(items)


def sentinel_lists(w: Workload):
    """Append lists that write the sentinel row (row 0) into the sentinel slot."""
    return AppendLists(rows4=[0], slots4=[w.sentinel_slot])


@dataclasses.dataclass
class PrefillKQ:
    """Keys of a finished prefill and its tail queries, padded to a batch."""
    k: torch.Tensor          # [batch, max_tokens, hkv, 128]
    q_tail: torch.Tensor     # [batch, max_tail, hq, 128]
    n_tokens: np.ndarray     # int32 [batch]
    n_tail: np.ndarray       # int32 [batch]
    note: str


def vl_prefill(seed=6, batch=32, n_tokens=65536, hkv=8, hq=32, max_tail=64, lengths=None, n_tail=None,
               planted=0.03, dtype=torch.bfloat16, device="cpu") -> PrefillKQ:
    """Keys and tail queries shaped like the hybrid-anchor prefill (Llama-3.1-8B:
    Hq 32 / Hkv 8, 65536 tokens, 64 tail queries).  K, q ~ N(0, 1); the tail queries of
    each (request, KV-head group) share a random direction c (q = c + noise), and a
    seeded `planted` fraction of each head's tokens carries 4 c / |c| on top of its key,
    the columns many queries attend to.  `lengths` / `n_tail` (per request) may be
    ragged; rows past a request's length are zero."""
    g = hq // hkv
    lens = np.full(batch, n_tokens, np.int64) if lengths is None else np.asarray(lengths, np.int64)
    tails = np.full(batch, max_tail, np.int64) if n_tail is None else np.asarray(n_tail, np.int64)
    mt = int(lens.max()) if batch else 0
    c = randn((batch, 1, hkv, 1, 128), seed, 61, device=device)
    q = randn((batch, max_tail, hkv, g, 128), seed, 62, device=device) + c
    k = randn((batch, mt, hkv, 128), seed, 63, device=device)
    unit = (c / c.norm(dim=-1, keepdim=True)).reshape(batch, 1, hkv, 128)
    mark = torch.rand((batch, mt, hkv, 1), generator=torch_gen(seed, 64, device=device), device=device) < planted
    k.add_(mark.float() * 4.0 * unit)
    for b in range(batch):
        k[b, int(lens[b]):] = 0.0
        q[b, int(tails[b]):] = 0.0
    q = q.reshape(batch, max_tail, hq, 128)
    return PrefillKQ(k.to(dtype).contiguous(), q.to(dtype).contiguous(), lens.astype(np.int32),
                     tails.astype(np.int32), f"{batch} requests, {mt} tokens max, Hq {hq} / Hkv {hkv}, "
                     f"{max_tail} tail queries, {planted:.0%} planted lines")


@dataclasses.dataclass
class TokenStream:
    """Token ids of a synthetic agentic conversation and the template's boundary ids."""
    tokens: np.ndarray       # int32 [n]
    markers: dict            # token id -> event name (system, user, assistant, ...)


_STREAM_EVENTS = ("system", "user", "assistant", "observation", "end", "think_begin", "think_end",
                  "tool_call_begin", "tool_call_end", "image_begin", "image_end")


def agentic_token_stream(seed=0, n_turns=8, tokens_per_turn=400, vocab=900) -> TokenStream:
    """A seeded multi-turn agent conversation as token ids: a system prompt, then per turn
    a user message (sometimes with an image span), an assistant reply with think and
    tool-call spans, and tool observations (sometimes with images).  Boundary tokens are
    ids vocab .. vocab + 10; about 5 % of spans are left open or closed twice, as
    truncated or malformed template output would."""
    rng = np_rng(seed, 71)
    markers = {vocab + i: e for i, e in enumerate(_STREAM_EVENTS)}
    mid = {e: vocab + i for i, e in enumerate(_STREAM_EVENTS)}
    out = []
    text = lambda n: out.extend(rng.integers(0, vocab, max(1, int(n))).tolist())  # noqa: E731

    def span(name, n):
        out.append(mid[name + "_begin"])
        text(n)
        if rng.random() > 0.05:
            out.append(mid[name + "_end"])
        if rng.random() < 0.05:
            out.append(mid[name + "_end"])

    out.append(mid["system"]); text(tokens_per_turn); out.append(mid["end"])
    for _ in range(n_turns):
        m = tokens_per_turn
        out.append(mid["user"]); text(rng.exponential(m / 4))
        if rng.random() < 0.3:
            span("image", rng.exponential(m / 3))
        out.append(mid["end"])
        out.append(mid["assistant"])
        if rng.random() < 0.7:
            span("think", rng.exponential(m / 4))
        text(rng.exponential(m / 8))
        for _ in range(int(rng.integers(0, 3))):
            span("tool_call", rng.exponential(m / 16))
            out.append(mid["end"])
            out.append(mid["observation"]); text(rng.exponential(m / 4))
            if rng.random() < 0.2:
                span("image", rng.exponential(m / 4))
            out.append(mid["end"])
            out.append(mid["assistant"]); text(rng.exponential(m / 16))
        out.append(mid["end"])
    return TokenStream(np.array(out, np.int32), markers)


def prefill_qkv(seed=7, batch=2, n_max=256, hq=8, hkv=2, lengths=None, vl_frac=0.05, device="cpu"):
    """Prompt queries, keys and values (bf16, ~N(0,1); keys of a few seeded channels
    x4, an outlier pattern INT8 tiles must carry), per-request lengths (default n_max),
    and seeded vertical-line flags (uint8 [batch, hkv, n_max], 1 for vl_frac of the
    positions) for the prefill operator."""
    lens = np.full(batch, n_max, np.int32) if lengths is None else np.asarray(lengths, np.int32)
    q = randn((batch, n_max, hq, HEAD_DIM), seed, 81, device=device)
    k = randn((batch, n_max, hkv, HEAD_DIM), seed, 82, device=device)
    v = randn((batch, n_max, hkv, HEAD_DIM), seed, 83, device=device)
    ch = np_rng(seed, 84).choice(HEAD_DIM, 4, replace=False)
    k[..., torch.as_tensor(ch, device=device)] *= 4.0
    cls = (np_rng(seed, 85).random((batch, hkv, n_max)) < vl_frac).astype(np.uint8)
    return _bf16(q).contiguous(), _bf16(k).contiguous(), _bf16(v).contiguous(), lens, cls
