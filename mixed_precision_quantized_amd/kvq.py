"""Thin Python binding of libkvq (ctypes).  Argument marshalling only: every step of
the decode path runs in the library's HIP kernels or its host C++ code.

Device arrays are torch tensors on a ROCm device; host arrays are numpy arrays.
Calls enqueue on torch's current stream unless a stream is given.  The binding
raises ImportError when libkvq.so is missing: there is no fallback path.

The operations and their sources are documented in include/kvq.h.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
# KVQ_LIBRARY may name another build of the same sources (the host-sanitizer build).
LIB_PATH = os.environ.get("KVQ_LIBRARY") or os.path.join(HERE, "libkvq.so")

INT2, INT4, FP16 = 0, 1, 2
F32, BF16, F16 = 0, 1, 2
TABLE_PAGES, TABLE_SLOTS = 0, 1
ANCHOR_FP16, ANCHOR_FP8 = 0, 1  # kvq_cache.anchor_format
DEVERR_ID, DEVERR_RANGE, DEVERR_PAIR, DEVERR_SPLIT = 1, 2, 4, 8
HEAD_DIM = 128
FP8_ANCHOR_BLOCK = 3   # kvq_block_bytes class of an FP8 anchor block
PAGE = 16

SPLIT_DTYPE = np.dtype([("table", "<i4"), ("head", "<i4"), ("cls", "<i4"),
                        ("tok_begin", "<i4"), ("tok_end", "<i4")])

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built: run __graft_entry__.build() "
                      "(the decode path has no fallback)")
_lib = ctypes.CDLL(LIB_PATH)


class KvqError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = _lib.kvq_status_string(status).decode()
        detail = _lib.kvq_last_error().decode()
        super().__init__(f"{where}: {msg} ({status}): {detail}")


class _CacheC(ctypes.Structure):
    _fields_ = [("head_dim", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("heads_per_page", ctypes.c_int32), ("n_pages", ctypes.c_int32 * 3),
                ("pool", ctypes.c_void_p * 3), ("sentinel_slot", ctypes.c_int32), ("anchor_format", ctypes.c_int32)]


class _SplitC(ctypes.Structure):
    _fields_ = [("table", ctypes.c_int32), ("head", ctypes.c_int32), ("cls", ctypes.c_int32),
                ("tok_begin", ctypes.c_int32), ("tok_end", ctypes.c_int32)]


_P, _i32, _i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
_SIGS = {
    "kvq_block_bytes": ([_i32], ctypes.c_size_t),
    "kvq_route_tokens": ([_P, _i32, _P, _P, _P, _P], ctypes.c_int),
    "kvq_tag_tokens": ([_P, _i32, _P, _i32, _P, _P], ctypes.c_int),
    "kvq_allocate_bits": ([_P, _P, _P, _i32, ctypes.c_double, _P, _P], ctypes.c_int),
    "kvq_count_tags": ([_P, _i32, _P], ctypes.c_int),
    "kvq_tag_flags": ([_P, _i32, _P, _i32, _P], ctypes.c_int),
    "kvq_quantize_append": ([_P, _P, _P, _i32, _i64, _i64, _i64, _i32, _P, _P, _i32, _P, _P, _i32, _P, _P,
                             _P, _P], ctypes.c_int),
    "kvq_reorder_pages": ([_P, _P, _i32, _i32, _P, _P, _P, _P], ctypes.c_int),
    "kvq_compact_slots": ([_P, _P, _i32, _i32, _P, _P, _P, _P, _P], ctypes.c_int),
    "kvq_prefill_prepare": ([_P, _P, _i32, _i32, _i32, _i32, _P, _P, _P, _P, _P, _P, _P,
                             ctypes.c_size_t, _P, _P], ctypes.c_int),
    "kvq_prefill_attn": ([_P, _P, _i32, _i32, _i32, _i32, _i32, _P, _P, _i32, _P, _P,
                          ctypes.c_size_t, _P, _P, _P], ctypes.c_int),
    "kvq_prefill_workspace_bytes": ([_i32, _i32, _i32], ctypes.c_size_t),
    "kvq_select_vertical_lines": ([_P, _i32, _P, _i32, _i32, _i32, _i32, _i32, _i32, _P, _P, _i32,
                                   ctypes.c_float, _P, _P, _P, _P, _P, _P], ctypes.c_int),
    "kvq_plan_balanced": ([_P, _i32, _i32, _i32, _i32, _i32, _i32, _P, _P, _i32, _P, _P, _P], ctypes.c_int),
    "kvq_wave_timeline": ([_P], ctypes.c_int),
    "kvq_decode_attn": ([_P, _P, _i32, _i32, _i32, _i32, _P, _i32, _i32, _i32, _P, _i32, _P, _P, _P,
                         _P], ctypes.c_int),
    "kvq_lse_merge": ([_P, _P, _i32, _P, _i32, _i32, _i32, _P, _i32, _P, _P], ctypes.c_int),
    "kvq_plan_splits": ([_P, _i32, _i32, _i32, _i32, _P, _P, _P, _i64, _P, _i32, _P, _P], ctypes.c_int),
    "kvq_plan_workers": ([_P, _i32, _i32, _i32, _i32, _P, _P, _P, _P, _i32, _P, _P, _P], ctypes.c_int),
    "kvq_decode_attn_shared": ([_P, _P, _i32, _i32, _i32, _i32, _P, _i32, _i32, _i32, _P, _P, _i32, _i32, _P, _P,
                                _P, _P, _P], ctypes.c_int),
    "kvq_decode_work_bytes": ([_i32], ctypes.c_size_t),
    "kvq_decode_attn_shared_noalloc": ([_P, _P, _i32, _i32, _i32, _i32, _P, _i32, _i32, _i32, _P, _P, _i32, _i32,
                                        _P, _P, _P, _P], ctypes.c_int),
    "kvq_aot_split_counts": ([_P, _i32, _i32, _i32, _P], ctypes.c_int),
    "kvq_balanced_split_counts": ([_P, _i32, _i32, _P], ctypes.c_int),
    "kvq_decode_occupancy": ([_i32, _i32, _P, _P], ctypes.c_int),
    "kvq_decode_fp16_occupancy": ([_i32, _i32, _P, _P], ctypes.c_int),
    "kvq_plan_splits_per_kernel": ([_P, _i32, _i32, _i32, _i32, _P, _P, _P, _P, _i32, _P, _P], ctypes.c_int),
    "kvq_head_group_plan": ([_P, _i32, _i32, _i64, _i32, _P, _P, _P], ctypes.c_int),
    "kvq_status_string": ([_i32], ctypes.c_char_p),
    "kvq_last_error": ([], ctypes.c_char_p),
}
for _name, (_args, _res) in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.argtypes = _args
    _fn.restype = _res

EXPORTED = tuple(_SIGS)


def _check(status: int, where: str):
    if status != 0:
        raise KvqError(status, where)


def _dptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    assert t.is_cuda, "device array expected"
    return ctypes.c_void_p(t.data_ptr())


def _hptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


_DTYPES = {torch.float32: F32, torch.bfloat16: BF16, torch.float16: F16}


def block_bytes(cls: int) -> int:
    return int(_lib.kvq_block_bytes(cls))


class Cache:
    """Device pools of a mixed-precision paged KV cache (allocated by torch)."""

    def __init__(self, heads_per_page: int, n_pages, device="cuda", sentinel_slot: int = -1,
                 pools=None, anchor_fp8: bool = False):
        self.heads_per_page = int(heads_per_page)
        self.n_pages = tuple(int(n) for n in n_pages)
        self.sentinel_slot = int(sentinel_slot)
        self.anchor_fp8 = bool(anchor_fp8)
        self.block_bytes = (block_bytes(0), block_bytes(1), block_bytes(FP8_ANCHOR_BLOCK if anchor_fp8 else 2))
        if pools is None:
            pools = [torch.zeros(max(1, n * self.heads_per_page * self.block_bytes[c]), dtype=torch.uint8,
                                 device=device) for c, n in enumerate(self.n_pages)]
        self.pools = pools
        self._c = _CacheC()
        self._c.head_dim = HEAD_DIM
        self._c.page_size = PAGE
        self._c.heads_per_page = self.heads_per_page
        for i in range(3):
            self._c.n_pages[i] = self.n_pages[i]
            self._c.pool[i] = self.pools[i].data_ptr()
        self._c.sentinel_slot = self.sentinel_slot
        self._c.anchor_format = ANCHOR_FP8 if self.anchor_fp8 else ANCHOR_FP16

    @property
    def struct(self):
        return ctypes.byref(self._c)

    def pool_bytes(self, cls: int) -> torch.Tensor:
        return self.pools[cls][: self.n_pages[cls] * self.heads_per_page * self.block_bytes[cls]]


def route_tokens(flags: np.ndarray):
    """flags uint8 [n] (0 INT2, 1 INT4, 2 FP16) -> (classes, n_int2_groups, n_int4, n_fp16)."""
    flags = np.ascontiguousarray(flags, dtype=np.uint8)
    cls = np.zeros(flags.shape[0], np.uint8)
    n2, n4, n16 = _i32(), _i32(), _i32()
    _check(_lib.kvq_route_tokens(_hptr(flags), flags.shape[0], _hptr(cls), ctypes.byref(n2),
                                 ctypes.byref(n4), ctypes.byref(n16)), "kvq_route_tokens")
    return cls, n2.value, n4.value, n16.value


N_TEMPORAL, N_MODAL, N_SEMANTIC, N_TAGS = 4, 2, 7, 56
(EV_SYSTEM, EV_USER, EV_ASSISTANT, EV_OBSERVATION, EV_END, EV_THINK_BEGIN, EV_THINK_END,
 EV_TOOL_CALL_BEGIN, EV_TOOL_CALL_END, EV_IMAGE_BEGIN, EV_IMAGE_END) = range(11)


class _MarkerC(ctypes.Structure):
    _fields_ = [("token_id", ctypes.c_int32), ("event", ctypes.c_int32)]


def tag_tokens(tokens: np.ndarray, markers):
    """tokens int32 [n]; markers: {token id: EV_*}.  Returns (tags uint8 [n], turns)."""
    tokens = np.ascontiguousarray(tokens, dtype=np.int32)
    arr = (_MarkerC * max(1, len(markers)))(*[_MarkerC(int(t), int(e)) for t, e in markers.items()])
    tags = np.zeros(tokens.shape[0], np.uint8)
    turns = _i32()
    _check(_lib.kvq_tag_tokens(_hptr(tokens), tokens.shape[0], ctypes.cast(arr, _P), len(markers), _hptr(tags),
                               ctypes.byref(turns)), "kvq_tag_tokens")
    return tags, turns.value


def count_tags(tags: np.ndarray, counts: Optional[np.ndarray] = None) -> np.ndarray:
    """Adds the tokens per tag of tags (uint8) into counts (int64 [N_TAGS], new if None)."""
    tags = np.ascontiguousarray(tags, np.uint8)
    if counts is None:
        counts = np.zeros(N_TAGS, np.int64)
    assert counts.dtype == np.int64 and counts.flags.c_contiguous and counts.shape[0] >= N_TAGS
    _check(_lib.kvq_count_tags(_hptr(tags), tags.shape[0], _hptr(counts)), "kvq_count_tags")
    return counts


def allocate_bits(d2, d4, counts, budget_bits: float):
    """Greedy 2 / 4-bit widths per tag; returns (bits uint8 [n_tags], average width)."""
    d2 = np.ascontiguousarray(d2, np.float64).reshape(-1)
    d4 = np.ascontiguousarray(d4, np.float64).reshape(-1)
    counts = np.ascontiguousarray(counts, np.int64).reshape(-1)
    bits = np.zeros(counts.shape[0], np.uint8)
    avg = ctypes.c_double()
    _check(_lib.kvq_allocate_bits(_hptr(d2), _hptr(d4), _hptr(counts), counts.shape[0], float(budget_bits),
                                  _hptr(bits), ctypes.byref(avg)), "kvq_allocate_bits")
    return bits, avg.value


def tag_flags(tags: np.ndarray, bits: np.ndarray) -> np.ndarray:
    """Routing flags (0 INT2, 1 INT4) of tagged tokens under per-tag widths."""
    tags = np.ascontiguousarray(tags, np.uint8)
    bits = np.ascontiguousarray(bits, np.uint8)
    flags = np.zeros(tags.shape[0], np.uint8)
    _check(_lib.kvq_tag_flags(_hptr(tags), tags.shape[0], _hptr(bits), bits.shape[0], _hptr(flags)),
           "kvq_tag_flags")
    return flags


def quantize_append(cache: Cache, k: torch.Tensor, v: torch.Tensor, rows4=None, slots4=None,
                    rows2=None, pages2=None, rows16=None, slots16=None, dev_err=None, stream=None):
    """k, v [R, heads_per_page, 128] (any strides with unit channel stride); lists are
    int32 device tensors (or None)."""
    assert k.shape == v.shape and k.stride() == v.stride() and k.dtype == v.dtype
    assert k.shape[-1] == HEAD_DIM and k.stride(-1) == 1
    n = lambda t: 0 if t is None else int(t.numel())  # noqa: E731
    head_stride = k.stride(1) if k.dim() == 3 else HEAD_DIM
    _check(_lib.kvq_quantize_append(
        cache.struct, _dptr(k), _dptr(v), _DTYPES[k.dtype], k.shape[0], k.stride(0), head_stride,
        n(rows4), _dptr(rows4), _dptr(slots4), n(pages2), _dptr(rows2), _dptr(pages2),
        n(rows16), _dptr(rows16), _dptr(slots16), _dptr(dev_err), _stream(stream)),
        "kvq_quantize_append")


def reorder_pages(cache: Cache, tables: torch.Tensor, n_entries: torch.Tensor,
                  class_counts: Optional[torch.Tensor] = None, dev_err=None, stream=None):
    assert tables.dtype == torch.int32 and tables.is_contiguous() and tables.dim() == 2
    _check(_lib.kvq_reorder_pages(cache.struct, _dptr(tables), tables.shape[0], tables.shape[1],
                                  _dptr(n_entries), _dptr(class_counts), _dptr(dev_err),
                                  _stream(stream)), "kvq_reorder_pages")


def compact_slots(cache: Cache, tables: torch.Tensor, n_entries: torch.Tensor, head_tokens: torch.Tensor,
                  live_tokens: Optional[torch.Tensor] = None, dev_err=None, stream=None) -> torch.Tensor:
    """Slot tables int32 [n_tables, max_entries], compacted in place; returns the live
    counts int32 [n_tables, heads_per_page] (device)."""
    assert tables.dtype == torch.int32 and tables.is_contiguous() and tables.dim() == 2
    assert head_tokens.dtype == torch.int32 and head_tokens.is_contiguous()
    assert n_entries.dtype == torch.int32 and n_entries.numel() >= tables.shape[0]
    assert head_tokens.numel() >= tables.shape[0] * cache.heads_per_page
    if live_tokens is None:
        live_tokens = torch.empty_like(head_tokens)
    assert live_tokens.dtype == torch.int32 and live_tokens.numel() >= head_tokens.numel()
    _check(_lib.kvq_compact_slots(cache.struct, _dptr(tables), tables.shape[0], tables.shape[1],
                                  _dptr(n_entries), _dptr(head_tokens), _dptr(live_tokens), _dptr(dev_err),
                                  _stream(stream)), "kvq_compact_slots")
    return live_tokens


CLASS_QUANTIZED, CLASS_VERTICAL_LINE, CLASS_WINDOW = 0, 1, 2


def select_vertical_lines(k: torch.Tensor, q_tail: torch.Tensor, n_tokens: torch.Tensor, n_tail: torch.Tensor,
                          window: int = 128, rho: float = 0.05, out=None, dev_err=None, stream=None):
    """k [batch, max_tokens, hkv, 128], q_tail [batch, max_tail, hq, 128] (device);
    returns (proxy [batch, hkv, 128], scores [batch, hkv, max_tokens], token_class uint8
    [batch, hkv, max_tokens], n_vl [batch, hkv]), or fills `out` (the same four)."""
    assert k.is_contiguous() and q_tail.is_contiguous() and k.dim() == 4 and q_tail.dim() == 4
    batch, max_tokens, hkv = k.shape[:3]
    max_tail, hq = q_tail.shape[1:3]
    assert n_tokens.dtype == torch.int32 and n_tail.dtype == torch.int32
    if out is None:
        dev = k.device
        out = (torch.empty((batch, hkv, HEAD_DIM), dtype=torch.float32, device=dev),
               torch.empty((batch, hkv, max_tokens), dtype=torch.float32, device=dev),
               torch.empty((batch, hkv, max_tokens), dtype=torch.uint8, device=dev),
               torch.empty((batch, hkv), dtype=torch.int32, device=dev))
    proxy, scores, cls, n_vl = out
    _check(_lib.kvq_select_vertical_lines(_dptr(k), _DTYPES[k.dtype], _dptr(q_tail), _DTYPES[q_tail.dtype], batch,
                                          max_tokens, hkv, hq, max_tail, _dptr(n_tokens), _dptr(n_tail), window,
                                          float(rho), _dptr(proxy), _dptr(scores), _dptr(cls), _dptr(n_vl),
                                          _dptr(dev_err), _stream(stream)), "kvq_select_vertical_lines")
    return out


def prefill_workspace(batch: int, n_max: int, hq: int, hkv: int, device="cuda"):
    """Outputs and scratch of prefill_attn: (k_codes, k_scales, v_codes, v_scales,
    scratch, out); scratch is kvq_prefill_workspace_bytes bytes."""
    tiles = n_max // 64
    nbytes = _lib.kvq_prefill_workspace_bytes(batch, n_max, hkv)
    if nbytes == 0:
        raise KvqError(-1, f"kvq_prefill_workspace_bytes({batch}, {n_max}, {hkv})")
    return (torch.empty((batch, n_max, hkv, HEAD_DIM), dtype=torch.int8, device=device),
            torch.empty((batch, hkv, tiles), dtype=torch.float32, device=device),
            torch.empty((batch, n_max, hkv, HEAD_DIM), dtype=torch.int8, device=device),
            torch.empty((batch, hkv, tiles), dtype=torch.float32, device=device),
            torch.empty(nbytes, dtype=torch.uint8, device=device),
            torch.empty((batch, n_max, hq, HEAD_DIM), dtype=torch.float32, device=device))


def prefill_prepare(k: torch.Tensor, v: torch.Tensor, n_tokens: torch.Tensor,
                    token_class: Optional[torch.Tensor], ws, dev_err=None, stream=None):
    """The INT8 codes and scales of k, v and the attention's scratch, into ws
    (prefill_workspace's tuple)."""
    assert k.dtype == v.dtype == torch.bfloat16
    assert k.is_contiguous() and v.is_contiguous()
    batch, n_max, hkv = k.shape[:3]
    kc, ks, vc, vs, scratch, _ = ws
    if token_class is not None:
        assert token_class.dtype == torch.uint8 and token_class.is_contiguous()
    _check(_lib.kvq_prefill_prepare(_dptr(k), _dptr(v), BF16, batch, n_max, hkv, _dptr(n_tokens),
                                    _dptr(token_class), _dptr(kc), _dptr(ks), _dptr(vc), _dptr(vs),
                                    _dptr(scratch), scratch.numel(), _dptr(dev_err), _stream(stream)),
           "kvq_prefill_prepare")


def prefill_attend(q: torch.Tensor, k: torch.Tensor, n_tokens: torch.Tensor, token_class: Optional[torch.Tensor],
                   window: int, ws, dev_err=None, stream=None):
    """The attention over what prefill_prepare left in ws; fills ws[5]."""
    assert q.dtype == torch.bfloat16 and q.is_contiguous()
    batch, n_max, hq = q.shape[:3]
    hkv = k.shape[2]
    _, ks, _, _, scratch, out = ws
    _check(_lib.kvq_prefill_attn(_dptr(q), _dptr(k), BF16, batch, n_max, hq, hkv, _dptr(n_tokens),
                                 _dptr(token_class), window, _dptr(ks), _dptr(scratch), scratch.numel(),
                                 _dptr(out), _dptr(dev_err), _stream(stream)),
           "kvq_prefill_attn")


def prefill_attn(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, n_tokens: torch.Tensor,
                 token_class: Optional[torch.Tensor] = None, window: int = 128, ws=None, dev_err=None,
                 stream=None):
    """q [batch, n_max, hq, 128], k, v [batch, n_max, hkv, 128] bf16 (device); token_class
    uint8 [batch, hkv, n_max] or None.  prepare then attend; returns prefill_workspace's
    tuple, filled."""
    batch, n_max, hq = q.shape[:3]
    if ws is None:
        ws = prefill_workspace(batch, n_max, hq, k.shape[2], q.device)
    prefill_prepare(k, v, n_tokens, token_class, ws, dev_err, stream)
    prefill_attend(q, k, n_tokens, token_class, window, ws, dev_err, stream)
    return ws


def decode_attn(cache: Cache, q: torch.Tensor, hkv: int, tables: torch.Tensor, table_kind: int,
                splits: torch.Tensor, part_o: torch.Tensor, part_lse: torch.Tensor, dev_err=None,
                stream=None):
    """q [batch, hq, 128]; splits int32 device [n, 5]; part_o float [n, g, 128]; part_lse [n, g]."""
    assert q.is_contiguous() and tables.is_contiguous() and splits.is_contiguous()
    assert splits.dtype == torch.int32 and splits.shape[-1] == 5
    batch, hq = q.shape[0], q.shape[1]
    n_splits = splits.shape[0]
    g = hq // hkv
    assert part_o.numel() >= n_splits * g * HEAD_DIM and part_lse.numel() >= n_splits * g
    assert part_o.dtype == torch.float32 and part_lse.dtype == torch.float32
    _check(_lib.kvq_decode_attn(cache.struct, _dptr(q), _DTYPES[q.dtype], batch, hq, hkv,
                                _dptr(tables), tables.shape[0], tables.shape[1], table_kind,
                                _dptr(splits), n_splits, _dptr(part_o), _dptr(part_lse),
                                _dptr(dev_err), _stream(stream)), "kvq_decode_attn")


def decode_attn_shared(cache: Cache, q: torch.Tensor, hkv: int, tables: torch.Tensor, table_kind: int,
                       workers: torch.Tensor, groups: torch.Tensor, n_groups: int, work: torch.Tensor,
                       part_o: torch.Tensor, part_lse: torch.Tensor, dev_err=None, stream=None):
    """Shared-window decode: workers int32 device [n, 5] (each its group's range), groups
    int32 device [n], work from decode_work(n_groups) (zero before the first call; zero
    again after each)."""
    assert q.is_contiguous() and tables.is_contiguous() and workers.is_contiguous() and groups.is_contiguous()
    assert workers.dtype == groups.dtype == work.dtype == torch.int32 and workers.shape[-1] == 5
    batch, hq = q.shape[0], q.shape[1]
    n = workers.shape[0]
    assert groups.numel() >= n and work.numel() * 4 >= _lib.kvq_decode_work_bytes(n_groups)
    assert part_o.numel() >= n * (hq // hkv) * HEAD_DIM and part_lse.numel() >= n * (hq // hkv)
    _check(_lib.kvq_decode_attn_shared(cache.struct, _dptr(q), _DTYPES[q.dtype], batch, hq, hkv, _dptr(tables),
                                       tables.shape[0], tables.shape[1], table_kind, _dptr(workers), _dptr(groups),
                                       n, n_groups, _dptr(work), _dptr(part_o), _dptr(part_lse), _dptr(dev_err),
                                       _stream(stream)), "kvq_decode_attn_shared")


def decode_attn_shared_noalloc(cache: Cache, q: torch.Tensor, hkv: int, tables: torch.Tensor, table_kind: int,
                               workers: torch.Tensor, groups: torch.Tensor, n_groups: int, part_o: torch.Tensor,
                               part_lse: torch.Tensor, dev_err=None, stream=None):
    """decode_attn_shared with the library's own counters (no work argument, nothing
    allocated by the library)."""
    assert q.is_contiguous() and tables.is_contiguous() and workers.is_contiguous() and groups.is_contiguous()
    assert workers.dtype == groups.dtype == torch.int32 and workers.shape[-1] == 5
    batch, hq = q.shape[0], q.shape[1]
    n = workers.shape[0]
    assert groups.numel() >= n
    assert part_o.numel() >= n * (hq // hkv) * HEAD_DIM and part_lse.numel() >= n * (hq // hkv)
    _check(_lib.kvq_decode_attn_shared_noalloc(cache.struct, _dptr(q), _DTYPES[q.dtype], batch, hq, hkv,
                                               _dptr(tables), tables.shape[0], tables.shape[1], table_kind,
                                               _dptr(workers), _dptr(groups), n, n_groups, _dptr(part_o),
                                               _dptr(part_lse), _dptr(dev_err), _stream(stream)),
           "kvq_decode_attn_shared_noalloc")


def decode_work(n_groups: int, device="cuda") -> torch.Tensor:
    """Zeroed work counters for decode_attn_shared."""
    nbytes = _lib.kvq_decode_work_bytes(n_groups)
    if nbytes == 0:
        raise KvqError(-1, f"kvq_decode_work_bytes({n_groups})")
    return torch.zeros(nbytes // 4, dtype=torch.int32, device=device)


def lse_merge(part_o: torch.Tensor, part_lse: torch.Tensor, n_splits: int, split_offsets: torch.Tensor,
              batch: int, hq: int, hkv: int, out: torch.Tensor, out_lse=None, stream=None):
    assert out.is_contiguous() and out.numel() >= batch * hq * HEAD_DIM
    _check(_lib.kvq_lse_merge(_dptr(part_o), _dptr(part_lse), n_splits, _dptr(split_offsets), batch,
                              hq, hkv, _dptr(out), _DTYPES[out.dtype], _dptr(out_lse),
                              _stream(stream)), "kvq_lse_merge")


def plan_splits(ranges: np.ndarray, batch: int, hkv: int, heads_per_page: int,
                splits_per_head: Optional[np.ndarray] = None, tokens_per_split=None,
                target_bytes: int = 0, max_out: Optional[int] = None, class_cost=None):
    """ranges: structured (SPLIT_DTYPE) or int32 [n, 5], sorted by (table, head).
    Returns (splits int32 [n_out, 5], split_offsets int32 [batch*hkv + 1])."""
    r = np.ascontiguousarray(np.asarray(ranges).view(np.int32).reshape(-1, 5))
    if max_out is None:
        n_units = int(np.maximum(0, (r[:, 4] - r[:, 3])).sum()) if len(r) else 0
        max_out = max(1, n_units + len(r))
        if splits_per_head is not None:
            max_out = max(max_out, int(np.asarray(splits_per_head).sum()) + len(r))
    out = np.zeros((max_out, 5), np.int32)
    offsets = np.zeros(batch * hkv + 1, np.int32)
    n_out = _i32()
    sph = None if splits_per_head is None else np.ascontiguousarray(splits_per_head, np.int32)
    tps = None if tokens_per_split is None else np.ascontiguousarray(tokens_per_split, np.int32)
    cc = None if class_cost is None else np.ascontiguousarray(class_cost, np.float32)
    _check(_lib.kvq_plan_splits(_hptr(r), r.shape[0], batch, hkv, heads_per_page, _hptr(sph), _hptr(cc),
                                _hptr(tps), int(target_bytes), _hptr(out), max_out,
                                ctypes.byref(n_out), _hptr(offsets)), "kvq_plan_splits")
    return out[: n_out.value].copy(), offsets


def plan_splits_per_kernel(ranges: np.ndarray, batch: int, hkv: int, heads_per_page: int,
                           int_splits: np.ndarray, fp16_splits: np.ndarray, class_cost=None,
                           max_out: Optional[int] = None):
    """ranges as for plan_splits; int_splits / fp16_splits int32 [n_tables*heads_per_page]:
    pieces per (table, head) for its INT2 / INT4 ranges and for its FP16 ranges.
    Returns (splits int32 [n_out, 5], split_offsets int32 [batch*hkv + 1])."""
    r = np.ascontiguousarray(np.asarray(ranges).view(np.int32).reshape(-1, 5))
    n_heads = batch * hkv
    ints = np.ascontiguousarray(np.broadcast_to(np.asarray(int_splits, np.int32), (n_heads,)))
    fp16 = np.ascontiguousarray(np.broadcast_to(np.asarray(fp16_splits, np.int32), (n_heads,)))
    if max_out is None:
        max_out = max(1, int(ints.sum()) + int(fp16.sum()) + len(r))
    out = np.zeros((max_out, 5), np.int32)
    offsets = np.zeros(batch * hkv + 1, np.int32)
    n_out = _i32()
    cc = None if class_cost is None else np.ascontiguousarray(class_cost, np.float32)
    _check(_lib.kvq_plan_splits_per_kernel(_hptr(r), r.shape[0], batch, hkv, heads_per_page, _hptr(ints),
                                           _hptr(fp16), _hptr(cc), _hptr(out), max_out, ctypes.byref(n_out),
                                           _hptr(offsets)), "kvq_plan_splits_per_kernel")
    return out[: n_out.value].copy(), offsets


def plan_workers(ranges: np.ndarray, batch: int, hkv: int, heads_per_page: int, workers_per_head: np.ndarray,
                 class_cost=None):
    """ranges as for plan_splits.  Returns (workers int32 [n, 5], groups int32 [n], n_groups,
    split_offsets int32 [batch*hkv + 1])."""
    r = np.ascontiguousarray(np.asarray(ranges).view(np.int32).reshape(-1, 5))
    wph = np.ascontiguousarray(workers_per_head, np.int32)
    max_out = max(1, int(wph.sum()) + len(r))
    out = np.zeros((max_out, 5), np.int32)
    grp = np.zeros(max_out, np.int32)
    offsets = np.zeros(batch * hkv + 1, np.int32)
    n_out, n_groups = _i32(), _i32()
    cc = None if class_cost is None else np.ascontiguousarray(class_cost, np.float32)
    _check(_lib.kvq_plan_workers(_hptr(r), r.shape[0], batch, hkv, heads_per_page, _hptr(wph), _hptr(cc), _hptr(out),
                                 _hptr(grp), max_out, ctypes.byref(n_out), ctypes.byref(n_groups), _hptr(offsets)),
           "kvq_plan_workers")
    return out[: n_out.value].copy(), grp[: n_out.value].copy(), n_groups.value, offsets


def head_group_plan(budgets: np.ndarray, heads_per_group: int, n_tokens: int, cls: int = 1):
    """(order int32 [hkv], table_slots int32 [hkv / H], bytes int64 [3]: grouped,
    per-head, no eviction) for ragged head-group tables (host)."""
    b = np.ascontiguousarray(budgets, np.float32)
    hkv = b.shape[0]
    order = np.zeros(hkv, np.int32)
    slots = np.zeros(max(hkv // max(heads_per_group, 1), 1), np.int32)
    nbytes = np.zeros(3, np.int64)
    _check(_lib.kvq_head_group_plan(_hptr(b), hkv, heads_per_group, n_tokens, cls, _hptr(order), _hptr(slots),
                                    _hptr(nbytes)), "kvq_head_group_plan")
    return order, slots, nbytes


def aot_split_counts(budgets: np.ndarray, batch: int, total_work: int) -> np.ndarray:
    b = np.ascontiguousarray(budgets, np.float32)
    out = np.zeros(batch * b.shape[0], np.int32)
    _check(_lib.kvq_aot_split_counts(_hptr(b), b.shape[0], batch, total_work, _hptr(out)),
           "kvq_aot_split_counts")
    return out


def plan_balanced(ranges: np.ndarray, batch: int, hkv: int, heads_per_page: int, g: int, total_splits: int,
                  class_cost=None, max_out: Optional[int] = None):
    """Split counts per (table, head) balanced over tokens x class cost (kvq_plan_balanced).
    Returns (splits int32 [n_out, 5], split_offsets int32 [batch*hkv + 1],
    splits_per_head int32 [n_tables*heads_per_page])."""
    r = np.ascontiguousarray(np.asarray(ranges).view(np.int32).reshape(-1, 5))
    n_heads = batch * hkv  # n_tables * heads_per_page
    if max_out is None:  # a head may get one piece per non-empty range beyond its count
        max_out = max(int(total_splits), n_heads) + len(r) + 1
    out = np.zeros((max_out, 5), np.int32)
    offsets = np.zeros(batch * hkv + 1, np.int32)
    sph = np.zeros(n_heads, np.int32)
    n_out = _i32()
    cc = None if class_cost is None else np.ascontiguousarray(class_cost, np.float32)
    _check(_lib.kvq_plan_balanced(_hptr(r), r.shape[0], batch, hkv, heads_per_page, g, total_splits, _hptr(cc),
                                  _hptr(out), max_out, ctypes.byref(n_out), _hptr(offsets), _hptr(sph)),
           "kvq_plan_balanced")
    return out[: n_out.value].copy(), offsets, sph


def balanced_split_counts(work, total_work: int) -> np.ndarray:
    """Split counts such that no piece holds more than the smallest cap that fits
    total_work work groups (work: per-entry cost, e.g. live tokens per (table, head))."""
    w = np.ascontiguousarray(np.asarray(work).reshape(-1), np.int64)
    out = np.zeros(w.shape[0], np.int32)
    _check(_lib.kvq_balanced_split_counts(_hptr(w), w.shape[0], total_work, _hptr(out)),
           "kvq_balanced_split_counts")
    return out


def wave_timeline(buffer: Optional[torch.Tensor]):
    """Profiling builds (libkvq_timeline.so) only: later fixed-split page-table decode
    launches record 8 uint64 words per split into buffer (int64 [n_splits, 8], device);
    None stops the recording."""
    if buffer is not None:
        assert buffer.dtype == torch.int64 and buffer.is_contiguous() and buffer.shape[-1] == 8
    _check(_lib.kvq_wave_timeline(_dptr(buffer)), "kvq_wave_timeline")


def decode_occupancy(g: int, table_kind: int = 0):
    per_cu, n_cu = _i32(), _i32()
    _check(_lib.kvq_decode_occupancy(g, table_kind, ctypes.byref(per_cu), ctypes.byref(n_cu)),
           "kvq_decode_occupancy")
    return per_cu.value, n_cu.value


def decode_fp16_occupancy(g: int, anchor_fp8: bool = False):
    per_cu, n_cu = _i32(), _i32()
    _check(_lib.kvq_decode_fp16_occupancy(g, ANCHOR_FP8 if anchor_fp8 else ANCHOR_FP16, ctypes.byref(per_cu),
                                          ctypes.byref(n_cu)), "kvq_decode_fp16_occupancy")
    return per_cu.value, n_cu.value


def status_string(status: int) -> str:
    return _lib.kvq_status_string(status).decode()


def raw_library():
    """The loaded ctypes library (for tests of the ABI itself)."""
    return _lib


class BoundCall:
    """A library call with its ctypes arguments marshalled once (for tight launch loops:
    replaying a decode step costs one ctypes call per kernel).  The tensors passed at
    construction must stay alive and in place."""

    def __init__(self, name: str, args, keep=()):
        self._fn = getattr(_lib, name)
        self._args = tuple(args)
        self._keep = keep
        self._name = name

    def __call__(self):
        st = self._fn(*self._args)
        if st != 0:
            raise KvqError(st, self._name)


def bind_decode_attn(cache: Cache, q: torch.Tensor, hkv: int, tables: torch.Tensor, table_kind: int,
                     splits: torch.Tensor, part_o: torch.Tensor, part_lse: torch.Tensor,
                     dev_err=None, stream=None) -> BoundCall:
    assert q.is_contiguous() and tables.is_contiguous() and splits.is_contiguous()
    batch, hq = q.shape[0], q.shape[1]
    args = (cache.struct, _dptr(q), _DTYPES[q.dtype], batch, hq, hkv, _dptr(tables), tables.shape[0],
            tables.shape[1], table_kind, _dptr(splits), splits.shape[0], _dptr(part_o),
            _dptr(part_lse), _dptr(dev_err), _stream(stream))
    return BoundCall("kvq_decode_attn", args, keep=(cache, q, tables, splits, part_o, part_lse, dev_err))


def bind_decode_attn_shared(cache: Cache, q: torch.Tensor, hkv: int, tables: torch.Tensor, table_kind: int,
                            workers: torch.Tensor, groups: torch.Tensor, n_groups: int, work: torch.Tensor,
                            part_o: torch.Tensor, part_lse: torch.Tensor, dev_err=None, stream=None) -> BoundCall:
    assert q.is_contiguous() and tables.is_contiguous() and workers.is_contiguous() and groups.is_contiguous()
    batch, hq = q.shape[0], q.shape[1]
    args = (cache.struct, _dptr(q), _DTYPES[q.dtype], batch, hq, hkv, _dptr(tables), tables.shape[0],
            tables.shape[1], table_kind, _dptr(workers), _dptr(groups), workers.shape[0], n_groups, _dptr(work),
            _dptr(part_o), _dptr(part_lse), _dptr(dev_err), _stream(stream))
    return BoundCall("kvq_decode_attn_shared", args,
                     keep=(cache, q, tables, workers, groups, work, part_o, part_lse, dev_err))


def bind_quantize_append(cache: Cache, k: torch.Tensor, v: torch.Tensor, rows4=None, slots4=None,
                         rows2=None, pages2=None, rows16=None, slots16=None, dev_err=None,
                         stream=None) -> BoundCall:
    assert k.shape == v.shape and k.stride() == v.stride() and k.dtype == v.dtype
    assert k.shape[-1] == HEAD_DIM and k.stride(-1) == 1
    n = lambda t: 0 if t is None else int(t.numel())  # noqa: E731
    head_stride = k.stride(1) if k.dim() == 3 else HEAD_DIM
    args = (cache.struct, _dptr(k), _dptr(v), _DTYPES[k.dtype], k.shape[0], k.stride(0), head_stride,
            n(rows4), _dptr(rows4), _dptr(slots4), n(pages2), _dptr(rows2), _dptr(pages2),
            n(rows16), _dptr(rows16), _dptr(slots16), _dptr(dev_err), _stream(stream))
    return BoundCall("kvq_quantize_append", args,
                     keep=(cache, k, v, rows4, slots4, rows2, pages2, rows16, slots16, dev_err))


def bind_lse_merge(part_o, part_lse, n_splits, split_offsets, batch, hq, hkv, out, out_lse=None,
                   stream=None) -> BoundCall:
    args = (_dptr(part_o), _dptr(part_lse), n_splits, _dptr(split_offsets), batch, hq, hkv, _dptr(out),
            _DTYPES[out.dtype], _dptr(out_lse), _stream(stream))
    return BoundCall("kvq_lse_merge", args, keep=(part_o, part_lse, split_offsets, out, out_lse))
