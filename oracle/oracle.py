"""ctypes wrapper of the CPU oracle (TEST INFRASTRUCTURE ONLY).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this module.  The product path (the HIP library and its binding) never
imports it.  Inputs and outputs are numpy arrays on the host.

Citations of the operations wrapped here are in kvq_oracle.h.
"""
import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
# ORACLE_LIBRARY may name another build of the same source (the sanitizer build).
LIB_PATH = os.environ.get("ORACLE_LIBRARY") or os.path.join(HERE, "liboracle.so")

INT2, INT4, FP16 = 0, 1, 2
F32, BF16, F16 = 0, 1, 2
PAGES, SLOTS = 0, 1
PAGE = 16
HEAD_DIM = 128
BLOCK_BYTES = {INT2: 1536, INT4: 2560, FP16: 8192}
FP8_ANCHOR_BYTES = 4160   # an FP16-class block of a cache with FP8 anchors

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            from . import build as _build  # noqa: WPS433 (build on first use)
            _build.build()
        _lib = ctypes.CDLL(LIB_PATH)
        _declare(_lib)
    return _lib


class _Cache(ctypes.Structure):
    _fields_ = [("heads_per_page", ctypes.c_int32),
                ("n_pages", ctypes.c_int32 * 3),
                ("pool", ctypes.c_void_p * 3),
                ("sentinel_slot", ctypes.c_int32),
                ("anchor_fp8", ctypes.c_int32)]


class _Range(ctypes.Structure):
    _fields_ = [("table", ctypes.c_int32), ("head", ctypes.c_int32),
                ("cls", ctypes.c_int32), ("tok_begin", ctypes.c_int32),
                ("tok_end", ctypes.c_int32)]


RANGE_DTYPE = np.dtype([("table", "<i4"), ("head", "<i4"), ("cls", "<i4"),
                        ("tok_begin", "<i4"), ("tok_end", "<i4")])


def _declare(L):
    P = ctypes.c_void_p
    i32, i64 = ctypes.c_int32, ctypes.c_int64
    L.orc_f16_down.argtypes = [ctypes.c_float]
    L.orc_f16_down.restype = ctypes.c_uint16
    L.orc_f16_up.argtypes = [ctypes.c_float]
    L.orc_f16_up.restype = ctypes.c_uint16
    L.orc_f16_up4.argtypes = [ctypes.c_float]
    L.orc_f16_up4.restype = ctypes.c_uint16
    L.orc_f16_nearest.argtypes = [ctypes.c_float]
    L.orc_f16_nearest.restype = ctypes.c_uint16
    L.orc_f16_value.argtypes = [ctypes.c_uint16]
    L.orc_f16_value.restype = ctypes.c_double
    L.orc_block_bytes.argtypes = [i32]
    L.orc_block_bytes.restype = i64
    L.orc_e4m3_value.argtypes = [ctypes.c_uint8]
    L.orc_e4m3_value.restype = ctypes.c_double
    L.orc_e4m3_nearest.argtypes = [ctypes.c_double]
    L.orc_e4m3_nearest.restype = ctypes.c_uint8
    L.orc_fp8_row.argtypes = [P, i32, P, P]
    L.orc_fp8_row.restype = None
    L.orc_quantize.argtypes = [P, i32, i64, i32, P, P, P]
    L.orc_quantize.restype = None
    L.orc_quantize_k2.argtypes = [P, i32, i64, P, P, P]
    L.orc_quantize_k2.restype = None
    L.orc_route.argtypes = [P, i32, P, P, P, P]
    L.orc_append.argtypes = [P, P, P, i32, i64, i64, i32, P, P, i32, P, P, i32, P, P]
    L.orc_reorder.argtypes = [P, P, i32, i32, P, P]
    L.orc_compact_slots.argtypes = [P, P, i32, i32, P, P, i32, P]
    L.orc_token.argtypes = [P, i32, i32, i32, P, P]
    L.orc_select_vl.argtypes = [P, P, i32, i32, i32, i32, i32, P, P, i32, ctypes.c_double, P, P, P]
    L.orc_prefill_attend.argtypes = [P, P, P, i32, i32, i32, i32, P, P, i32, P, P, P, P, P]
    L.orc_prefill_attend_rows.argtypes = [P, P, P, i32, i32, i32, i32, P, P, i32, i32, P, P, P, P, P, P, P]
    L.orc_attend.argtypes = [P, P, i32, i32, i32, P, i32, i32, i32, P, i32, P, P, i32]
    L.orc_attend_ranges.argtypes = [P, P, i32, i32, i32, P, i32, i32, i32, P, i32, P, P, i32]
    L.orc_merge.argtypes = [P, P, P, i32, i32, i32, P, P]
    for name in ("orc_route", "orc_append", "orc_reorder", "orc_compact_slots", "orc_token", "orc_select_vl",
                 "orc_prefill_attend", "orc_prefill_attend_rows",
                 "orc_attend",
                 "orc_attend_ranges", "orc_merge"):
        getattr(L, name).restype = ctypes.c_int


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(rc, what):
    if rc != 0:
        raise RuntimeError(f"oracle {what} failed with code {rc}")


def _c_array(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# --- fp16 helpers ------------------------------------------------------------

def e4m3_value(code: int) -> float:
    return float(lib().orc_e4m3_value(int(code)))


def e4m3_nearest(y: float) -> int:
    return int(lib().orc_e4m3_nearest(float(y)))


def fp8_row(x):
    """(codes uint8 [n], scale fp16 bits) of one FP8 anchor row."""
    x = _c_array(x, np.float32)
    codes = np.zeros(x.shape[0], np.uint8)
    scale = np.zeros(1, np.uint16)
    lib().orc_fp8_row(_ptr(x), x.shape[0], _ptr(codes), _ptr(scale))
    return codes, int(scale[0])


def f16_down(x: float) -> int:
    return int(lib().orc_f16_down(float(x)))


def f16_up(x: float) -> int:
    return int(lib().orc_f16_up(float(x)))


def f16_nearest(x: float) -> int:
    return int(lib().orc_f16_nearest(float(x)))


def f16_value(bits: int) -> float:
    return float(lib().orc_f16_value(int(bits)))


def f16_up4(x: float) -> int:
    return int(lib().orc_f16_up4(float(x)))


def quantize_k2(x):
    """Quantize one INT2 key group (one channel over 32 tokens); returns (codes, scale
    bits, zero bits)."""
    x = _c_array(x, np.float32)
    codes = np.zeros(x.shape[0], np.uint8)
    s = ctypes.c_uint16()
    z = ctypes.c_uint16()
    lib().orc_quantize_k2(_ptr(x), x.shape[0], 1, _ptr(codes), ctypes.byref(s), ctypes.byref(z))
    return codes, int(s.value), int(z.value)


def quantize(x, bits: int):
    """Quantize one group; returns (codes uint8[n], scale bits, zero bits)."""
    x = _c_array(x, np.float32)
    codes = np.zeros(x.shape[0], np.uint8)
    s = ctypes.c_uint16()
    z = ctypes.c_uint16()
    lib().orc_quantize(_ptr(x), x.shape[0], 1, bits, _ptr(codes), ctypes.byref(s), ctypes.byref(z))
    return codes, int(s.value), int(z.value)


def route(flags):
    """Route per-token flags (0 INT2, 1 INT4, 2 FP16); returns (cls, n2_groups, n4, n16)."""
    flags = _c_array(flags, np.uint8)
    cls = np.zeros(flags.shape[0], np.uint8)
    n2, n4, n16 = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    _check(lib().orc_route(_ptr(flags), flags.shape[0], _ptr(cls), ctypes.byref(n2),
                           ctypes.byref(n4), ctypes.byref(n16)), "route")
    return cls, n2.value, n4.value, n16.value


def merge(part_out, part_lse, offsets, batch, hq, hkv):
    part_out = _c_array(part_out, np.float64)
    part_lse = _c_array(part_lse, np.float64)
    offsets = _c_array(offsets, np.int32)
    out = np.zeros((batch, hq, HEAD_DIM), np.float64)
    lse = np.zeros((batch, hq), np.float64)
    _check(lib().orc_merge(_ptr(part_out), _ptr(part_lse), _ptr(offsets), batch, hq, hkv,
                           _ptr(out), _ptr(lse)), "merge")
    return out, lse


def select_vl(k, q_tail, n_tokens, n_tail, window=128, rho=0.05):
    """Vertical-line selection + FREEZE routing.  k float32 [batch, max_tokens, hkv, 128],
    q_tail float32 [batch, max_tail, hq, 128]; returns (scores fp64 [batch, hkv, max_tokens],
    classes uint8 (0 quantized, 1 vertical line, 2 window) same shape, n_vl [batch, hkv])."""
    k = _c_array(k, np.float32)
    q_tail = _c_array(q_tail, np.float32)
    batch, max_tokens, hkv = k.shape[:3]
    max_tail, hq = q_tail.shape[1:3]
    scores = np.zeros((batch, hkv, max_tokens), np.float64)
    cls = np.zeros((batch, hkv, max_tokens), np.uint8)
    n_vl = np.zeros((batch, hkv), np.int32)
    _check(lib().orc_select_vl(_ptr(k), _ptr(q_tail), batch, max_tokens, hkv, hq, max_tail,
                               _ptr(_c_array(n_tokens, np.int32)), _ptr(_c_array(n_tail, np.int32)),
                               window, float(rho), _ptr(scores), _ptr(cls), _ptr(n_vl)), "select_vl")
    return scores, cls, n_vl


def prefill_attend(q, k, v, n_tokens, cls=None, window=128):
    """Prefill attention with an INT8 prefix (q plain, prefix K and V quantized).  q
    [batch, n_max, hq, 128], k, v [batch, n_max, hkv, 128] float32; cls uint8 [batch,
    hkv, n_max] (1 = vertical line) or None.  Returns (out fp64 like q, k_codes,
    k_scales, v_codes, v_scales)."""
    q, k, v = (_c_array(a, np.float32) for a in (q, k, v))
    batch, n_max, hq = q.shape[:3]
    hkv = k.shape[2]
    tiles = (n_max + 63) // 64
    out = np.zeros(q.shape, np.float64)
    kc, vc = np.zeros(k.shape, np.int8), np.zeros(k.shape, np.int8)
    ks, vs = np.zeros((batch, hkv, tiles), np.float32), np.zeros((batch, hkv, tiles), np.float32)
    c = None if cls is None else _c_array(cls, np.uint8)
    _check(lib().orc_prefill_attend(_ptr(q), _ptr(k), _ptr(v), batch, n_max, hq, hkv,
                                    _ptr(_c_array(n_tokens, np.int32)), _ptr(c), window, _ptr(out),
                                    _ptr(kc), _ptr(ks), _ptr(vc), _ptr(vs)), "prefill_attend")
    return out, kc, ks, vc, vs


def prefill_attend_rows(q, k, v, n_tokens, cls, window, rows):
    """prefill_attend for the listed (request, position) rows only: (out fp64 [n_rows,
    hq, 128], k_codes, k_scales, v_codes, v_scales)."""
    q, k, v = (_c_array(a, np.float32) for a in (q, k, v))
    batch, n_max, hq = q.shape[:3]
    hkv = k.shape[2]
    tiles = (n_max + 63) // 64
    rows = np.asarray(rows, np.int32).reshape(-1, 2)
    rb, rt = np.ascontiguousarray(rows[:, 0]), np.ascontiguousarray(rows[:, 1])
    out = np.zeros((rows.shape[0], hq, HEAD_DIM), np.float64)
    kc, vc = np.zeros(k.shape, np.int8), np.zeros(k.shape, np.int8)
    ks, vs = np.zeros((batch, hkv, tiles), np.float32), np.zeros((batch, hkv, tiles), np.float32)
    c = None if cls is None else _c_array(cls, np.uint8)
    _check(lib().orc_prefill_attend_rows(_ptr(q), _ptr(k), _ptr(v), batch, n_max, hq, hkv,
                                         _ptr(_c_array(n_tokens, np.int32)), _ptr(c), window, rows.shape[0],
                                         _ptr(rb), _ptr(rt), _ptr(out), _ptr(kc), _ptr(ks), _ptr(vc), _ptr(vs)),
           "prefill_attend_rows")
    return out, kc, ks, vc, vs


class Cache:
    """Host-side pools laid out exactly as the GPU pools (one per class)."""

    def __init__(self, heads_per_page, n_int2, n_int4, n_fp16, sentinel_slot=-1, anchor_fp8=False):
        self.heads_per_page = int(heads_per_page)
        self.n_pages = (int(n_int2), int(n_int4), int(n_fp16))
        self.anchor_fp8 = bool(anchor_fp8)
        self.block_bytes = (BLOCK_BYTES[INT2], BLOCK_BYTES[INT4], FP8_ANCHOR_BYTES if anchor_fp8 else BLOCK_BYTES[FP16])
        self.pools = [np.zeros(max(1, n * self.heads_per_page * self.block_bytes[c]), np.uint8)
                      for c, n in zip((INT2, INT4, FP16), self.n_pages)]
        self.sentinel_slot = int(sentinel_slot)

    def _struct(self):
        c = _Cache()
        c.heads_per_page = self.heads_per_page
        for i in range(3):
            c.n_pages[i] = self.n_pages[i]
            c.pool[i] = self.pools[i].ctypes.data
        c.sentinel_slot = self.sentinel_slot
        c.anchor_fp8 = 1 if self.anchor_fp8 else 0
        return c

    def pool_bytes(self, cls):
        n = self.n_pages[cls] * self.heads_per_page * self.block_bytes[cls]
        return self.pools[cls][:n]

    def append(self, k, v, dtype, row_stride, head_stride, rows4=(), slots4=(),
               rows2=(), pages2=(), rows16=(), slots16=()):
        """k, v: numpy arrays (float32, or uint16 bit patterns for bf16/f16)."""
        k = np.ascontiguousarray(k)
        v = np.ascontiguousarray(v)
        r4, s4 = _c_array(rows4, np.int32), _c_array(slots4, np.int32)
        r2, p2 = _c_array(rows2, np.int32), _c_array(pages2, np.int32)
        r16, s16 = _c_array(rows16, np.int32), _c_array(slots16, np.int32)
        assert r4.shape == s4.shape and r16.shape == s16.shape and r2.shape[0] == 32 * p2.shape[0]
        c = self._struct()
        _check(lib().orc_append(ctypes.byref(c), _ptr(k), _ptr(v), dtype, row_stride, head_stride,
                                r4.shape[0], _ptr(r4), _ptr(s4), p2.shape[0], _ptr(r2), _ptr(p2),
                                r16.shape[0], _ptr(r16), _ptr(s16)), "append")

    def reorder(self, tables, n_entries):
        """In-place stable partition of int32 tables [n_tables, max_entries]; returns counts."""
        assert tables.dtype == np.int32 and tables.flags.c_contiguous
        n_entries = _c_array(n_entries, np.int32)
        counts = np.zeros((tables.shape[0], 3), np.int32)
        c = self._struct()
        _check(lib().orc_reorder(ctypes.byref(c), _ptr(tables), tables.shape[0], tables.shape[1],
                                 _ptr(n_entries), _ptr(counts)), "reorder")
        return counts

    def compact_slots(self, tables, n_entries, head_tokens):
        """In-place stable compaction of int32 slot tables [n_tables, max_entries]
        (live entries first); returns the live counts [n_tables, heads]."""
        assert tables.dtype == np.int32 and tables.flags.c_contiguous
        n_entries = _c_array(n_entries, np.int32)
        head_tokens = _c_array(head_tokens, np.int32)
        live = np.zeros(head_tokens.shape, np.int32)
        c = self._struct()
        _check(lib().orc_compact_slots(ctypes.byref(c), _ptr(tables), tables.shape[0], tables.shape[1],
                                       _ptr(n_entries), _ptr(head_tokens), head_tokens.shape[1],
                                       _ptr(live)), "compact_slots")
        return live

    def token(self, page, off, head):
        k = np.zeros(HEAD_DIM, np.float64)
        v = np.zeros(HEAD_DIM, np.float64)
        c = self._struct()
        _check(lib().orc_token(ctypes.byref(c), page, off, head, _ptr(k), _ptr(v)), "token")
        return k, v

    def attend(self, q, batch, hq, hkv, tables, kind, ranges, n_threads=1):
        q = _c_array(q, np.float32)
        tables = _c_array(tables, np.int32)
        ranges = np.ascontiguousarray(ranges, dtype=RANGE_DTYPE)
        out = np.zeros((batch, hq, HEAD_DIM), np.float64)
        lse = np.zeros((batch, hq), np.float64)
        c = self._struct()
        _check(lib().orc_attend(ctypes.byref(c), _ptr(q), batch, hq, hkv, _ptr(tables),
                                tables.shape[0], tables.shape[1], kind, _ptr(ranges),
                                ranges.shape[0], _ptr(out), _ptr(lse), n_threads), "attend")
        return out, lse

    def attend_ranges(self, q, batch, hq, hkv, tables, kind, ranges, n_threads=1):
        q = _c_array(q, np.float32)
        tables = _c_array(tables, np.int32)
        ranges = np.ascontiguousarray(ranges, dtype=RANGE_DTYPE)
        g = hq // hkv
        out = np.zeros((ranges.shape[0], g, HEAD_DIM), np.float64)
        lse = np.zeros((ranges.shape[0], g), np.float64)
        c = self._struct()
        _check(lib().orc_attend_ranges(ctypes.byref(c), _ptr(q), batch, hq, hkv, _ptr(tables),
                                       tables.shape[0], tables.shape[1], kind, _ptr(ranges),
                                       ranges.shape[0], _ptr(out), _ptr(lse), n_threads),
               "attend_ranges")
        return out, lse
