// Decode path of libkvq for gfx950: split-K GQA decode attention read directly from
// the INT2 / INT4 / FP16 pools (dequantization inside the attention loop), and the
// log-sum-exp merge of the split partials.
//
// Method (pages): TriAxialKV key design 4, phase 2 -- every split covers tokens of one
// precision, so a split's loop has no precision branch, and splits are merged by a
// global log-sum-exp reduction.  HyQuant background / Algorithm 3 -- online softmax
// state (m, l, acc) with O = acc / l; the g query heads sharing a KV head are packed
// together (GQA); the FP16 anchor segments are more splits of the same launch.
// IntentKV layout-preserving eviction -- a slot-map entry equal to the sentinel slot
// contributes nothing.
//
// Kernel (one 64-lane wavefront per split; lane l = 16*lb + lr):
//   QK^T on MFMA (v_mfma_f32_16x16x32_f16).  Rows of the 16x16 tile are (query j',
//   channel group i) = 4j' + i; the query operand is block-diagonal (row (j', i) only
//   sees channels of group i), so the result keeps the four per-group partial dot
//   products of every (query, token) apart and the per-token INT4 group scales are
//   applied after the product: lane (lr, lb) ends with query lb's four group partials
//   of token lr.  q enters unscaled (bf16 / fp16 queries are exact in fp16) and the
//   softmax scale is applied to the fp32 result.  INT4 K codes enter as exact
//   offset-coded fp16 values (2^e + c, see below) and the offset's share of the dot
//   product is removed per group together with the zero term z * sum(q).  INT2 K has
//   per-channel scales of at most 9 significant bits: the code operand becomes
//   2^-9 c s, exact in fp16 (one fma per pair of values, see k2_field), and the zero
//   term sum q z of the 32-token pair is added to the logits.
//   Online softmax in base 2 per query with 16-lane DPP row reductions; the running
//   state is rescaled only when a row maximum grows.
//   P V on MFMA.  Rows (query j', group i); the weight operand is p * s (fp16) for
//   group i, the value operand the offset-coded codes with small offsets (64 / 16), and
//   the zero term p * z is accumulated with v_dot2_f32_f16; the offsets' share, 2^e
//   times the sum of the fp16 weights that entered the product, is removed at the end.
//   Lane (lr, lb) ends with query lb's outputs for channels 8 lr .. 8 lr + 7.
//   Tokens come 32 at a time (two 16-token pages, or one INT2 page pair).  Page-table
//   INT2 / INT4 splits stage their bytes through an LDS ring filled by direct
//   HBM -> LDS copies (decode_ring_kernel); FP16 splits and slot maps load into two
//   alternating register windows (decode_kernel).
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>
#include <type_traits>

#include "kvq_internal.h"

namespace kvq {
namespace {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4v __attribute__((ext_vector_type(4)));
// Pool bytes through the global address space (vector memory counters only), and
// page-table entries through the constant address space: wave-uniform entries become
// scalar loads that never wait on the vector loads in flight.
typedef const __attribute__((address_space(1))) uint8_t *gbytes;
typedef const __attribute__((address_space(4))) int32_t *cints;

typedef uint32_t u2v __attribute__((ext_vector_type(2)));

// Per-wave timeline of the fixed-split page-table decode, compiled in only when
// KVQ_WAVE_TIMELINE is defined (the profiling build libkvq_timeline.so): per split, 8
// words: the wave's start, its first window landed and its end (s_memrealtime, 100 MHz),
// the shader clock (s_memtime) at start and end, XCC_ID, HW_ID and the split's window
// count.  Every lane stores the same value.
#ifdef KVQ_WAVE_TIMELINE
__device__ uint64_t *g_timeline = nullptr;
__device__ __forceinline__ void timeline_put(int s_idx, int k, uint64_t v) {
  uint64_t *p = g_timeline;
  if (p) p[(size_t)s_idx * 8 + k] = v;
}
#define KVQ_TIMELINE(s_idx, k, v) timeline_put((s_idx), (k), (v))
#else
#define KVQ_TIMELINE(s_idx, k, v) ((void)0)
#endif
// Cache bytes (codes, scales, zeros, anchors) are read once per launch: their loads and
// copies are non-temporal, so that they do not displace what is read again from the L2
// and the Infinity Cache (page and slot tables, queries, and the split partials the merge
// reads back); measured on the Qwen3-8B-shaped decode: 93.8 -> 91.1 us per launch,
// 98.4 -> 94.0 us per step and layer.  Table entries and queries keep the default policy.
__device__ __forceinline__ uint4 ld4(gbytes p) {
  const u4v v = __builtin_nontemporal_load(reinterpret_cast<const __attribute__((address_space(1))) u4v *>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ uint2 ld2(gbytes p) {
  const u2v v = __builtin_nontemporal_load(reinterpret_cast<const __attribute__((address_space(1))) u2v *>(p));
  return make_uint2(v[0], v[1]);
}
__device__ __forceinline__ uint32_t ld1(gbytes p) {
  return __builtin_nontemporal_load(reinterpret_cast<const __attribute__((address_space(1))) uint32_t *>(p));
}
__device__ __forceinline__ uint32_t ld1_keep(gbytes p) {  // table entries
  return *reinterpret_cast<const __attribute__((address_space(1))) uint32_t *>(p);
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ void report(int32_t *err, int32_t bit) {
  if (err) atomicOr(err, bit);
}

__device__ __forceinline__ h2 as_h2(uint32_t u) { return __builtin_bit_cast(h2, u); }
__device__ __forceinline__ uint32_t as_u32(h2 h) { return __builtin_bit_cast(uint32_t, h); }
__device__ __forceinline__ h8 h8_of(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  const u4v v = {a, b, c, d};
  return __builtin_bit_cast(h8, v);
}
__device__ __forceinline__ h8 h8_of(uint4 v) { return h8_of(v.x, v.y, v.z, v.w); }
__device__ __forceinline__ f4 mfma(h8 a, h8 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ float dot2(h2 a, h2 b, float c) { return __builtin_amdgcn_fdot2(a, b, c, false); }
__device__ __forceinline__ float h2f(uint32_t bits) {
  return __half2float(__ushort_as_half((unsigned short)(bits & 0xffffu)));
}

// Row (16-lane) reductions by DPP row rotations; every lane of the row gets the result.
template <int N>
__device__ __forceinline__ float dpp_ror(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x120 + N, 0xf, 0xf, true));
}
__device__ __forceinline__ float row_max16(float x) {
  x = fmaxf(x, dpp_ror<8>(x));
  x = fmaxf(x, dpp_ror<4>(x));
  x = fmaxf(x, dpp_ror<2>(x));
  return fmaxf(x, dpp_ror<1>(x));
}
__device__ __forceinline__ float row_sum16(float x) {
  x += dpp_ror<8>(x);
  x += dpp_ror<4>(x);
  x += dpp_ror<2>(x);
  return x + dpp_ror<1>(x);
}
// Sum over the 4 lanes of a quad (quad_perm xor 1, then xor 2).
__device__ __forceinline__ float quad_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xf, 0xf, true));
  return x + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xf, 0xf, true));
}

// Lane within the wavefront (a work group may hold several waves).
__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63u); }

// ------------------------------------------------------------ code -> fp16 ----

// A code OR-ed into the low mantissa bits of a power of two gives 2^e + c exactly
// in fp16 (1024 + c for bits 0-3 / 0-1, 256 + c for bits 2-3, 64 + c for bits 4-7 /
// 4-5, 16 + c for bits 6-7).  The K operand of INT2 subtracts 2^e + 2 to get the
// exact centered code; the INT4 K and all V operands keep the offset 2^e and
// remove its contribution after the product: the query is exact in fp16, and the
// V side subtracts 2^e times the sum of the very fp16 weights that entered the
// product, so only fp32 rounding of the larger sums remains.

// v_perm selector giving byte b of the first word in bits 0-7 and byte b of the
// second in bits 16-23 (bytes 1 and 3 zero).
__host__ __device__ constexpr uint32_t pair_sel(uint32_t b) {
  return b | (0x0Cu << 8) | ((4u + b) << 16) | (0x0Cu << 24);
}

// ------------------------------------------------------------------ args ------

struct DecodeArgs {
  int32_t heads, n2, n4, n16;
  gbytes pool2, pool4, pool16;
  int32_t sentinel;
  const void *q;
  int32_t q_dtype, batch, hq, hkv, g, tpr;
  const int32_t *tables;
  int32_t n_tables, max_entries;
  const kvq_split *splits;
  int32_t n_splits;
  float *part_o, *part_lse;
  int32_t *err;
  int32_t only_fp16;  // page mode with the LDS-staged kernel present: this kernel takes FP16 splits only
  int32_t fp8;        // the FP16 class holds FP8 anchors (e4m3 codes and a power-of-two scale per token)
  int32_t q_lds;      // 16-bit queries on a 16-byte boundary: the LDS-staged kernels copy them in (stage_q_issue)
  int32_t *work;            // shared mode: window counters of the groups, then the count of finished workers
  const int32_t *wgroup;    // shared mode: group of each worker
  int32_t n_groups;
};

// FP8 anchors: 8 e4m3 codes (two words) to 8 fp16 (one uint4, channel order kept), times
// the token's power-of-two scale s: exact while the values stay inside fp16's range.
__device__ __forceinline__ uint4 fp8x8_h(uint32_t w0, uint32_t w1, float s) {
  typedef _Float16 hv2 __attribute__((ext_vector_type(2)));
  const hv2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, s, false), b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, s, true);
  const hv2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, s, false), d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, s, true);
  return make_uint4(__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b), __builtin_bit_cast(uint32_t, c),
                    __builtin_bit_cast(uint32_t, d));
}

// The pages of one class: ids first .. first + count - 1 of the unified numbering,
// blocks of head `head` at base + (id - first) * stride.  The host keeps every unified
// slot id (16 x page id) inside int32, so ids relative to `first` fit 32 bits.
template <int CLS>
struct ClassPages {
  gbytes base;
  uint32_t first, count, stride;
  __device__ ClassPages(const DecodeArgs &a, int head) {
    const uint32_t bytes = CLS == KVQ_INT2 ? kI2Bytes : CLS == KVQ_INT4 ? kI4Bytes : a.fp8 ? kF8Bytes : kF16Bytes;
    first = CLS == KVQ_INT2 ? 0u : CLS == KVQ_INT4 ? (uint32_t)a.n2 : (uint32_t)(a.n2 + a.n4);
    count = (uint32_t)(CLS == KVQ_INT2 ? a.n2 : CLS == KVQ_INT4 ? a.n4 : a.n16);
    stride = (uint32_t)a.heads * bytes;
    base = (CLS == KVQ_INT2 ? a.pool2 : CLS == KVQ_INT4 ? a.pool4 : a.pool16) + (uint32_t)head * bytes;
  }
  // Page id -> class-relative index; ids outside the class (negative included) are
  // not `< count` after the unsigned wrap.
  __device__ __forceinline__ uint32_t rel(int32_t id) const { return (uint32_t)id - first; }
  __device__ __forceinline__ gbytes block(uint32_t r) const { return base + (uint64_t)r * stride; }
};

template <int QT>
struct Lds {
  _Float16 q[4 * QT][kHeadDim];      // queries x 2^k (per row), rounded to fp16 (rows beyond g zero)
  float qs[4 * QT];                  // 2^-k of each row: back onto its logits
  _Float16 zero[32];                 // zeros: the off-diagonal blocks of the query operand
  // softmax weights of the current 32 tokens: [query tile][query][token] for one tile;
  // for two tiles [query][token] over the 8 queries (the weights operand's rows 8-15
  // are zero, read from `zero`)
  _Float16 p[QT == 2 ? 1 : QT][QT == 2 ? 8 : 4][32];
};

// ------------------------------------------------------------- per window -----

// What one lane loads for 32 tokens (the next window is loaded while the current one
// is computed).
struct Win {
  uint4 k[2][4];     // K codes: [page half][up to 64 B]
  uint4 km[2];       // INT4 K meta of token lr (per page half)
  uint4 kz;          // INT2 per-channel zeros of channels 8 lr .. 8 lr + 7
  uint4 kg[4];       // INT2 per-channel scales of channels 32 lb .. 32 lb + 31
  uint4 v[8];        // V words / FP16 rows of this lane's 8 tokens
  uint4 vm[2];       // V meta of this lane's 8 tokens, group lr & 3: INT4 (scale, zero) pairs;
                     // INT2 the 8 scales, then the 8 zeros
  uint32_t ok;       // bit h: page half h exists and has the right class
  uint32_t live;     // bit h: the QK token T + 16 h + lr is live
  uint32_t vlive;    // bit q: this lane's P V token q (0..7) is live
};

// The fp16 scale of token t in a block's scale row (2 bytes each, the row 4-byte
// aligned): its 16 bits, or as float bits.
__device__ __forceinline__ uint32_t scale_half(gbytes row, int t) {
  const uint32_t w = ld1(row + 4 * (t >> 1));
  return t & 1 ? w >> 16 : w & 0xffffu;
}
__device__ __forceinline__ float half_value(uint32_t h) { return (float)__builtin_bit_cast(_Float16, (uint16_t)h); }
__device__ __forceinline__ uint32_t scale_bits(gbytes row, int t) { return __float_as_uint(half_value(scale_half(row, t))); }

template <int CLS, bool SLOTS>
struct Loader {
  const DecodeArgs &a;
  const kvq_split sp;
  const int lr, lb;
  const int32_t *trow;
  cints crow;
  const ClassPages<CLS> pages;
  int32_t e_first, e_last;    // page-table entries of the split
  mutable uint32_t errs = 0;  // KVQ_DEVERR_* met so far (reported once, after the loop)
  const int vg;               // channel group whose V scale / zero this lane loads

  // vg_by_channel: the group of the lane's V channels (lr / 4) instead of the group of
  // its weights row (lr % 4), for the P V form that scales the codes.
  __device__ Loader(const DecodeArgs &a_, const kvq_split &s_, int lane, bool vg_by_channel = false)
      : a(a_), sp(s_), lr(lane & 15), lb(lane >> 4),
        trow(a_.tables + (int64_t)s_.table * a_.max_entries), crow((cints)trow), pages(a_, s_.head),
        e_first(s_.tok_begin >> 4), e_last((s_.tok_end - 1) >> 4),
        vg(vg_by_channel ? (lane & 15) >> 2 : lane & 3) {}

  // Page-table mode: the block of a 16-token page half, clamped to the split's entries
  // (a bad id reads the class's first block and is flagged).
  __device__ __forceinline__ gbytes half_page(int32_t T, int h, bool &ok) const {
    const int32_t e = min(max((T >> 4) + h, e_first), e_last);
    const uint32_t r = pages.rel(crow[__builtin_amdgcn_readfirstlane(e)]);
    ok = r < pages.count;
    return pages.block(ok ? r : 0u);
  }

  // Slot-map mode: the block and offset of token t (clamped into the split); live is
  // false for dead, absent or bad entries.
  __device__ __forceinline__ gbytes token_block(int32_t t, int &off, bool &live) const {
    const int32_t tc = min(max(t, sp.tok_begin), sp.tok_end - 1);
    const int32_t slot = (int32_t)ld1_keep((gbytes)(trow + tc));
    const bool dead = a.sentinel >= 0 && slot == a.sentinel;
    const uint32_t r = pages.rel(slot >> 4);
    const bool ok = slot >= 0 && r < pages.count;
    live = ok && !dead && t >= sp.tok_begin && t < sp.tok_end;
    errs |= (!ok && !dead) ? (uint32_t)KVQ_DEVERR_ID : 0u;
    off = ok ? (slot & 15) : 0;
    return pages.block(ok ? r : 0u);
  }

  __device__ void load(int32_t T, Win &w) const {
    const int ti = lb * 8;  // first of this lane's 8 P V tokens
    w.ok = 0;
    w.live = 0;
    w.vlive = 0;
    if (!SLOTS) {
      bool ok0, ok1;
      const gbytes blk0 = half_page(T, 0, ok0), blk1 = half_page(T, 1, ok1);
      errs |= (ok0 && ok1) ? 0u : (uint32_t)KVQ_DEVERR_ID;
      w.ok = (ok0 ? 1u : 0u) | (ok1 ? 2u : 0u);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const gbytes bh = h ? blk1 : blk0;
        if (CLS == KVQ_INT4) {
          w.k[h][0] = ld4(bh + kI4KC + lr * 64 + lb * 16);
          w.km[h] = ld4(bh + kI4KM + lr * 16);
        } else if (CLS == KVQ_INT2) {
          const uint2 x = ld2(bh + kI2KC + lr * 32 + lb * 8);
          w.k[h][0] = make_uint4(x.x, x.y, 0, 0);
        } else if (a.fp8) {  // raw codes of channels 32 lb .. + 31 and the token's scale
          w.k[h][0] = ld4(bh + kF8K + lr * 128 + lb * 32);
          w.k[h][1] = ld4(bh + kF8K + lr * 128 + lb * 32 + 16);
          w.k[h][2].x = scale_bits(bh + kF8KS, lr);
        } else {
#pragma unroll
          for (int m = 0; m < 4; ++m) w.k[h][m] = ld4(bh + kF16K + lr * 256 + lb * 64 + m * 16);
        }
      }
      if (CLS == KVQ_INT2) {  // per-channel meta of the pair: even page ch 0-63, odd 64-127
        const gbytes mb = (lr >> 3) ? blk1 : blk0;
        w.kz = ld4(mb + kI2KZ + (lr & 7) * 16);
        const gbytes g = ((lb >> 1) ? blk1 : blk0) + kI2KS + (lb & 1) * 64;
#pragma unroll
        for (int m = 0; m < 4; ++m) w.kg[m] = ld4(g + 16 * m);
      }
      // P V lanes: 8 tokens of page half lb / 2, offsets 8 (lb & 1) .. + 7.
      const gbytes vb = (lb >> 1) ? blk1 : blk0;
      const int o0 = 8 * (lb & 1);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        if (CLS == KVQ_INT4) w.v[q].x = ld1(vb + kI4VC + (o0 + q) * 64 + lr * 4);
        else if (CLS == KVQ_INT2) w.v[q].x = ld1(vb + kI2VC + (o0 + q) * 32 + (lr >> 1) * 4);
        else if (a.fp8) {  // codes of channels 8 lr .. + 7
          const uint2 c = ld2(vb + kF8V + (o0 + q) * 128 + lr * 8);
          w.v[q] = make_uint4(c.x, c.y, 0u, 0u);
        } else w.v[q] = ld4(vb + kF16V + (o0 + q) * 256 + lr * 16);
      }
      if (CLS == KVQ_FP16 && a.fp8) w.vm[0] = ld4(vb + kF8VS + 2 * o0);  // the 8 tokens' fp16 scales
      if (CLS == KVQ_INT4) {  // (scale, zero) pairs of the 8 tokens
        const gbytes m = vb + kI4VM + (vg * kPage + o0) * 4;
        w.vm[0] = ld4(m);
        w.vm[1] = ld4(m + 16);
      } else if (CLS == KVQ_INT2) {  // the 8 tokens' scales, then their zeros
        const gbytes m = vb + kI2VM + 64 * vg + 2 * o0;
        w.vm[0] = ld4(m);
        w.vm[1] = ld4(m + 32);
      }
    } else {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        int off;
        bool live;
        const gbytes b = token_block(T + 16 * h + lr, off, live);
        if (live) w.live |= 1u << h;
        if (CLS == KVQ_INT4) {
          w.k[h][0] = ld4(b + kI4KC + off * 64 + lb * 16);
          w.km[h] = ld4(b + kI4KM + off * 16);
        } else if (a.fp8) {
          w.k[h][0] = ld4(b + kF8K + off * 128 + lb * 32);
          w.k[h][1] = ld4(b + kF8K + off * 128 + lb * 32 + 16);
          w.k[h][2].x = scale_bits(b + kF8KS, off);
        } else {
#pragma unroll
          for (int m = 0; m < 4; ++m) w.k[h][m] = ld4(b + kF16K + off * 256 + lb * 64 + m * 16);
        }
      }
      uint32_t vm[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        int off;
        bool live;
        const gbytes b = token_block(T + ti + q, off, live);
        if (live) w.vlive |= 1u << q;
        if (CLS == KVQ_INT4) {
          w.v[q].x = ld1(b + kI4VC + off * 64 + lr * 4);
          vm[q] = ld1(b + kI4VM + (vg * kPage + off) * 4);
        } else {
          if (a.fp8) {
            const uint2 c = ld2(b + kF8V + off * 128 + lr * 8);
            w.v[q] = make_uint4(c.x, c.y, 0u, 0u);
            vm[q] = scale_half(b + kF8VS, off);
          } else {
            w.v[q] = ld4(b + kF16V + off * 256 + lr * 16);
          }
        }
      }
      if (CLS == KVQ_INT4) {
        w.vm[0] = make_uint4(vm[0], vm[1], vm[2], vm[3]);
        w.vm[1] = make_uint4(vm[4], vm[5], vm[6], vm[7]);
      } else if (a.fp8) {  // the 8 tokens' fp16 scales, two per word
        w.vm[0] = make_uint4(vm[0] | (vm[1] << 16), vm[2] | (vm[3] << 16), vm[4] | (vm[5] << 16), vm[6] | (vm[7] << 16));
      }
    }
  }
};

// Keeps a 32-bit constant in a VGPR, so that (x & mask) | magic can be one
// v_and_or_b32 (a VOP3 instruction may read only one scalar / literal operand).
__device__ __forceinline__ uint32_t in_vgpr(uint32_t c) {
  asm volatile("" : "+v"(c));
  return c;
}

struct Consts {
  uint32_t m000F, m00F0, m0003, m000C, m0030, m00C0;
  __device__ Consts()
      : m000F(in_vgpr(0x000F000Fu)), m00F0(in_vgpr(0x00F000F0u)), m0003(in_vgpr(0x00030003u)),
        m000C(in_vgpr(0x000C000Cu)), m0030(in_vgpr(0x00300030u)), m00C0(in_vgpr(0x00C000C0u)) {}
};

// INT4 word (channels 8w .. 8w + 7, even ones in the low half) -> 8 fp16 values in
// channel order: 1024 + c for channels with (ch & 2) == 0, 64 + c for the others.
__device__ __forceinline__ h8 cvt_k4(uint32_t x, const Consts &k) {
  const uint32_t y = x >> 8;
  return h8_of((x & k.m000F) | 0x64006400u, (x & k.m00F0) | 0x54005400u, (y & k.m000F) | 0x64006400u,
               (y & k.m00F0) | 0x54005400u);
}
// INT2 byte pair (bits 0-7 and 16-23) -> its 8 codes c as off + 2^-9 c: each 2-bit
// field OR-ed into the mantissa of off = 2, 1/2, 1/8, 1/32 (bits 0-1, 2-3, 4-5, 6-7),
// whose last place is 2^-9 where the field lands.  The K operand is then
// fma(off + 2^-9 c, s, -off s) = 2^-9 c s, exact: -off s is s times a power of two, and
// an INT2 key scale has at most 9 significant bits (the write path rounds it so), so
// c s is an fp16 value for c = 0..3; both are finite while 2 s is.  (For scales below
// 2^-7 the operand lies on fp16's subnormal grid and may round, by at most 2^-24 in all,
// 2^-15 of a key value.)
__device__ __forceinline__ h8 k2_field(uint32_t x, const Consts &k) {
  return h8_of((x & k.m0003) | 0x40004000u, (x & k.m000C) | 0x38003800u, (x & k.m0030) | 0x30003000u,
               (x & k.m00C0) | 0x28002800u);
}
constexpr float kI2Unit = 0x1p-9f;  // unit of the INT2 K operand (above)

constexpr float kNegBig = -1.0e30f;  // running-max start: finite, so no exp2 ever sees -inf - -inf

// One split: writes part_o / part_lse of split s_idx.
template <int QT, int CLS, bool SLOTS>
struct SplitRun {
  const DecodeArgs &a;
  const kvq_split &sp;
  Lds<QT> &L;
  const int lane, lr, lb;
  const Consts k;
  uint32_t sel2[2];    // INT2 V: byte pairs of this lane's even / odd channels
  float scale;         // softmax scale (base 2)
  float qscale[QT];    // and with the staged row's 2^-k: logits of query 4 qt + lb
  h8 Aq[QT][4];        // block-diagonal query operand
  h2 qn[QT][4];        // natural-order q pairs: query 4 qt + lb, channels 8 lr .. 8 lr + 7
  float qsum[QT][4];   // per-group sum of q of query 4 qt + lb (INT4 zero term)
  f4 qoff[QT];         // minus the per-group sum of q x code offset (1024 / 64) of query 4 qt + lb
  // Two query tiles (g = 5..8) form P V with the weights as they are (rows = the 8
  // queries) and the V scale and zero applied to the codes: one set of accumulators
  // for both tiles instead of one per tile with the weights scaled per channel group.
  static constexpr bool kVS = QT == 2;
  f4 acc[kVS ? 1 : QT][8];  // P V accumulators
  float m_run[QT], l_run[QT];  // running maximum of the raw logits, sum of the weights
  float nmq[QT];       // -m_run qscale (minus the base-2 maximum the weights are taken against)
  int qbase = 0;       // first query head (of the g) this wave computes
  float zacc[QT];      // row lr: sum of p z over this lane's tokens (V zero term)
  f4 aone[QT];         // rows 4 lb + e: sums of the fp16 operand weights p s (V code offset),
                       // the product of the weights operand with a ones operand
  h8 ones;             // that operand
  static constexpr int kFold = 16;  // windows between folds of those two into acc
  int since = 0;       // windows since the last fold

  __device__ SplitRun(const DecodeArgs &a_, const kvq_split &sp_, Lds<QT> &L_)
      : a(a_), sp(sp_), L(L_), lane(lane_id()), lr(lane_id() & 15), lb(lane_id() >> 4) {
    scale = kLog2e / sqrtf((float)kHeadDim);
#pragma unroll
    for (int qt = 0; qt < QT; ++qt)  // (INT2 logits come in the K operand's unit 2^-9)
      qscale[qt] = scale * L.qs[4 * qt + lb] * (CLS == KVQ_INT2 ? 1.0f / kI2Unit : 1.0f);
    {
      const uint32_t one = in_vgpr(0x3C003C00u);
      ones = h8_of(one, one, one, one);
    }
    sel2[0] = pair_sel(lr & 1);  // byte lr & 1: even channels of the lane's half word
    sel2[1] = pair_sel((lr & 1) + 2);
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      // lanes of query row jr hold its channels 32 lb .. 32 lb + 31 where lb is the
      // lane's group (lr % 4), zeros (L.zero) elsewhere
      const int jr = 4 * qt + (lr >> 2), gi = lr & 3;
      const _Float16 *src = lb == gi ? &L.q[jr][32 * lb] : L.zero;
#pragma unroll
      for (int m = 0; m < 4; ++m) Aq[qt][m] = *reinterpret_cast<const h8 *>(src + 8 * m);
      float ps = 0.0f, po = 0.0f;
      const h2 *qrow = reinterpret_cast<const h2 *>(&L.q[4 * qt + lb][8 * lr]);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        qn[qt][u] = qrow[u];
        const float pair = (float)qn[qt][u][0] + (float)qn[qt][u][1];
        ps += pair;
        po += (u & 1 ? 64.0f : 1024.0f) * pair;  // channels 8 lr + 2 u, + 1: (ch & 2) == 2 u & 2
      }
      ps = quad_sum(ps);  // lanes (lb, lr): query 4 qt + lb, group lr / 4
      po = quad_sum(po);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        qsum[qt][r] = __shfl(ps, 16 * lb + 4 * r);
        qoff[qt][r] = -__shfl(po, 16 * lb + 4 * r);
      }
      m_run[qt] = kNegBig;
      nmq[qt] = -kNegBig;
      l_run[qt] = 0.0f;
      zacc[qt] = 0.0f;
      aone[qt] = f4{0.0f, 0.0f, 0.0f, 0.0f};
      if (!kVS || qt == 0) {
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) acc[kVS ? 0 : qt][nt] = f4{0.0f, 0.0f, 0.0f, 0.0f};
      }
    }
  }

  __device__ __forceinline__ void window(const Win &w, int32_t T) {
    window(w, T, [] {});
  }

  // 32 tokens starting at T, from the loaded window `w`; `mid()` runs once the
  // window's words have all been used (before the softmax).
  template <typename F>
  __device__ __forceinline__ void window(const Win &w, int32_t T, F &&mid) {
    const bool partial = (T < sp.tok_begin) || (T + 32 > sp.tok_end) || w.ok != 3u;  // (slot maps: ok = 0)
    // live bit h: QK token T + 16 h + lr counts; vlive bit q: P V token T + 8 lb + q counts.
    // Formed inside each branch of a partial window that needs them, so that a full
    // window carries no masks.
    auto live_bits = [&]() -> uint32_t {
      if (SLOTS) return w.live;
      uint32_t l = 0u;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int32_t t = T + 16 * h + lr;
        if (t >= sp.tok_begin && t < sp.tok_end && (w.ok >> h & 1)) l |= 1u << h;
      }
      return l;
    };
    auto vlive_bits = [&]() -> uint32_t {
      if (SLOTS) return w.vlive;
      const int32_t t0 = T + 8 * lb;
      const int32_t lo = min(max(sp.tok_begin - t0, 0), 8), hi = min(max(sp.tok_end - t0, 0), 8);
      return (w.ok >> (lb >> 1) & 1) ? (0xFFu >> (8 - hi)) & (0xFFu << lo) & 0xFFu : 0u;
    };
    // V metadata (scale, zero) of this lane's 8 P V tokens; a token that does not count
    // may sit in an unwritten slot, so its pair is cleared (its weight is 0, and 0 times
    // a non-finite scale would not be).
    uint32_t mv[8] = {w.vm[0].x, w.vm[0].y, w.vm[0].z, w.vm[0].w, w.vm[1].x, w.vm[1].y, w.vm[1].z, w.vm[1].w};
    if (CLS == KVQ_INT4 && partial) {  // word q: token q's (scale, zero)
      const uint32_t vlive = vlive_bits();
#pragma unroll
      for (int q = 0; q < 8; ++q) mv[q] = (vlive >> q & 1) ? mv[q] : 0u;
    } else if (CLS == KVQ_INT2 && partial) {  // words u and 4 + u: tokens 2 u, 2 u + 1 in the halves
      const uint32_t vlive = vlive_bits();
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint32_t mk = ((vlive >> (2 * u) & 1) ? 0x0000ffffu : 0u) | ((vlive >> (2 * u + 1) & 1) ? 0xffff0000u : 0u);
        mv[u] &= mk;
        mv[4 + u] &= mk;
      }
    }
    // The scales and the zeros of tokens 2 u, 2 u + 1 as fp16 pairs.
    auto meta_pair = [&](int u, uint32_t &s2, uint32_t &z2) {
      if (CLS == KVQ_INT2) {
        s2 = mv[u];
        z2 = mv[4 + u];
      } else {
        s2 = __builtin_amdgcn_perm(mv[2 * u + 1], mv[2 * u], 0x05040100u);
        z2 = __builtin_amdgcn_perm(mv[2 * u + 1], mv[2 * u], 0x07060302u);
      }
    };

    // INT2: zero term of the pair, q . z summed over the 128 channels (the 16 lanes of
    // row lb hold 8 channels each); added to the logits of query 4 qt + lb in the K
    // operand's unit 2^-9.  And -off s for the 8 values of each K operand register (k2_field).
    float c2[QT];
    h8 nofs[4];
    if (CLS == KVQ_INT2) {
      const uint32_t kz[4] = {w.kz.x, w.kz.y, w.kz.z, w.kz.w};
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        float bz = 0.0f;
#pragma unroll
        for (int u = 0; u < 4; ++u) bz = dot2(qn[qt][u], as_h2(kz[u]), bz);
        c2[qt] = row_sum16(bz);
      }
      const h8 noff = {(_Float16)-2.0f, (_Float16)-2.0f, (_Float16)-0.5f, (_Float16)-0.5f,
                       (_Float16)-0.125f, (_Float16)-0.125f, (_Float16)-0.03125f, (_Float16)-0.03125f};
#pragma unroll
      for (int m = 0; m < 4; ++m) nofs[m] = h8_of(w.kg[m]) * noff;
    }

    // QK^T: logit (base 2) of query 4 qt + lb and token T + 16 h + lr.
    float x[QT][2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      h8 kb[4];
      if (CLS == KVQ_INT4) {
        const uint4 v = w.k[h][0];
        kb[0] = cvt_k4(v.x, k);
        kb[1] = cvt_k4(v.y, k);
        kb[2] = cvt_k4(v.z, k);
        kb[3] = cvt_k4(v.w, k);
      } else if (CLS == KVQ_INT2) {
        const uint4 v = w.k[h][0];
        kb[0] = __builtin_elementwise_fma(k2_field(v.x, k), h8_of(w.kg[0]), nofs[0]);  // 2^-9 c s
        kb[1] = __builtin_elementwise_fma(k2_field(v.x >> 8, k), h8_of(w.kg[1]), nofs[1]);
        kb[2] = __builtin_elementwise_fma(k2_field(v.y, k), h8_of(w.kg[2]), nofs[2]);
        kb[3] = __builtin_elementwise_fma(k2_field(v.y >> 8, k), h8_of(w.kg[3]), nofs[3]);
      } else if (a.fp8) {
        const float sk = __uint_as_float(w.k[h][2].x);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const uint4 c = w.k[h][m >> 1];
          kb[m] = h8_of(m & 1 ? fp8x8_h(c.z, c.w, sk) : fp8x8_h(c.x, c.y, sk));
        }
      } else {
#pragma unroll
        for (int m = 0; m < 4; ++m) kb[m] = h8_of(w.k[h][m]);
      }
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        // INT4: the accumulators start at minus the offsets' share of the dot products
        f4 d = CLS == KVQ_INT4 ? qoff[qt] : f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < 4; ++m) d = mfma(Aq[qt][m], kb[m], d);
        float s;
        if (CLS == KVQ_INT4) {
          const uint32_t mm[4] = {w.km[h].x, w.km[h].y, w.km[h].z, w.km[h].w};
          s = 0.0f;
#pragma unroll
          for (int r = 0; r < 4; ++r)  // s (q . (offset + c) - q . offset) + z sum(q)
            s = fmaf(h2f(mm[r]), d[r], fmaf(h2f(mm[r] >> 16), qsum[qt][r], s));
        } else if (CLS == KVQ_INT2) {
          s = fmaf(c2[qt], kI2Unit, (d[0] + d[1]) + (d[2] + d[3]));
        } else {
          s = (d[0] + d[1]) + (d[2] + d[3]);
        }
        x[qt][h] = s;  // raw: the softmax applies qscale
      }
    }
    if (partial) {  // tokens that do not count get logit -inf (weight 0)
      // (partial is wave-uniform and rare: the empty asm keeps this a branch instead of
      // selects that every window would execute)
      asm volatile("" ::: "memory");
      const uint32_t live = live_bits();
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) x[qt][h] = (live >> h & 1) ? x[qt][h] : -INFINITY;
    }

    // V operand: this lane's channels 8 lr + nt, its 8 tokens as 4 pairs.
    h8 vb[8];
    {
      uint32_t t[8][4];  // [nt][token pair]
      // Codes go to bits 4-7 / 4-5 / 6-7 only (offset 64 / 64 / 16): the offsets'
      // share of the fp32 accumulators, and so its rounding, stays small.
      if (CLS == KVQ_INT4) {  // 64 + c for every channel
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const uint32_t wa = w.v[2 * u].x, wb = w.v[2 * u + 1].x;
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            const uint32_t y = __builtin_amdgcn_perm(wb, wa, pair_sel(b));
            const int c = b == 0 ? 0 : b == 1 ? 4 : b == 2 ? 1 : 5;  // channel in the low nibble
            t[c][u] = ((y << 4) & k.m00F0) | 0x54005400u;
            t[c + 2][u] = (y & k.m00F0) | 0x54005400u;
          }
        }
      } else if (CLS == KVQ_INT2) {  // 64 + c for channels with (nt >> 1) even, 16 + c for odd
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const uint32_t wa = w.v[2 * u].x, wb = w.v[2 * u + 1].x;
#pragma unroll
          for (int par = 0; par < 2; ++par) {
            const uint32_t y = __builtin_amdgcn_perm(wb, wa, sel2[par]), y4 = y << 4;
            t[par + 0][u] = (y4 & k.m0030) | 0x54005400u;
            t[par + 2][u] = (y4 & k.m00C0) | 0x4C004C00u;
            t[par + 4][u] = (y & k.m0030) | 0x54005400u;
            t[par + 6][u] = (y & k.m00C0) | 0x4C004C00u;
          }
        }
      } else {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          uint4 ra = w.v[2 * u], rb = w.v[2 * u + 1];
          if (a.fp8) {  // tokens 2u, 2u + 1: scales in the halves of word u
            const uint32_t sw = u == 0 ? w.vm[0].x : u == 1 ? w.vm[0].y : u == 2 ? w.vm[0].z : w.vm[0].w;
            ra = fp8x8_h(ra.x, ra.y, half_value(sw & 0xffffu));
            rb = fp8x8_h(rb.x, rb.y, half_value(sw >> 16));
          }
          const uint32_t da[4] = {ra.x, ra.y, ra.z, ra.w}, db[4] = {rb.x, rb.y, rb.z, rb.w};
#pragma unroll
          for (int nt = 0; nt < 8; ++nt) {
            const uint32_t xa = da[nt >> 1], xb = db[nt >> 1];
            t[nt][u] = (nt & 1) ? ((xa >> 16) | (xb & 0xffff0000u)) : ((xa & 0xffffu) | (xb << 16));
          }
        }
        if (partial) {  // absent or dead tokens: keep the operand finite
          const uint32_t vlive = vlive_bits();
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const uint32_t mk = ((vlive >> (2 * u) & 1) ? 0x0000ffffu : 0u) |
                                ((vlive >> (2 * u + 1) & 1) ? 0xffff0000u : 0u);
#pragma unroll
            for (int nt = 0; nt < 8; ++nt) t[nt][u] &= mk;
          }
        }
      }
      if (kVS && CLS != KVQ_FP16) {
        // v = s c + z (fp16, one rounding) with the scale and zero of this lane's channel
        // group (lr / 4) for each token; c = (offset + c) - offset exactly
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          uint32_t s2w, z2w;
          meta_pair(u, s2w, z2w);
          const h2 s2 = as_h2(s2w), z2 = as_h2(z2w);
#pragma unroll
          for (int nt = 0; nt < 8; ++nt) {
            const _Float16 o = (_Float16)v_offset(nt);
            const h2 c = as_h2(t[nt][u]) - h2{o, o};
            t[nt][u] = as_u32(__builtin_elementwise_fma(c, s2, z2));
          }
        }
      }
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) vb[nt] = h8_of(t[nt][0], t[nt][1], t[nt][2], t[nt][3]);
    }
    mid();

    // Online softmax per query (the 16 lanes of row lb) on the raw logits: the base-2
    // logit is x qscale.  The row maximum is taken only when a logit of the wave exceeds
    // its row's running maximum m_run (rare after the first windows); the weights are
    // exp2(x qscale - m_run qscale), one rounding (fma), so at most 1 up to that
    // rounding.
    float alpha_q[QT];  // (kVS) this window's rescale of query 4 qt + lb
    bool rescaled = false;
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      const float t = fmaxf(x[qt][0], x[qt][1]);
      alpha_q[qt] = 1.0f;
      if (__any(t > m_run[qt])) {
        const float mn = fmaxf(m_run[qt], row_max16(t));
        const float mqn = mn * qscale[qt];
        // rows whose maximum stays keep alpha 1 (no -inf - -inf); the first rise from
        // the start values gives 0, which meets an empty state
        const float alpha = mn > m_run[qt] ? __builtin_amdgcn_exp2f(-mqn - nmq[qt]) : 1.0f;
        l_run[qt] *= alpha;
        if (kVS) {
          alpha_q[qt] = alpha;
          rescaled = true;
        } else {
#pragma unroll
          for (int nt = 0; nt < 8; ++nt) acc[kVS ? 0 : qt][nt] *= alpha;
          if (CLS != KVQ_FP16) {
            aone[qt] *= alpha;  // rows 4 lb .. 4 lb + 3: query lb, this lane's own
            zacc[qt] *= __shfl(alpha, 16 * (lr >> 2));  // row lr belongs to query lr / 4
          }
        }
        nmq[qt] = mn > m_run[qt] ? -mqn : nmq[qt];
        m_run[qt] = mn;
      }
      // v_exp_f32: exp2(-inf) = 0; results below 2^-126 may flush to zero, which no
      // softmax weight of consequence is.
      const float p0 = __builtin_amdgcn_exp2f(fmaf(x[qt][0], qscale[qt], nmq[qt]));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(x[qt][1], qscale[qt], nmq[qt]));
      l_run[qt] += p0 + p1;
      L.p[kVS ? 0 : qt][kVS ? 4 * qt + lb : lb][lr] = (_Float16)p0;
      L.p[kVS ? 0 : qt][kVS ? 4 * qt + lb : lb][16 + lr] = (_Float16)p1;
    }
    if (kVS && rescaled) {  // accumulator row 4 lb + r is query 4 lb + r: tile lb, row r
      f4 ar;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float a0 = __shfl(alpha_q[0], 16 * r), a1 = __shfl(alpha_q[kVS ? 1 : 0], 16 * r);
        ar[r] = lb == 0 ? a0 : a1;
      }
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) acc[0][nt] *= ar;
    }

    __syncthreads();  // the weights of this window are in LDS

    // P V.
    if (kVS) {  // weights of query lr (rows 8-15 zero), tokens 8 lb .. 8 lb + 7
      const _Float16 *prow = lr < 8 ? &L.p[0][lr & 7][8 * lb] : L.zero;
      const h8 ap = h8_of(*reinterpret_cast<const uint4 *>(prow));
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) acc[0][nt] = mfma(ap, vb[nt], acc[0][nt]);
      return;
    }
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      const uint4 pw = *reinterpret_cast<const uint4 *>(&L.p[kVS ? 0 : qt][lr >> 2][8 * lb]);
      h8 ap;
      if (CLS == KVQ_FP16) {
        ap = h8_of(pw);
      } else {
        const uint32_t p2[4] = {pw.x, pw.y, pw.z, pw.w};
        uint32_t aw[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          uint32_t s2, z2;  // scales, zeros
          meta_pair(u, s2, z2);
          const h2 pp = as_h2(p2[u]), ap2 = pp * as_h2(s2);
          aw[u] = as_u32(ap2);
          zacc[qt] = dot2(pp, as_h2(z2), zacc[qt]);
        }
        ap = h8_of(aw[0], aw[1], aw[2], aw[3]);
        aone[qt] = mfma(ap, ones, aone[qt]);
      }
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) acc[kVS ? 0 : qt][nt] = mfma(ap, vb[nt], acc[kVS ? 0 : qt][nt]);
    }
    if (CLS != KVQ_FP16 && ++since == kFold) {
      fold();
      since = 0;
    }
  }

  // Row (query lb, group lr / 4) total of the lanes' V zero-term sums (they are kept per
  // P-operand row, lane (lr, lb) for row lr).
  __device__ __forceinline__ float row_zero(int qt) const {
    float z = zacc[qt];
    z += __shfl_xor(z, 16);
    z += __shfl_xor(z, 32);
    return __shfl(z, 4 * lb + (lr >> 2));
  }

  // Code offset of channel 8 lr + nt in the V operand.
  __device__ __forceinline__ static float v_offset(int nt) {
    return CLS == KVQ_INT4 ? 64.0f : CLS == KVQ_INT2 ? ((nt >> 1) & 1 ? 16.0f : 64.0f) : 0.0f;
  }

  // Folds the V zero term and the code offsets into the accumulators every kFold
  // windows, so that they hold sum p v-hat itself: with the offsets in them, an
  // accumulator runs some hundreds of times larger than the result (the offset is 64
  // against codes of 0-15, and the code term cancels most of the zero term), and the
  // fp32 rounding of a long split's additions would grow with its length (measured:
  // row error 2.2e-3 for 6,800-token splits, 9.5e-3 for 27,000, against 6e-4 folded
  // every 8 windows).  Every 16 windows (512 tokens) the 32K-token Qwen3-8B-shaped rows
  // measure 8.2e-4 against 7.6e-4 at 8, and a launch takes about 0.5 % less time.
  // (Only element lr / 4 of an accumulator is a row this lane reports; the others, rows
  // of the block-diagonal product that no lane reads, take additions of no meaning.)
  __device__ __forceinline__ void fold() {
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      const float zrow = row_zero(qt);
      f4 c64, c16;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        c64[e] = fmaf(-64.0f, aone[qt][e], zrow);
        c16[e] = fmaf(-16.0f, aone[qt][e], zrow);
      }
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) acc[kVS ? 0 : qt][nt] += v_offset(nt) == 64.0f ? c64 : c16;
      zacc[qt] = 0.0f;
      aone[qt] = f4{0.0f, 0.0f, 0.0f, 0.0f};
    }
  }

  // Normalize and store: lane (lr, lb) owns query 4 qt + lb, channels 8 lr .. 8 lr + 7
  // (kVS: queries 4 lb .. 4 lb + 3 of the wave's eight, for lb < 2).
  __device__ void finish(int s_idx) {
    if (kVS) {
      float lt[QT];
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) lt[qt] = row_sum16(l_run[qt]);  // query 4 qt + lb, every lane of row lb
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float l0 = __shfl(lt[0], 16 * r), l1 = __shfl(lt[QT - 1], 16 * r);
        const float m0 = -__shfl(nmq[0], 16 * r), m1 = -__shfl(nmq[QT - 1], 16 * r);
        const float l_tot = lb == 0 ? l0 : l1, m = lb == 0 ? m0 : m1;
        const int j = qbase + 4 * lb + r;
        const bool any = l_tot > 0.0f;
        const float inv = any ? 1.0f / l_tot : 0.0f;
        float o[8];
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) o[nt] = any ? acc[0][nt][r] * inv : 0.0f;
        if (lb < 2 && j < a.g) {
          float4 *dst = reinterpret_cast<float4 *>(a.part_o + ((int64_t)s_idx * a.g + j) * kHeadDim + 8 * lr);
          dst[0] = make_float4(o[0], o[1], o[2], o[3]);
          dst[1] = make_float4(o[4], o[5], o[6], o[7]);
          if (lr == 0) a.part_lse[(int64_t)s_idx * a.g + j] = any ? (m + log2f(l_tot)) * kLn2 : -INFINITY;
        }
      }
      return;
    }
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      const float l_tot = row_sum16(l_run[qt]);
      const float zrow = CLS == KVQ_FP16 ? 0.0f : row_zero(qt);  // row (query lb, group lr / 4)
      const int j = qbase + 4 * qt + lb;
      const bool any = l_tot > 0.0f;
      const float inv = any ? 1.0f / l_tot : 0.0f;
      const int r = lr >> 2;
      float o[8];
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) {
        const f4 d = acc[kVS ? 0 : qt][nt];
        const float v = r == 0 ? d[0] : r == 1 ? d[1] : r == 2 ? d[2] : d[3];
        const f4 ao = aone[qt];
        const float arow = r == 0 ? ao[0] : r == 1 ? ao[1] : r == 2 ? ao[2] : ao[3];
        o[nt] = any ? (CLS == KVQ_FP16 ? v : fmaf(-v_offset(nt), arow, v) + zrow) * inv : 0.0f;
      }
      if (j < a.g) {
        float4 *dst = reinterpret_cast<float4 *>(a.part_o + ((int64_t)s_idx * a.g + j) * kHeadDim + 8 * lr);
        dst[0] = make_float4(o[0], o[1], o[2], o[3]);
        dst[1] = make_float4(o[4], o[5], o[6], o[7]);
        if (lr == 0) a.part_lse[(int64_t)s_idx * a.g + j] = any ? (log2f(l_tot) - nmq[qt]) * kLn2 : -INFINITY;
      }
    }
  }
};

template <int QT, int CLS, bool SLOTS>
__device__ void run_split(const DecodeArgs &a, const kvq_split &sp, int s_idx, Lds<QT> &L) {
  const Loader<CLS, SLOTS> ld(a, sp, lane_id(), QT == 2);
  SplitRun<QT, CLS, SLOTS> R(a, sp, L);
  // Two window buffers used alternately: the loads of the next 32 tokens are issued
  // before the current 32 are computed, unconditionally (the last step reloads the
  // current window), so no wait ever has to drain them early.
  const int32_t end = sp.tok_end;
  int32_t T = SLOTS ? sp.tok_begin : (sp.tok_begin & ~15);
  Win wa, wb;
  ld.load(T, wa);
  for (;;) {
    const int32_t T1 = T + 32;
    ld.load(T1 < end ? T1 : T, wb);
    R.window(wa, T);
    if (T1 >= end) break;
    const int32_t T2 = T1 + 32;
    ld.load(T2 < end ? T2 : T1, wa);
    R.window(wb, T1);
    if (T2 >= end) break;
    T = T2;
  }
  if (ld.errs) report(a.err, (int32_t)ld.errs);  // bad ids met by this lane (rare)
  R.finish(s_idx);
}

// ------------------------------------------------------- LDS-staged path -----
//
// Page-table mode, INT2 / INT4 splits.  Every 32-token window is copied HBM -> LDS
// by global_load_lds_dwordx4 (each lane moves 16 B, one instruction fills a 1 KB
// chunk at M0) into a per-wave ring of window slots, several windows ahead of the
// one being computed; no registers hold bytes in flight, so the prefetch depth is
// set by LDS, not by the register file.  The copies are issued from inline assembly
// and waited for with explicit vmcnt counts (the compiler would otherwise wait for
// every copy in flight before each LDS read); the compute is the register path's.

// A split's g query heads are spread over W waves of one work group, 4 QT each (one
// wave up to g = 8, two for g = 16); the waves share the ring, each wave issues the
// copies of every W-th chunk, and a barrier per window publishes the chunks.  With
// one wave no barrier is needed.

template <int W>
constexpr int ring_bytes() { return W == 1 ? 10240 : 15360; }

// Ring geometry tag of the FP16 class when a cache stores its anchors as FP8 (a copy
// layout of its own; the window compute is the FP16 class's).
constexpr int kAnchorF8 = 3;
template <int CLS>
constexpr int compute_class() { return CLS == kAnchorF8 ? KVQ_FP16 : CLS; }

template <int CLS, int W>
struct RingGeom {
  // Copies per window, each from one page block (see RingLoader::issue):
  // INT4: K codes x2, V codes x2, metadata x2 (half-wave each); INT2: the first KB of
  // each page, then the last 512 B of each page (half-wave each); FP16 (one wave, its
  // own kernel with a 32 KB ring): K x4 and V x4 per page.
  // FP8 anchors: K codes x2 and V codes x2 per page, then each page's K and V scales
  // (lanes 0-3).
  static constexpr int kChunks = CLS == KVQ_INT4 ? 6 : CLS == KVQ_INT2 ? 4 : CLS == kAnchorF8 ? 10 : 16;
  static constexpr int kSlotBytes = CLS == KVQ_INT4 ? 5120 : CLS == KVQ_INT2 ? 3072 : CLS == kAnchorF8 ? 8320 : 16384;
  static constexpr int kRingBytes = CLS == KVQ_FP16 ? 2 * 16384 : CLS == kAnchorF8 ? 2 * 8320 : ring_bytes<W>();
  static constexpr int kSlots = kRingBytes / kSlotBytes;
  // Windows copied ahead of the one computed.  One wave refills a slot as soon as its
  // window sits in registers, so every slot is in flight during a compute; with
  // several waves the slot refilled is the previous window's, which the block barrier
  // of the current window shows every wave to have read.
  static constexpr int kAhead = kSlots - (W == 1 ? 0 : 1);
  static_assert(kAhead >= 1, "ring too small");
  // Copies wave w issues per window: chunks c with c % W == w.
  static constexpr int chunks_of(int w) { return (kChunks - w + W - 1) / W; }
};

// One 1 KB chunk of cache bytes: lane L copies 16 B from src to LDS byte lds + 16 L,
// non-temporal (see ld4).  The LDS base goes in M0 (an input the compiler sets, so it may
// reuse the value across copies); an LDS-bound global load needs one wait state after a
// write of M0, hence the s_nop.
__device__ __forceinline__ void dma_chunk(uint32_t lds, gbytes src) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt" : : "v"((uint64_t)src), "{m0}"(lds) : "memory");
}

// One 1 KB chunk from one page block: lane L copies 16 B from base + voff (base
// wave-uniform in SGPRs, voff per lane) to LDS byte lds + 16 L, non-temporal.
__device__ __forceinline__ void dma_block(uint32_t lds, gbytes base, uint32_t voff) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt" : : "v"(voff), "s"((uint64_t)base), "{m0}"(lds) : "memory");
}

// The same with the default cache policy (query rows, read by every split of a head, and
// anchor rows, whose lines several copies share).
__device__ __forceinline__ void dma_block_keep(uint32_t lds, gbytes base, uint32_t voff) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(voff), "s"((uint64_t)base), "{m0}"(lds) : "memory");
}

// Half of a chunk: lanes 0-31 (HI false) or 32-63 (HI true) copy 16 B from base + voff
// to LDS byte lds + 16 L, non-temporal.  The other half is masked off by clearing its half of EXEC
// around the copy (restored after it), with no lane test: every lane of the wave is
// active where this is called.
template <bool HI>
__device__ __forceinline__ void dma_block_half(uint32_t lds, gbytes base, uint32_t voff) {
  uint64_t saved;
  if (HI)
    asm volatile("s_mov_b64 %0, exec\n\ts_mov_b32 exec_lo, 0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2 nt\n\ts_mov_b64 exec, %0"
                 : "=&s"(saved) : "v"(voff), "s"((uint64_t)base), "{m0}"(lds) : "memory");
  else
    asm volatile("s_mov_b64 %0, exec\n\ts_mov_b32 exec_hi, 0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2 nt\n\ts_mov_b64 exec, %0"
                 : "=&s"(saved) : "v"(voff), "s"((uint64_t)base), "{m0}"(lds) : "memory");
}

// One 256 B chunk of cache bytes: lane L copies 4 B from src to LDS byte lds + 4 L,
// non-temporal.
__device__ __forceinline__ void dma_dword(uint32_t lds, gbytes src) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, off nt" : : "v"((uint64_t)src), "{m0}"(lds) : "memory");
}

// The same for table entries (default cache policy).
__device__ __forceinline__ void dma_dword_keep(uint32_t lds, gbytes src) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, off" : : "v"((uint64_t)src), "{m0}"(lds) : "memory");
}

// Lanes 0 and 1 copy the dwords at base + voff to LDS bytes lds, lds + 4 (the other
// lanes copy nothing).
__device__ __forceinline__ void dma_pair(uint32_t lds, gbytes base, uint32_t voff, int lane) {
  if (lane < 2)
    asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, %1" : : "v"(voff), "s"((uint64_t)base), "{m0}"(lds) : "memory");
}

// Waits until at most N copies issued by this wave are still in flight (they complete
// in issue order).
template <int N>
__device__ __forceinline__ void wait_copies() {
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

template <int QT>
__device__ void stage_q(const DecodeArgs &a, const kvq_split &sp, Lds<QT> &L, int q_first);
template <int QT>
__device__ void stage_q_issue(const DecodeArgs &a, const kvq_split &sp, Lds<QT> &L, int q_first);
template <int QT>
__device__ void stage_q_convert(const DecodeArgs &a, Lds<QT> &L, int q_first);

// Issue priority by progress.  A SIMD's waves issue oldest first among equal
// priorities, so waves given equal work would finish one after another and leave the
// SIMD to a single wave at the end.  A wave lowers its priority when half, three
// quarters and seven eighths of its split are done: waves ahead yield to waves behind
// at each of these points, and only the last eighth runs oldest first.
struct ProgressPriority {
  int32_t next, level = 3;
  const int32_t nw;
  __device__ explicit ProgressPriority(int32_t nw_) : next(nw_ >> 1), nw(nw_) {
    __builtin_amdgcn_s_setprio(3);
  }
  __device__ __forceinline__ void step(int32_t n) {  // before window n
    if (n == next && level > 0) {
      --level;
      if (level == 2) __builtin_amdgcn_s_setprio(2);
      else if (level == 1) __builtin_amdgcn_s_setprio(1);
      else __builtin_amdgcn_s_setprio(0);
      next = nw - (nw >> (4 - level));  // 3/4, then 7/8 of the windows
    }
  }
};

// 1 if a < b, else 0 (unsigned), computed on the scalar unit: a and b are wave-uniform.
__device__ __forceinline__ uint32_t s_below(uint32_t a, uint32_t b) {
  uint32_t r;
  asm("s_cmp_lt_u32 %1, %2\n\ts_cselect_b32 %0, 1, 0" : "=s"(r) : "s"(a), "s"(b) : "scc");
  return r;
}

template <int CLS, int W>
struct RingLoader {
  using G = RingGeom<CLS, W>;
  static constexpr int kAhead = G::kAhead;
  const kvq_split sp;
  cints crow;
  const ClassPages<compute_class<CLS>()> pages;
  const int32_t e_last;
  const int lane, lr, lb, wave;
  const uint32_t ring;  // LDS byte address of the ring
  const uint8_t *lds;   // the same, as a pointer
  const uint32_t idr;   // LDS byte address of this wave's page-id ring (kIdSlots x 2 ids)
  const int32_t *lds_idr;
  uint32_t voff[3];     // per-lane source offsets of this class's copies (within a block)
  uint32_t errs = 0;
  const int vg;         // channel group whose V scale / zero this lane reads (see Loader)

  __device__ RingLoader(const DecodeArgs &a, const kvq_split &s_, uint8_t *ring_, int32_t *idr_, int wave_,
                        bool vg_by_channel = false)
      : sp(s_), crow((cints)(a.tables + (int64_t)s_.table * a.max_entries)), pages(a, s_.head),
        e_last((s_.tok_end - 1) >> 4), lane(lane_id()), lr(lane_id() & 15), lb(lane_id() >> 4), wave(wave_),
        ring((uint32_t)(uintptr_t)ring_), lds(ring_), idr((uint32_t)(uintptr_t)idr_), lds_idr(idr_),
        vg(vg_by_channel ? (lane_id() & 15) >> 2 : lane_id() & 3) {
    if (CLS == KVQ_INT4) {
      voff[0] = kI4KC + lr * 64 + lb * 16;                                 // K codes, reader-lane order
      voff[1] = kI4VC + lane * 16;                                         // V codes, natural
      voff[2] = (lane & 15) * 16 + ((lane >> 4) & 1 ? kI4VM : kI4KM);     // K meta | V meta
    } else if (CLS == KVQ_FP16) {
      voff[0] = kF16K + lr * 256 + lb * 64;                                // K rows, reader-lane order
      voff[1] = kF16V + lane * 16;                                         // V rows, natural
      voff[2] = 0;
    } else if (CLS == kAnchorF8) {
      voff[0] = kF8K + lr * 128 + lb * 32;                                 // K codes, reader-lane order
      voff[1] = kF8V + lane * 16;                                          // V codes, natural
      voff[2] = (lane & 1) * 16 + ((lane & 2) ? kF8VS : kF8KS);            // lanes 0-3: K, V scales
    } else {
      voff[0] = lane * 16;                                                 // bytes 0 .. 1023 (and 1024 ..)
      voff[1] = 0;
      voff[2] = 0;
    }
  }

  // Page-table entry of page half h of window T (T is never before the split's first
  // page; past its last page the last entry is repeated).
  __device__ __forceinline__ int32_t entry(int32_t T, int h) const {
    return crow[(uint32_t)__builtin_amdgcn_readfirstlane(min((T >> 4) + h, e_last))];
  }

  // Copies the two entries of window T into id slot `slot` (lanes 0, 1), clamped the
  // same way as entry().
  __device__ __forceinline__ void issue_ids(int32_t T, int slot) const {
    const int32_t e = min((T >> 4) + (lane & 1), e_last);
    dma_pair(idr + 8u * (uint32_t)slot, (gbytes)crow, 4u * (uint32_t)e, lane);
  }
  // The two entries of id slot `slot` (its copy has landed).
  __device__ __forceinline__ void ids(int slot, int32_t &id0, int32_t &id1) const {
    const int2 v = *reinterpret_cast<const int2 *>(lds_idr + 2 * slot);
    id0 = __builtin_amdgcn_readfirstlane(v.x);
    id1 = __builtin_amdgcn_readfirstlane(v.y);
  }

  // Copy c of a window whose page halves live in blocks b0, b1, with per-lane source
  // offsets voff (LDS slot layout in read()).
  __device__ __forceinline__ void copy(int c, uint32_t base, gbytes b0, gbytes b1, const uint32_t (&vo)[3]) const {
    if (CLS == KVQ_INT4) {
      switch (c) {
        case 0: dma_block(base, b0, vo[0]); break;
        case 1: dma_block(base + 1024, b1, vo[0]); break;
        case 2: dma_block(base + 2048, b0, vo[1]); break;
        case 3: dma_block(base + 3072, b1, vo[1]); break;
        case 4: dma_block_half<false>(base + 4096, b0, vo[2]); break;
        default: dma_block_half<true>(base + 4096, b1, vo[2]); break;
      }
    } else if (CLS == KVQ_FP16) {
      // (anchor copies keep the default cache policy: a K row's 128-byte lines are read by
      // four of these copies, 16 B of every 64 at a time, and non-temporal reads fetched
      // them again for each: 119 against 88 us per hybrid-anchor layer)
      // chunk c: region c / 4 (K of page half 0, K of half 1, V of half 0, V of half 1),
      // part c % 4 (K: channels 8 (c % 4) + 32 lb .. + 7 of every token; V: tokens
      // 4 (c % 4) .. + 3)
      const int r = c >> 2, m = c & 3;
      const gbytes b = (r & 1) ? b1 : b0;
      dma_block_keep(base + 1024 * c, r < 2 ? b + 16 * m : b + 1024 * m, r < 2 ? vo[0] : vo[1]);
    } else if (CLS == kAnchorF8) {
      // chunks 0-3: K codes of half c / 2, part c % 2 (channels 32 lb + 16 (c % 2) .. + 15
      // of every token); 4-7: V codes of half (c - 4) / 2, tokens 8 ((c - 4) % 2) .. + 7;
      // 8, 9: the scales of half c - 8 (lanes 0-3)
      if (c < 4) {
        dma_block_keep(base + 1024 * c, ((c >> 1) ? b1 : b0) + 16 * (c & 1), vo[0]);
      } else if (c < 8) {
        dma_block_keep(base + 4096 + 1024 * (c - 4), (((c - 4) >> 1) ? b1 : b0) + 1024 * (c & 1), vo[1]);
      } else if (lane < 4) {
        dma_block_keep(base + 8192 + 64 * (c - 8), c == 8 ? b0 : b1, vo[2]);
      }
    } else {
      switch (c) {
        case 0: dma_block(base, b0, vo[0]); break;
        case 1: dma_block(base + 1024, b1, vo[0]); break;
        // bytes 1024 .. 1535 of page half 0 (lanes 0-31), then of half 1 (lanes 32-63):
        // lane L reads base + 16 L of a base moved by 1024, or by 1024 - 512
        case 2: dma_block_half<false>(base + 2048, b0 + 1024, vo[0]); break;
        default: dma_block_half<true>(base + 2048, b1 + 512, vo[0]); break;
      }
    }
  }

  // Copies this wave's share of window T (page ids id0, id1 of its two halves) into
  // slot `slot`; returns the window's page-half validity bits.  The copy count per
  // window is fixed: a window past the split's end copies the class's first 16-byte
  // line to every lane.
  __device__ __forceinline__ uint32_t issue(int32_t id0, int32_t id1, bool real, int slot) {
    const uint32_t base = ring + (uint32_t)slot * G::kSlotBytes;
    asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory");  // this wave's reads of the slot are done
    if (real) {
      // Validity bits on the scalar unit (a comparison the compiler keeps as a lane mask
      // would be turned into an integer by vector instructions); an invalid id reads the
      // class's first block.
      const uint32_t r0 = pages.rel(id0), r1 = pages.rel(id1);
      const uint32_t ok0 = s_below(r0, pages.count), ok1 = s_below(r1, pages.count);
      const gbytes b0 = pages.block(r0 & (0u - ok0)), b1 = pages.block(r1 & (0u - ok1));
#pragma unroll
      for (int c = 0; c < G::kChunks; ++c)
        if (c % W == wave) copy(c, base, b0, b1, voff);
      errs |= (ok0 & ok1) ^ 1u;  // KVQ_DEVERR_ID (1) unless both halves are valid
      return ok0 | (ok1 << 1);
    }
    const uint32_t zero[3] = {0u, 0u, 0u};
#pragma unroll
    for (int c = 0; c < G::kChunks; ++c)
      if (c % W == wave) copy(c, base, pages.base, pages.base, zero);
    return 0u;
  }

  // Waits for this wave's copies of the oldest window in flight (kAhead windows are,
  // each followed by one id copy).
  __device__ __forceinline__ void wait() const {
    if (W == 1 || wave == 0) wait_copies<(kAhead - 1) * (G::chunks_of(0) + 1)>();
    else if (wave == 1) wait_copies<(kAhead - 1) * (G::chunks_of(1) + 1)>();
    else if (wave == 2) wait_copies<(kAhead - 1) * (G::chunks_of(2) + 1)>();
    else wait_copies<(kAhead - 1) * (G::chunks_of(3) + 1)>();
  }

  // Waits for the copies this wave issued before the prologue's windows (the query rows
  // of stage_q_issue): the kAhead windows and their id copies may still be in flight.
  __device__ __forceinline__ void wait_before_windows() const {
    if (W == 1 || wave == 0) wait_copies<kAhead * (G::chunks_of(0) + 1)>();
    else if (wave == 1) wait_copies<kAhead * (G::chunks_of(1) + 1)>();
    else if (wave == 2) wait_copies<kAhead * (G::chunks_of(2) + 1)>();
    else wait_copies<kAhead * (G::chunks_of(3) + 1)>();
  }

  // Reads window T from slot `slot` into the register window of the compute.
  __device__ __forceinline__ void read(int32_t T, int slot, uint32_t ok, Win &w) const {
    const uint8_t *S = lds + slot * G::kSlotBytes;
    w.ok = ok;
    const int o0 = 8 * (lb & 1);
    if (CLS == KVQ_INT4) {
      // [K codes A][K codes B][V codes A][V codes B][K meta A, V meta A][K meta B, V meta B]
      const uint8_t *M = S + 4096;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        w.k[h][0] = *reinterpret_cast<const uint4 *>(S + 1024 * h + 16 * lane);
        w.km[h] = *reinterpret_cast<const uint4 *>(M + 512 * h + 16 * lr);
      }
      const uint8_t *V = S + 2048 + 1024 * (lb >> 1) + 64 * o0 + 4 * lr;
#pragma unroll
      for (int q = 0; q < 8; ++q) w.v[q].x = *reinterpret_cast<const uint32_t *>(V + 64 * q);
      const uint8_t *VM = M + 512 * (lb >> 1) + 256 + (vg * kPage + o0) * 4;
      w.vm[0] = *reinterpret_cast<const uint4 *>(VM);
      w.vm[1] = *reinterpret_cast<const uint4 *>(VM + 16);
    } else if (CLS == kAnchorF8) {
      // [K A][K B] (2 chunks each, reader-lane order), [V A][V B] (rows of 128 B),
      // [K scales A, V scales A][K scales B, V scales B] (32 B each)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        w.k[h][0] = *reinterpret_cast<const uint4 *>(S + 2048 * h + 16 * lane);
        w.k[h][1] = *reinterpret_cast<const uint4 *>(S + 2048 * h + 1024 + 16 * lane);
        w.k[h][2].x = __float_as_uint(half_value(*reinterpret_cast<const uint16_t *>(S + 8192 + 64 * h + 2 * lr)));
      }
      const uint8_t *V = S + 4096 + 2048 * (lb >> 1) + 128 * o0 + 8 * lr;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const uint2 c = *reinterpret_cast<const uint2 *>(V + 128 * q);
        w.v[q] = make_uint4(c.x, c.y, 0u, 0u);
      }
      w.vm[0] = *reinterpret_cast<const uint4 *>(S + 8192 + 64 * (lb >> 1) + 32 + 2 * o0);
    } else if (CLS == KVQ_FP16) {
      // [K A][K B] (chunk m of a half: lane L's 16 B of the reader lane L), [V A][V B]
      // (token rows of 256 B)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int m = 0; m < 4; ++m) w.k[h][m] = *reinterpret_cast<const uint4 *>(S + 4096 * h + 1024 * m + 16 * lane);
      const uint8_t *V = S + 8192 + 4096 * (lb >> 1) + 256 * o0 + 16 * lr;
#pragma unroll
      for (int q = 0; q < 8; ++q) w.v[q] = *reinterpret_cast<const uint4 *>(V + 256 * q);
    } else {
      // Page P's bytes 0 .. 1023 at 1024 P, its bytes 1024 .. 1535 at 2048 + 512 P.
      auto at = [S](int P, int byte) { return byte < 1024 ? S + 1024 * P + byte : S + 2048 + 512 * P + (byte - 1024); };
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint2 x = *reinterpret_cast<const uint2 *>(S + 1024 * h + kI2KC + 32 * lr + 8 * lb);
        w.k[h][0] = make_uint4(x.x, x.y, 0, 0);
      }
      w.kz = *reinterpret_cast<const uint4 *>(S + 1024 * (lr >> 3) + kI2KZ + 16 * (lr & 7));  // zeros
      const uint8_t *KG = S + 1024 * (lb >> 1) + kI2KS + 64 * (lb & 1);
#pragma unroll
      for (int m = 0; m < 4; ++m) w.kg[m] = *reinterpret_cast<const uint4 *>(KG + 16 * m);
      // V codes of tokens o0 .. o0 + 7: tokens 0-7 sit in the first KB, 8-15 after it
      const uint8_t *V = at(lb >> 1, kI2VC + 32 * o0) + 4 * (lr >> 1);
#pragma unroll
      for (int q = 0; q < 8; ++q) w.v[q].x = *reinterpret_cast<const uint32_t *>(V + 32 * q);
      const uint8_t *VM = at(lb >> 1, kI2VM + 64 * vg + 2 * o0);  // 8 scales, the zeros 32 B on
      w.vm[0] = *reinterpret_cast<const uint4 *>(VM);
      w.vm[1] = *reinterpret_cast<const uint4 *>(VM + 32);
    }
  }
};

template <int CLS, int W, int QT>
__device__ void run_split_ring(const DecodeArgs &a, const kvq_split &sp, int s_idx, Lds<QT> &L, uint8_t *ring,
                               int32_t *idr, int wave) {
  using G = RingGeom<CLS, W>;
  constexpr int A = G::kAhead;
  RingLoader<CLS, W> ld(a, sp, ring, idr, wave, QT == 2);
  const int32_t T0 = sp.tok_begin & ~15;  // INT2 splits start on 32-token pairs
  const int32_t nw = (sp.tok_end - T0 + 31) >> 5;
  // Window i is copied into slot i mod kSlots, A windows ahead of its compute; the page
  // ids of window i are copied into id slot i mod kIdSlots another A windows earlier
  // (before the copies of window i - A, so they have landed when those have).
  constexpr int kIdSlots = 8;  // ids of windows n + A .. n + 2A are live; the first A go to slots A .. 2A - 1
  static_assert(2 * A <= kIdSlots, "id ring too small");
  uint32_t okq = 0;  // validity bits of the windows in flight, 2 per window, newest lowest
  // The start is a chain of dependent memory round trips (split, page ids, data), each
  // long while every wave of the launch starts at once: the query rows are copied first
  // and the page ids of the first windows loaded together, before any window's copies.
  const bool q_lds = a.q_lds != 0;
  if (q_lds) stage_q_issue<QT>(a, sp, L, 4 * QT * wave);
  int32_t pid[A][2];
#pragma unroll
  for (int i = 0; i < A; ++i) {
    pid[i][0] = ld.entry(T0 + 32 * i, 0);
    pid[i][1] = ld.entry(T0 + 32 * i, 1);
  }
#pragma unroll
  for (int i = 0; i < A; ++i) {
    const int32_t Ti = T0 + 32 * i;
    ld.issue_ids(Ti + 32 * A, i + A);
    okq = (okq << 2) | ld.issue(pid[i][0], pid[i][1], i < nw, i);
  }
  // The queries are staged while the first windows are on their way.
  if (q_lds) {
    ld.wait_before_windows();
    stage_q_convert<QT>(a, L, 4 * QT * wave);
  } else {
    stage_q<QT>(a, sp, L, 4 * QT * wave);
  }
  SplitRun<QT, compute_class<CLS>(), false> R(a, sp, L);
  R.qbase = 4 * QT * wave;
  int id_slot = A;  // id slot of window n + A
  ProgressPriority prio(nw);
  // Window n: wait for its copies, read it, compute it; the copies of window n + A go
  // into window n - 1's slot (several waves) or into window n's own slot once its
  // words are used (one wave).
  auto step = [&](int32_t n, int slot_c, int slot_i) {
    if (W == 1) prio.step(n);  // (the waves of one block move in step anyway)
    ld.wait();
    if (n == 0) KVQ_TIMELINE(s_idx, 1, __builtin_amdgcn_s_memrealtime());
    if (W > 1) __syncthreads();  // every wave's chunks of window n have landed, window n - 1 is read
    const uint32_t ok = (okq >> (2 * (A - 1))) & 3u;
    const int32_t Tn = T0 + 32 * (n + A);
    int32_t id0, id1;
    ld.ids(id_slot, id0, id1);  // window n + A
    Win w;
    const int32_t T = T0 + 32 * n;
    const int id_next = (id_slot + A) & (kIdSlots - 1);
    if (W > 1) {
      ld.issue_ids(Tn + 32 * A, id_next);
      okq = (okq << 2) | ld.issue(id0, id1, n + A < nw, slot_i);
      ld.read(T, slot_c, ok, w);
      R.window(w, T);
    } else {  // (issue() waits for the LDS reads)
      ld.read(T, slot_c, ok, w);
      R.window(w, T, [&] {
        ld.issue_ids(Tn + 32 * A, id_next);
        okq = (okq << 2) | ld.issue(id0, id1, n + A < nw, slot_i);
      });
    }
    id_slot = (id_slot + 1) & (kIdSlots - 1);
  };
  if (W == 1) {
    // Unrolled over the ring so that every slot address is a compile-time offset.
    for (int32_t n0 = 0; n0 < nw; n0 += G::kSlots) {
#pragma unroll
      for (int k = 0; k < G::kSlots; ++k)
        if (n0 + k < nw) step(n0 + k, k, k);
    }
  } else {
    int slot_c = 0, slot_i = A;  // slots of the window computed and of the next copy
    for (int32_t n = 0; n < nw; ++n) {
      step(n, slot_c, slot_i);
      slot_c = slot_c + 1 == G::kSlots ? 0 : slot_c + 1;
      slot_i = slot_i + 1 == G::kSlots ? 0 : slot_i + 1;
    }
  }
  wait_copies<0>();  // no copy outlives the wave
  if (ld.errs) report(a.err, (int32_t)ld.errs);
  R.finish(s_idx);
  KVQ_TIMELINE(s_idx, 2, __builtin_amdgcn_s_memrealtime());
  KVQ_TIMELINE(s_idx, 4, __builtin_amdgcn_s_memtime());
  KVQ_TIMELINE(s_idx, 7, (uint64_t)nw);
}


// ------------------------------------------------------------- shared windows -----
//
// Shared mode (page tables, INT2 / INT4, one wave per worker): the workers of a group
// (one token range of one (table, head, class)) take its 32-token windows from the
// group's counter, kSlots windows per claim, so a worker on a part of the chip that
// streams faster takes more windows.  A worker's partial is the softmax over the
// windows it took.  The schedule of run_split_ring is kept: a window's page ids are
// copied two ring depths before its compute and its data one ring depth before; a block
// of windows is claimed one block before its page ids are needed, at the start of a
// block, and its result is read at the start of the next block, where the wait for that
// block's first window already covers it (vector-memory operations of a wave complete
// in issue order).  Claims are per block, not per window: atomics on one address
// serialize (about 250 ns each on MI355X), and a claim per window was measured slower.

// Claims the next n windows of a group: a vector atomic add from lane 0, returning the
// counter before the add, issued from inline assembly so that it joins the ring copies
// in the vector-memory counter (the compiler would wait for every copy in flight before
// the first use of its own atomic's result).  The result register may be read only
// after a wait that covers the atomic.
__device__ __forceinline__ uint32_t claim_issue(int32_t *ctr, uint32_t n) {
  uint32_t old;
  uint64_t save;
  asm volatile(
      "s_mov_b64 %1, exec\n\t"
      "s_mov_b64 exec, 1\n\t"
      "global_atomic_add %0, %2, %3, %4 sc0\n\t"
      "s_mov_b64 exec, %1"
      : "=&v"(old), "=&s"(save)
      : "v"(0u), "v"(n), "s"((uint64_t)(uintptr_t)ctr)
      : "memory");
  return old;
}

// Waits until at most N vector-memory operations of this wave are in flight, then
// returns lane 0's value of x (a claim result the wait covers) in a scalar register.
template <int N>
__device__ __forceinline__ uint32_t wait_take(uint32_t x) {
  uint32_t r;
  asm volatile("s_waitcnt vmcnt(%2)\n\tv_readfirstlane_b32 %0, %1" : "=s"(r) : "v"(x), "n"(N) : "memory");
  return r;
}

// Issue priority by the progress of the worker's group.  A group's windows are shared by
// its workers only, so a group whose waves sit behind others on their SIMDs (a SIMD
// issues the oldest of equal-priority waves first) would end late while the others idle;
// a wave whose group has handed out more of its windows yields to waves of groups that
// are further behind: priority 3 below half the windows claimed, 2 below three quarters,
// 1 below seven eighths, 0 after.
struct GroupPriority {
  int level = -1;
  __device__ __forceinline__ void set(uint32_t claimed, uint32_t nw) {
    const int want = 8u * claimed < 4u * nw ? 3 : 8u * claimed < 6u * nw ? 2 : 8u * claimed < 7u * nw ? 1 : 0;
    if (want == level) return;
    level = want;
    if (want == 3) __builtin_amdgcn_s_setprio(3);
    else if (want == 2) __builtin_amdgcn_s_setprio(2);
    else if (want == 1) __builtin_amdgcn_s_setprio(1);
    else __builtin_amdgcn_s_setprio(0);
  }
};

template <int CLS, int QT>
__device__ void run_shared_ring(const DecodeArgs &a, const kvq_split &sp, int s_idx, Lds<QT> &L, uint8_t *ring,
                                int32_t *idr, int32_t *win, int32_t *ctr) {
  using G = RingGeom<CLS, 1>;
  constexpr int S = G::kSlots;      // windows per claim, per unrolled pass, and in flight
  constexpr int A = G::kAhead;
  static_assert(A == S, "one wave refills a slot as soon as its window sits in registers");
  constexpr int C = G::chunks_of(0);  // data copies per window (plus one id copy)
  constexpr int kWin = 16;            // window-start ring: window i at i % kWin
  static_assert(4 * S <= kWin, "window ring too small");
  constexpr int kIdSlots = 8;  // ids of windows n + A .. n + 2A are live; the first A go to slots A .. 2A - 1
  static_assert(2 * A <= kIdSlots, "id ring too small");
  RingLoader<CLS, 1> ld(a, sp, ring, idr, 0, QT == 2);
  const int lane = lane_id();
  const int32_t T0 = sp.tok_begin & ~15;
  const uint32_t nw = (uint32_t)((sp.tok_end - T0 + 31) >> 5);  // windows of the group
  // Window i of this worker starts at token win[i % kWin], or -1 once the group is
  // exhausted (claims only grow, so every later window is -1 too).
  auto put = [&](int32_t i, uint32_t k0) {  // windows i .. i + S - 1 are the group's k0 ..
    if (lane < S) win[(i + lane) & (kWin - 1)] = k0 + (uint32_t)lane < nw ? T0 + 32 * (int32_t)(k0 + lane) : -1;
  };
  auto start = [&](int32_t i) { return win[i & (kWin - 1)]; };
  // The first three blocks in one claim: nothing is in flight yet, so waiting for it
  // costs its own latency only.
  // (the query rows are copied first, alongside the claim; the first windows' page ids
  // are loaded together, as in run_split_ring)
  const bool q_lds = a.q_lds != 0;
  if (q_lds) stage_q_issue<QT>(a, sp, L, 0);
  uint32_t k0 = 0u;
  if (lane == 0) k0 = (uint32_t)atomicAdd(ctr, 3 * S);
  k0 = (uint32_t)__builtin_amdgcn_readfirstlane((int)k0);
#pragma unroll
  for (int b = 0; b < 3; ++b) put(b * S, k0 + (uint32_t)(b * S));
  uint32_t okq = 0;
  int32_t pid[A][2];
#pragma unroll
  for (int i = 0; i < A; ++i) {
    const int32_t Ti = start(i);
    const int32_t Te = Ti >= 0 ? Ti : T0;
    pid[i][0] = ld.entry(Te, 0);
    pid[i][1] = ld.entry(Te, 1);
  }
#pragma unroll
  for (int i = 0; i < A; ++i) {
    const int32_t Ti = start(i), Tn = start(i + A);
    ld.issue_ids(Tn >= 0 ? Tn : T0, i + A);
    okq = (okq << 2) | ld.issue(pid[i][0], pid[i][1], Ti >= 0, i);
  }
  if (q_lds) {
    ld.wait_before_windows();
    stage_q_convert<QT>(a, L, 0);
  } else {
    stage_q<QT>(a, sp, L, 0);
  }
  SplitRun<QT, CLS, false> R(a, sp, L);
  int id_slot = A;     // id slot of window n + A
  uint32_t pend = 0u;  // the claim issued at the start of the current block
  GroupPriority prio;
  // Window n = block start + r: wait for its data (and, at a block start, for the claim
  // issued one block earlier), read it, compute it; the copies of window n + A go into
  // its slot once its words are in registers.  Returns false once the group is
  // exhausted.
  auto step = [&](int32_t n, auto rc) -> bool {
    constexpr int r = decltype(rc)::value;
    const int32_t Tw = start(n);
    if (Tw < 0) return false;
    if (r == 0) {
      if (n >= S) {
        const uint32_t k = wait_take<(S - 1) * (C + 1)>(pend);
        put(n + 2 * S, k);  // the block two ahead
        prio.set(k, nw);
      } else {
        wait_copies<(S - 1) * (C + 1)>();
      }
    } else {
      wait_copies<(S - 1) * (C + 1) + 1>();  // (a claim was issued since window n's copies)
    }
    const uint32_t ok = (okq >> (2 * (A - 1))) & 3u;
    int32_t id0, id1;
    ld.ids(id_slot, id0, id1);  // window n + A
    const int id_next = (id_slot + A) & (kIdSlots - 1);
    Win w;
    ld.read(Tw, r, ok, w);
    R.window(w, Tw, [&] {
      if (r == 0) pend = claim_issue(ctr, S);  // block three ahead
      const int32_t Tf = start(n + 2 * A);
      ld.issue_ids(Tf >= 0 ? Tf : T0, id_next);
      okq = (okq << 2) | ld.issue(id0, id1, start(n + A) >= 0, r);
    });
    id_slot = (id_slot + 1) & (kIdSlots - 1);
    return true;
  };
  bool more = true;
  for (int32_t n0 = 0; more; n0 += S) {
    more = step(n0, std::integral_constant<int, 0>{});
    if (more && S > 1) more = step(n0 + 1, std::integral_constant<int, (S > 1 ? 1 : 0)>{});
    if (more && S > 2) more = step(n0 + 2, std::integral_constant<int, (S > 2 ? 2 : 0)>{});
  }
  wait_copies<0>();  // no copy or claim outlives the wave
  if (ld.errs) report(a.err, (int32_t)ld.errs);
  R.finish(s_idx);
}

// Every worker of a shared launch counts itself out, and the last one resets the counters
// for the next launch (every other worker has stopped claiming by then).  The count is
// two-level, so that no address takes more than 64 of the workers' atomics, all of
// which arrive at about the same time: worker s counts into sub-counter s % 64, and the
// last worker of each sub-counter into the top one.
constexpr int kDoneSubs = 64;

__device__ void shared_exit(const DecodeArgs &a, int s_idx) {
  const int lane = lane_id();
  int32_t *sub = a.work + a.n_groups, *top = sub + kDoneSubs;
  const int32_t k = s_idx % kDoneSubs;
  const int32_t members = (a.n_splits - 1 - k) / kDoneSubs + 1;  // workers k, k + 64, ...
  const int32_t subs = min(a.n_splits, kDoneSubs);
  int last = 0;
  if (lane == 0 && atomicAdd(sub + k, 1) == members - 1) last = atomicAdd(top, 1) == subs - 1;
  last = __builtin_amdgcn_readfirstlane(last);
  if (last)
    for (int i = lane; i <= a.n_groups + kDoneSubs; i += 64)
      __hip_atomic_store(a.work + i, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Slot maps, INT4 splits, one wave.  Every token of a window may live in a different
// page, so the window's 32 slot ids are copied into LDS one window ahead of its data
// (lanes 0-31, 4 B each), and the data copies gather per token into the INT4 window
// layout of the page-table path: K codes (2 x 1 KB, reader-lane order), V codes
// (2 x 1 KB), K metadata (lanes 0-31, 16 B per token), V metadata (2 x 256 B of 4-byte
// (token, group) pieces).  Eight copies per window, slot ids first.
struct SlotRingLoader {
  using G = RingGeom<KVQ_INT4, 1>;
  static constexpr int kCopies = 8;
  static constexpr int kIdBlocks = 4;  // slot-id blocks of 128 B, window i in block i mod 4
  const kvq_split sp;
  gbytes trow;
  const ClassPages<KVQ_INT4> pages;
  const int32_t sentinel;
  const int lane, lr, lb;
  const uint32_t ring, ids;  // LDS byte addresses of the data ring and of the slot-id blocks
  const uint8_t *lds_ring;
  const int32_t *lds_ids;
  uint32_t errs = 0;
  const int vg;  // channel group whose V scale / zero this lane reads (see Loader)

  __device__ SlotRingLoader(const DecodeArgs &a, const kvq_split &s_, uint8_t *ring_, int32_t *ids_,
                            bool vg_by_channel = false)
      : sp(s_), trow((gbytes)(a.tables + (int64_t)s_.table * a.max_entries)), pages(a, s_.head),
        sentinel(a.sentinel), lane(lane_id()), lr(lane_id() & 15), lb(lane_id() >> 4),
        ring((uint32_t)(uintptr_t)ring_), ids((uint32_t)(uintptr_t)ids_), lds_ring(ring_), lds_ids(ids_),
        vg(vg_by_channel ? (lane_id() & 15) >> 2 : lane_id() & 3) {}

  // Slot ids of window T (entries clamped into the split) into id block `blk`.
  __device__ __forceinline__ void issue_ids(int32_t T, int blk) {
    const int32_t e = min(T + (lane & 31), sp.tok_end - 1);
    if (lane < 32) dma_dword_keep(ids + 128u * (uint32_t)blk, trow + 4 * (int64_t)e);
  }

  // Block of a slot id (the class's first block for ids outside the class).
  __device__ __forceinline__ gbytes block_of(int32_t id, int &off) const {
    const uint32_t r = pages.rel(id >> 4);
    const bool ok = id >= 0 && r < pages.count;
    off = ok ? (id & 15) : 0;
    return pages.block(ok ? r : 0u);
  }

  // Copies the data of window T, whose slot ids sit in block `blk`, into data slot
  // `slot`; returns the window's live mask (bit i: token T + i counts).  A window past
  // the split's end (`real` false) copies one 16-byte line to every lane.
  __device__ __forceinline__ uint32_t issue_data(int32_t T, int blk, bool real, int slot) {
    const int32_t *I = lds_ids + 32 * blk;
    const uint32_t base = ring + (uint32_t)slot * G::kSlotBytes;
    asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory");  // reads of the slot are done
    if (!real) {
      for (int c = 0; c < 5; ++c) dma_chunk(base + 1024 * c, pages.base);
      dma_dword(base + 4608, pages.base);
      dma_dword(base + 4864, pages.base);
      return 0u;
    }
    const int32_t idk0 = I[lr], idk1 = I[16 + lr], idv0 = I[lane >> 2], idv1 = I[16 + (lane >> 2)];
    const int32_t idm = I[lane & 31];
    int ok0, ok1, ov0, ov1, om;
    const gbytes bk0 = block_of(idk0, ok0), bk1 = block_of(idk1, ok1);
    const gbytes bv0 = block_of(idv0, ov0), bv1 = block_of(idv1, ov1), bm = block_of(idm, om);
    dma_chunk(base, bk0 + kI4KC + ok0 * 64 + lb * 16);
    dma_chunk(base + 1024, bk1 + kI4KC + ok1 * 64 + lb * 16);
    dma_chunk(base + 2048, bv0 + kI4VC + ov0 * 64 + (lane & 3) * 16);
    dma_chunk(base + 3072, bv1 + kI4VC + ov1 * 64 + (lane & 3) * 16);
    if (lane < 32) dma_chunk(base + 4096, bm + kI4KM + om * 16);
    dma_dword(base + 4608, bk0 + kI4VM + ((lane >> 4) * kPage + ok0) * 4);
    dma_dword(base + 4864, bk1 + kI4VM + ((lane >> 4) * kPage + ok1) * 4);
    // live mask from lanes 0-31 (token T + lane)
    const int32_t t = T + (lane & 31);
    const bool dead = sentinel >= 0 && idm == sentinel;
    const uint32_t r = pages.rel(idm >> 4);
    const bool ok = idm >= 0 && r < pages.count;
    const bool in = lane < 32 && t >= sp.tok_begin && t < sp.tok_end;
    if (in && !dead && !ok) errs |= KVQ_DEVERR_ID;
    return (uint32_t)__ballot(in && !dead && ok);
  }

  // Reads window T from data slot `slot`; live mask `mask`.
  __device__ __forceinline__ void read(int slot, uint32_t mask, Win &w) const {
    const uint8_t *S = lds_ring + slot * G::kSlotBytes;
    const uint8_t *M = S + 4096;
    w.ok = mask == 0xFFFFFFFFu ? 3u : 0u;  // a window with every token live needs no masks
    w.live = ((mask >> lr) & 1u) | (((mask >> (16 + lr)) & 1u) << 1);
    w.vlive = (mask >> (8 * lb)) & 0xFFu;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      w.k[h][0] = *reinterpret_cast<const uint4 *>(S + 1024 * h + 16 * lane);
      w.km[h] = *reinterpret_cast<const uint4 *>(M + 256 * h + 16 * lr);
    }
    const int o0 = 8 * (lb & 1);
    const uint8_t *V = S + 2048 + 1024 * (lb >> 1) + 64 * o0 + 4 * lr;
#pragma unroll
    for (int q = 0; q < 8; ++q) w.v[q].x = *reinterpret_cast<const uint32_t *>(V + 64 * q);
    const uint8_t *VM = M + 512 + 256 * (lb >> 1) + (vg * kPage + o0) * 4;
    w.vm[0] = *reinterpret_cast<const uint4 *>(VM);
    w.vm[1] = *reinterpret_cast<const uint4 *>(VM + 16);
  }
};

template <int QT>
__device__ void run_split_slots_ring(const DecodeArgs &a, const kvq_split &sp, int s_idx, Lds<QT> &L,
                                     uint8_t *ring, int32_t *id_blocks) {
  using G = RingGeom<KVQ_INT4, 1>;
  static_assert(G::kSlots == 2, "two data slots");
  constexpr int C = SlotRingLoader::kCopies - 1;  // data copies per window (the eighth: its ids)
  SlotRingLoader ld(a, sp, ring, id_blocks, QT == 2);
  const int32_t T0 = sp.tok_begin;
  const int32_t nw = (sp.tok_end - T0 + 31) >> 5;
  // Window i: slot ids copied at iteration i - 4 into id block i mod 4, data at
  // iteration i - 2 into data slot i mod 2 (as soon as window i - 2 sits in registers),
  // computed at iteration i, so two windows are in flight during every compute and a
  // window's ids have two iterations to land before its data copies need them.  Per
  // iteration: (wait: data of i, and so the ids of i + 2, copied before it), read i,
  // ids of i + 4, data of i + 2, compute i.  Copies complete in issue order; the wait
  // counts what follows: the ids of i + 3 and the data of i + 1.
  static_assert(SlotRingLoader::kIdBlocks == 4, "ids of windows i + 2 .. i + 4 are live");
  // The query rows are copied before the first ids (a.q_lds), so the wait for the ids
  // of window 0 covers them (copies complete in issue order).
  const bool q_lds = a.q_lds != 0;
  if (q_lds) stage_q_issue<QT>(a, sp, L, 0);
  ld.issue_ids(T0, 0);
  ld.issue_ids(T0 + 32, 1);
  ld.issue_ids(T0 + 64, 2);
  wait_copies<2>();  // ids of window 0
  uint32_t mask0 = ld.issue_data(T0, 0, true, 0);
  ld.issue_ids(T0 + 96, 3);
  wait_copies<C + 2>();  // ids of window 1 (then: ids of 2, data of 0, ids of 3)
  uint32_t mask1 = ld.issue_data(T0 + 32, 1, 1 < nw, 1);
  if (q_lds) stage_q_convert<QT>(a, L, 0);
  else stage_q<QT>(a, sp, L, 0);
  SplitRun<QT, KVQ_INT4, true> R(a, sp, L);
  ProgressPriority prio(nw);
  for (int32_t n = 0; n < nw; ++n) {
    prio.step(n);
    wait_copies<C + 1>();  // the data of window n and the ids of n + 2 (then: ids of n + 3, data of n + 1)
    Win w;
    ld.read(n & 1, mask0, w);
    ld.issue_ids(T0 + 32 * (n + 4), (n + 4) & 3);
    const uint32_t mask2 = ld.issue_data(T0 + 32 * (n + 2), (n + 2) & 3, n + 2 < nw, n & 1);
    R.window(w, T0 + 32 * n);
    mask0 = mask1;
    mask1 = mask2;
  }
  wait_copies<0>();  // no copy outlives the wave
  if (ld.errs) report(a.err, (int32_t)ld.errs);
  R.finish(s_idx);
}

// Checks split s_idx.  A split this launch does not own returns false at once; an
// owned split that is malformed or empty (or of a class with no pages) gets O = 0,
// lse = -inf (and an error bit when malformed) and returns false.
template <int QT, bool SLOTS, bool RING>
__device__ bool split_check(const DecodeArgs &a, int s_idx, kvq_split &sp, int q_first = 0) {
  const int lane = lane_id();
  sp = a.splits[s_idx];
  const int64_t cap = SLOTS ? (int64_t)a.max_entries : (int64_t)a.max_entries * kPage;
  const bool ok = sp.table >= 0 && sp.table < a.n_tables && sp.head >= 0 && sp.head < a.heads &&
                  sp.cls >= 0 && sp.cls <= 2 && sp.tok_begin >= 0 && sp.tok_end >= sp.tok_begin &&
                  sp.tok_end <= cap &&
                  (sp.cls != KVQ_INT2 || (!SLOTS && sp.tok_begin % kGroup == 0 && sp.tok_end % kGroup == 0));
  // With the LDS-staged kernel in the launch, it owns every split except the FP16 ones
  // of a cache that has FP16 pages, which the register-staged one takes.
  const bool fp16_elsewhere = ok && sp.cls == KVQ_FP16 && a.n16 > 0;
  if (RING ? fp16_elsewhere : (a.only_fp16 && !fp16_elsewhere)) return false;
  const int32_t n_cls = !ok ? 0 : sp.cls == KVQ_INT2 ? a.n2 : sp.cls == KVQ_INT4 ? a.n4 : a.n16;
  if (!ok || sp.tok_end == sp.tok_begin || n_cls == 0) {
    if (lane == 0 && (!ok || sp.tok_end > sp.tok_begin))  // (a class with no pages: its ids are bad)
      report(a.err, ok ? KVQ_DEVERR_ID : KVQ_DEVERR_SPLIT);
    for (int j = q_first; j < min(q_first + 4 * QT, a.g); ++j) {
      float *o = a.part_o + ((int64_t)s_idx * a.g + j) * kHeadDim;
      *reinterpret_cast<float2 *>(o + 2 * lane) = make_float2(0.0f, 0.0f);
      if (lane == 0) a.part_lse[(int64_t)s_idx * a.g + j] = -INFINITY;
    }
    return false;
  }
  return true;
}

// Stages the split's query heads q_first .. q_first + 4 QT - 1 in LDS rows 0 .. 4 QT - 1
// (rows past g zero) as fp16, each row multiplied by the power of two 2^k that brings
// its largest magnitude into [2^14, 2^15): exact, so any finite query fits fp16's range
// and keeps 11 significant bits relative to its largest channel; L.qs holds 2^-k, which
// the row's logits take back.  Every wave of the work group calls it alike.
// Row j of the staged queries from its channels lane and lane + 64 (v), given the
// row's largest magnitude mx.
template <int QT>
__device__ __forceinline__ void stage_row(Lds<QT> &L, int j, const float (&v)[2], float mx) {
  const int lane = lane_id();
  int k = 0;
  if (mx > 0.0f) {  // mx = f 2^e with f in [0.5, 1)
    int e;
    (void)frexpf(mx, &e);
    k = min(15 - e, 100);
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) L.q[j][lane + 64 * i] = (_Float16)ldexpf(v[i], k);
  if (lane == 0) L.qs[j] = ldexpf(1.0f, -k);
}

template <int QT>
__device__ void stage_q(const DecodeArgs &a, const kvq_split &sp, Lds<QT> &L, int q_first) {
  const int lane = lane_id();
  const int b = sp.table / a.tpr;
  const int kvh = (sp.table % a.tpr) * a.heads + sp.head;
  // Every load is issued before any value is used (rows at or past g read row g - 1).
  float v[4 * QT][2], mx[4 * QT];
  const int64_t row0 = (int64_t)b * a.hq + (int64_t)kvh * a.g;
  if (a.q_dtype == KVQ_F32) {
    const float *q = static_cast<const float *>(a.q);
#pragma unroll
    for (int j = 0; j < 4 * QT; ++j)
#pragma unroll
      for (int i = 0; i < 2; ++i) v[j][i] = q[(row0 + min(q_first + j, a.g - 1)) * kHeadDim + lane + 64 * i];
  } else {
    const uint16_t *q = static_cast<const uint16_t *>(a.q);
    uint32_t h[4 * QT][2];
#pragma unroll
    for (int j = 0; j < 4 * QT; ++j)
#pragma unroll
      for (int i = 0; i < 2; ++i) h[j][i] = q[(row0 + min(q_first + j, a.g - 1)) * kHeadDim + lane + 64 * i];
#pragma unroll
    for (int j = 0; j < 4 * QT; ++j)
#pragma unroll
      for (int i = 0; i < 2; ++i) v[j][i] = a.q_dtype == KVQ_BF16 ? __uint_as_float(h[j][i] << 16) : h2f(h[j][i]);
  }
#pragma unroll
  for (int j = 0; j < 4 * QT; ++j) {
#pragma unroll
    for (int i = 0; i < 2; ++i) v[j][i] = q_first + j < a.g ? v[j][i] : 0.0f;
    mx[j] = fmaxf(fabsf(v[j][0]), fabsf(v[j][1]));
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1)  // the rows' reductions side by side
#pragma unroll
    for (int j = 0; j < 4 * QT; ++j) mx[j] = fmaxf(mx[j], __shfl_xor(mx[j], off));
#pragma unroll
  for (int j = 0; j < 4 * QT; ++j) stage_row(L, j, v[j], mx[j]);
  if (lane < 32) L.zero[lane] = (_Float16)0.0f;
  __syncthreads();
}

// The same in two steps for 16-bit queries on a 16-byte boundary (a.q_lds): the raw
// rows go to L.q by LDS-bound copies (one per four rows: lane L takes row 4 c + L / 16,
// bytes 16 (L % 16) .. + 15), issued before the split's first windows; rows at or past g
// copy row g - 1, a valid row of the same head (they are staged as zeros).  Once the
// copies have landed, stage_q_convert stages the rows in place.
template <int QT>
__device__ void stage_q_issue(const DecodeArgs &a, const kvq_split &sp, Lds<QT> &L, int q_first) {
  const int lane = lane_id();
  const int b = sp.table / a.tpr;
  const int kvh = (sp.table % a.tpr) * a.heads + sp.head;
  const gbytes base = (gbytes)a.q + ((int64_t)b * a.hq + (int64_t)kvh * a.g) * (kHeadDim * 2);
  const uint32_t lds = (uint32_t)(uintptr_t)&L.q[0][0];
#pragma unroll
  for (int c = 0; c < QT; ++c) {
    const int row = min(q_first + 4 * c + (lane >> 4), a.g - 1);
    dma_block_keep(lds + 1024u * (uint32_t)c, base, (uint32_t)row * (kHeadDim * 2) + 16u * (uint32_t)(lane & 15));
  }
}

template <int QT>
__device__ void stage_q_convert(const DecodeArgs &a, Lds<QT> &L, int q_first) {
  const int lane = lane_id();
  uint32_t raw[4 * QT][2];
#pragma unroll
  for (int j = 0; j < 4 * QT; ++j)
#pragma unroll
    for (int i = 0; i < 2; ++i) raw[j][i] = reinterpret_cast<const uint16_t *>(&L.q[j][0])[lane + 64 * i];
  float v[4 * QT][2], mx[4 * QT];
#pragma unroll
  for (int j = 0; j < 4 * QT; ++j) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
      v[j][i] = q_first + j >= a.g ? 0.0f : a.q_dtype == KVQ_BF16 ? __uint_as_float(raw[j][i] << 16) : h2f(raw[j][i]);
    mx[j] = fmaxf(fabsf(v[j][0]), fabsf(v[j][1]));
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1)  // the rows' reductions side by side
#pragma unroll
    for (int j = 0; j < 4 * QT; ++j) mx[j] = fmaxf(mx[j], __shfl_xor(mx[j], off));
#pragma unroll
  for (int j = 0; j < 4 * QT; ++j) stage_row(L, j, v[j], mx[j]);
  if (lane < 32) L.zero[lane] = (_Float16)0.0f;
  __syncthreads();
}

template <int QT, bool SLOTS, bool RING>
__device__ bool split_prologue(const DecodeArgs &a, int s_idx, kvq_split &sp, Lds<QT> &L, int q_first = 0) {
  if (!split_check<QT, SLOTS, RING>(a, s_idx, sp, q_first)) return false;
  stage_q<QT>(a, sp, L, q_first);
  return true;
}

// The split block b runs.  With FP16 pages a plan's splits go to two launches, and each
// launch's blocks of the other kind return at once.  Block b goes to XCD b mod 8, so in
// plan order (a fixed class pattern per (table, head)) the splits a launch runs can
// fall unevenly on the XCDs; instead the blocks of XCD x take the x-th eighth of the
// plan, in order, which holds its even share of every class.
__device__ __forceinline__ int split_of_block(const DecodeArgs &a) {
  const int b = (int)blockIdx.x;
  if (a.n16 == 0) return b;
  const int q = a.n_splits >> 3, r = a.n_splits & 7, x = b & 7;
  return x * q + min(x, r) + (b >> 3);
}

// Register-staged kernel: slot-map mode (all classes), and FP16 splits in page mode.
template <int QT, bool SLOTS>
__global__ void __launch_bounds__(64) decode_kernel(DecodeArgs a) {
  __shared__ Lds<QT> L;
  const int s_idx = split_of_block(a);
  kvq_split sp;
  if (!split_prologue<QT, SLOTS, false>(a, s_idx, sp, L)) return;
  if (sp.cls == KVQ_INT4) run_split<QT, KVQ_INT4, SLOTS>(a, sp, s_idx, L);
  else if (sp.cls == KVQ_FP16) run_split<QT, KVQ_FP16, SLOTS>(a, sp, s_idx, L);
  else if (!SLOTS) run_split<QT, KVQ_INT2, false>(a, sp, s_idx, L);
}

// LDS-staged kernel: page-table mode, INT2 and INT4 splits; W waves per split with 4 QT
// query heads each; three waves per SIMD at QT = 1 (at most 168 registers a lane), two
// at QT = 2 (three, with the query operand read from LDS at each window to fit the
// registers, measured slower: 208 against 187 us on the agentic shape).
template <int W, int QT, bool SHARED>
__global__ void __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(QT == 1 ? 3 : 2)))
decode_ring_kernel(DecodeArgs a) {
  __shared__ Lds<QT> L[W];
  __shared__ __attribute__((aligned(16))) uint8_t ring[ring_bytes<W>()];
  __shared__ __attribute__((aligned(16))) int32_t idr[W][16];
  __shared__ int32_t win[SHARED ? 16 : 1];
  // Shared mode: block b runs worker b P mod n (P the prime 2^31 - 1, so a bijection
  // for any worker count below it).  Blocks are handed to the SIMDs in order and a SIMD
  // issues its oldest waves first, so in worker order the early requests' groups would
  // hold the oldest waves everywhere and end first; spread, every group's workers span
  // all ages.
  const int s_idx = SHARED ? (int)(((uint64_t)blockIdx.x * 2147483647ull) % (uint64_t)a.n_splits) : split_of_block(a);
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  kvq_split sp;
  if (SHARED) {
    static_assert(!SHARED || W == 1, "shared windows: one wave per worker");
    const int32_t grp = a.wgroup[s_idx];
    if (grp < 0 || grp >= a.n_groups) {  // a worker with no group: O = 0, lse = -inf
      if (lane_id() == 0) report(a.err, KVQ_DEVERR_SPLIT);
      for (int j = 0; j < min(4 * QT, a.g); ++j) {
        *reinterpret_cast<float2 *>(a.part_o + ((int64_t)s_idx * a.g + j) * kHeadDim + 2 * lane_id()) =
            make_float2(0.0f, 0.0f);
        if (lane_id() == 0) a.part_lse[(int64_t)s_idx * a.g + j] = -INFINITY;
      }
    } else if (split_check<QT, false, true>(a, s_idx, sp, 0)) {
      if (sp.cls == KVQ_INT4) run_shared_ring<KVQ_INT4, QT>(a, sp, s_idx, L[0], ring, idr[0], win, a.work + grp);
      else if (sp.cls == KVQ_INT2) run_shared_ring<KVQ_INT2, QT>(a, sp, s_idx, L[0], ring, idr[0], win, a.work + grp);
    }
    shared_exit(a, s_idx);
    return;
  }
#ifdef KVQ_WAVE_TIMELINE
  {
    KVQ_TIMELINE(s_idx, 0, __builtin_amdgcn_s_memrealtime());
    KVQ_TIMELINE(s_idx, 3, __builtin_amdgcn_s_memtime());
    uint32_t xcc, hwid;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_HW_ID)" : "=s"(hwid));
    KVQ_TIMELINE(s_idx, 5, xcc);
    KVQ_TIMELINE(s_idx, 6, hwid);
  }
#endif
  if (!split_check<QT, false, true>(a, s_idx, sp, 4 * QT * wave)) return;
  if (sp.cls == KVQ_INT4) run_split_ring<KVQ_INT4, W, QT>(a, sp, s_idx, L[wave], ring, idr[wave], wave);
  else if (sp.cls == KVQ_INT2) run_split_ring<KVQ_INT2, W, QT>(a, sp, s_idx, L[wave], ring, idr[wave], wave);
}

// LDS-staged kernel for the FP16 splits of a page-table launch (FP16 anchors, g <= 8):
// a 32 KB ring of two 16 KB windows per wave, one wave per SIMD; the FP16 window has
// no unpacking, so one wave's compute keeps ahead of its copies.
// FP8 anchors: 8.3 KB windows, two per wave, two waves per SIMD.
template <int QT, bool F8>
__global__ void __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(F8 ? 2 : 1)))
decode_anchor_ring_kernel(DecodeArgs a) {
  constexpr int RC = F8 ? kAnchorF8 : KVQ_FP16;
  __shared__ Lds<QT> L;
  __shared__ __attribute__((aligned(16))) uint8_t ring[RingGeom<RC, 1>::kRingBytes];
  __shared__ __attribute__((aligned(16))) int32_t idr[16];
  const int s_idx = split_of_block(a);
  kvq_split sp;
  // (a.only_fp16 is set: this kernel takes the FP16 splits, the other one the rest)
  if (!split_check<QT, false, false>(a, s_idx, sp, 0)) return;
  run_split_ring<RC, 1, QT>(a, sp, s_idx, L, ring, idr, 0);
}

// LDS-staged kernel for slot maps (INT4 splits, g <= 8).
template <int QT>
__global__ void __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(QT == 1 ? 3 : 2)))
decode_slots_ring_kernel(DecodeArgs a) {
  __shared__ Lds<QT> L;
  __shared__ __attribute__((aligned(16))) uint8_t ring[ring_bytes<1>()];
  __shared__ __attribute__((aligned(16))) int32_t id_blocks[SlotRingLoader::kIdBlocks * 32];
  const int s_idx = split_of_block(a);
  kvq_split sp;
  if (!split_check<QT, true, true>(a, s_idx, sp)) return;
  if (sp.cls == KVQ_INT4) run_split_slots_ring<QT>(a, sp, s_idx, L, ring, id_blocks);
}

// ------------------------------------------------------------------ merge -----

// One wavefront per (request, query head); lane = channel pair.  Splits come 32 at a
// time: their lse values (lane = split) and partial rows are loaded together before any
// is used, so a row costs about one memory latency per 32 splits after the offsets;
// the maximum and the weights exp(lse - max) are formed across the wave and broadcast
// with v_readlane.
__global__ void __launch_bounds__(64) lse_merge_kernel(const float *part_o, const float *part_lse,
                                                       int32_t n_splits, const int32_t *offsets, int32_t hq,
                                                       int32_t hkv, void *out, int32_t out_dtype,
                                                       float *out_lse) {
  const int lane = threadIdx.x;
  const int64_t row = blockIdx.x;
  const int b = (int)(row / hq), qh = (int)(row % hq);
  const int g = hq / hkv, kvh = qh / g, j = qh % g;
  const int32_t s0 = min(max(offsets[(int64_t)b * hkv + kvh], 0), n_splits);
  const int32_t s1 = min(max(offsets[(int64_t)b * hkv + kvh + 1], s0), n_splits);
  // Up to 32 splits at a time: their lse values (lane = split) and partial rows are
  // loaded together, then folded into a running (max, sum, row).
  float m = -INFINITY, tot = 0.0f, o0 = 0.0f, o1 = 0.0f;
  for (int32_t base = s0; base < s1; base += 32) {
    const int32_t n = min(s1 - base, 32);
    const float l = lane < n ? part_lse[(int64_t)(base + lane) * g + j] : -INFINITY;
    float2 po[32];
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      const int32_t kk = min(k, n - 1);  // past the end: a repeated row, weight 0
      po[k] = *reinterpret_cast<const float2 *>(part_o + ((int64_t)(base + kk) * g + j) * kHeadDim + 2 * lane);
    }
    float mc = l;
    for (int off = 32; off > 0; off >>= 1) mc = fmaxf(mc, __shfl_xor(mc, off));
    const float mn = fmaxf(m, mc);
    if (mn == -INFINITY) continue;  // every split so far is empty
    const float r = expf(m - mn);   // 0 while m is -inf
    const float w = expf(l - mn);   // lane k: split base + k (0 past the end)
    float ws = w;
    for (int off = 32; off > 0; off >>= 1) ws += __shfl_xor(ws, off);
    tot = fmaf(tot, r, ws);
    o0 *= r;
    o1 *= r;
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      const float wk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), k));
      o0 = fmaf(wk, po[k].x, o0);
      o1 = fmaf(wk, po[k].y, o1);
    }
    m = mn;
  }
  float lse = -INFINITY;
  if (m != -INFINITY) {
    o0 /= tot;
    o1 /= tot;
    lse = m + logf(tot);
  }
  const int64_t at = row * kHeadDim + 2 * lane;
  if (out_dtype == KVQ_F32) {
    *reinterpret_cast<float2 *>(static_cast<float *>(out) + at) = make_float2(o0, o1);
  } else if (out_dtype == KVQ_BF16) {
    auto bf = [](float f) {
      const uint32_t u = __float_as_uint(f);
      return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;  // round to nearest even
    };
    *reinterpret_cast<uint32_t *>(static_cast<uint16_t *>(out) + at) = bf(o0) | (bf(o1) << 16);
  } else {
    const uint32_t h0 = __half_as_ushort(__float2half_rn(o0)), h1 = __half_as_ushort(__float2half_rn(o1));
    *reinterpret_cast<uint32_t *>(static_cast<uint16_t *>(out) + at) = h0 | (h1 << 16);
  }
  if (out_lse && lane == 0) out_lse[row] = lse;
}

kvq_status launched(const char *what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(KVQ_ERR_HIP, "%s launch failed: %s", what, hipGetErrorString(e));
  return KVQ_OK;
}

}  // namespace
}  // namespace kvq

using namespace kvq;

namespace {

// Checks shared by both decode entry points; fills the argument block.
kvq_status decode_setup(DecodeArgs &a, const kvq_cache *c, const void *q, int32_t q_dtype, int32_t batch, int32_t hq,
                        int32_t hkv, const int32_t *tables, int32_t n_tables, int32_t max_entries, int32_t table_kind,
                        const kvq_split *splits, int32_t n_splits, float *part_o, float *part_lse, int32_t *dev_err) {
  kvq_status st = check_cache(c);
  if (st != KVQ_OK) return st;
  if (batch < 0 || hq <= 0 || hkv <= 0 || hq % hkv)
    return fail(KVQ_ERR_INVALID_ARG, "bad head counts hq=%d hkv=%d", hq, hkv);
  if (hkv % c->heads_per_page)
    return fail(KVQ_ERR_INVALID_ARG, "hkv %d is not a multiple of heads_per_page %d", hkv, c->heads_per_page);
  const int g = hq / hkv;
  if (g > kMaxG) return fail(KVQ_ERR_UNSUPPORTED, "g = %d query heads per KV head exceeds %d", g, kMaxG);
  if (q_dtype < KVQ_F32 || q_dtype > KVQ_F16) return fail(KVQ_ERR_INVALID_ARG, "bad q dtype %d", q_dtype);
  if (table_kind != KVQ_TABLE_PAGES && table_kind != KVQ_TABLE_SLOTS)
    return fail(KVQ_ERR_INVALID_ARG, "bad table kind %d", table_kind);
  const int tpr = hkv / c->heads_per_page;
  if ((int64_t)n_tables != (int64_t)batch * tpr)
    return fail(KVQ_ERR_INVALID_ARG, "n_tables %d != batch * hkv / heads_per_page = %lld", n_tables,
                (long long)batch * tpr);
  if (n_splits < 0 || max_entries < 0) return fail(KVQ_ERR_INVALID_ARG, "negative size");
  if (n_splits > 0 && (!q || !tables || !splits || !part_o || !part_lse))
    return fail(KVQ_ERR_INVALID_ARG, "NULL device array");
  a.heads = c->heads_per_page;
  a.n2 = c->n_pages[0];
  a.n4 = c->n_pages[1];
  a.n16 = c->n_pages[2];
  a.pool2 = (gbytes)c->pool[0];
  a.pool4 = (gbytes)c->pool[1];
  a.pool16 = (gbytes)c->pool[2];
  a.sentinel = c->sentinel_slot;
  a.fp8 = c->anchor_format == KVQ_ANCHOR_FP8 ? 1 : 0;
  a.q = q;
  a.q_dtype = q_dtype;
  a.q_lds = q_dtype != KVQ_F32 && ((uintptr_t)q & 15u) == 0 ? 1 : 0;
  a.batch = batch;
  a.hq = hq;
  a.hkv = hkv;
  a.g = g;
  a.tpr = tpr;
  a.tables = tables;
  a.n_tables = n_tables;
  a.max_entries = max_entries;
  a.splits = splits;
  a.n_splits = n_splits;
  a.part_o = part_o;
  a.part_lse = part_lse;
  a.err = dev_err;
  a.only_fp16 = 0;
  a.work = nullptr;
  a.wgroup = nullptr;
  a.n_groups = 0;
  return KVQ_OK;
}

// The kernel for the FP16 splits of a page-table launch (when the cache has FP16 pages;
// the INT2 / INT4 kernel leaves them): LDS-staged up to g = 8 (FP16 or FP8 anchors),
// register-staged at g = 16.
kvq_status launch_fp16_pages(DecodeArgs a, hipStream_t s) {
  if (a.n16 == 0) return KVQ_OK;
  a.only_fp16 = 1;
  const dim3 grid(a.n_splits), block(64);
  if (a.g <= 8) {
    if (a.fp8 && a.g <= 4) hipLaunchKernelGGL((decode_anchor_ring_kernel<1, true>), grid, block, 0, s, a);
    else if (a.fp8) hipLaunchKernelGGL((decode_anchor_ring_kernel<2, true>), grid, block, 0, s, a);
    else if (a.g <= 4) hipLaunchKernelGGL((decode_anchor_ring_kernel<1, false>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((decode_anchor_ring_kernel<2, false>), grid, block, 0, s, a);
    return launched("decode_anchor_ring_kernel");
  }
  if (a.g <= 4) hipLaunchKernelGGL((decode_kernel<1, false>), grid, block, 0, s, a);
  else if (a.g <= 8) hipLaunchKernelGGL((decode_kernel<2, false>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((decode_kernel<4, false>), grid, block, 0, s, a);
  return launched("decode_kernel");
}

}  // namespace

extern "C" kvq_status kvq_decode_attn(const kvq_cache *c, const void *q, int32_t q_dtype, int32_t batch,
                                      int32_t hq, int32_t hkv, const int32_t *tables, int32_t n_tables,
                                      int32_t max_entries, int32_t table_kind, const kvq_split *splits,
                                      int32_t n_splits, float *part_o, float *part_lse, int32_t *dev_err,
                                      void *stream) {
  DecodeArgs a;
  kvq_status st = decode_setup(a, c, q, q_dtype, batch, hq, hkv, tables, n_tables, max_entries, table_kind, splits,
                               n_splits, part_o, part_lse, dev_err);
  if (st != KVQ_OK || n_splits == 0) return st;
  const int g = a.g;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid(n_splits), block(64);
  if (table_kind == KVQ_TABLE_SLOTS) {
    if (g > 8) {  // register-staged kernel for every split
      hipLaunchKernelGGL((decode_kernel<4, true>), grid, block, 0, s, a);
      return launched("decode_kernel");
    }
    // INT4 splits (and every malformed one) in the LDS-staged kernel, FP16 splits in
    // the register-staged one when the cache has FP16 pages.
    if (g <= 4) hipLaunchKernelGGL((decode_slots_ring_kernel<1>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((decode_slots_ring_kernel<2>), grid, block, 0, s, a);
    st = launched("decode_slots_ring_kernel");
    if (st != KVQ_OK || a.n16 == 0) return st;
    a.only_fp16 = 1;
    if (g <= 4) hipLaunchKernelGGL((decode_kernel<1, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((decode_kernel<2, true>), grid, block, 0, s, a);
    return launched("decode_kernel");
  }
  // Page mode: INT2 / INT4 splits (and every malformed one) in the LDS-staged kernel,
  // FP16 splits in the register-staged one when the cache has FP16 pages.
  if (g <= 4) hipLaunchKernelGGL((decode_ring_kernel<1, 1, false>), grid, dim3(64), 0, s, a);
  else if (g <= 8) hipLaunchKernelGGL((decode_ring_kernel<1, 2, false>), grid, dim3(64), 0, s, a);
  else hipLaunchKernelGGL((decode_ring_kernel<2, 2, false>), grid, dim3(128), 0, s, a);
  st = launched("decode_ring_kernel");
  if (st != KVQ_OK) return st;
  return launch_fp16_pages(a, s);
}

extern "C" kvq_status kvq_decode_attn_shared(const kvq_cache *c, const void *q, int32_t q_dtype, int32_t batch,
                                             int32_t hq, int32_t hkv, const int32_t *tables, int32_t n_tables,
                                             int32_t max_entries, int32_t table_kind, const kvq_split *workers,
                                             const int32_t *worker_group, int32_t n_workers, int32_t n_groups,
                                             int32_t *work, float *part_o, float *part_lse, int32_t *dev_err,
                                             void *stream) {
  DecodeArgs a;
  kvq_status st = decode_setup(a, c, q, q_dtype, batch, hq, hkv, tables, n_tables, max_entries, table_kind, workers,
                               n_workers, part_o, part_lse, dev_err);
  if (st != KVQ_OK) return st;
  if (table_kind != KVQ_TABLE_PAGES) return fail(KVQ_ERR_UNSUPPORTED, "shared windows need page tables");
  if (a.g > 8) return fail(KVQ_ERR_UNSUPPORTED, "shared windows: g = %d > 8", a.g);
  if (n_workers == 0) return KVQ_OK;
  if (n_groups < 1 || !work || !worker_group) return fail(KVQ_ERR_INVALID_ARG, "shared windows need groups and counters");
  a.work = work;
  a.wgroup = worker_group;
  a.n_groups = n_groups;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid(n_workers), block(64);
  if (a.g <= 4) hipLaunchKernelGGL((decode_ring_kernel<1, 1, true>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((decode_ring_kernel<1, 2, true>), grid, block, 0, s, a);
  st = launched("decode_ring_kernel");
  if (st != KVQ_OK) return st;
  return launch_fp16_pages(a, s);
}

namespace kvq {
namespace {

// ------------------------------------------------------------- no allocation -----
//
// The shared-window decode with its counters in a file-scope device array instead of a
// caller's workspace, for callers that cannot allocate (code under graph capture, tight
// serving loops).  Each GPU holds its own copy of the array, at its own address, until
// the process ends; the address is looked up once per device with that device current.
// Every call on a GPU uses that GPU's array, so calls that overlap on one GPU race.

constexpr int kNoAllocGroups = 16384;  // groups one call may have
constexpr int kMaxDevices = 64;
__device__ __align__(256) int32_t scratch[kNoAllocGroups + kDoneSubs + 1];

// Clears n counters (a fill kernel rather than a memset: safe under graph capture).
__global__ void __launch_bounds__(256) clear_kernel(int32_t *p, int32_t n) {
  for (int32_t i = (int32_t)(blockIdx.x * 256 + threadIdx.x); i < n; i += (int32_t)(gridDim.x * 256)) p[i] = 0;
}

int32_t *scratch_address(kvq_status &st) {
  static std::mutex mu;
  static int32_t *addr[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    st = fail(KVQ_ERR_NO_DEVICE, "hipGetDevice failed");
    return nullptr;
  }
  if (dev >= kMaxDevices) {
    st = fail(KVQ_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void *ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      st = fail(KVQ_ERR_HIP, "hipGetSymbolAddress(scratch) failed: %s", hipGetErrorString(e));
      return nullptr;
    }
    addr[dev] = static_cast<int32_t *>(ptr);
  }
  return addr[dev];
}

}  // namespace
}  // namespace kvq

extern "C" kvq_status kvq_decode_attn_shared_noalloc(const kvq_cache *c, const void *q, int32_t q_dtype,
                                                     int32_t batch, int32_t hq, int32_t hkv, const int32_t *tables,
                                                     int32_t n_tables, int32_t max_entries, int32_t table_kind,
                                                     const kvq_split *workers, const int32_t *worker_group,
                                                     int32_t n_workers, int32_t n_groups, float *part_o,
                                                     float *part_lse, int32_t *dev_err, void *stream) {
  using namespace kvq;
  if (n_groups > kNoAllocGroups)
    return fail(KVQ_ERR_CAPACITY, "%d groups: this entry point holds counters for at most %d", n_groups,
                kNoAllocGroups);
  if (n_workers > 0 && n_groups < 1) return fail(KVQ_ERR_INVALID_ARG, "shared windows need groups");
  kvq_status st = KVQ_OK;
  int32_t *work = n_workers > 0 ? scratch_address(st) : nullptr;
  if (st != KVQ_OK) return st;
  if (work) {
    const int32_t n = n_groups + kDoneSubs + 1;
    hipLaunchKernelGGL(clear_kernel, dim3((n + 255) / 256), dim3(256), 0, static_cast<hipStream_t>(stream), work, n);
    if ((st = launched("clear_kernel")) != KVQ_OK) return st;
  }
  return kvq_decode_attn_shared(c, q, q_dtype, batch, hq, hkv, tables, n_tables, max_entries, table_kind, workers,
                                worker_group, n_workers, n_groups, work, part_o, part_lse, dev_err, stream);
}

extern "C" kvq_status kvq_lse_merge(const float *part_o, const float *part_lse, int32_t n_splits,
                                    const int32_t *split_offsets,
                                    int32_t batch, int32_t hq, int32_t hkv, void *out, int32_t out_dtype,
                                    float *out_lse, void *stream) {
  if (batch < 0 || hq <= 0 || hkv <= 0 || hq % hkv)
    return fail(KVQ_ERR_INVALID_ARG, "bad head counts hq=%d hkv=%d", hq, hkv);
  if (out_dtype < KVQ_F32 || out_dtype > KVQ_F16) return fail(KVQ_ERR_INVALID_ARG, "bad out dtype %d", out_dtype);
  if (n_splits < 0) return fail(KVQ_ERR_INVALID_ARG, "negative n_splits");
  if (batch == 0) return KVQ_OK;
  if (!split_offsets || !out || (n_splits > 0 && (!part_o || !part_lse)))
    return fail(KVQ_ERR_INVALID_ARG, "NULL device array");
  if ((int64_t)batch * hq > INT32_MAX) return fail(KVQ_ERR_UNSUPPORTED, "too many rows");
  hipLaunchKernelGGL(lse_merge_kernel, dim3(batch * hq), dim3(64), 0, static_cast<hipStream_t>(stream), part_o,
                     part_lse, n_splits, split_offsets, hq, hkv, out, out_dtype, out_lse);
  return launched("lse_merge_kernel");
}

extern "C" kvq_status kvq_wave_timeline(void *buffer) {
#ifdef KVQ_WAVE_TIMELINE
  uint64_t *p = static_cast<uint64_t *>(buffer);
  const hipError_t e = hipMemcpyToSymbol(HIP_SYMBOL(g_timeline), &p, sizeof p);
  if (e != hipSuccess) return fail(KVQ_ERR_HIP, "timeline buffer: %s", hipGetErrorString(e));
  return KVQ_OK;
#else
  (void)buffer;
  return fail(KVQ_ERR_UNSUPPORTED, "this build records no wave timeline (build with KVQ_WAVE_TIMELINE)");
#endif
}

extern "C" kvq_status kvq_decode_occupancy(int32_t g, int32_t table_kind, int32_t *per_cu, int32_t *n_cu) {
  if (!per_cu || !n_cu || g < 1 || g > kMaxG || (table_kind != KVQ_TABLE_PAGES && table_kind != KVQ_TABLE_SLOTS))
    return fail(KVQ_ERR_INVALID_ARG, "bad occupancy query");
  int dev = 0, count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess || count == 0) return fail(KVQ_ERR_NO_DEVICE, "no HIP device");
  if (hipGetDevice(&dev) != hipSuccess) return fail(KVQ_ERR_NO_DEVICE, "hipGetDevice failed");
  int blocks = 0, cus = 0;
  hipError_t e;
  const bool slots = table_kind == KVQ_TABLE_SLOTS;
  if (g <= 4)
    e = slots ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, decode_slots_ring_kernel<1>, 64, 0)
              : hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, decode_ring_kernel<1, 1, false>, 64, 0);
  else if (g <= 8)
    e = slots ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, decode_slots_ring_kernel<2>, 64, 0)
              : hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, decode_ring_kernel<1, 2, false>, 64, 0);
  else
    e = slots ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, decode_kernel<4, true>, 64, 0)
              : hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, decode_ring_kernel<2, 2, false>, 128, 0);
  if (e != hipSuccess) return fail(KVQ_ERR_HIP, "occupancy query failed: %s", hipGetErrorString(e));
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return fail(KVQ_ERR_HIP, "CU count query failed");
  *per_cu = blocks;
  *n_cu = cus;
  return KVQ_OK;
}

extern "C" kvq_status kvq_decode_fp16_occupancy(int32_t g, int32_t anchor_format, int32_t *per_cu, int32_t *n_cu) {
  if (!per_cu || !n_cu || g < 1 || g > kMaxG || (anchor_format != KVQ_ANCHOR_FP16 && anchor_format != KVQ_ANCHOR_FP8))
    return fail(KVQ_ERR_INVALID_ARG, "bad occupancy query");
  int dev = 0, count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess || count == 0) return fail(KVQ_ERR_NO_DEVICE, "no HIP device");
  if (hipGetDevice(&dev) != hipSuccess) return fail(KVQ_ERR_NO_DEVICE, "hipGetDevice failed");
  int blocks = 0, cus = 0;
  hipError_t e;
  const bool f8 = anchor_format == KVQ_ANCHOR_FP8;
  if (g <= 4)
    e = f8 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, decode_anchor_ring_kernel<1, true>, 64, 0)
           : hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, decode_anchor_ring_kernel<1, false>, 64, 0);
  else if (g <= 8)
    e = f8 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, decode_anchor_ring_kernel<2, true>, 64, 0)
           : hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, decode_anchor_ring_kernel<2, false>, 64, 0);
  else
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, decode_kernel<4, false>, 64, 0);
  if (e != hipSuccess) return fail(KVQ_ERR_HIP, "occupancy query failed: %s", hipGetErrorString(e));
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return fail(KVQ_ERR_HIP, "CU count query failed");
  *per_cu = blocks;
  *n_cu = cus;
  return KVQ_OK;
}
