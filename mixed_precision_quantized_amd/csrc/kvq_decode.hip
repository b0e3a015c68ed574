// Decode path of libkvq for gfx950: split-K decode attention read directly from
// the INT2 / INT4 / FP16 pools (dequantization inside the attention loop), and
// the log-sum-exp merge of the split partials.
//
// TriAxialKV key design 4 (phase 2): every split covers tokens of one precision,
// so the loop over a split has no precision branch; splits are merged by a
// global log-sum-exp reduction.  HyQuant background / Algorithm 3: online
// softmax state (m, l, acc) with O = acc / l; the g query heads that share a KV
// head are processed together (GQA packing); the FP16 anchor segments are more
// splits of the same launch.  IntentKV layout-preserving eviction: a slot-map
// entry equal to the sentinel slot contributes nothing.
//
// Reference kernel (one 64-lane wavefront per split):
//   - tokens are taken 64 at a time, lane = token: each lane dequantizes its own
//     K row and forms the g logits in fp32 (q pre-scaled by log2(e)/sqrt(128) so
//     the softmax runs on exp2);
//   - chunk maximum and sum by wavefront butterflies; the running (m, l, acc)
//     is rescaled only when the maximum moves;
//   - P V with lane = channel pair: each lane dequantizes its two channels of
//     every V row of the chunk and accumulates g outputs.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ void report(int32_t *err, int32_t bit) {
  if (err) atomicOr(err, bit);
}

__device__ __forceinline__ float h2f(uint32_t bits) {
  return __half2float(__ushort_as_half((unsigned short)(bits & 0xffffu)));
}

__device__ __forceinline__ float load_q(const void *q, int32_t dtype, int64_t idx) {
  if (dtype == KVQ_F32) return static_cast<const float *>(q)[idx];
  const uint32_t h = static_cast<const uint16_t *>(q)[idx];
  return dtype == KVQ_BF16 ? __uint_as_float(h << 16) : h2f(h);
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m);
  return x;
}

struct DecodeArgs {
  int32_t heads, n2, n4, n16;
  const uint8_t *pool2, *pool4, *pool16;
  int32_t sentinel;
  const void *q;
  int32_t q_dtype, batch, hq, hkv, g, tpr;
  const int32_t *tables;
  int32_t n_tables, max_entries, kind;
  const kvq_split *splits;
  int32_t n_splits;
  float *part_o, *part_lse;
  int32_t *err;
};

__device__ __forceinline__ int page_class(const DecodeArgs &a, int64_t p) {
  if (p < 0) return -1;
  if (p < a.n2) return KVQ_INT2;
  if (p < (int64_t)a.n2 + a.n4) return KVQ_INT4;
  if (p < (int64_t)a.n2 + a.n4 + a.n16) return KVQ_FP16;
  return -1;
}

__device__ __forceinline__ const uint8_t *block_of(const DecodeArgs &a, int cls, int64_t page, int head) {
  if (cls == KVQ_INT2) return a.pool2 + (page * a.heads + head) * (int64_t)kI2Bytes;
  if (cls == KVQ_INT4) return a.pool4 + ((page - a.n2) * a.heads + head) * (int64_t)kI4Bytes;
  return a.pool16 + ((page - a.n2 - a.n4) * a.heads + head) * (int64_t)kF16Bytes;
}

// Bit of the code of channel index k (0 .. 32/b - 1) inside its 32-bit word.
template <int BITS>
__device__ __forceinline__ int word_bit(int k) {
  return (k & 1) * 16 + (k >> 1) * BITS;
}

// Logits of the GP (padded) query rows against one dequantized K row.
template <int GP, int CLS>
__device__ __forceinline__ void k_logits(const DecodeArgs &a, const uint8_t *blk, int off, int64_t page,
                                         int head, const float (*qs)[kHeadDim], float *x) {
#pragma unroll
  for (int j = 0; j < GP; ++j) x[j] = 0.0f;
  if (CLS == KVQ_INT4) {
    const uint4 *row = reinterpret_cast<const uint4 *>(blk + kI4KC + off * 64);
    const uint4 meta = *reinterpret_cast<const uint4 *>(blk + kI4KM + off * 16);
    const uint32_t metas[4] = {meta.x, meta.y, meta.z, meta.w};
#pragma unroll
    for (int grp = 0; grp < 4; ++grp) {
      const float s = h2f(metas[grp]), z = h2f(metas[grp] >> 16);
      const uint4 w = row[grp];
      const uint32_t words[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int wi = 0; wi < 4; ++wi)
#pragma unroll
        for (int n = 0; n < 8; ++n) {
          const int ch = grp * 32 + wi * 8 + n;
          const float kv = fmaf((float)((words[wi] >> word_bit<4>(n)) & 15u), s, z);
#pragma unroll
          for (int j = 0; j < GP; ++j) x[j] = fmaf(qs[j][ch], kv, x[j]);
        }
    }
  } else if (CLS == KVQ_INT2) {
    const uint4 *row = reinterpret_cast<const uint4 *>(blk + kI2KC + off * 32);
    const int64_t even = page & ~1ll;
    const uint8_t *m_even = block_of(a, KVQ_INT2, even, head);
    const uint8_t *m_odd = block_of(a, KVQ_INT2, even + 1, head);
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const uint4 w = row[half];
      const uint32_t words[4] = {w.x, w.y, w.z, w.w};
      const uint8_t *mb = half ? m_odd : m_even;  // channels 64*half .. 64*half+63
#pragma unroll
      for (int wi = 0; wi < 4; ++wi)
#pragma unroll
        for (int n = 0; n < 16; ++n) {
          const int ch = half * 64 + wi * 16 + n;
          const float s = h2f(*reinterpret_cast<const uint16_t *>(mb + kI2KS + (ch & 63) * 2));
          const float z = h2f(*reinterpret_cast<const uint16_t *>(mb + kI2KZ + (ch & 63) * 2));
          const float kv = fmaf((float)((words[wi] >> word_bit<2>(n)) & 3u), s, z);
#pragma unroll
          for (int j = 0; j < GP; ++j) x[j] = fmaf(qs[j][ch], kv, x[j]);
        }
    }
  } else {
    const uint4 *row = reinterpret_cast<const uint4 *>(blk + kF16K + off * 256);
#pragma unroll 4
    for (int wi = 0; wi < 16; ++wi) {
      const uint4 w = row[wi];
      const uint32_t words[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int n = 0; n < 8; ++n) {
        const int ch = wi * 8 + n;
        const float kv = h2f(words[n >> 1] >> (16 * (n & 1)));
#pragma unroll
        for (int j = 0; j < GP; ++j) x[j] = fmaf(qs[j][ch], kv, x[j]);
      }
    }
  }
}

// This lane's two V channels (2l, 2l+1) of one token: the even and odd members of
// pair (l % (16/b)) of word l / (16/b).
template <int CLS>
__device__ __forceinline__ void v_pair(const uint8_t *blk, int off, int lane, float &v0, float &v1) {
  if (CLS == KVQ_INT4) {
    const uint32_t w = *reinterpret_cast<const uint32_t *>(blk + kI4VC + off * 64 + (lane >> 2) * 4);
    const uint32_t meta = *reinterpret_cast<const uint32_t *>(blk + kI4VM + ((lane >> 4) * kPage + off) * 4);
    const float s = h2f(meta), z = h2f(meta >> 16);
    const int sh = (lane & 3) * 4;
    v0 = fmaf((float)((w >> sh) & 15u), s, z);
    v1 = fmaf((float)((w >> (16 + sh)) & 15u), s, z);
  } else if (CLS == KVQ_INT2) {
    const uint32_t w = *reinterpret_cast<const uint32_t *>(blk + kI2VC + off * 32 + (lane >> 3) * 4);
    const uint32_t meta = *reinterpret_cast<const uint32_t *>(blk + kI2VM + ((lane >> 4) * kPage + off) * 4);
    const float s = h2f(meta), z = h2f(meta >> 16);
    const int sh = (lane & 7) * 2;
    v0 = fmaf((float)((w >> sh) & 3u), s, z);
    v1 = fmaf((float)((w >> (16 + sh)) & 3u), s, z);
  } else {
    const uint32_t w = *reinterpret_cast<const uint32_t *>(blk + kF16V + off * 256 + lane * 4);
    v0 = h2f(w);
    v1 = h2f(w >> 16);
  }
}

template <int GP, int CLS>
__device__ void decode_split(const DecodeArgs &a, const kvq_split &sp, int s_idx, float (*qs)[kHeadDim],
                             float (*ps)[64], const uint8_t **tok_blk, int *tok_off) {
  const int lane = threadIdx.x;
  const int32_t *trow = a.tables + (int64_t)sp.table * a.max_entries;
  float m[GP], l[GP], acc0[GP], acc1[GP];
#pragma unroll
  for (int j = 0; j < GP; ++j) {
    m[j] = -INFINITY;
    l[j] = 0.0f;
    acc0[j] = acc1[j] = 0.0f;
  }
  for (int32_t base = sp.tok_begin; base < sp.tok_end; base += 64) {
    const int32_t t = base + lane;
    bool live = t < sp.tok_end;
    int64_t page = 0;
    int off = 0;
    if (live) {
      if (a.kind == KVQ_TABLE_PAGES) {
        page = trow[t >> 4];
        off = t & 15;
      } else {
        const int32_t slot = trow[t];
        live = !(a.sentinel >= 0 && slot == a.sentinel);
        page = slot >> 4;
        off = slot & 15;
        if (slot < 0) live = false;
      }
      if (live && page_class(a, page) != CLS) {
        report(a.err, KVQ_DEVERR_ID);
        live = false;
      }
    }
    const uint8_t *blk = live ? block_of(a, CLS, page, sp.head) : nullptr;
    float x[GP];
    if (live) {
      k_logits<GP, CLS>(a, blk, off, page, sp.head, qs, x);
    } else {
#pragma unroll
      for (int j = 0; j < GP; ++j) x[j] = -INFINITY;
    }
    tok_blk[lane] = blk;
    tok_off[lane] = off;
#pragma unroll
    for (int j = 0; j < GP; ++j) {
      const float mc = wave_max(x[j]);
      const float mn = fmaxf(m[j], mc);
      float p = 0.0f, alpha = 1.0f;
      if (mn != -INFINITY) {
        alpha = exp2f(m[j] - mn);  // 0 while nothing was live before
        p = live ? exp2f(x[j] - mn) : 0.0f;
      }
      ps[j][lane] = p;
      l[j] = l[j] * alpha + wave_sum(p);
      acc0[j] *= alpha;
      acc1[j] *= alpha;
      m[j] = mn;
    }
    __syncthreads();
    const int n_here = min(64, sp.tok_end - base);
    for (int tt = 0; tt < n_here; ++tt) {
      const uint8_t *b = tok_blk[tt];
      if (!b) continue;  // dead or invalid token: weight 0
      float v0, v1;
      v_pair<CLS>(b, tok_off[tt], lane, v0, v1);
#pragma unroll
      for (int j = 0; j < GP; ++j) {
        acc0[j] = fmaf(ps[j][tt], v0, acc0[j]);
        acc1[j] = fmaf(ps[j][tt], v1, acc1[j]);
      }
    }
    __syncthreads();
  }
  for (int j = 0; j < a.g; ++j) {
    const bool any = l[j] > 0.0f;
    const float inv = any ? 1.0f / l[j] : 0.0f;
    float *o = a.part_o + ((int64_t)s_idx * a.g + j) * kHeadDim;
    *reinterpret_cast<float2 *>(o + 2 * lane) = make_float2(acc0[j] * inv, acc1[j] * inv);
    if (lane == 0) a.part_lse[(int64_t)s_idx * a.g + j] = any ? (m[j] + log2f(l[j])) * kLn2 : -INFINITY;
  }
}

template <int GP>
__global__ void __launch_bounds__(64) decode_ref_kernel(DecodeArgs a) {
  __shared__ float qs[GP][kHeadDim];
  __shared__ float ps[GP][64];
  __shared__ const uint8_t *tok_blk[64];
  __shared__ int tok_off[64];
  const int lane = threadIdx.x;
  const int s_idx = blockIdx.x;
  const kvq_split sp = a.splits[s_idx];
  const int64_t cap = a.kind == KVQ_TABLE_PAGES ? (int64_t)a.max_entries * kPage : a.max_entries;
  const bool ok = sp.table >= 0 && sp.table < a.n_tables && sp.head >= 0 && sp.head < a.heads &&
                  sp.cls >= 0 && sp.cls <= 2 && sp.tok_begin >= 0 && sp.tok_end >= sp.tok_begin &&
                  sp.tok_end <= cap &&
                  (sp.cls != KVQ_INT2 ||
                   (a.kind == KVQ_TABLE_PAGES && sp.tok_begin % kGroup == 0 && sp.tok_end % kGroup == 0));
  if (!ok) {
    if (lane == 0) report(a.err, KVQ_DEVERR_SPLIT);
    for (int j = 0; j < a.g; ++j) {
      float *o = a.part_o + ((int64_t)s_idx * a.g + j) * kHeadDim;
      *reinterpret_cast<float2 *>(o + 2 * lane) = make_float2(0.0f, 0.0f);
      if (lane == 0) a.part_lse[(int64_t)s_idx * a.g + j] = -INFINITY;
    }
    return;
  }
  const int b = sp.table / a.tpr;
  const int kvh = (sp.table % a.tpr) * a.heads + sp.head;
  const float scale = kLog2e / sqrtf((float)kHeadDim);
#pragma unroll
  for (int j = 0; j < GP; ++j)
    for (int c = lane; c < kHeadDim; c += 64)
      qs[j][c] = j < a.g ? load_q(a.q, a.q_dtype, ((int64_t)b * a.hq + kvh * a.g + j) * kHeadDim + c) * scale
                         : 0.0f;
  __syncthreads();
  if (sp.cls == KVQ_INT2) decode_split<GP, KVQ_INT2>(a, sp, s_idx, qs, ps, tok_blk, tok_off);
  else if (sp.cls == KVQ_INT4) decode_split<GP, KVQ_INT4>(a, sp, s_idx, qs, ps, tok_blk, tok_off);
  else decode_split<GP, KVQ_FP16>(a, sp, s_idx, qs, ps, tok_blk, tok_off);
}

// ------------------------------------------------------------------ merge -----

// One wavefront per (request, query head); lane = channel pair.
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
  float mx = -INFINITY;
  for (int32_t s = s0; s < s1; ++s) mx = fmaxf(mx, part_lse[(int64_t)s * g + j]);
  float o0 = 0.0f, o1 = 0.0f, lse = -INFINITY;
  if (mx != -INFINITY) {
    float tot = 0.0f;
    for (int32_t s = s0; s < s1; ++s) {
      const float w = expf(part_lse[(int64_t)s * g + j] - mx);
      const float2 po = *reinterpret_cast<const float2 *>(part_o + ((int64_t)s * g + j) * kHeadDim + 2 * lane);
      tot += w;
      o0 = fmaf(w, po.x, o0);
      o1 = fmaf(w, po.y, o1);
    }
    o0 /= tot;
    o1 /= tot;
    lse = mx + logf(tot);
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

extern "C" kvq_status kvq_decode_attn(const kvq_cache *c, const void *q, int32_t q_dtype, int32_t batch,
                                      int32_t hq, int32_t hkv, const int32_t *tables, int32_t n_tables,
                                      int32_t max_entries, int32_t table_kind, const kvq_split *splits,
                                      int32_t n_splits, float *part_o, float *part_lse, int32_t *dev_err,
                                      void *stream) {
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
  if (n_splits == 0) return KVQ_OK;
  if (!q || !tables || !splits || !part_o || !part_lse)
    return fail(KVQ_ERR_INVALID_ARG, "NULL device array");
  DecodeArgs a;
  a.heads = c->heads_per_page;
  a.n2 = c->n_pages[0];
  a.n4 = c->n_pages[1];
  a.n16 = c->n_pages[2];
  a.pool2 = static_cast<const uint8_t *>(c->pool[0]);
  a.pool4 = static_cast<const uint8_t *>(c->pool[1]);
  a.pool16 = static_cast<const uint8_t *>(c->pool[2]);
  a.sentinel = c->sentinel_slot;
  a.q = q;
  a.q_dtype = q_dtype;
  a.batch = batch;
  a.hq = hq;
  a.hkv = hkv;
  a.g = g;
  a.tpr = tpr;
  a.tables = tables;
  a.n_tables = n_tables;
  a.max_entries = max_entries;
  a.kind = table_kind;
  a.splits = splits;
  a.n_splits = n_splits;
  a.part_o = part_o;
  a.part_lse = part_lse;
  a.err = dev_err;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (g <= 4) hipLaunchKernelGGL(decode_ref_kernel<4>, dim3(n_splits), dim3(64), 0, s, a);
  else if (g <= 8) hipLaunchKernelGGL(decode_ref_kernel<8>, dim3(n_splits), dim3(64), 0, s, a);
  else hipLaunchKernelGGL(decode_ref_kernel<16>, dim3(n_splits), dim3(64), 0, s, a);
  return launched("decode_ref_kernel");
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

extern "C" kvq_status kvq_decode_occupancy(int32_t g, int32_t *per_cu, int32_t *n_cu) {
  if (!per_cu || !n_cu || g < 1 || g > kMaxG) return fail(KVQ_ERR_INVALID_ARG, "bad occupancy query");
  int dev = 0, count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess || count == 0) return fail(KVQ_ERR_NO_DEVICE, "no HIP device");
  if (hipGetDevice(&dev) != hipSuccess) return fail(KVQ_ERR_NO_DEVICE, "hipGetDevice failed");
  int blocks = 0, cus = 0;
  hipError_t e;
  if (g <= 4) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, decode_ref_kernel<4>, 64, 0);
  else if (g <= 8) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, decode_ref_kernel<8>, 64, 0);
  else e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, decode_ref_kernel<16>, 64, 0);
  if (e != hipSuccess) return fail(KVQ_ERR_HIP, "occupancy query failed: %s", hipGetErrorString(e));
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return fail(KVQ_ERR_HIP, "CU count query failed");
  *per_cu = blocks;
  *n_cu = cus;
  return KVQ_OK;
}
