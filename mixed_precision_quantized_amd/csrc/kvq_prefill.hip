// Prefill attention with an INT8 prefix (HyQuant Algorithm 2).
//
// For query position t of a request, query head j and its KV head h = j / g, the keys
// k <= t are read in full precision when k is a vertical line of h or lies in the window
// k > t - W, and through INT8 otherwise; all of them share one online softmax.  INT8
// tiles are 64 positions with the symmetric scale max|x| / 127 (queries per query head,
// keys per KV head with the vertical lines left out of the maximum).  V is not
// quantized: it enters P.V as fp16 (exact for bf16 values in fp16's normal range), with
// fp16 weights (bf16 weights would lose too much for the 2e-3 bar).
//
// Three launches: the INT8 codes and scales (one work group per 64-position tile and
// head); V transposed to fp16 [b][h][channel][position] so the P.V operand reads whole
// channels; the attention: one wave per (request, query head, 16 query positions), 32
// keys a step, S^T = K Q^T on MFMA (i32 16x16x64 for the INT8 pairs, f32 16x16x32 bf16
// for the full-precision pairs, each only when the step has such a pair), so a lane holds
// its query's scores in the layout the P operand of O^T = V^T P^T wants.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "kvq.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kTile = 64;       // INT8 tile (positions)
constexpr int kQBlock = 16;     // query positions per wave
constexpr int kKStep = 32;      // keys per step

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 bf8 __attribute__((ext_vector_type(8)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ void report(int32_t *err, int32_t bit) {
  if (err) atomicOr(err, bit);
}

__device__ __forceinline__ float bf16_value(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

struct PfArgs {
  const uint16_t *q, *k, *v;     // bf16 [batch][n_max][heads][128]
  const uint8_t *cls;            // [batch][hkv][n_max] (1 = vertical line) or null
  const int32_t *n_tokens;
  int32_t batch, n_max, hq, hkv, window, tiles;
  int8_t *q_codes, *k_codes;     // like q, k
  float *q_scales, *k_scales;    // [batch][hq][tiles], [batch][hkv][tiles]
  uint16_t *vt;                  // fp16 [batch][hkv][128][n_max]
  float *out;                    // [batch][n_max][hq][128]
  int32_t *err;
};

__device__ __forceinline__ int32_t checked_n(const PfArgs &a, int b) {
  const int32_t n = a.n_tokens[b];
  return (n < 0 || n > a.n_max) ? -1 : n;
}

// Codes and scale of one 64-position tile of one head (blockIdx.z < hq: query head z,
// else KV head z - hq).  Thread: row tid / 4, channels 32 (tid % 4) .. + 31.
__global__ void __launch_bounds__(256) pf_quant_kernel(PfArgs a) {
  __shared__ float wmax[4];
  const int tid = threadIdx.x, tile = blockIdx.x, b = blockIdx.y, z = blockIdx.z;
  const bool is_q = z < a.hq;
  const int heads = is_q ? a.hq : a.hkv, head = is_q ? z : z - a.hq;
  int32_t n = checked_n(a, b);
  if (n < 0) {
    if (tid == 0) report(a.err, KVQ_DEVERR_RANGE);
    n = 0;
  }
  const int row = tile * kTile + tid / 4, c0 = 32 * (tid % 4);
  const uint16_t *src = (is_q ? a.q : a.k) + (((int64_t)b * a.n_max + row) * heads + head) * kHeadDim + c0;
  const bool live = row < n;
  const bool counts = live && (is_q || !a.cls || a.cls[((int64_t)b * a.hkv + head) * a.n_max + row] != 1);
  float x[32];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 w = reinterpret_cast<const uint4 *>(src)[i];
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[8 * i + 2 * e] = bf16_value((uint16_t)(ww[e] & 0xFFFFu));
      x[8 * i + 2 * e + 1] = bf16_value((uint16_t)(ww[e] >> 16));
    }
  }
  float m = 0.0f;
  if (counts)
#pragma unroll
    for (int i = 0; i < 32; ++i) m = fmaxf(m, fabsf(x[i]));
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if ((tid & 63) == 0) wmax[tid >> 6] = m;
  __syncthreads();
  const float amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  const float s = __fdiv_rn(amax, 127.0f);
  if (tid == 0) (is_q ? a.q_scales : a.k_scales)[((int64_t)b * heads + head) * a.tiles + tile] = s;
  uint32_t packed[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t w = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float c = 0.0f;
      if (live && s != 0.0f) c = fminf(fmaxf(rintf(__fdiv_rn(x[4 * i + e], s)), -127.0f), 127.0f);
      w |= ((uint32_t)(uint8_t)(int8_t)c) << (8 * e);
    }
    packed[i] = w;
  }
  int8_t *dst = (is_q ? a.q_codes : a.k_codes) + (((int64_t)b * a.n_max + row) * heads + head) * kHeadDim + c0;
  reinterpret_cast<uint4 *>(dst)[0] = make_uint4(packed[0], packed[1], packed[2], packed[3]);
  reinterpret_cast<uint4 *>(dst)[1] = make_uint4(packed[4], packed[5], packed[6], packed[7]);
}

// V [b][t][h][c] (bf16) -> vt [b][h][c][t] (fp16, exact in fp16's normal range) through
// LDS, 64 positions x 128 channels a group; positions at or past the request's length
// are written as 0.
__global__ void __launch_bounds__(256) pf_vt_kernel(PfArgs a) {
  __shared__ uint16_t tileb[kTile][kHeadDim + 2];
  const int tid = threadIdx.x, tile = blockIdx.x, b = blockIdx.y, h = blockIdx.z;
  int32_t n = checked_n(a, b);
  if (n < 0) n = 0;
  for (int i = tid; i < kTile * kHeadDim / 2; i += 256) {  // 2 channels per step
    const int r = i / (kHeadDim / 2), c = 2 * (i % (kHeadDim / 2));
    const int t = tile * kTile + r;
    uint32_t w = 0;
    if (t < n) w = *reinterpret_cast<const uint32_t *>(a.v + (((int64_t)b * a.n_max + t) * a.hkv + h) * kHeadDim + c);
    tileb[r][c] = __builtin_bit_cast(uint16_t, (_Float16)bf16_value((uint16_t)(w & 0xFFFFu)));
    tileb[r][c + 1] = __builtin_bit_cast(uint16_t, (_Float16)bf16_value((uint16_t)(w >> 16)));
  }
  __syncthreads();
  for (int i = tid; i < kHeadDim * kTile / 2; i += 256) {  // 2 positions per step
    const int c = i / (kTile / 2), r = 2 * (i % (kTile / 2));
    const uint32_t w = (uint32_t)tileb[r][c] | ((uint32_t)tileb[r + 1][c] << 16);
    *reinterpret_cast<uint32_t *>(a.vt + (((int64_t)b * a.hkv + h) * kHeadDim + c) * a.n_max + tile * kTile + r) = w;
  }
}

__device__ __forceinline__ uint32_t pack_f16(float lo, float hi) {  // round to nearest even
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)lo) | ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)hi) << 16);
}

__global__ void __launch_bounds__(64) pf_attn_kernel(PfArgs a) {
  const int lane = threadIdx.x, col = lane & 15, rg = lane >> 4;
  const int b = blockIdx.y / a.hq, j = blockIdx.y % a.hq, h = j / (a.hq / a.hkv);
  const int t0 = blockIdx.x * kQBlock, t = t0 + col;  // this lane's query (column)
  int32_t n = checked_n(a, b);
  if (n < 0) n = 0;
  float *outq = a.out + (((int64_t)b * a.n_max + t) * a.hq + j) * kHeadDim;
  if (t0 >= n) {
#pragma unroll
    for (int ct = 0; ct < 8; ++ct)
      *reinterpret_cast<float4 *>(outq + 16 * ct + 4 * rg) = make_float4(0.f, 0.f, 0.f, 0.f);
    return;
  }
  // Query operands (B of S^T = K Q^T): lane (query col, k group rg).
  const int tq = min(t, n - 1);
  const uint16_t *qrow = a.q + (((int64_t)b * a.n_max + tq) * a.hq + j) * kHeadDim;
  const int8_t *qcrow = a.q_codes + (((int64_t)b * a.n_max + tq) * a.hq + j) * kHeadDim;
  bf8 qf[4];
  v4i qi[2];
#pragma unroll
  for (int m = 0; m < 4; ++m) qf[m] = *reinterpret_cast<const bf8 *>(qrow + 32 * m + 8 * rg);
#pragma unroll
  for (int m = 0; m < 2; ++m) qi[m] = *reinterpret_cast<const v4i *>(qcrow + 64 * m + 16 * rg);
  const float sq = a.q_scales[((int64_t)b * a.hq + j) * a.tiles + t0 / kTile];
  const float scale = 1.4426950408889634f / sqrtf((float)kHeadDim);  // log2(e) / sqrt(d)
  const uint8_t *vl = a.cls ? a.cls + ((int64_t)b * a.hkv + h) * a.n_max : nullptr;
  const uint16_t *vt = a.vt + (int64_t)(b * a.hkv + h) * kHeadDim * a.n_max;

  float m_run = -1.0e30f, l_run = 0.0f;
  v4f acc[8];
#pragma unroll
  for (int ct = 0; ct < 8; ++ct) acc[ct] = v4f{0.f, 0.f, 0.f, 0.f};
  const int32_t k_last = min(t0 + kQBlock - 1, n - 1);
  for (int32_t k0 = 0; k0 <= k_last; k0 += kKStep) {
    // Lane (query col, rg) holds keys k0 + 16 u + 4 rg + i (u = 0, 1; i = 0 .. 3).
    uint32_t vlw[2] = {0u, 0u};
    if (vl) {
#pragma unroll
      for (int u = 0; u < 2; ++u) vlw[u] = *reinterpret_cast<const uint32_t *>(vl + k0 + 16 * u + 4 * rg);
    }
    bool vis[2][4], fp[2][4];
    bool any_q = false, any_f = false;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int32_t kk = k0 + 16 * u + 4 * rg + i;
        vis[u][i] = kk <= t && kk < n;
        fp[u][i] = ((vlw[u] >> (8 * i)) & 0xFFu) == 1u || kk > t - a.window;
        any_q |= vis[u][i] && !fp[u][i];
        any_f |= vis[u][i] && fp[u][i];
      }
    const bool need_q = __any(any_q), need_f = __any(any_f);
    v4f sf[2], sqv[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int32_t kr = k0 + 16 * u + col;  // A-operand row: key
      const int64_t krow = (((int64_t)b * a.n_max + kr) * a.hkv + h) * kHeadDim;
      sf[u] = v4f{0.f, 0.f, 0.f, 0.f};
      sqv[u] = v4f{0.f, 0.f, 0.f, 0.f};
      if (need_f) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const bf8 kf = *reinterpret_cast<const bf8 *>(a.k + krow + 32 * m + 8 * rg);
          sf[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[m], sf[u], 0, 0, 0);
        }
      }
      if (need_q) {
        v4i s32 = v4i{0, 0, 0, 0};
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const v4i kc = *reinterpret_cast<const v4i *>(a.k_codes + krow + 64 * m + 16 * rg);
          s32 = __builtin_amdgcn_mfma_i32_16x16x64_i8(kc, qi[m], s32, 0, 0, 0);
        }
        const float sk = a.k_scales[((int64_t)b * a.hkv + h) * a.tiles + k0 / kTile];
#pragma unroll
        for (int i = 0; i < 4; ++i) sqv[u][i] = (float)s32[i] * (sq * sk);
      }
    }
    // Logits (base 2), masked; the step's maximum per query over its 4 lanes.
    float x[2][4], bmax = -INFINITY;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float s = fp[u][i] ? sf[u][i] : sqv[u][i];
        x[u][i] = vis[u][i] ? s * scale : -INFINITY;
        bmax = fmaxf(bmax, x[u][i]);
      }
    bmax = fmaxf(bmax, __shfl_xor(bmax, 16));
    bmax = fmaxf(bmax, __shfl_xor(bmax, 32));
    const float m_new = fmaxf(m_run, bmax);
    if (m_new > m_run) {
      const float alpha = exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) acc[ct] *= alpha;
      m_run = m_new;
    }
    float p[2][4];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[u][i] = exp2f(x[u][i] - m_run);
        l_run += p[u][i];
      }
    // P^T operand (fp16 weights): k slot 8 rg + i <-> key 4 rg + i (i < 4), 16 + 4 rg +
    // (i - 4) (i >= 4): the lane's own eight weights, in order.
    const h8 pw = __builtin_bit_cast(h8, make_uint4(pack_f16(p[0][0], p[0][1]), pack_f16(p[0][2], p[0][3]),
                                                    pack_f16(p[1][0], p[1][1]), pack_f16(p[1][2], p[1][3])));
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) {
      const uint16_t *vrow = vt + (int64_t)(16 * ct + col) * a.n_max + k0 + 4 * rg;
      const uint2 lo = *reinterpret_cast<const uint2 *>(vrow), hi = *reinterpret_cast<const uint2 *>(vrow + 16);
      const h8 vw = __builtin_bit_cast(h8, make_uint4(lo.x, lo.y, hi.x, hi.y));
      acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vw, pw, acc[ct], 0, 0, 0);
    }
  }
  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
  const float inv = (t < n && l_tot > 0.0f) ? 1.0f / l_tot : 0.0f;
#pragma unroll
  for (int ct = 0; ct < 8; ++ct)
    *reinterpret_cast<float4 *>(outq + 16 * ct + 4 * rg) =
        make_float4(acc[ct][0] * inv, acc[ct][1] * inv, acc[ct][2] * inv, acc[ct][3] * inv);
}

kvq_status launched(const char *what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(KVQ_ERR_HIP, "%s launch failed: %s", what, hipGetErrorString(e));
  return KVQ_OK;
}

}  // namespace
}  // namespace kvq

using namespace kvq;

extern "C" kvq_status kvq_prefill_attn(const void *q, const void *k, const void *v, int32_t dtype, int32_t batch,
                                       int32_t n_max, int32_t hq, int32_t hkv, const int32_t *n_tokens,
                                       const uint8_t *token_class, int32_t window, int8_t *q_codes,
                                       float *q_scales, int8_t *k_codes, float *k_scales, void *v_t, float *out,
                                       int32_t *dev_err, void *stream) {
  if (dtype != KVQ_BF16) return fail(KVQ_ERR_UNSUPPORTED, "prefill attention takes bf16 q, k, v");
  if (batch < 0 || n_max < 0 || n_max % kTile) return fail(KVQ_ERR_INVALID_ARG, "n_max %d: a multiple of 64", n_max);
  if (hkv <= 0 || hq <= 0 || hq % hkv) return fail(KVQ_ERR_INVALID_ARG, "hq %d is not a multiple of hkv %d", hq, hkv);
  if (window < 0) return fail(KVQ_ERR_INVALID_ARG, "negative window");
  if (batch == 0 || n_max == 0) return KVQ_OK;
  if (!q || !k || !v || !n_tokens || !q_codes || !q_scales || !k_codes || !k_scales || !v_t || !out)
    return fail(KVQ_ERR_INVALID_ARG, "NULL buffer");
  if ((int64_t)batch * hq > 65535 || (int64_t)hq + hkv > 65535) return fail(KVQ_ERR_UNSUPPORTED, "grid too large");
  PfArgs a;
  a.q = static_cast<const uint16_t *>(q);
  a.k = static_cast<const uint16_t *>(k);
  a.v = static_cast<const uint16_t *>(v);
  a.cls = token_class;
  a.n_tokens = n_tokens;
  a.batch = batch;
  a.n_max = n_max;
  a.hq = hq;
  a.hkv = hkv;
  a.window = window;
  a.tiles = n_max / kTile;
  a.q_codes = q_codes;
  a.k_codes = k_codes;
  a.q_scales = q_scales;
  a.k_scales = k_scales;
  a.vt = static_cast<uint16_t *>(v_t);
  a.out = out;
  a.err = dev_err;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(pf_quant_kernel, dim3(a.tiles, batch, hq + hkv), dim3(256), 0, s, a);
  kvq_status st = launched("pf_quant_kernel");
  if (st != KVQ_OK) return st;
  hipLaunchKernelGGL(pf_vt_kernel, dim3(a.tiles, batch, hkv), dim3(256), 0, s, a);
  st = launched("pf_vt_kernel");
  if (st != KVQ_OK) return st;
  hipLaunchKernelGGL(pf_attn_kernel, dim3(n_max / kQBlock, batch * hq), dim3(64), 0, s, a);
  return launched("pf_attn_kernel");
}
