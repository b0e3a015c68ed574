// Vertical-line selection and FREEZE routing (HyQuant Algorithm 1 and Algorithm 4).
//
// Per request b and KV head h: the tail-query proxy u (the mean over the request's
// tail queries of the sum of the g query heads of h), the score u . K of every token,
// and, over the non-window prefix (the last `window` tokens excluded), the
// round(rho * prefix) tokens of highest score (ties: lower index) as vertical lines.
// The class written per token is the FREEZE routing: vertical lines and window stay
// FP16, the rest of the prefix is quantized.
//
// Three launches: the proxy (one wave per (b, h)); the scores (HBM-bound: every K row
// read once, a token's hkv x 128 values across the 64 lanes of a wave, a dot product
// per lane and a reduction over the lanes of one head); the selection (one work group
// per (b, h): a four-pass 8-bit radix select of the threshold key over the prefix
// scores in LDS histograms, then one ordered pass that ranks the keys equal to the
// threshold by index).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "kvq.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kMaxTail = 64;  // tail queries kept by the proxy
constexpr int kScoreWaves = 4;
constexpr int kTokensPerWave = 64;
constexpr int kSelectThreads = 1024;

__device__ __forceinline__ void report(int32_t *err, int32_t bit) {
  if (err) atomicOr(err, bit);
}

template <int DT>
__device__ __forceinline__ float elem(const void *p, int64_t i) {
  if (DT == KVQ_F32) return static_cast<const float *>(p)[i];
  const uint16_t h = static_cast<const uint16_t *>(p)[i];
  if (DT == KVQ_BF16) return __uint_as_float((uint32_t)h << 16);
  return (float)__builtin_bit_cast(_Float16, h);
}

// u[b][h][c] = (1 / n_tail) sum_i sum_j q[b][i][h g + j][c].  Lane = channel pair; the
// four waves take every fourth (i, j) term and add their sums through LDS.
template <int QD>
__global__ void __launch_bounds__(256) vl_proxy_kernel(const void *q, int32_t hkv, int32_t hq, int32_t max_tail,
                                                       const int32_t *n_tail, float *u, int32_t *err) {
  __shared__ float part[4][kHeadDim];
  const int b = blockIdx.x / hkv, h = blockIdx.x % hkv, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = hq / hkv;
  int32_t nt = n_tail[b];
  if (nt < 0 || nt > max_tail) {
    if (threadIdx.x == 0) report(err, KVQ_DEVERR_RANGE);
    nt = 0;
  }
  float s0 = 0.0f, s1 = 0.0f;
  const int terms = nt * g;
#pragma unroll 8
  for (int x = wave; x < terms; x += 4) {
    const int i = x / g, j = x % g;
    const int64_t at = (((int64_t)b * max_tail + i) * hq + h * g + j) * kHeadDim + 2 * lane;
    s0 += elem<QD>(q, at);
    s1 += elem<QD>(q, at + 1);
  }
  part[wave][2 * lane] = s0;
  part[wave][2 * lane + 1] = s1;
  __syncthreads();
  if (wave == 0) {
    const float inv = nt > 0 ? 1.0f / (float)nt : 0.0f;
    float *dst = u + ((int64_t)b * hkv + h) * kHeadDim + 2 * lane;
#pragma unroll
    for (int c = 0; c < 2; ++c)
      dst[c] = (((part[0][2 * lane + c] + part[1][2 * lane + c]) + part[2][2 * lane + c]) + part[3][2 * lane + c]) *
               inv;
  }
}

// NW consecutive 32-bit words at p (16-byte aligned when NW >= 4), in the widest loads.
template <int NW>
__device__ __forceinline__ void load_words(const uint32_t *p, uint32_t (&w)[NW]) {
  if constexpr (NW >= 4) {
#pragma unroll
    for (int i = 0; i < NW / 4; ++i) {
      const uint4 v = reinterpret_cast<const uint4 *>(p)[i];
      w[4 * i] = v.x, w[4 * i + 1] = v.y, w[4 * i + 2] = v.z, w[4 * i + 3] = v.w;
    }
  } else if constexpr (NW == 2) {
    const uint2 v = *reinterpret_cast<const uint2 *>(p);
    w[0] = v.x, w[1] = v.y;
  } else {
    w[0] = *p;
  }
}

// Words one lane loads per token row: E values of type KD.
template <int KD, int E>
constexpr int words_of() { return KD == KVQ_F32 ? E : E / 2; }

// The E values of one lane, from its words, as fp32.
template <int KD, int E>
__device__ __forceinline__ void values_of(const uint32_t (&w)[words_of<KD, E>()], float (&v)[E]) {
  if constexpr (KD == KVQ_F32) {
#pragma unroll
    for (int e = 0; e < E; ++e) v[e] = __uint_as_float(w[e]);
  } else {
#pragma unroll
    for (int e = 0; e < E / 2; ++e) {
      if (KD == KVQ_BF16) {
        v[2 * e] = __uint_as_float(w[e] << 16);
        v[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
      } else {
        v[2 * e] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[e] & 0xFFFFu));
        v[2 * e + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[e] >> 16));
      }
    }
  }
}

// Sum over the LPH consecutive lanes of a head; lane 0 of each group gets the total.
// Within 16-lane rows by DPP (quad swaps, then row rotations that bring lane i + 4 and
// lane i + 8 to lane i), across rows by a lane shuffle.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

template <int LPH>
__device__ __forceinline__ float head_sum(float s) {
  if constexpr (LPH >= 2) s += dpp_mov<0xB1>(s);   // quad_perm [1, 0, 3, 2]
  if constexpr (LPH >= 4) s += dpp_mov<0x4E>(s);   // quad_perm [2, 3, 0, 1]
  if constexpr (LPH >= 8) s += dpp_mov<0x12C>(s);  // row_ror:12 (lane i reads lane i + 4 of its row)
  if constexpr (LPH >= 16) s += dpp_mov<0x128>(s); // row_ror:8
  if constexpr (LPH >= 32) s += __shfl_xor(s, 16);
  if constexpr (LPH >= 64) s += __shfl_xor(s, 32);
  return s;
}

// Scores of 64 consecutive tokens per wave.  A token row holds HKV x 128 values; lane
// l takes E = 2 HKV consecutive ones (all of one head: 64 / HKV lanes per head), so a
// wave reads each row as one contiguous block.  U rows are loaded per step, the next
// step's rows before the current ones are reduced; rows past the request's length
// are clamped to its last row (read, never scored), so no load sits under a branch.
template <int KD, int HKV>
__global__ void __launch_bounds__(64 * kScoreWaves) vl_score_kernel(const void *k, int32_t max_tokens,
                                                                    const int32_t *n_tokens, const float *u,
                                                                    float *scores) {
  constexpr int E = 2 * HKV, LPH = 64 / HKV, NW = words_of<KD, E>(), U = 4;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int b = blockIdx.y, h = lane / LPH;
  const int32_t n = min(max(n_tokens[b], 0), max_tokens);
  const int32_t t0 = (blockIdx.x * kScoreWaves + wave) * kTokensPerWave;
  if (t0 >= max_tokens) return;
  const int32_t t_end = min(t0 + kTokensPerWave, max_tokens);
  float *out = scores + ((int64_t)b * HKV + h) * max_tokens;
  const bool writer = lane % LPH == 0;
  if (n <= t0) {  // nothing of this request here
    for (int32_t t = t0; t < t_end; ++t)
      if (writer) out[t] = 0.0f;
    return;
  }
  float uu[E];
#pragma unroll
  for (int e = 0; e < E; ++e) uu[e] = u[((int64_t)b * HKV + h) * kHeadDim + (lane % LPH) * E + e];
  const uint32_t *kw = static_cast<const uint32_t *>(k);
  const int64_t row0 = (int64_t)b * max_tokens;
  auto load = [&](int32_t t, uint32_t (&w)[U][NW]) {
#pragma unroll
    for (int r = 0; r < U; ++r) {
      const int64_t row = row0 + min(t + r, n - 1);
      load_words<NW>(kw + row * (HKV * kHeadDim * NW / E) + (int64_t)lane * NW, w[r]);
    }
  };
  auto score = [&](int32_t t, const uint32_t (&w)[U][NW]) {
#pragma unroll
    for (int r = 0; r < U; ++r) {
      float v[E];
      values_of<KD, E>(w[r], v);
      float s = 0.0f;
#pragma unroll
      for (int e = 0; e < E; ++e) s = fmaf(uu[e], v[e], s);
      s = head_sum<LPH>(s);
      const int32_t tt = t + r;
      if (writer && tt < t_end) out[tt] = tt < n ? s : 0.0f;
    }
  };
  uint32_t wa[U][NW], wb[U][NW];
  load(t0, wa);
  for (int32_t t = t0; t < t_end; t += 2 * U) {
    load(t + U < t_end ? t + U : t, wb);
    score(t, wa);
    if (t + U >= t_end) break;
    load(t + 2 * U < t_end ? t + 2 * U : t + U, wa);
    score(t + U, wb);
  }
}

// Order-preserving key of a score (+0 and -0 alike).
__device__ __forceinline__ uint32_t key_of(float s) {
  const uint32_t x = __float_as_uint(s == 0.0f ? 0.0f : s);
  return (x & 0x80000000u) ? ~x : (x | 0x80000000u);
}

__global__ void __launch_bounds__(kSelectThreads) vl_select_kernel(const float *scores, int32_t hkv,
                                                                   int32_t max_tokens, const int32_t *n_tokens,
                                                                   int32_t window, float rho, uint8_t *cls,
                                                                   int32_t *n_vl, int32_t *err) {
  constexpr int kWaves = kSelectThreads / 64;
  __shared__ uint32_t hist[kWaves][256];  // one histogram per wave (the top bits of the keys
                                          // of nearby scores collide: few distinct bins)
  __shared__ uint32_t suffix[256];
  __shared__ uint32_t wave_eq[kWaves];
  __shared__ uint32_t sel[2];  // threshold prefix, keys still needed at it
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = blockIdx.x / hkv;
  const int64_t row = (int64_t)blockIdx.x * max_tokens;
  int32_t n = n_tokens[b];
  if (n < 0 || n > max_tokens) {
    if (tid == 0) report(err, KVQ_DEVERR_RANGE);
    n = 0;
  }
  const int32_t n_pre = max(n - window, 0);
  const int32_t m = (int32_t)floor((double)rho * (double)n_pre + 0.5);
  const float *S = scores + row;

  // Radix select of the m-th largest key, 8 bits a pass from the top: per-wave
  // histograms of the next digit among the keys that match the prefix so far, their
  // per-bin totals, suffix sums over the bins (a log-step scan), and the one bin where
  // the suffix sum first reaches the count still needed.
  uint32_t prefix = 0, need = (uint32_t)m;
  if (m > 0) {
    for (int shift = 24; shift >= 0; shift -= 8) {
      const uint32_t hi_mask = shift == 24 ? 0u : (~0u << (shift + 8));
      for (int i = tid; i < kWaves * 256; i += kSelectThreads) (&hist[0][0])[i] = 0;
      __syncthreads();
      for (int32_t t = tid; t < n_pre; t += kSelectThreads) {
        const uint32_t key = key_of(S[t]);
        if ((key & hi_mask) == prefix) atomicAdd(&hist[wave][(key >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (tid < 256) {
        uint32_t c = 0;
        for (int w = 0; w < kWaves; ++w) c += hist[w][tid];
        suffix[tid] = c;
      }
      __syncthreads();
      for (int d = 1; d < 256; d <<= 1) {  // suffix[t] = sum of bins t .. 255
        const uint32_t add = (tid < 256 && tid + d < 256) ? suffix[tid + d] : 0u;
        __syncthreads();
        if (tid < 256) suffix[tid] += add;
        __syncthreads();
      }
      if (tid < 256) {
        const uint32_t here = suffix[tid], next = tid < 255 ? suffix[tid + 1] : 0u;
        if (here >= need && next < need) {
          sel[0] = prefix | ((uint32_t)tid << shift);
          sel[1] = need - next;
        }
      }
      __syncthreads();
      prefix = sel[0];
      need = sel[1];
      __syncthreads();  // the histograms are cleared again next pass
    }
  }
  // Classes in token order: above the threshold, or at it among the first `need`.
  const uint64_t below = lane ? (~0ull >> (64 - lane)) : 0ull;
  uint32_t eq_before = 0;
  for (int32_t base = 0; base < max_tokens; base += kSelectThreads) {
    const int32_t t = base + tid;
    const bool in_pre = t < n_pre;
    const uint32_t key = in_pre && m > 0 ? key_of(S[t]) : 0u;
    const bool gt = in_pre && m > 0 && key > prefix, eq = in_pre && m > 0 && key == prefix;
    const uint64_t eq_mask = __ballot(eq);
    if (lane == 0) wave_eq[wave] = (uint32_t)__popcll(eq_mask);
    __syncthreads();
    uint32_t off = eq_before, total = 0;
    for (int w = 0; w < kSelectThreads / 64; ++w) {
      if (w < wave) off += wave_eq[w];
      total += wave_eq[w];
    }
    const uint32_t rank = off + (uint32_t)__popcll(eq_mask & below);
    if (t < max_tokens) {
      uint8_t c = 0;
      if (t < n && t >= n_pre) c = 2;
      else if (gt || (eq && rank < need)) c = 1;
      cls[row + t] = c;
    }
    eq_before += total;
    __syncthreads();  // wave_eq is rewritten by the next chunk
  }
  if (tid == 0) n_vl[blockIdx.x] = m;
}

kvq_status launched(const char *what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(KVQ_ERR_HIP, "%s launch failed: %s", what, hipGetErrorString(e));
  return KVQ_OK;
}

template <int KD>
void launch_scores(int hkv, dim3 grid, hipStream_t s, const void *k, int32_t max_tokens, const int32_t *n_tokens,
                   const float *u, float *scores) {
  const dim3 block(64 * kScoreWaves);
  switch (hkv) {
    case 1: hipLaunchKernelGGL((vl_score_kernel<KD, 1>), grid, block, 0, s, k, max_tokens, n_tokens, u, scores); break;
    case 2: hipLaunchKernelGGL((vl_score_kernel<KD, 2>), grid, block, 0, s, k, max_tokens, n_tokens, u, scores); break;
    case 4: hipLaunchKernelGGL((vl_score_kernel<KD, 4>), grid, block, 0, s, k, max_tokens, n_tokens, u, scores); break;
    case 8: hipLaunchKernelGGL((vl_score_kernel<KD, 8>), grid, block, 0, s, k, max_tokens, n_tokens, u, scores); break;
    default: hipLaunchKernelGGL((vl_score_kernel<KD, 16>), grid, block, 0, s, k, max_tokens, n_tokens, u, scores);
  }
}

}  // namespace
}  // namespace kvq

using namespace kvq;

extern "C" kvq_status kvq_select_vertical_lines(const void *k, int32_t k_dtype, const void *q_tail, int32_t q_dtype,
                                                int32_t batch, int32_t max_tokens, int32_t hkv, int32_t hq,
                                                int32_t max_tail, const int32_t *n_tokens, const int32_t *n_tail,
                                                int32_t window, float rho, float *proxy, float *scores,
                                                uint8_t *token_class, int32_t *n_vl, int32_t *dev_err,
                                                void *stream) {
  auto dtype_ok = [](int32_t d) { return d == KVQ_F32 || d == KVQ_BF16 || d == KVQ_F16; };
  if (!dtype_ok(k_dtype) || !dtype_ok(q_dtype)) return fail(KVQ_ERR_INVALID_ARG, "unknown K or query dtype");
  if (batch < 0 || max_tokens < 0) return fail(KVQ_ERR_INVALID_ARG, "negative batch or max_tokens");
  if (hkv <= 0 || hq <= 0 || hq % hkv) return fail(KVQ_ERR_INVALID_ARG, "hq %d is not a multiple of hkv %d", hq, hkv);
  if (hkv != 1 && hkv != 2 && hkv != 4 && hkv != 8 && hkv != 16)
    return fail(KVQ_ERR_UNSUPPORTED, "hkv %d: 1, 2, 4, 8 or 16 KV heads", hkv);
  if (max_tail < 1 || max_tail > kMaxTail) return fail(KVQ_ERR_INVALID_ARG, "max_tail %d outside [1, 64]", max_tail);
  if (window < 0 || !(rho >= 0.0f && rho <= 1.0f)) return fail(KVQ_ERR_INVALID_ARG, "window < 0 or rho outside [0, 1]");
  if (batch == 0 || max_tokens == 0) return KVQ_OK;
  if (!k || !q_tail || !n_tokens || !n_tail || !proxy || !scores || !token_class || !n_vl)
    return fail(KVQ_ERR_INVALID_ARG, "NULL buffer");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 pgrid(batch * hkv), pblock(256);
  if (q_dtype == KVQ_F32)
    hipLaunchKernelGGL(vl_proxy_kernel<KVQ_F32>, pgrid, pblock, 0, s, q_tail, hkv, hq, max_tail, n_tail, proxy, dev_err);
  else if (q_dtype == KVQ_BF16)
    hipLaunchKernelGGL(vl_proxy_kernel<KVQ_BF16>, pgrid, pblock, 0, s, q_tail, hkv, hq, max_tail, n_tail, proxy, dev_err);
  else
    hipLaunchKernelGGL(vl_proxy_kernel<KVQ_F16>, pgrid, pblock, 0, s, q_tail, hkv, hq, max_tail, n_tail, proxy, dev_err);
  kvq_status st = launched("vl_proxy_kernel");
  if (st != KVQ_OK) return st;
  const int per_block = kScoreWaves * kTokensPerWave;
  const dim3 sgrid((max_tokens + per_block - 1) / per_block, batch);
  if (k_dtype == KVQ_F32) launch_scores<KVQ_F32>(hkv, sgrid, s, k, max_tokens, n_tokens, proxy, scores);
  else if (k_dtype == KVQ_BF16) launch_scores<KVQ_BF16>(hkv, sgrid, s, k, max_tokens, n_tokens, proxy, scores);
  else launch_scores<KVQ_F16>(hkv, sgrid, s, k, max_tokens, n_tokens, proxy, scores);
  st = launched("vl_score_kernel");
  if (st != KVQ_OK) return st;
  hipLaunchKernelGGL(vl_select_kernel, dim3(batch * hkv), dim3(kSelectThreads), 0, s, scores, hkv, max_tokens,
                     n_tokens, window, rho, token_class, n_vl, dev_err);
  return launched("vl_select_kernel");
}
