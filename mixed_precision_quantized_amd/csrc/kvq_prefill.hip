// Prefill attention with an INT8 prefix (HyQuant: the fused operator of the core method,
// softmax([Q K-hat_Q^T || Q K_FP^T] / sqrt(d)) [V-hat_Q || V_FP], and Algorithm 2).
//
// For query position t of a request, query head j and its KV head h = j / g, the keys
// k <= t are read in full precision (K and V as given) when k is a vertical line of h or
// lies in the window k > t - W, and through INT8 otherwise (K-hat = s_K code_K, V-hat =
// s_V code_V); the query is used as given; all of them share one online softmax.  INT8
// tiles are 64 positions per KV head, separately for K and V, with the symmetric scale
// max|x| / 127 over the tile's live non-line values.
//
// The three segments of the scan are three key lists:
//   INT8    keys k <= t - W that are not vertical lines: K codes as exact bf16 integers
//           (the tile's s_K scales the fp32 logit), and V-hat^T (s_V code_V in fp16,
//           formed once per tile) with the vertical-line columns zeroed, so their
//           weights drop out of P.V; their softmax weights enter the row sum through a
//           0 / 1 keep mask;
//   VL      the vertical lines k <= t, gathered per KV head into a compact list (bf16
//           K rows, fp16 V^T columns, positions);
//   window  keys t - W < k <= t that are not vertical lines, bf16 K and fp16 V^T.
// Their union is every key k <= t, each in the precision the method gives it.  Q . K
// is a bf16 product (exact products, fp32 sums) in every segment; V enters P.V in fp16
// (exact for bf16 values in fp16's normal range; V-hat rounded once to fp16) with fp16
// weights (bf16 weights would lose too much for the 2e-3 bar).
//
// Launches: K codes and scales with their bf16 copy (one work group per 64-position
// tile and KV head); V codes and scales, V-hat^T and V^T with the keep mask (the same
// grid); the vertical-line list (one work group per request and KV head); its gather;
// the attention.  An attention work group (4 waves, two groups per CU) takes one
// request, one KV head and 128 / g positions of all g of its query heads (of half of
// them, for g = 16): 8 column blocks of 16 (position, head) rows, two per wave.  K and
// V^T stages of 64 keys go to LDS by LDS-bound global loads, double-buffered across all
// three segments; S^T = K Q^T on MFMA (f32 16x16x32 bf16) puts a lane's scores where
// the P operand of O^T = V^T P^T wants them (f32 16x16x32 f16).  The softmax rescales
// lazily: the running maximum moves only when a score exceeds it by 2^8.
#include <hip/hip_runtime.h>

#include <cfloat>
#include <cmath>
#include <cstdint>

#include "kvq.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kTile = 64;       // INT8 tile = LDS stage (positions)
constexpr int kGroupRows = 128; // (position, query head) rows per attention work group
constexpr int kAttnWaves = 4;   // attention waves per work group
constexpr int kAttnThreads = 64 * kAttnWaves;
constexpr int kCB = kGroupRows / 16 / kAttnWaves;  // 16-row column blocks per wave
constexpr float kLazy = 8.0f;   // log2 headroom of the running maximum
constexpr int kRing = 2;        // LDS stages: the copy of stage s + 1 overlaps stage s
static_assert(kRing == 2, "the clean INT8 loop takes its LDS stages in pairs");
constexpr int kColBlocks = kGroupRows / 16;

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 bf8 __attribute__((ext_vector_type(8)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef const __attribute__((address_space(1))) uint8_t *gbytes;

__device__ __forceinline__ void report(int32_t *err, int32_t bit) {
  if (err) atomicOr(err, bit);
}

__device__ __forceinline__ float bf16_value(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

struct PfArgs {
  const uint16_t *q, *k, *v;     // bf16 [batch][n_max][heads][128]
  const uint8_t *cls;            // [batch][hkv][n_max] (1 = vertical line) or null
  const int32_t *n_tokens;
  int32_t batch, n_max, hq, hkv, g, window, tiles;
  int32_t hsplit;                // attention work groups per (position block, KV head)
  int8_t *k_codes, *v_codes;     // like k, v
  float *k_scales, *v_scales;    // [batch][hkv][tiles]
  uint16_t *kq;                  // bf16 [batch][n_max][hkv][128]: K codes as exact bf16 integers
  uint16_t *vt;                  // fp16 [batch][hkv][128][n_max]: V; vertical lines, t >= n: 0
  uint16_t *vtq;                 // fp16 [batch][hkv][128][n_max]: V-hat = s_V code_V; lines, t >= n: 0
  uint16_t *keep;                // fp16 [batch][hkv][n_max]: 1 for live keys that are not lines
  int32_t *vl_pos;               // [batch][hkv][n_max]: line positions in order, then INT32_MAX
  int32_t *vl_cnt;               // [batch][hkv][tiles]: lines at positions < 64 (tile + 1)
  uint16_t *vl_k;                // bf16 [batch][hkv][n_max][128]: line K rows, then 0
  uint16_t *vl_vt;               // fp16 [batch][hkv][128][n_max]: line V columns, then 0
  float *out;                    // [batch][n_max][hq][128]
  int32_t *err;
};

__device__ __forceinline__ int32_t checked_n(const PfArgs &a, int b) {
  const int32_t n = a.n_tokens[b];
  return (n < 0 || n > a.n_max) ? -1 : n;
}

// INT8 code of x in a tile of scale s (Algorithm 2's symmetric scale): clamp(rint(x / s),
// -127, 127) with a correctly rounded fp32 quotient, 0 when s = 0.
__device__ __forceinline__ float int8_code(float x, float s) {
  return s != 0.0f ? fminf(fmaxf(rintf(__fdiv_rn(x, s)), -127.0f), 127.0f) : 0.0f;
}

// K codes and scale of one 64-position tile of one KV head, and the codes as exact bf16
// integers (the attention's K operand).  Thread: row tid / 4, channels 32 (tid % 4) ..
// + 31.
__global__ void __launch_bounds__(256) pf_quant_k_kernel(PfArgs a) {
  __shared__ float wmax[4];
  const int tid = threadIdx.x, tile = blockIdx.x, b = blockIdx.y, head = blockIdx.z;
  int32_t n = checked_n(a, b);
  if (n < 0) {
    if (tid == 0) report(a.err, KVQ_DEVERR_RANGE);
    n = 0;
  }
  const int row = tile * kTile + tid / 4, c0 = 32 * (tid % 4);
  const int64_t at = (((int64_t)b * a.n_max + row) * a.hkv + head) * kHeadDim + c0;
  const bool live = row < n;
  const bool counts = live && !(a.cls && a.cls[((int64_t)b * a.hkv + head) * a.n_max + row] == 1);
  float x[32];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 w = live ? reinterpret_cast<const uint4 *>(a.k + at)[i] : make_uint4(0u, 0u, 0u, 0u);
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
  if (tid == 0) a.k_scales[((int64_t)b * a.hkv + head) * a.tiles + tile] = s;
  uint32_t packed[8], wide[16] = {};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t w = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float c = live ? int8_code(x[4 * i + e], s) : 0.0f;
      w |= ((uint32_t)(uint8_t)(int8_t)c) << (8 * e);
      // an integer of at most 8 bits is exact in bf16: the top half of its fp32 bits
      const uint32_t hb = __float_as_uint(c) >> 16;
      wide[2 * i + (e >> 1)] |= hb << (16 * (e & 1));
    }
    packed[i] = w;
  }
  int8_t *dst = a.k_codes + at;
  reinterpret_cast<uint4 *>(dst)[0] = make_uint4(packed[0], packed[1], packed[2], packed[3]);
  reinterpret_cast<uint4 *>(dst)[1] = make_uint4(packed[4], packed[5], packed[6], packed[7]);
  uint4 *kd = reinterpret_cast<uint4 *>(a.kq + at);
#pragma unroll
  for (int i = 0; i < 4; ++i) kd[i] = make_uint4(wide[4 * i], wide[4 * i + 1], wide[4 * i + 2], wide[4 * i + 3]);
}

// V of one 64-position tile of one KV head, through LDS: its codes and scale (vertical
// lines left out of the maximum, as for K), then transposed to [channel][position]
// twice, as given (fp16, exact in fp16's normal range) for the full-precision segments
// and as V-hat = s_V code_V (rounded once to fp16) for the INT8 segment; vertical lines
// and positions at or past the request's length are 0 in both.  Also the keep mask of
// the INT8 and window segments: 1 for live positions that are not vertical lines.
__global__ void __launch_bounds__(256) pf_quant_v_kernel(PfArgs a) {
  __shared__ uint16_t tileb[kTile][kHeadDim + 2];  // bf16 bits
  __shared__ int8_t codes[kTile][kHeadDim + 4];
  __shared__ uint8_t kept[kTile], live[kTile];
  __shared__ float wmax[4];
  const int tid = threadIdx.x, tile = blockIdx.x, b = blockIdx.y, h = blockIdx.z;
  int32_t n = checked_n(a, b);  // (the K kernel reports a bad length)
  if (n < 0) n = 0;
  const int64_t bh = (int64_t)b * a.hkv + h;
  if (tid < kTile) {
    const int t = tile * kTile + tid;
    const bool lv = t < n;
    const bool k = lv && !(a.cls && a.cls[bh * a.n_max + t] == 1);
    kept[tid] = k ? 1 : 0;
    live[tid] = lv ? 1 : 0;
    a.keep[bh * a.n_max + t] = k ? 0x3C00u : 0u;  // fp16 1.0, 0.0
  }
  __syncthreads();
  float m = 0.0f;
  for (int i = tid; i < kTile * kHeadDim / 2; i += 256) {  // 2 channels per step
    const int r = i / (kHeadDim / 2), c = 2 * (i % (kHeadDim / 2));
    const int t = tile * kTile + r;
    uint32_t w = 0;
    if (live[r]) w = *reinterpret_cast<const uint32_t *>(a.v + (((int64_t)b * a.n_max + t) * a.hkv + h) * kHeadDim + c);
    tileb[r][c] = (uint16_t)(w & 0xFFFFu);
    tileb[r][c + 1] = (uint16_t)(w >> 16);
    if (kept[r]) m = fmaxf(m, fmaxf(fabsf(bf16_value((uint16_t)(w & 0xFFFFu))), fabsf(bf16_value((uint16_t)(w >> 16)))));
  }
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if ((tid & 63) == 0) wmax[tid >> 6] = m;
  __syncthreads();
  const float amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  const float s = __fdiv_rn(amax, 127.0f);
  if (tid == 0) a.v_scales[bh * a.tiles + tile] = s;
  for (int i = tid; i < kTile * kHeadDim / 4; i += 256) {  // 4 channels (one code word) per step
    const int r = i / (kHeadDim / 4), c = 4 * (i % (kHeadDim / 4));
    const int t = tile * kTile + r;
    uint32_t w = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float cd = live[r] ? int8_code(bf16_value(tileb[r][c + e]), s) : 0.0f;
      codes[r][c + e] = (int8_t)cd;
      w |= ((uint32_t)(uint8_t)(int8_t)cd) << (8 * e);
    }
    *reinterpret_cast<uint32_t *>(a.v_codes + (((int64_t)b * a.n_max + t) * a.hkv + h) * kHeadDim + c) = w;
  }
  __syncthreads();
  auto f16 = [](float x) { return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x); };
  for (int i = tid; i < kHeadDim * kTile / 2; i += 256) {  // 2 positions per step
    const int c = i / (kTile / 2), r = 2 * (i % (kTile / 2));
    uint32_t raw = 0, deq = 0;
#pragma unroll
    for (int e = 0; e < 2; ++e)
      if (kept[r + e]) {
        raw |= f16(bf16_value(tileb[r + e][c])) << (16 * e);
        deq |= f16(s * (float)codes[r + e][c]) << (16 * e);
      }
    const int64_t at = (bh * kHeadDim + c) * a.n_max + tile * kTile + r;
    *reinterpret_cast<uint32_t *>(a.vt + at) = raw;
    *reinterpret_cast<uint32_t *>(a.vtq + at) = deq;
  }
}

// The vertical-line list of one (request, KV head): positions t < n with class 1, in
// order, then INT32_MAX up to n_max; vl_cnt[tile] = lines at positions < 64 (tile + 1).
constexpr int kScanThreads = 1024;
__global__ void __launch_bounds__(kScanThreads) pf_vl_scan_kernel(PfArgs a) {
  __shared__ int32_t wsum[kScanThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int b = blockIdx.x / a.hkv;
  const int64_t bh = blockIdx.x;
  int32_t n = checked_n(a, b);
  if (n < 0) n = 0;
  int32_t *pos = a.vl_pos + bh * a.n_max;
  int32_t running = 0;
  for (int base = 0; base < a.n_max; base += kScanThreads) {
    const int t = base + tid;
    const bool f = t < n && a.cls && a.cls[bh * a.n_max + t] == 1;
    const uint64_t m = __ballot(f);
    const int below = __popcll(m & ((1ull << lane) - 1ull));
    if (lane == 0) wsum[wv] = __popcll(m);
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int i = 0; i < kScanThreads / 64; ++i) {
      before += i < wv ? wsum[i] : 0;
      total += wsum[i];
    }
    if (f) pos[running + before + below] = t;
    if (t < a.n_max && (t & (kTile - 1)) == kTile - 1)
      a.vl_cnt[bh * a.tiles + t / kTile] = running + before + below + (f ? 1 : 0);
    running += total;
    __syncthreads();
  }
  for (int i = running + tid; i < a.n_max; i += kScanThreads) pos[i] = INT32_MAX;
}

// Gathers 64 entries of one vertical-line list: K rows (bf16, as they are) and V
// columns (fp16, transposed); entries past the list's length up to the next multiple of
// 64 are zeros.
__global__ void __launch_bounds__(256) pf_vl_gather_kernel(PfArgs a) {
  __shared__ uint16_t tileb[kTile][kHeadDim + 2];
  const int tid = threadIdx.x, it = blockIdx.x;
  const int b = blockIdx.y / a.hkv, h = blockIdx.y % a.hkv;
  const int64_t bh = blockIdx.y;
  const int32_t total = a.vl_cnt[bh * a.tiles + a.tiles - 1];
  if (it * kTile >= ((total + kTile - 1) & ~(kTile - 1))) return;
  const int32_t *pos = a.vl_pos + bh * a.n_max;
  for (int i = tid; i < kTile * kHeadDim / 8; i += 256) {  // 8 channels per step
    const int r = i / (kHeadDim / 8), c = 8 * (i % (kHeadDim / 8));
    const int32_t e = it * kTile + r;
    uint4 kw = make_uint4(0u, 0u, 0u, 0u), vw = kw;
    if (e < total) {
      const int64_t src = (((int64_t)b * a.n_max + pos[e]) * a.hkv + h) * kHeadDim + c;
      kw = *reinterpret_cast<const uint4 *>(a.k + src);
      vw = *reinterpret_cast<const uint4 *>(a.v + src);
    }
    *reinterpret_cast<uint4 *>(a.vl_k + (bh * a.n_max + e) * kHeadDim + c) = kw;
    const uint32_t ww[4] = {vw.x, vw.y, vw.z, vw.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      tileb[r][c + 2 * q] = __builtin_bit_cast(uint16_t, (_Float16)bf16_value((uint16_t)(ww[q] & 0xFFFFu)));
      tileb[r][c + 2 * q + 1] = __builtin_bit_cast(uint16_t, (_Float16)bf16_value((uint16_t)(ww[q] >> 16)));
    }
  }
  __syncthreads();
  for (int i = tid; i < kHeadDim * kTile / 2; i += 256) {
    const int c = i / (kTile / 2), r = 2 * (i % (kTile / 2));
    const uint32_t w = (uint32_t)tileb[r][c] | ((uint32_t)tileb[r + 1][c] << 16);
    *reinterpret_cast<uint32_t *>(a.vl_vt + (bh * kHeadDim + c) * a.n_max + it * kTile + r) = w;
  }
}

// ---- attention ----------------------------------------------------------------------

// One stage in LDS: 64 keys of K (bf16 rows of 256 B: codes or values), V^T (128 channel
// rows of 64 fp16 keys) and 256 B of side data (fp16 keep weights, or line positions).
// 16-byte chunks are XOR-swizzled within a row so that the 16 lanes a 16-byte LDS read
// serves at once hit 16 different banks quads: a key row's chunk c sits at c ^ swz_w(key),
// a channel row's at c ^ swz_v(ch).
struct __align__(16) PfStage {
  uint8_t k[kTile * 256];
  uint8_t v[kHeadDim * kTile * 2];
  uint32_t aux[kTile];
};

// The A-operand rows a 16-lane group reads are keys {0..3, 8..11, 16..19, 24..27} (+4,
// +32): the low three bits give the 8 keys of each parity 8 different chunks, and as
// 256-byte rows span every bank, the parity picks the other half of the 16 chunks.
__device__ __forceinline__ int swz_w(int key) {
  return ((key >> 1) & 1) | (((key >> 3) & 1) << 1) | (((key >> 4) & 1) << 2) | ((key & 1) << 3);
}
// Channel rows 16 ct .. 16 ct + 15: parity picks the bank half, ch / 2 the chunk.
__device__ __forceinline__ int swz_v(int ch) { return (ch >> 1) & 7; }

__device__ __forceinline__ uint32_t lds_addr(const void *p) { return (uint32_t)(uintptr_t)p; }

// 1 KB to LDS: lane L copies 16 B from base + voff to LDS byte lds + 16 L.  The LDS base
// goes in M0; an LDS-bound global load needs one wait state after a write of M0.
__device__ __forceinline__ void dma_block(uint32_t lds, gbytes base, uint32_t voff) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(voff), "s"((uint64_t)base), "{m0}"(lds) : "memory");
}

// The work group's stage list: INT8 stages 0 .. n8 - 1 (key tiles 0 ..), line stages
// (64 list entries each), window stages (key tiles w_first ..).
struct PfPlan {
  int32_t n8, n8_clean, nvl, nwin, w_first;
};

// A wave-uniform pointer, held in scalar registers.
__device__ __forceinline__ gbytes uniform(const void *p) {
  const uint64_t x = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x), hi = __builtin_amdgcn_readfirstlane((uint32_t)(x >> 32));
  return (gbytes)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// Copies of one stage into LDS.  Each lane's offsets within a stage are fixed, so they
// are computed once; a stage only moves the (wave-uniform) base pointers.
struct PfCopier {
  gbytes kq, kin, kvl, vt, vtq, vlvt, keep, vlpos;  // this (request, KV head)'s arrays
  uint32_t krow16;                                  // K row stride (codes and input alike)
  uint32_t ow[16 / kAttnWaves];                     // K rows: key * krow16 + 16 c
  uint32_t ov[16 / kAttnWaves];                     // V^T: ch * n_max * 2 + 16 c
  int w, lane;

  __device__ PfCopier(const PfArgs &a, int b, int h, int w_, int lane_) : w(w_), lane(lane_) {
    const int64_t bh = (int64_t)b * a.hkv + h;
    kq = uniform(a.kq + ((int64_t)b * a.n_max * a.hkv + h) * kHeadDim);
    kin = uniform(a.k + ((int64_t)b * a.n_max * a.hkv + h) * kHeadDim);
    kvl = uniform(a.vl_k + bh * a.n_max * kHeadDim);
    vt = uniform(a.vt + bh * kHeadDim * a.n_max);
    vtq = uniform(a.vtq + bh * kHeadDim * a.n_max);
    vlvt = uniform(a.vl_vt + bh * kHeadDim * a.n_max);
    keep = uniform(a.keep + bh * a.n_max);
    vlpos = uniform(a.vl_pos + bh * a.n_max);
    krow16 = 2u * (uint32_t)a.hkv * kHeadDim;
#pragma unroll
    for (int i = 0; i < 16 / kAttnWaves; ++i) {  // 1 KB = 4 keys of 256 B
      const int key = 4 * (w + kAttnWaves * i) + (lane >> 4);
      ow[i] = (uint32_t)key * krow16 + 16u * (uint32_t)((lane & 15) ^ swz_w(key));
    }
#pragma unroll
    for (int i = 0; i < 16 / kAttnWaves; ++i) {  // 1 KB = 8 channels x 64 keys
      const int ch = 8 * (w + kAttnWaves * i) + (lane >> 3);
      ov[i] = (uint32_t)ch * (uint32_t)a.n_max * 2u + 16u * (uint32_t)((lane & 7) ^ swz_v(ch));
    }
  }

  __device__ __forceinline__ void issue(const PfPlan &pl, int sigma, PfStage &S) const {
    const uint32_t kl = lds_addr(S.k), vl = lds_addr(S.v), xl = lds_addr(S.aux);
    if (sigma < pl.n8) {  // K codes (bf16), V-hat^T, keep weights
      const int32_t k0 = sigma * kTile;
      const gbytes kb = kq + (uint64_t)k0 * krow16, vb = vtq + 2 * k0;
#pragma unroll
      for (int i = 0; i < 16 / kAttnWaves; ++i) dma_block(kl + 1024u * (w + kAttnWaves * i), kb, ow[i]);
#pragma unroll
      for (int i = 0; i < 16 / kAttnWaves; ++i) dma_block(vl + 1024u * (w + kAttnWaves * i), vb, ov[i]);
      if (w == 0 && lane < 8) dma_block(xl, keep + 2 * k0, 16u * lane);
    } else if (sigma < pl.n8 + pl.nvl) {  // gathered line rows, their V^T, positions
      const int32_t e0 = (sigma - pl.n8) * kTile;
      const gbytes kb = kvl + (uint64_t)e0 * (kHeadDim * 2), vb = vlvt + 2 * e0;
#pragma unroll
      for (int i = 0; i < 16 / kAttnWaves; ++i) {
        const int key = 4 * (w + kAttnWaves * i) + (lane >> 4);
        dma_block(kl + 1024u * (w + kAttnWaves * i), kb, (uint32_t)key * 256u + 16u * (uint32_t)((lane & 15) ^ swz_w(key)));
      }
#pragma unroll
      for (int i = 0; i < 16 / kAttnWaves; ++i) dma_block(vl + 1024u * (w + kAttnWaves * i), vb, ov[i]);
      if (w == 0 && lane < 16) dma_block(xl, vlpos + 4 * e0, 16u * lane);
    } else {  // bf16 K rows of the input, V^T, keep weights
      const int32_t k0 = (pl.w_first + sigma - pl.n8 - pl.nvl) * kTile;
      const gbytes kb = kin + (uint64_t)k0 * krow16, vb = vt + 2 * k0;
#pragma unroll
      for (int i = 0; i < 16 / kAttnWaves; ++i) dma_block(kl + 1024u * (w + kAttnWaves * i), kb, ow[i]);
#pragma unroll
      for (int i = 0; i < 16 / kAttnWaves; ++i) dma_block(vl + 1024u * (w + kAttnWaves * i), vb, ov[i]);
      if (w == 0 && lane < 8) dma_block(xl, keep + 2 * k0, 16u * lane);
    }
  }
};

// Per-lane softmax state and output accumulators of the wave's four column blocks.
// The row sums ride along as a ninth P.V tile whose A operand is the keep weight of each
// key in every row: row 0 of it (lane (col, 0), element 0) is column col's sum.
struct PfState {
  v4f acc[8][kCB];  // O^T tiles: [channel tile][column block]
  v4f sum[kCB];     // row sums
  float m[kCB];
};

enum PfKind { kInt8 = 0, kInt8Edge = 1, kLines = 2, kWindow = 3 };

__device__ __forceinline__ float col_max(float x) {  // over the 4 lanes of a column
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ uint32_t pack_f16(float lo, float hi) {  // round to nearest even
  return __builtin_bit_cast(uint32_t, h2{(_Float16)lo, (_Float16)hi});
}

// One stage (64 keys, two halves of 32) of one segment.  Lane (col, rg) of column block
// cb holds the scores of keys 32 half + 8 rg + e (e = 0 .. 7) for its query: the A
// operand row r of block u (u = 0, 1) is key 8 (r / 4) + 4 u + r % 4.
template <int kKind>
__device__ __forceinline__ void attend_stage(const PfStage &S, PfState &st, const bf8 (&qf)[kCB][4],
                                             const float (&coef)[kCB], const int32_t (&tq)[kCB], int32_t k0,
                                             int32_t window, int lane) {
  constexpr bool kMasked = kKind != kInt8;
  const int r = lane & 15, rg = lane >> 4;
  // Scores of both halves first: the second half's products run on the matrix cores
  // while the first half's softmax runs on the vector ALUs.
  v4f raw[2][2][kCB];  // [half][u][column block]
#pragma unroll
  for (int half = 0; half < 2; ++half)
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int key = 32 * half + 8 * (r >> 2) + 4 * u + (r & 3);
      bf8 ka[4];
#pragma unroll
      for (int m = 0; m < 4; ++m)
        ka[m] = *reinterpret_cast<const bf8 *>(S.k + key * 256 + 16 * ((4 * m + rg) ^ swz_w(key)));
#pragma unroll
      for (int cb = 0; cb < kCB; ++cb) {
        v4f sf = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < 4; ++m) sf = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[m], qf[cb][m], sf, 0, 0, 0);
        raw[half][u][cb] = sf;
      }
    }
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    float x[kCB][8];
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb)
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i) x[cb][4 * u + i] = raw[half][u][cb][i];
    // Side data of this lane's 8 keys: keep weights (INT8 and window stages; the A
    // operand of the row-sum tile), or positions (line stages).
    const int e0 = 32 * half + 8 * rg;
    h8 keep8;
    int32_t pos8[8];
    if constexpr (kKind == kLines) {
      const v4i p0 = *reinterpret_cast<const v4i *>(S.aux + e0), p1 = *reinterpret_cast<const v4i *>(S.aux + e0 + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pos8[e] = p0[e];
        pos8[4 + e] = p1[e];
      }
      keep8 = h8{1, 1, 1, 1, 1, 1, 1, 1};  // masked entries weigh 0 already
    } else {
      keep8 = *reinterpret_cast<const h8 *>(reinterpret_cast<const uint8_t *>(S.aux) + 2 * e0);
    }
    if constexpr (kMasked) {
#pragma unroll
      for (int cb = 0; cb < kCB; ++cb)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int32_t key = k0 + e0 + e;
          bool ok;
          if constexpr (kKind == kInt8Edge) ok = key <= tq[cb] - window;
          else if constexpr (kKind == kLines) ok = pos8[e] <= tq[cb];
          else ok = key <= tq[cb] && key > tq[cb] - window && keep8[e] > (_Float16)0;
          x[cb][e] = ok ? x[cb][e] : -INFINITY;
        }
    }
    // The running maximum moves only when a score passes it by more than kLazy: each
    // lane tests its own 8 scores (coef >= FLT_MIN, so -inf stays -inf), and only then
    // do the 4 lanes of a column agree on its new maximum.
    float lmax[kCB];
    bool grow = false;
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb) {
      float mx = __builtin_fmaxf(__builtin_fmaxf(x[cb][0], x[cb][1]), x[cb][2]);
      mx = __builtin_fmaxf(__builtin_fmaxf(mx, x[cb][3]), x[cb][4]);
      mx = __builtin_fmaxf(__builtin_fmaxf(mx, x[cb][5]), x[cb][6]);
      mx = __builtin_fmaxf(mx, x[cb][7]);
      lmax[cb] = mx * coef[cb];
      grow |= lmax[cb] > st.m[cb] + kLazy;
    }
    if (__any(grow)) {
#pragma unroll
      for (int cb = 0; cb < kCB; ++cb) {
        const float mn = fmaxf(st.m[cb], col_max(lmax[cb]));
        const float al = __builtin_amdgcn_exp2f(st.m[cb] - mn);
        st.m[cb] = mn;
        st.sum[cb] *= al;
        // One tile at a time: the accumulators stay in the matrix registers, with a
        // few temporaries, instead of all moving out at once.
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) {
          st.acc[ct][cb] *= al;
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    // Weights: p = 2^(x coef - m), fp16 for P.V and the row sums; INT8 keys enter the
    // row sum through the keep weights (their lines' and dead keys' V columns are 0).
    h8 pw[kCB];
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb) {
      float p[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) p[e] = __builtin_amdgcn_exp2f(fmaf(x[cb][e], coef[cb], -st.m[cb]));
      pw[cb] = __builtin_bit_cast(h8, make_uint4(pack_f16(p[0], p[1]), pack_f16(p[2], p[3]), pack_f16(p[4], p[5]),
                                                 pack_f16(p[6], p[7])));
    }
    // O^T += V^T P^T: lane (channel row r, key group rg) reads keys 32 half + 8 rg ...+7.
    h8 va[8];
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) {
      const int ch = 16 * ct + r;
      va[ct] = *reinterpret_cast<const h8 *>(S.v + ch * 128 + 16 * ((4 * half + rg) ^ swz_v(ch)));
    }
#pragma unroll
    for (int ct = 0; ct < 8; ++ct)
#pragma unroll
      for (int cb = 0; cb < kCB; ++cb) st.acc[ct][cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va[ct], pw[cb], st.acc[ct][cb], 0, 0, 0);
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb) st.sum[cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(keep8, pw[cb], st.sum[cb], 0, 0, 0);
  }
}

__global__ void __launch_bounds__(kAttnThreads, 2) pf_attn_kernel(PfArgs a) {
  __shared__ PfStage stage[kRing];
  const int tid = threadIdx.x, lane = tid & 63, col = lane & 15, rg = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, in a scalar register
  const int n_bh = a.batch * a.hkv;
  const int hw = a.g / a.hsplit;                       // query heads per work group
  const int per_head = kColBlocks / hw;                // column blocks per query head
  const int qp = 16 * per_head;                        // positions per work group
  const int n_blk = (a.n_max + qp - 1) / qp;
  const int rest = (int)(blockIdx.x / n_bh), hs = rest % a.hsplit;
  const int blk = n_blk - 1 - rest / a.hsplit;         // longest rows first
  const int bh = (int)(blockIdx.x % n_bh), b = bh / a.hkv, h = bh % a.hkv;
  const int32_t p0 = blk * qp;
  int32_t n = checked_n(a, b);
  if (n < 0) n = 0;
  // Column blocks kCB w + c: query head h g + hs hw + hg, positions pos0 .. pos0 + 15.
  int32_t tq[kCB], jq[kCB], pos0[kCB];
#pragma unroll
  for (int c = 0; c < kCB; ++c) {
    const int cbg = kCB * w + c;
    jq[c] = h * a.g + hs * hw + cbg / per_head;
    pos0[c] = p0 + 16 * (cbg % per_head);
    tq[c] = pos0[c] + col;
  }
  auto store = [&](int c, const float *vals) {
    const int32_t t = tq[c];
    if (t >= a.n_max) return;
    float *o = a.out + (((int64_t)b * a.n_max + t) * a.hq + jq[c]) * kHeadDim + 4 * rg;
#pragma unroll
    for (int ct = 0; ct < 8; ++ct)
      *reinterpret_cast<float4 *>(o + 16 * ct) = make_float4(vals[4 * ct], vals[4 * ct + 1], vals[4 * ct + 2], vals[4 * ct + 3]);
  };
  if (p0 >= n) {
    float zero[32] = {};
#pragma unroll
    for (int c = 0; c < kCB; ++c) store(c, zero);
    return;
  }
  const int32_t kmax = min(p0 + qp, n) - 1;  // the last key any live row reads
  PfPlan pl;
  const int32_t q_hi = kmax - a.window;       // the last INT8 key
  pl.n8 = q_hi >= 0 ? q_hi / kTile + 1 : 0;
  pl.n8_clean = min(pl.n8, max(p0 - a.window + 1, 0) / kTile);
  // (clamped, so that a list left by another call cannot send the copies past it)
  pl.nvl = a.cls ? (min(max(a.vl_cnt[(int64_t)bh * a.tiles + kmax / kTile], 0), a.n_max) + kTile - 1) / kTile : 0;
  pl.w_first = max(p0 - a.window + 1, 0) / kTile;
  pl.nwin = a.window > 0 ? kmax / kTile - pl.w_first + 1 : 0;
  const int total = pl.n8 + pl.nvl + pl.nwin;

  PfState st;
#pragma unroll
  for (int c = 0; c < kCB; ++c) {
    st.m[c] = -1.0e30f;
    st.sum[c] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) st.acc[ct][c] = v4f{0.f, 0.f, 0.f, 0.f};
  }
  constexpr float kScale = 1.4426950408889634f * 0.08838834764831845f;  // log2(e) / sqrt(128)
  // The queries as given (bf16; 0 for rows past the request's length), for every segment.
  bf8 qf[kCB][4];
  float coef[kCB];
#pragma unroll
  for (int c = 0; c < kCB; ++c) {
    const bool live = tq[c] < n;
    const int32_t t = min(tq[c], a.n_max - 1);
    const uint16_t *row = a.q + (((int64_t)b * a.n_max + t) * a.hq + jq[c]) * kHeadDim;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint4 v = live ? *reinterpret_cast<const uint4 *>(row + 32 * m + 8 * rg) : make_uint4(0u, 0u, 0u, 0u);
      qf[c][m] = __builtin_bit_cast(bf8, v);
    }
  }
  const float *ks = a.k_scales + (int64_t)bh * a.tiles;

  const PfCopier cp(a, b, h, w, lane);
  // A wave's copies per stage: K and V^T blocks, and the side words on wave 0.  Before
  // stage s is read, only the copies of the stages after it may still be in flight.
  auto copies = [&](int sg) {
    if (sg >= total) return 0;
    return 16 / kAttnWaves + 16 / kAttnWaves + (w == 0 ? 1 : 0);
  };
  auto wait_for = [&](int sg) {
    int later = 0;
#pragma unroll
    for (int i = 1; i < kRing - 1; ++i) later += copies(sg + i);
    switch (later) {
#define KVQ_WAIT(N) case N: asm volatile("s_waitcnt vmcnt(" #N ")" ::: "memory"); break;
      KVQ_WAIT(1) KVQ_WAIT(2) KVQ_WAIT(3) KVQ_WAIT(4) KVQ_WAIT(5) KVQ_WAIT(6) KVQ_WAIT(7) KVQ_WAIT(8)
      KVQ_WAIT(9) KVQ_WAIT(10) KVQ_WAIT(11) KVQ_WAIT(12) KVQ_WAIT(13) KVQ_WAIT(14) KVQ_WAIT(15) KVQ_WAIT(16)
#undef KVQ_WAIT
      default: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    }
    __syncthreads();
    if (sg + kRing - 1 < total) cp.issue(pl, sg + kRing - 1, stage[(sg + kRing - 1) % kRing]);
  };
#pragma unroll
  for (int i = 0; i < kRing - 1; ++i)
    if (i < total) cp.issue(pl, i, stage[i]);
  int sigma = 0;
  // INT8 stages: first those whose keys every row reads in INT8, then the ones that
  // reach the window.
  // Two stages a pass (stage 2i in LDS stage 0, 2i + 1 in LDS stage 1), so that every
  // LDS address is a lane base plus a constant.
  // The logit of an INT8 key is s_K (q . code) / sqrt(128): the tile's scale joins the
  // softmax scale (kept >= FLT_MIN so that a masked -inf never meets a zero factor).
  auto clean = [&](int sg, const PfStage &S) {
    wait_for(sg);
    const float c8 = fmaxf(kScale * ks[sg], FLT_MIN);
#pragma unroll
    for (int c = 0; c < kCB; ++c) coef[c] = c8;
    attend_stage<kInt8>(S, st, qf, coef, tq, sg * kTile, a.window, lane);
  };
  for (; sigma + 1 < pl.n8_clean; sigma += 2) {
    clean(sigma, stage[0]);
    clean(sigma + 1, stage[1]);
  }
  if (sigma < pl.n8_clean) {
    clean(sigma, stage[0]);
    ++sigma;
  }
  for (; sigma < pl.n8; ++sigma) {
    wait_for(sigma);
    const float c8 = fmaxf(kScale * ks[sigma], FLT_MIN);
#pragma unroll
    for (int c = 0; c < kCB; ++c) coef[c] = c8;
    attend_stage<kInt8Edge>(stage[sigma % kRing], st, qf, coef, tq, sigma * kTile, a.window, lane);
  }
  // Full-precision segments.
#pragma unroll
  for (int c = 0; c < kCB; ++c) coef[c] = kScale;
  for (; sigma < pl.n8 + pl.nvl; ++sigma) {
    wait_for(sigma);
    attend_stage<kLines>(stage[sigma % kRing], st, qf, coef, tq, 0, a.window, lane);
  }
  for (; sigma < total; ++sigma) {
    wait_for(sigma);
    attend_stage<kWindow>(stage[sigma % kRing], st, qf, coef, tq,
                          (pl.w_first + sigma - pl.n8 - pl.nvl) * kTile, a.window, lane);
  }
#pragma unroll
  for (int c = 0; c < kCB; ++c) {
    const float l = __shfl(st.sum[c][0], col);  // lane (col, 0) holds the column's sum
    const bool live = tq[c] < n && l > 0.0f;
    const float inv = live ? 1.0f / l : 0.0f;
    float vals[32];
#pragma unroll
    for (int ct = 0; ct < 8; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i) vals[4 * ct + i] = live ? st.acc[ct][c][i] * inv : 0.0f;
    store(c, vals);
  }
}

kvq_status launched(const char *what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(KVQ_ERR_HIP, "%s launch failed: %s", what, hipGetErrorString(e));
  return KVQ_OK;
}

// Workspace regions (each 256-byte aligned), in this order: vt, vtq (fp16), keep (fp16),
// vl_pos, vl_cnt (int32), vl_k (bf16), vl_vt (fp16), kq (bf16).
struct PfLayout {
  size_t vt, vtq, keep, vl_pos, vl_cnt, vl_k, vl_vt, kq, total;
};

PfLayout pf_layout(int64_t batch, int64_t n_max, int64_t hkv) {
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t bh = (size_t)(batch * hkv), n = (size_t)n_max;
  PfLayout L;
  size_t o = 0;
  L.vt = o;
  o = up(o + bh * kHeadDim * n * 2);
  L.vtq = o;
  o = up(o + bh * kHeadDim * n * 2);
  L.keep = o;
  o = up(o + bh * n * 2);
  L.vl_pos = o;
  o = up(o + bh * n * 4);
  L.vl_cnt = o;
  o = up(o + bh * (n / kTile) * 4);
  L.vl_k = o;
  o = up(o + bh * n * kHeadDim * 2);
  L.vl_vt = o;
  o = up(o + bh * kHeadDim * n * 2);
  L.kq = o;
  o = up(o + bh * n * kHeadDim * 2);
  L.total = o;
  return L;
}

}  // namespace
}  // namespace kvq

using namespace kvq;

extern "C" size_t kvq_prefill_workspace_bytes(int32_t batch, int32_t n_max, int32_t hkv) {
  if (batch <= 0 || n_max <= 0 || hkv <= 0 || n_max % kTile) return 0;
  return pf_layout(batch, n_max, hkv).total;
}

namespace {

// Validation shared by both entry points, then the argument block.
kvq_status pf_setup(PfArgs &a, const void *q, const void *k, const void *v, int32_t dtype, int32_t batch,
                    int32_t n_max, int32_t hq, int32_t hkv, const int32_t *n_tokens, const uint8_t *token_class,
                    int32_t window, int8_t *k_codes, float *k_scales, int8_t *v_codes, float *v_scales,
                    void *workspace, size_t workspace_bytes, float *out, int32_t *dev_err, bool &empty) {
  empty = false;
  if (dtype != KVQ_BF16) return fail(KVQ_ERR_UNSUPPORTED, "prefill attention takes bf16 q, k, v");
  if (batch < 0 || n_max < 0 || n_max % kTile) return fail(KVQ_ERR_INVALID_ARG, "n_max %d: a multiple of 64", n_max);
  if (hkv <= 0 || hq <= 0 || hq % hkv) return fail(KVQ_ERR_INVALID_ARG, "hq %d is not a multiple of hkv %d", hq, hkv);
  const int32_t g = hq / hkv;
  if (g != 1 && g != 2 && g != 4 && g != 8 && g != 16)
    return fail(KVQ_ERR_UNSUPPORTED, "hq / hkv = %d: 1, 2, 4, 8 or 16 query heads per KV head", g);
  if (window < 0) return fail(KVQ_ERR_INVALID_ARG, "negative window");
  if (batch == 0 || n_max == 0) {
    empty = true;
    return KVQ_OK;
  }
  if (!k || !n_tokens || !k_scales || !workspace) return fail(KVQ_ERR_INVALID_ARG, "NULL buffer");
  // 16-byte LDS-bound copies and vector loads read q, k, v, the codes and the workspace
  // regions.
  auto misaligned = [](const void *p, uintptr_t to) { return p && (reinterpret_cast<uintptr_t>(p) & (to - 1)); };
  if (misaligned(q, 16) || misaligned(k, 16) || misaligned(v, 16) || misaligned(k_codes, 16) ||
      misaligned(v_codes, 16) || misaligned(workspace, 256))
    return fail(KVQ_ERR_INVALID_ARG, "q, k, v and the codes must be 16-byte aligned, the workspace 256-byte aligned");
  // LDS-bound loads address one (request, head)'s K rows, V^T rows and lists with 32-bit
  // byte offsets.
  if ((int64_t)n_max * hkv * kHeadDim * 2 > INT32_MAX) return fail(KVQ_ERR_UNSUPPORTED, "n_max * hkv too large");
  if ((int64_t)batch * hq > 65535 || (int64_t)batch * hkv > 65535) return fail(KVQ_ERR_UNSUPPORTED, "grid too large");
  const PfLayout L = pf_layout(batch, n_max, hkv);
  if (workspace_bytes < L.total)
    return fail(KVQ_ERR_CAPACITY, "prefill workspace of %zu bytes, %zu needed", workspace_bytes, L.total);
  uint8_t *ws = static_cast<uint8_t *>(workspace);
  a.q = static_cast<const uint16_t *>(q);
  a.k = static_cast<const uint16_t *>(k);
  a.v = static_cast<const uint16_t *>(v);
  a.cls = token_class;
  a.n_tokens = n_tokens;
  a.batch = batch;
  a.n_max = n_max;
  a.hq = hq;
  a.hkv = hkv;
  a.g = g;
  a.hsplit = g > kColBlocks ? g / kColBlocks : 1;
  a.window = window;
  a.tiles = n_max / kTile;
  a.k_codes = k_codes;
  a.v_codes = v_codes;
  a.k_scales = k_scales;
  a.v_scales = v_scales;
  a.kq = reinterpret_cast<uint16_t *>(ws + L.kq);
  a.vt = reinterpret_cast<uint16_t *>(ws + L.vt);
  a.vtq = reinterpret_cast<uint16_t *>(ws + L.vtq);
  a.keep = reinterpret_cast<uint16_t *>(ws + L.keep);
  a.vl_pos = reinterpret_cast<int32_t *>(ws + L.vl_pos);
  a.vl_cnt = reinterpret_cast<int32_t *>(ws + L.vl_cnt);
  a.vl_k = reinterpret_cast<uint16_t *>(ws + L.vl_k);
  a.vl_vt = reinterpret_cast<uint16_t *>(ws + L.vl_vt);
  a.out = out;
  a.err = dev_err;
  return KVQ_OK;
}

}  // namespace

extern "C" kvq_status kvq_prefill_prepare(const void *k, const void *v, int32_t dtype, int32_t batch, int32_t n_max,
                                          int32_t hkv, const int32_t *n_tokens, const uint8_t *token_class,
                                          int8_t *k_codes, float *k_scales, int8_t *v_codes, float *v_scales,
                                          void *workspace, size_t workspace_bytes, int32_t *dev_err, void *stream) {
  PfArgs a;
  bool empty;
  // (hq = hkv: the query heads play no part in the preparation)
  kvq_status st = pf_setup(a, nullptr, k, v, dtype, batch, n_max, hkv, hkv, n_tokens, token_class, 0, k_codes,
                           k_scales, v_codes, v_scales, workspace, workspace_bytes, nullptr, dev_err, empty);
  if (st != KVQ_OK || empty) return st;
  if (!v || !k_codes || !v_codes || !v_scales) return fail(KVQ_ERR_INVALID_ARG, "NULL buffer");
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(pf_quant_k_kernel, dim3(a.tiles, batch, hkv), dim3(256), 0, s, a);
  if ((st = launched("pf_quant_k_kernel")) != KVQ_OK) return st;
  hipLaunchKernelGGL(pf_quant_v_kernel, dim3(a.tiles, batch, hkv), dim3(256), 0, s, a);
  if ((st = launched("pf_quant_v_kernel")) != KVQ_OK) return st;
  if (token_class) {
    hipLaunchKernelGGL(pf_vl_scan_kernel, dim3(batch * hkv), dim3(kScanThreads), 0, s, a);
    if ((st = launched("pf_vl_scan_kernel")) != KVQ_OK) return st;
    hipLaunchKernelGGL(pf_vl_gather_kernel, dim3(a.tiles, batch * hkv), dim3(256), 0, s, a);
    if ((st = launched("pf_vl_gather_kernel")) != KVQ_OK) return st;
  }
  return KVQ_OK;
}

extern "C" kvq_status kvq_prefill_attn(const void *q, const void *k, int32_t dtype, int32_t batch, int32_t n_max,
                                       int32_t hq, int32_t hkv, const int32_t *n_tokens, const uint8_t *token_class,
                                       int32_t window, const float *k_scales, const void *workspace,
                                       size_t workspace_bytes, float *out, int32_t *dev_err, void *stream) {
  PfArgs a;
  bool empty;
  kvq_status st = pf_setup(a, q, k, nullptr, dtype, batch, n_max, hq, hkv, n_tokens, token_class, window, nullptr,
                           const_cast<float *>(k_scales), nullptr, nullptr, const_cast<void *>(workspace),
                           workspace_bytes, out, dev_err, empty);
  if (st != KVQ_OK || empty) return st;
  if (!q || !out) return fail(KVQ_ERR_INVALID_ARG, "NULL q or out");
  const int64_t qp = 16 * (kColBlocks / (a.g / a.hsplit));
  const int64_t n_blk = (n_max + qp - 1) / qp, groups = n_blk * a.hsplit * batch * hkv;
  if (groups > INT32_MAX) return fail(KVQ_ERR_UNSUPPORTED, "grid too large");
  hipLaunchKernelGGL(pf_attn_kernel, dim3((uint32_t)groups), dim3(kAttnThreads), 0, static_cast<hipStream_t>(stream), a);
  return launched("pf_attn_kernel");
}
