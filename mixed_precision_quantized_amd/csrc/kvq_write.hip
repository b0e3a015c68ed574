// Write path of libkvq for gfx950: quantize + pack into the INT2 / INT4 / FP16
// pools, and the phase-1 page-table reorder.
//
// Quantizer (TriAxialKV key design 3): asymmetric groups of G = 32, scale and
// zero stored as fp16: z = largest fp16 <= min, s = smallest fp16 >=
// fl32(fl32(max - z) / L), code = clamp(rint(fl32(fl32(x - z) / s)), 0, L).
// This translation unit is compiled with -ffp-contract=off and keeps fp32
// denormals, so every operation rounds exactly as IEEE fp32 does.
//
// Work mapping: one 64-lane wavefront per (token, head) for per-token groups;
// lane l owns channels 2l and 2l+1 (one load), so a 32-channel group is one 16-lane
// DPP row and its min / max four row rotations; codes are packed into words across
// 4 (INT4) or 8 (INT2) lanes by DPP as well.  One wavefront per
// (INT2 group, head) for the per-channel INT2 K groups (each lane keeps its two
// channels of all 32 tokens in registers).
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include <cstdint>

#include "kvq_internal.h"

namespace kvq {
namespace {

__device__ __forceinline__ void report(int32_t *err, int32_t bit) {
  if (err) atomicOr(err, bit);
}

// ---------------------------------------------------------------- fp16 --------

// fp16 bits -> fp32, exact (including fp16 subnormals), by integer arithmetic.
__device__ __forceinline__ float half_bits_to_float(uint32_t h) {
  const uint32_t sign = (h & 0x8000u) << 16;
  const uint32_t ex = (h >> 10) & 31u, man = h & 1023u;
  float mag;
  if (ex == 0) {
    mag = (float)man * 5.9604644775390625e-08f;  // man * 2^-24, exact
  } else {
    mag = __uint_as_float(((ex + 112u) << 23) | (man << 13));
  }
  return __uint_as_float(__float_as_uint(mag) | sign);
}

// Directed rounding of a finite fp32 value to fp16 bits: up = false gives the
// largest fp16 <= x, up = true the smallest fp16 >= x.  -0 is returned as +0.
__device__ __forceinline__ uint32_t float_to_half_directed(float x, bool up) {
  const uint32_t b = __float_as_uint(x);
  const uint32_t sign = b >> 31;
  const uint32_t a = b & 0x7fffffffu;
  if (a == 0) return 0;
  const int e = (int)(a >> 23) - 127;
  uint32_t mant = a & 0x7fffffu;
  int e_eff = e;
  if (e == -127) e_eff = -126;  // fp32 subnormal
  else mant |= 0x800000u;       // implicit bit
  uint32_t mag, lost;
  if (e_eff > 15) {
    mag = 0x7c00u;  // beyond fp16 range: only reachable when the caller's precondition fails
    lost = 0;
  } else if (e_eff >= -14) {  // fp16 normal: keep 10 fraction bits
    mag = ((uint32_t)(e_eff + 15) << 10) | ((mant >> 13) & 0x3ffu);
    lost = mant & 0x1fffu;
  } else {  // fp16 subnormal: value / 2^-24 = mant * 2^(e_eff + 1)
    const int sh = -(e_eff + 1);
    if (sh >= 32) {
      mag = 0;
      lost = mant;
    } else {
      mag = mant >> sh;
      lost = mant & ((1u << sh) - 1u);
    }
  }
  // Truncation rounded the magnitude toward zero; step away from zero when
  // the direction asks for it (a carry into the exponent field is correct).
  const bool away = lost != 0 && (up ? sign == 0 : sign == 1);
  mag += away ? 1u : 0u;
  return mag == 0 ? 0u : (mag | (sign << 15));
}

// Round-to-nearest-even fp32 -> fp16 bits (FP16 anchors).
__device__ __forceinline__ uint32_t float_to_half_rne(float x) {
  const uint32_t h = (uint32_t)__half_as_ushort(__float2half_rn(x));
  return h == 0x8000u ? 0u : h;
}

// Source values idx and idx + 1 (one lane's channel pair) in one load.
__device__ __forceinline__ float2 load_pair(const void *base, int32_t dtype, int64_t idx) {
  if (dtype == KVQ_F32) return *reinterpret_cast<const float2 *>(static_cast<const float *>(base) + idx);
  const uint32_t h = *reinterpret_cast<const uint32_t *>(static_cast<const uint16_t *>(base) + idx);
  if (dtype == KVQ_BF16) return make_float2(__uint_as_float(h << 16), __uint_as_float(h & 0xffff0000u));
  return make_float2(half_bits_to_float(h & 0xffffu), half_bits_to_float(h >> 16));
}

// DPP moves within a 16-lane row: rotation by N (every lane of the row gets the
// rotated value), shift towards lower lanes by N (lanes past the row's end read 0),
// and quad permutations.
template <int N>
__device__ __forceinline__ uint32_t row_ror(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x120 + N, 0xf, 0xf, true);
}
template <int N>
__device__ __forceinline__ uint32_t row_shl(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x100 + N, 0xf, 0xf, true);
}
template <int P>
__device__ __forceinline__ uint32_t quad_perm(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, P, 0xf, 0xf, true);
}
// Lane n of each 16-lane row to every lane of the row (n a constant once unrolled).
__device__ __forceinline__ float row_bcast(float x, int n) {
#define KVQ_BC(N) \
  case N: return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x150 + N, 0xf, 0xf, false));
  switch (n) {
    KVQ_BC(0) KVQ_BC(1) KVQ_BC(2) KVQ_BC(3) KVQ_BC(4) KVQ_BC(5) KVQ_BC(6) KVQ_BC(7)
    KVQ_BC(8) KVQ_BC(9) KVQ_BC(10) KVQ_BC(11) KVQ_BC(12) KVQ_BC(13) KVQ_BC(14)
    default: return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x150 + 15, 0xf, 0xf, false));
  }
#undef KVQ_BC
}

// Min and max over the 16 lanes of a group (one DPP row); every lane gets both.
__device__ __forceinline__ void group16_minmax(float &mn, float &mx) {
#define KVQ_STEP(N)                                                   \
  mn = fminf(mn, __uint_as_float(row_ror<N>(__float_as_uint(mn)))); \
  mx = fmaxf(mx, __uint_as_float(row_ror<N>(__float_as_uint(mx))));
  KVQ_STEP(8)
  KVQ_STEP(4)
  KVQ_STEP(2)
  KVQ_STEP(1)
#undef KVQ_STEP
}

struct Quant {
  float s, z;
  uint32_t sb, zb;
};

__device__ __forceinline__ Quant quant_params(float mn, float mx, float levels) {
  Quant q;
  q.zb = float_to_half_directed(mn, false);
  q.z = half_bits_to_float(q.zb);
  const float range = __fsub_rn(mx, q.z);
  const float step = __fdiv_rn(range, levels);
  q.sb = float_to_half_directed(step, true);
  q.s = half_bits_to_float(q.sb);
  return q;
}

// INT2 key groups (one channel over 32 tokens): the scale is rounded up further, to the
// next fp16 value whose two lowest mantissa bits are zero (at most 9 significant bits;
// a carry into the exponent field is correct), so that c s is an fp16 value for every
// code c = 0..3 and the decode can form its key operand with one fused multiply-add.
__device__ __forceinline__ Quant quant_params_k2(float mn, float mx) {
  Quant q = quant_params(mn, mx, 3.0f);
  q.sb = (q.sb + 3u) & ~3u;
  q.s = half_bits_to_float(q.sb);
  return q;
}

__device__ __forceinline__ uint32_t quant_code(float x, const Quant &q, float levels) {
  if (q.s == 0.0f) return 0;
  const float t = __fdiv_rn(__fsub_rn(x, q.z), q.s);
  const float r = fminf(fmaxf(rintf(t), 0.0f), levels);
  return (uint32_t)r;
}

__device__ __forceinline__ float canon(float x) { return x == 0.0f ? 0.0f : x; }  // -0 -> +0

struct CacheView {
  int32_t heads;
  int32_t n2, n4, n16;
  uint8_t *pool2, *pool4, *pool16;
  int32_t fp8;  // FP8 anchors instead of FP16
};

// ---------------------------------------------------------------- fp8 ---------
// OCP e4m3 code of y, |y| <= 448, rounded to nearest with ties to even (0 -> 0x00).
// Below 2^-6 the codes are multiples of 2^-9 (subnormals); in the binade 2^E they
// step by 2^(E-3), and the code of the value q 2^(E-3) (8 <= q <= 16) is 8 (E + 6) + q,
// so a carry into the next binade lands on the right code.  Scaling by powers of two
// is exact, so rintf does the only rounding.
__device__ __forceinline__ uint32_t e4m3_code(float y) {
  const float a = fabsf(y);
  uint32_t code;
  if (a < 0.015625f) {
    code = (uint32_t)rintf(a * 512.0f);
  } else {
    const int E = ilogbf(a);
    code = (uint32_t)(8 * (E + 6)) + (uint32_t)rintf(ldexpf(a, 3 - E));
  }
  return (code != 0 && y < 0.0f) ? (code | 0x80u) : code;
}

// The e of an anchor row: the smallest e >= -24 with max |x| <= 448 2^e.
__device__ __forceinline__ int fp8_exponent(float amax) {
  if (!(amax > 0.0f)) return -24;
  int E;
  (void)frexpf(amax, &E);  // amax in [2^(E-1), 2^E)
  int e = E - 9;           // 448 2^(E-10) < 2^(E-1) <= amax, so e is E - 9 or E - 8
  if (amax > ldexpf(448.0f, e)) ++e;
  return e < -24 ? -24 : e;
}

// fp16 bits of 2^e, -24 <= e <= 15.
__device__ __forceinline__ uint32_t pow2_half(int e) { return e >= -14 ? (uint32_t)(e + 15) << 10 : 1u << (e + 24); }

// One FP8 anchor row of a wavefront: lane L holds channels 2L, 2L + 1.
__device__ __forceinline__ void put_fp8_row(uint8_t *blk, int codes_at, int scales_at, int off, float x0, float x1,
                                            int lane) {
  float m = fmaxf(fabsf(x0), fabsf(x1));
  for (int d = 32; d > 0; d >>= 1) m = fmaxf(m, __shfl_xor(m, d));
  const int e = fp8_exponent(m);
  const uint32_t c0 = e4m3_code(ldexpf(x0, -e)), c1 = e4m3_code(ldexpf(x1, -e));
  *reinterpret_cast<uint16_t *>(blk + codes_at + off * 128 + 2 * lane) = (uint16_t)(c0 | (c1 << 8));
  if (lane == 0) *reinterpret_cast<uint16_t *>(blk + scales_at + off * 2) = (uint16_t)pow2_half(e);
}

__device__ __forceinline__ int page_class(const CacheView &c, int64_t p) {
  if (p < 0) return -1;
  if (p < c.n2) return KVQ_INT2;
  if (p < (int64_t)c.n2 + c.n4) return KVQ_INT4;
  if (p < (int64_t)c.n2 + c.n4 + c.n16) return KVQ_FP16;
  return -1;
}

// ---------------------------------------------------------- per-token path ----

// Packs this lane's two codes (channels 2l and 2l+1 of a row) into the row's 32-bit
// word: the word holds 32/BITS channels, so 16/BITS lanes share it; channel 2l is the
// even member of its pair (low half), 2l+1 the odd one (high half).  The first lane of
// each word stores it.
template <int BITS>
__device__ __forceinline__ void put_code_pair(uint8_t *row, uint32_t c0, uint32_t c1, int lane) {
  constexpr int kLanesPerWord = 16 / BITS;
  const int k = lane % kLanesPerWord;
  uint32_t w = (c0 << (k * BITS)) | (c1 << (16 + k * BITS));
  w |= quad_perm<0xB1>(w);  // lane ^ 1
  w |= quad_perm<0x4E>(w);  // lane ^ 2: each quad holds its 4 lanes' bits
  if (kLanesPerWord == 8) w |= row_shl<4>(w);  // the first lane of 8 adds the next quad's
  if (k == 0) *reinterpret_cast<uint32_t *>(row + (lane / kLanesPerWord) * 4) = w;
}

// Quantizes one 128-channel row (this lane: channels 2l, 2l+1) in per-token groups
// of 32 and writes codes + (scale, zero) of token `off` into a block; the metadata of
// (group g, token off) is entry off*4 + g (TOKEN_MAJOR) or g*16 + off.
template <int BITS, bool TOKEN_MAJOR>
__device__ __forceinline__ void put_token_row(uint8_t *blk, int codes_at, int meta_at, int off,
                                              float x0, float x1, int lane) {
  constexpr float kLevels = (float)((1 << BITS) - 1);
  float mn = fminf(canon(x0), canon(x1)), mx = fmaxf(canon(x0), canon(x1));
  group16_minmax(mn, mx);
  const Quant q = quant_params(mn, mx, kLevels);
  put_code_pair<BITS>(blk + codes_at + off * (kHeadDim * BITS / 8), quant_code(x0, q, kLevels),
                      quant_code(x1, q, kLevels), lane);
  if ((lane & 15) == 0) {
    const int g = lane >> 4;
    const int entry = TOKEN_MAJOR ? off * 4 + g : g * kPage + off;
    *reinterpret_cast<uint32_t *>(blk + meta_at + entry * 4) = q.sb | (q.zb << 16);
  }
}

// One wavefront per (item, head): items [0, n4) are INT4 tokens, then FP16 tokens.
__global__ void __launch_bounds__(256) append_tokens_kernel(
    CacheView c, const void *k, const void *v, int32_t dtype, int64_t n_rows, int64_t row_stride,
    int64_t head_stride,
    int32_t n4, const int32_t *rows4, const int32_t *slots4, int32_t n16, const int32_t *rows16,
    const int32_t *slots16, int32_t *err) {
  const int lane = threadIdx.x & 63;
  const int64_t work = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t total = (int64_t)(n4 + n16) * c.heads;
  if (work >= total) return;
  const int64_t item = work / c.heads;
  const int head = (int)(work % c.heads);
  const bool is4 = item < n4;
  const int32_t row = is4 ? rows4[item] : rows16[item - n4];
  const int32_t slot = is4 ? slots4[item] : slots16[item - n4];
  const int64_t page = slot >> 4;
  const int off = slot & 15;
  if (slot < 0 || row < 0 || row >= n_rows || page_class(c, page) != (is4 ? KVQ_INT4 : KVQ_FP16)) {
    if (lane == 0) report(err, KVQ_DEVERR_ID);
    return;
  }
  const int64_t src = (int64_t)row * row_stride + (int64_t)head * head_stride + 2 * lane;
  const float2 kp = load_pair(k, dtype, src), vp = load_pair(v, dtype, src);
  const float k0 = kp.x, k1 = kp.y, v0 = vp.x, v1 = vp.y;
  if (is4) {
    uint8_t *blk = c.pool4 + ((page - c.n2) * c.heads + head) * (int64_t)kI4Bytes;
    put_token_row<4, true>(blk, kI4KC, kI4KM, off, k0, k1, lane);
    put_token_row<4, false>(blk, kI4VC, kI4VM, off, v0, v1, lane);
  } else if (c.fp8) {
    uint8_t *blk = c.pool16 + ((page - c.n2 - c.n4) * c.heads + head) * (int64_t)kF8Bytes;
    put_fp8_row(blk, kF8K, kF8KS, off, k0, k1, lane);
    put_fp8_row(blk, kF8V, kF8VS, off, v0, v1, lane);
  } else {
    uint8_t *blk = c.pool16 + ((page - c.n2 - c.n4) * c.heads + head) * (int64_t)kF16Bytes;
    *reinterpret_cast<uint32_t *>(blk + kF16K + off * 256 + lane * 4) =
        float_to_half_rne(k0) | (float_to_half_rne(k1) << 16);
    *reinterpret_cast<uint32_t *>(blk + kF16V + off * 256 + lane * 4) =
        float_to_half_rne(v0) | (float_to_half_rne(v1) << 16);
  }
}

// ------------------------------------------------------------- INT2 groups ----

// One wavefront per (INT2 group, head).  K: per-channel groups across the 32
// tokens; V: per-token groups of 32 channels.
__global__ void __launch_bounds__(64) append_int2_kernel(
    CacheView c, const void *k, const void *v, int32_t dtype, int64_t n_rows, int64_t row_stride,
    int64_t head_stride,
    int32_t n_groups, const int32_t *rows2, const int32_t *pages2, int32_t *err) {
  const int lane = threadIdx.x;
  const int32_t grp = blockIdx.x / c.heads;
  const int head = blockIdx.x % c.heads;
  if (grp >= n_groups) return;
  const int64_t even = pages2[grp];
  if (page_class(c, even) != KVQ_INT2 || (even & 1) || even + 1 >= c.n2) {
    if (lane == 0) report(err, KVQ_DEVERR_PAIR);
    return;
  }
  uint8_t *blk[2];
  blk[0] = c.pool2 + (even * c.heads + head) * (int64_t)kI2Bytes;
  blk[1] = c.pool2 + ((even + 1) * c.heads + head) * (int64_t)kI2Bytes;
  const int32_t *rows = rows2 + (int64_t)grp * kGroup;

  // K, per channel: lane holds channels 2l, 2l+1 of all 32 tokens.
  float kx[kGroup][2];
  bool bad = false;
  float mn0 = 0.f, mx0 = 0.f, mn1 = 0.f, mx1 = 0.f;
#pragma unroll
  for (int t = 0; t < kGroup; ++t) {
    const int32_t r = rows[t];
    bad |= r < 0 || r >= n_rows;
    const int64_t src = (int64_t)(r < 0 || r >= n_rows ? 0 : r) * row_stride + (int64_t)head * head_stride + 2 * lane;
    const float2 kp = load_pair(k, dtype, src);
    kx[t][0] = kp.x;
    kx[t][1] = kp.y;
    const float a = canon(kx[t][0]), b = canon(kx[t][1]);
    mn0 = t ? fminf(mn0, a) : a;
    mx0 = t ? fmaxf(mx0, a) : a;
    mn1 = t ? fminf(mn1, b) : b;
    mx1 = t ? fmaxf(mx1, b) : b;
  }
  if (bad) {
    if (lane == 0) report(err, KVQ_DEVERR_ID);
    return;
  }
  const Quant q0 = quant_params_k2(mn0, mx0), q1 = quant_params_k2(mn1, mx1);
#pragma unroll
  for (int t = 0; t < kGroup; ++t)
    put_code_pair<2>(blk[t >> 4] + kI2KC + (t & 15) * 32, quant_code(kx[t][0], q0, 3.0f),
                     quant_code(kx[t][1], q1, 3.0f), lane);
  {
    // Channels 2l, 2l+1: scales and zeros of the even page (c < 64) or odd page.
    uint8_t *m = blk[lane >> 5];
    const int at = (lane & 31) * 4;
    *reinterpret_cast<uint32_t *>(m + kI2KS + at) = q0.sb | (q1.sb << 16);
    *reinterpret_cast<uint32_t *>(m + kI2KZ + at) = q0.zb | (q1.zb << 16);
  }

  // V, per token, one page (16 tokens) at a time.  The group of 32 channels (16 lanes)
  // of token t has its minimum and maximum in every lane of the group after the row
  // reduction; lane 16 g + i keeps token i's, forms its scale and zero (one of the 64
  // (token, group) pairs of the page per lane, not every pair in every lane), stores
  // them, and lends them to its group for the codes.
  const int li = lane & 15;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    float2 vx[kPage];
#pragma unroll
    for (int t = 0; t < kPage; ++t)
      vx[t] = load_pair(v, dtype, (int64_t)rows[16 * h + t] * row_stride + (int64_t)head * head_stride + 2 * lane);
    float kmn = 0.f, kmx = 0.f;
#pragma unroll
    for (int t = 0; t < kPage; ++t) {
      float mn = fminf(canon(vx[t].x), canon(vx[t].y)), mx = fmaxf(canon(vx[t].x), canon(vx[t].y));
      group16_minmax(mn, mx);
      kmn = li == t ? mn : kmn;
      kmx = li == t ? mx : kmx;
    }
    const Quant qv = quant_params(kmn, kmx, 3.0f);
    // per group (64 B) the 16 tokens' scales, then their 16 zeros: lane 16 g + t holds
    // group g, token t
    uint8_t *vm = blk[h] + kI2VM + 64 * (lane >> 4) + 2 * li;
    *reinterpret_cast<uint16_t *>(vm) = (uint16_t)qv.sb;
    *reinterpret_cast<uint16_t *>(vm + 32) = (uint16_t)qv.zb;
#pragma unroll
    for (int t = 0; t < kPage; ++t) {
      Quant q;
      q.s = row_bcast(qv.s, t);
      q.z = row_bcast(qv.z, t);
      put_code_pair<2>(blk[h] + kI2VC + t * 32, quant_code(vx[t].x, q, 3.0f), quant_code(vx[t].y, q, 3.0f), lane);
    }
  }
}

// --------------------------------------------------------------- reorder ------

// One wavefront per table: stable partition of the entries by class with ballot +
// popcount prefix sums.  The table is staged in LDS (4 B per entry) before anything is
// written, so the partitioned entries can go straight to the table in place: first
// the class counts, then the INT4 and FP16 entries to their places, then the INT2
// entries, which are also compacted at the front of the staged copy (an INT2 entry's
// place is at or before its input index, and every input of a 64-entry chunk is read
// before any lane writes) for the pair check.
__global__ void __launch_bounds__(64) reorder_kernel(CacheView c, int32_t *tables, int32_t max_entries,
                                                     const int32_t *n_entries, int32_t *class_counts,
                                                     int32_t *err) {
  extern __shared__ int32_t ent[];  // [max_entries]: the input order; then the INT2 entries in order
  const int lane = threadIdx.x;
  const int32_t t = blockIdx.x;
  int32_t *row = tables + (int64_t)t * max_entries;
  const int32_t n = n_entries[t];
  if (n < 0 || n > max_entries) {
    if (lane == 0) report(err, KVQ_DEVERR_RANGE);
    return;
  }
  bool bad = false;
  for (int32_t e = lane; e < n; e += 64) {
    ent[e] = row[e];
    bad |= page_class(c, ent[e]) < 0;
  }
  if (__any(bad)) {  // leave the table as it was
    if (lane == 0) report(err, KVQ_DEVERR_ID);
    return;
  }
  const uint64_t below = lane ? (~0ull >> (64 - lane)) : 0ull;
  int32_t counts[3] = {0, 0, 0};
  for (int32_t base = 0; base < n; base += 64) {  // each lane reads back what it staged
    const int32_t e = base + lane;
    const int cls = e < n ? page_class(c, ent[e]) : 3;
#pragma unroll
    for (int k = 0; k < 3; ++k) counts[k] += __popcll(__ballot(cls == k));
  }
  __syncthreads();  // entries are read across lanes below
  int32_t w4 = counts[0], w16 = counts[0] + counts[1];
  for (int32_t base = 0; base < n; base += 64) {
    const int32_t e = base + lane;
    const int32_t v = e < n ? ent[e] : 0;
    const int cls = e < n ? page_class(c, v) : 3;
    const uint64_t m4 = __ballot(cls == KVQ_INT4), m16 = __ballot(cls == KVQ_FP16);
    if (cls == KVQ_INT4) row[w4 + __popcll(m4 & below)] = v;
    if (cls == KVQ_FP16) row[w16 + __popcll(m16 & below)] = v;
    w4 += __popcll(m4);
    w16 += __popcll(m16);
  }
  int32_t w2 = 0;
  for (int32_t base = 0; base < n; base += 64) {
    const int32_t e = base + lane;
    const int32_t v = e < n ? ent[e] : 0;
    const bool mine = e < n && page_class(c, v) == KVQ_INT2;
    const uint64_t m2 = __ballot(mine);
    if (mine) {
      const int32_t at = w2 + __popcll(m2 & below);
      ent[at] = v;
      row[at] = v;
    }
    w2 += __popcll(m2);
  }
  __syncthreads();
  if (class_counts && lane == 0)
    for (int cls = 0; cls < 3; ++cls) class_counts[(int64_t)t * 3 + cls] = counts[cls];
  // INT2 entries must now be aligned pairs (even, even + 1).
  bool pair_bad = counts[0] & 1;
  for (int32_t e = 2 * lane; e + 1 < counts[0]; e += 128) {
    const int32_t p = ent[e];
    pair_bad |= (p & 1) || ent[e + 1] != p + 1;
  }
  if (__any(pair_bad) && lane == 0) report(err, KVQ_DEVERR_PAIR);
}

// Slot-map compaction: one wave per table streams its entries in 64-entry chunks, four
// chunks loaded at a time; a ballot over the live lanes gives each live entry its place
// (live entries so far + live lanes below).  In place: an entry only moves towards the
// front, to a position already read.  Lane h < heads keeps head h's live count, taken
// in the chunk where the head's prefix ends.
__global__ void __launch_bounds__(64) compact_slots_kernel(int32_t sentinel, int32_t heads, int32_t *tables,
                                                           int32_t max_entries, const int32_t *n_entries,
                                                           const int32_t *head_tokens, int32_t *live_tokens,
                                                           int32_t *err) {
  const int lane = threadIdx.x;
  const int32_t t = blockIdx.x;
  int32_t *row = tables + (int64_t)t * max_entries;
  const int32_t n = n_entries[t];
  const int32_t m = lane < heads ? head_tokens[(int64_t)t * heads + lane] : 0;
  if (__any(n < 0 || n > max_entries || m < 0 || m > n)) {  // leave the table as it was
    if (lane == 0) report(err, KVQ_DEVERR_RANGE);
    return;
  }
  const uint64_t below = lane ? (~0ull >> (64 - lane)) : 0ull;
  constexpr int kBatch = 4;
  int32_t w = 0, live_m = 0;
  for (int32_t base = 0; base < n; base += 64 * kBatch) {
    int32_t v[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int32_t e = base + 64 * i + lane;
      v[i] = e < n ? row[e] : sentinel;
    }
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int32_t cb = base + 64 * i;
      const bool live = cb + lane < n && v[i] != sentinel;
      const uint64_t mask = __ballot(live);
      if (m > cb && m <= cb + 64) {  // head lane's prefix ends in this chunk
        const int32_t k = m - cb;
        live_m = w + __popcll(mask & (k == 64 ? ~0ull : (1ull << k) - 1ull));
      }
      if (live) row[w + __popcll(mask & below)] = v[i];
      w += __popcll(mask);
    }
  }
  for (int32_t e = w + lane; e < n; e += 64) row[e] = sentinel;
  if (lane < heads) live_tokens[(int64_t)t * heads + lane] = live_m;
}

CacheView view_of(const kvq_cache *c) {
  CacheView v;
  v.heads = c->heads_per_page;
  v.n2 = c->n_pages[0];
  v.n4 = c->n_pages[1];
  v.n16 = c->n_pages[2];
  v.pool2 = static_cast<uint8_t *>(c->pool[0]);
  v.pool4 = static_cast<uint8_t *>(c->pool[1]);
  v.pool16 = static_cast<uint8_t *>(c->pool[2]);
  v.fp8 = c->anchor_format == KVQ_ANCHOR_FP8 ? 1 : 0;
  return v;
}

kvq_status launched(const char *what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(KVQ_ERR_HIP, "%s launch failed: %s", what, hipGetErrorString(e));
  return KVQ_OK;
}

}  // namespace
}  // namespace kvq

using namespace kvq;

extern "C" kvq_status kvq_quantize_append(const kvq_cache *c, const void *k, const void *v,
                                          int32_t src_dtype, int64_t n_rows, int64_t row_stride,
                                          int64_t head_stride,
                                          int32_t n_int4, const int32_t *int4_rows,
                                          const int32_t *int4_slots, int32_t n_int2_groups,
                                          const int32_t *int2_rows, const int32_t *int2_pages,
                                          int32_t n_fp16, const int32_t *fp16_rows,
                                          const int32_t *fp16_slots, int32_t *dev_err, void *stream) {
  kvq_status st = check_cache(c);
  if (st != KVQ_OK) return st;
  if (src_dtype < KVQ_F32 || src_dtype > KVQ_F16) return fail(KVQ_ERR_INVALID_ARG, "bad source dtype %d", src_dtype);
  if (n_int4 < 0 || n_int2_groups < 0 || n_fp16 < 0) return fail(KVQ_ERR_INVALID_ARG, "negative token count");
  if (row_stride < 0 || head_stride < 0 || n_rows < 0) return fail(KVQ_ERR_INVALID_ARG, "negative stride or row count");
  if ((n_int4 && (!int4_rows || !int4_slots)) || (n_int2_groups && (!int2_rows || !int2_pages)) ||
      (n_fp16 && (!fp16_rows || !fp16_slots)))
    return fail(KVQ_ERR_INVALID_ARG, "NULL destination list with a nonzero count");
  if ((n_int4 || n_int2_groups || n_fp16) && (!k || !v)) return fail(KVQ_ERR_INVALID_ARG, "NULL k or v");
  if (c->heads_per_page > 1 && head_stride < kHeadDim)
    return fail(KVQ_ERR_INVALID_ARG, "head_stride %lld overlaps heads", (long long)head_stride);
  const CacheView view = view_of(c);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t token_waves = (int64_t)(n_int4 + n_fp16) * c->heads_per_page;
  if (token_waves > 0) {
    const int64_t blocks = (token_waves + 3) / 4;
    if (blocks > INT32_MAX) return fail(KVQ_ERR_UNSUPPORTED, "too many tokens in one call");
    hipLaunchKernelGGL(append_tokens_kernel, dim3((uint32_t)blocks), dim3(256), 0, s, view, k, v, src_dtype,
                       n_rows, row_stride, head_stride, n_int4, int4_rows, int4_slots, n_fp16, fp16_rows,
                       fp16_slots, dev_err);
    if ((st = launched("append_tokens_kernel")) != KVQ_OK) return st;
  }
  if (n_int2_groups > 0) {
    const int64_t blocks = (int64_t)n_int2_groups * c->heads_per_page;
    if (blocks > INT32_MAX) return fail(KVQ_ERR_UNSUPPORTED, "too many INT2 groups in one call");
    hipLaunchKernelGGL(append_int2_kernel, dim3((uint32_t)blocks), dim3(64), 0, s, view, k, v, src_dtype,
                       n_rows, row_stride, head_stride, n_int2_groups, int2_rows, int2_pages, dev_err);
    if ((st = launched("append_int2_kernel")) != KVQ_OK) return st;
  }
  return KVQ_OK;
}

extern "C" kvq_status kvq_reorder_pages(const kvq_cache *c, int32_t *tables, int32_t n_tables,
                                        int32_t max_entries, const int32_t *n_entries,
                                        int32_t *class_counts, int32_t *dev_err, void *stream) {
  kvq_status st = check_cache(c);
  if (st != KVQ_OK) return st;
  if (n_tables < 0 || max_entries < 0) return fail(KVQ_ERR_INVALID_ARG, "negative table shape");
  if (n_tables == 0) return KVQ_OK;
  if (!tables || !n_entries) return fail(KVQ_ERR_INVALID_ARG, "NULL tables or n_entries");
  if (max_entries > kMaxReorderEntries)
    return fail(KVQ_ERR_UNSUPPORTED, "max_entries %d exceeds %d", max_entries, kMaxReorderEntries);
  const size_t lds = (size_t)(max_entries > 0 ? max_entries : 1) * 4;
  if (lds > 65536) {  // LDS beyond the default dynamic limit (MI355X: 160 KB per CU)
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&reorder_kernel),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return fail(KVQ_ERR_HIP, "reorder LDS of %zu bytes: %s", lds, hipGetErrorString(e));
  }
  hipLaunchKernelGGL(reorder_kernel, dim3(n_tables), dim3(64), lds, static_cast<hipStream_t>(stream), view_of(c),
                     tables, max_entries, n_entries, class_counts, dev_err);
  return launched("reorder_kernel");
}

extern "C" kvq_status kvq_compact_slots(const kvq_cache *c, int32_t *tables, int32_t n_tables,
                                        int32_t max_entries, const int32_t *n_entries,
                                        const int32_t *head_tokens, int32_t *live_tokens, int32_t *dev_err,
                                        void *stream) {
  kvq_status st = check_cache(c);
  if (st != KVQ_OK) return st;
  if (n_tables < 0 || max_entries < 0) return fail(KVQ_ERR_INVALID_ARG, "negative table shape");
  if (n_tables == 0) return KVQ_OK;
  if (!tables || !n_entries || !head_tokens || !live_tokens)
    return fail(KVQ_ERR_INVALID_ARG, "NULL tables, n_entries, head_tokens or live_tokens");
  if (c->heads_per_page > 64) return fail(KVQ_ERR_UNSUPPORTED, "more than 64 heads per table");
  hipLaunchKernelGGL(compact_slots_kernel, dim3(n_tables), dim3(64), 0, static_cast<hipStream_t>(stream),
                     c->sentinel_slot, c->heads_per_page, tables, max_entries, n_entries, head_tokens,
                     live_tokens, dev_err);
  return launched("compact_slots_kernel");
}
