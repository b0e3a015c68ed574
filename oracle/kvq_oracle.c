/*
 * kvq_oracle.c -- plain, slow CPU oracle (TEST INFRASTRUCTURE ONLY; see
 * kvq_oracle.h for the sources followed and the rules on who may use it).
 *
 * Written for clarity, not speed: every step follows the definitions on the
 * pages in their order.  Quantization is fp32 exactly as specified;
 * dequantization and attention are fp64.  Build flags: -O2 -ffp-contract=off
 * -fno-fast-math -fopenmp.
 */
#include "kvq_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

#define D 128        /* head dimension */
#define PAGE 16      /* tokens per page */
#define GRP 32       /* quantization group size G (TriAxialKV key design 3) */

/* ------------------------------------------------------------------------ */
/* fp16 values through exact fp64 scaling                                    */
/* ------------------------------------------------------------------------ */

/* Spacing of fp16 values in the binade of |x| (x != 0): 2^(lead-10), but no
 * finer than the subnormal step 2^-24. */
static double f16_quantum(double x)
{
    int e;
    frexp(fabs(x), &e);            /* |x| = f * 2^e, f in [0.5, 1) */
    int q = (e - 1) - 10;
    if (q < -24) q = -24;
    return ldexp(1.0, q);
}

static uint16_t f16_encode(double v)  /* v must be an fp16 value (or overflow) */
{
    if (v == 0.0) return 0;            /* canonical +0 */
    uint16_t sign = v < 0 ? 0x8000u : 0u;
    double a = fabs(v);
    if (a > 65504.0) return (uint16_t)(sign | 0x7c00u);
    int e;
    frexp(a, &e);
    int lead = e - 1;
    if (lead < -14)                    /* subnormal: a = m * 2^-24 */
        return (uint16_t)(sign | (uint16_t)(a / ldexp(1.0, -24)));
    uint16_t mant = (uint16_t)((a / ldexp(1.0, lead) - 1.0) * 1024.0);
    return (uint16_t)(sign | (uint16_t)((lead + 15) << 10) | mant);
}

double orc_f16_value(uint16_t h)
{
    int sign = (h >> 15) & 1, ex = (h >> 10) & 31, m = h & 1023;
    double v;
    if (ex == 0) v = ldexp((double)m, -24);
    else if (ex == 31) v = m ? NAN : INFINITY;
    else v = ldexp(1.0 + m / 1024.0, ex - 15);
    return sign ? -v : v;
}

uint16_t orc_f16_down(float x)
{
    double d = (double)x;
    if (d == 0.0) return 0;
    double q = f16_quantum(d);
    return f16_encode(floor(d / q) * q);
}

uint16_t orc_f16_up(float x)
{
    double d = (double)x;
    if (d == 0.0) return 0;
    double q = f16_quantum(d);
    return f16_encode(ceil(d / q) * q);
}

/* INT2 key scales: the smallest fp16 value >= x whose two lowest mantissa bits are
 * zero (a multiple of four units in the last place at x's fp16 exponent). */
uint16_t orc_f16_up4(float x)
{
    double d = (double)x;
    if (d == 0.0) return 0;
    double q = 4.0 * f16_quantum(d);
    return f16_encode(ceil(d / q) * q);
}

uint16_t orc_f16_nearest(float x)
{
    double d = (double)x;
    if (d == 0.0) return 0;
    double q = f16_quantum(d);
    return f16_encode(nearbyint(d / q) * q);   /* default mode: ties to even */
}

/* ------------------------------------------------------------------------ */
/* Quantizer (TriAxialKV key design 3: asymmetric groups, scale and zero)   */
/* ------------------------------------------------------------------------ */

static void quantize_with(const float *x, int32_t n, int64_t stride, int32_t bits,
                          uint16_t (*scale_up)(float), uint8_t *codes, uint16_t *scale, uint16_t *zero)
{
    const int levels = (1 << bits) - 1;
    float mn = 0.0f, mx = 0.0f;
    for (int32_t i = 0; i < n; ++i) {
        float v = x[i * stride];
        if (v == 0.0f) v = 0.0f;               /* -0 -> +0 */
        if (i == 0 || v < mn) mn = v;
        if (i == 0 || v > mx) mx = v;
    }
    uint16_t zb = orc_f16_down(mn);
    float z = (float)orc_f16_value(zb);
    float range = mx - z;                      /* fp32 subtract */
    float step = range / (float)levels;        /* fp32 correctly rounded divide */
    uint16_t sb = scale_up(step);
    float s = (float)orc_f16_value(sb);
    for (int32_t i = 0; i < n; ++i) {
        int code = 0;
        if (s != 0.0f) {
            float t = (x[i * stride] - z) / s; /* fp32 subtract, fp32 divide */
            float r = rintf(t);                /* ties to even */
            code = (int)r;
            if (code < 0) code = 0;
            if (code > levels) code = levels;
        }
        codes[i] = (uint8_t)code;
    }
    *scale = sb;
    *zero = zb;
}

void orc_quantize(const float *x, int32_t n, int64_t stride, int32_t bits,
                  uint8_t *codes, uint16_t *scale, uint16_t *zero)
{
    quantize_with(x, n, stride, bits, orc_f16_up, codes, scale, zero);
}

void orc_quantize_k2(const float *x, int32_t n, int64_t stride,
                     uint8_t *codes, uint16_t *scale, uint16_t *zero)
{
    quantize_with(x, n, stride, 2, orc_f16_up4, codes, scale, zero);
}

/* ------------------------------------------------------------------------ */
/* Byte layout of one head block of a page (written specification)          */
/* ------------------------------------------------------------------------ */
/* Code rows are sequences of little-endian 32-bit words.  With b bits per code,
 * word w holds the 32/b channels w*32/b ... (w+1)*32/b - 1; among them the
 * even-indexed ones fill the low 16 bits and the odd-indexed ones the high 16
 * bits, each half in ascending channel order, b bits per channel.
 * INT4 (2560 B): K codes [16 tok][64 B] at 0; K meta [16 tok][4 groups][scale,
 *   zero fp16] at 1024; V codes [16][64 B] at 1280; V meta [4 groups][16 tok]
 *   [scale, zero] at 2304.
 * INT2 (1536 B): K codes [16 tok][32 B] at 0; K per-channel meta of the page
 *   pair at 512: 64 fp16 scales then 64 fp16 zeros (the even page of the pair
 *   holds channels 0-63, the odd page 64-127); V codes [16 tok][32 B] at 768;
 *   V meta at 1280: per group (4 x 64 B) the 16 tokens' fp16 scales, then their
 *   16 fp16 zeros.
 * FP16 (8192 B): K [16 tok][128] fp16 at 0; V at 4096.
 * FP8 anchors (4160 B, the FP16 class of a cache with anchor_fp8): K codes
 *   [16 tok][128 B] at 0, K scales [16] fp16 at 2048, V codes [16][128 B] at
 *   2080, V scales [16] fp16 at 4128. */
enum {
    I4_KC = 0, I4_KM = 1024, I4_VC = 1280, I4_VM = 2304, I4_BYTES = 2560,
    I2_KC = 0, I2_KS = 512, I2_KZ = 640, I2_VC = 768, I2_VM = 1280, I2_BYTES = 1536,
    F16_K = 0, F16_V = 4096, F16_BYTES = 8192,
    F8_K = 0, F8_KS = 2048, F8_V = 2080, F8_VS = 4128, F8_BYTES = 4160
};

/* e4m3 by its definition: code s.EEEE.mmm is (-1)^s (1 + m/8) 2^(E-7) for E >= 1,
 * (-1)^s (m/8) 2^-6 for E = 0; the all-ones magnitude 0x7F is NaN. */
double orc_e4m3_value(uint8_t code)
{
    int E = (code >> 3) & 15, m = code & 7;
    double mag;
    if ((code & 0x7F) == 0x7F) return NAN;
    mag = E == 0 ? ldexp(m / 8.0, -6) : ldexp(1.0 + m / 8.0, E - 7);
    return (code & 0x80) ? -mag : mag;
}

/* Nearest e4m3 by trying every finite magnitude; an exact tie goes to the even
 * code (even mantissa).  Zero results are +0 (0x00). */
uint8_t orc_e4m3_nearest(double y)
{
    double a = fabs(y), best_d = INFINITY;
    int best = 0;
    for (int c = 0; c < 0x7F; ++c) {
        double d = fabs(orc_e4m3_value((uint8_t)c) - a);
        if (d < best_d || (d == best_d && (c & 1) == 0 && (best & 1) == 1)) { best_d = d; best = c; }
    }
    return (uint8_t)(best != 0 && y < 0 ? (best | 0x80) : best);
}

void orc_fp8_row(const float *x, int n, uint8_t *codes, uint16_t *scale)
{
    double amax = 0.0;
    int e = -24;
    for (int i = 0; i < n; ++i) if (fabs((double)x[i]) > amax) amax = fabs((double)x[i]);
    while (amax > ldexp(448.0, e)) ++e;
    for (int i = 0; i < n; ++i) codes[i] = orc_e4m3_nearest(ldexp((double)x[i], -e));
    *scale = orc_f16_nearest((float)ldexp(1.0, e));
}

/* Bit position of channel ch inside its code row (b bits per code). */
static int code_bit(int ch, int bits)
{
    int per_word = 32 / bits, k = ch % per_word;
    return (ch / per_word) * 32 + (k % 2) * 16 + (k / 2) * bits;
}

static int get_code(const uint8_t *row, int ch, int bits)
{
    int bit = code_bit(ch, bits);
    return (row[bit / 8] >> (bit % 8)) & ((1 << bits) - 1);
}

static void put_code(uint8_t *row, int ch, int bits, int code)
{
    int bit = code_bit(ch, bits);
    uint8_t mask = (uint8_t)(((1 << bits) - 1) << (bit % 8));
    row[bit / 8] = (uint8_t)((row[bit / 8] & ~mask) | (code << (bit % 8)));
}

int64_t orc_block_bytes(int32_t cls)
{
    return cls == ORC_INT2 ? I2_BYTES : cls == ORC_INT4 ? I4_BYTES
         : cls == ORC_FP16 ? F16_BYTES : cls == 3 ? F8_BYTES : 0;
}

static int32_t page_class(const orc_cache *c, int64_t page)
{
    int64_t n2 = c->n_pages[0], n4 = c->n_pages[1], n16 = c->n_pages[2];
    if (page < 0) return -1;
    if (page < n2) return ORC_INT2;
    if (page < n2 + n4) return ORC_INT4;
    if (page < n2 + n4 + n16) return ORC_FP16;
    return -1;
}

static int64_t class_base(const orc_cache *c, int32_t cls)
{
    int64_t b = 0;
    for (int32_t i = 0; i < cls; ++i) b += c->n_pages[i];
    return b;
}

static uint8_t *block_ptr(const orc_cache *c, int64_t page, int32_t head)
{
    int32_t cls = page_class(c, page);
    int64_t rel = page - class_base(c, cls);
    int64_t bytes = (cls == ORC_FP16 && c->anchor_fp8) ? F8_BYTES : orc_block_bytes(cls);
    return c->pool[cls] + (rel * c->heads_per_page + head) * bytes;
}

static void put_u16(uint8_t *p, uint16_t v) { p[0] = (uint8_t)(v & 255); p[1] = (uint8_t)(v >> 8); }
static uint16_t get_u16(const uint8_t *p) { return (uint16_t)(p[0] | (p[1] << 8)); }

/* Widen one source element to fp32 (exact for every supported dtype). */
static float src_value(const void *base, int32_t dtype, int64_t idx)
{
    if (dtype == ORC_F32) return ((const float *)base)[idx];
    if (dtype == ORC_BF16) {
        uint32_t b = (uint32_t)((const uint16_t *)base)[idx] << 16;
        float f;
        memcpy(&f, &b, 4);
        return f;
    }
    return (float)orc_f16_value(((const uint16_t *)base)[idx]);
}

static void load_row(float *dst, const void *src, int32_t dtype, int64_t row,
                     int64_t row_stride, int64_t head_stride, int32_t head)
{
    for (int ch = 0; ch < D; ++ch)
        dst[ch] = src_value(src, dtype, row * row_stride + head * head_stride + ch);
}

/* ------------------------------------------------------------------------ */
/* Routing                                                                   */
/* ------------------------------------------------------------------------ */

int orc_route(const uint8_t *flags, int32_t n, uint8_t *cls_out,
              int32_t *n_int2_groups, int32_t *n_int4, int32_t *n_fp16)
{
    if (n < 0 || (n > 0 && (!flags || !cls_out))) return ORC_EARG;
    int32_t want2 = 0;
    for (int32_t i = 0; i < n; ++i) {
        if (flags[i] > 2) return ORC_EARG;
        if (flags[i] == 0) ++want2;
    }
    int32_t full = (want2 / GRP) * GRP;        /* INT2 tokens that fill groups */
    int32_t seen2 = 0, c4 = 0, c16 = 0;
    for (int32_t i = 0; i < n; ++i) {
        if (flags[i] == 0) {
            cls_out[i] = seen2 < full ? ORC_INT2 : ORC_INT4;
            if (seen2 >= full) ++c4;
            ++seen2;
        } else if (flags[i] == 1) {
            cls_out[i] = ORC_INT4;
            ++c4;
        } else {
            cls_out[i] = ORC_FP16;
            ++c16;
        }
    }
    if (n_int2_groups) *n_int2_groups = full / GRP;
    if (n_int4) *n_int4 = c4;
    if (n_fp16) *n_fp16 = c16;
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Write path                                                                */
/* ------------------------------------------------------------------------ */

/* Per-token groups of 32 channels (INT4 K and V, INT2 V); the (scale, zero) of
 * (group g, token off) sits at meta_at + 4 * (off*4 + g) (META_TOKEN_MAJOR) or
 * 4 * (g*16 + off) (META_GROUP_MAJOR); META_GROUP_RUNS puts the scale at
 * meta_at + 64*g + 2*off and the zero 32 bytes after it. */
enum { META_TOKEN_MAJOR, META_GROUP_MAJOR, META_GROUP_RUNS };
static void put_token_groups(uint8_t *blk, int codes_at, int meta_at, int meta_kind, int bits,
                             int off, const float *row)
{
    const int row_bytes = D * bits / 8;
    for (int g = 0; g < D / GRP; ++g) {
        uint8_t codes[GRP];
        uint16_t s, z;
        orc_quantize(row + g * GRP, GRP, 1, bits, codes, &s, &z);
        for (int i = 0; i < GRP; ++i)
            put_code(blk + codes_at + off * row_bytes, g * GRP + i, bits, codes[i]);
        if (meta_kind == META_GROUP_RUNS) {
            put_u16(blk + meta_at + 64 * g + 2 * off, s);
            put_u16(blk + meta_at + 64 * g + 32 + 2 * off, z);
        } else {
            uint8_t *m = blk + meta_at + 4 * (meta_kind == META_TOKEN_MAJOR ? off * 4 + g : g * PAGE + off);
            put_u16(m, s);
            put_u16(m + 2, z);
        }
    }
}

int orc_append(orc_cache *c, const void *k, const void *v, int32_t dtype,
               int64_t row_stride, int64_t head_stride,
               int32_t n4, const int32_t *rows4, const int32_t *slots4,
               int32_t n2g, const int32_t *rows2, const int32_t *pages2,
               int32_t n16, const int32_t *rows16, const int32_t *slots16)
{
    if (!c || !k || !v || dtype < 0 || dtype > 2 || n4 < 0 || n2g < 0 || n16 < 0)
        return ORC_EARG;
    const int32_t H = c->heads_per_page;
    float kr[D], vr[D];

    for (int32_t i = 0; i < n4; ++i) {                 /* INT4 per-token */
        int64_t page = slots4[i] >> 4;
        int off = slots4[i] & 15;
        if (slots4[i] < 0 || page_class(c, page) != ORC_INT4) return ORC_ECLASS;
        for (int32_t h = 0; h < H; ++h) {
            uint8_t *blk = block_ptr(c, page, h);
            load_row(kr, k, dtype, rows4[i], row_stride, head_stride, h);
            load_row(vr, v, dtype, rows4[i], row_stride, head_stride, h);
            put_token_groups(blk, I4_KC, I4_KM, META_TOKEN_MAJOR, 4, off, kr);
            put_token_groups(blk, I4_VC, I4_VM, META_GROUP_MAJOR, 4, off, vr);
        }
    }

    for (int32_t g = 0; g < n2g; ++g) {                /* INT2 groups of 32 tokens */
        int64_t even = pages2[g];
        if (page_class(c, even) != ORC_INT2 || (even & 1) || even + 1 >= c->n_pages[0])
            return ORC_EPAIR;
        const int32_t *rows = rows2 + (int64_t)g * GRP;
        for (int32_t h = 0; h < H; ++h) {
            uint8_t *blk[2] = { block_ptr(c, even, h), block_ptr(c, even + 1, h) };
            /* K: one group per channel across the 32 tokens (per-channel). */
            float col[GRP];
            for (int ch = 0; ch < D; ++ch) {
                for (int t = 0; t < GRP; ++t)
                    col[t] = src_value(k, dtype, rows[t] * row_stride + h * head_stride + ch);
                uint8_t codes[GRP];
                uint16_t s, z;
                orc_quantize_k2(col, GRP, 1, codes, &s, &z);
                for (int t = 0; t < GRP; ++t)
                    put_code(blk[t / PAGE] + I2_KC + (t % PAGE) * 32, ch, 2, codes[t]);
                put_u16(blk[ch / 64] + I2_KS + (ch % 64) * 2, s);
                put_u16(blk[ch / 64] + I2_KZ + (ch % 64) * 2, z);
            }
            /* V: per-token groups. */
            for (int t = 0; t < GRP; ++t) {
                load_row(vr, v, dtype, rows[t], row_stride, head_stride, h);
                put_token_groups(blk[t / PAGE], I2_VC, I2_VM, META_GROUP_RUNS, 2, t % PAGE, vr);
            }
        }
    }

    for (int32_t i = 0; i < n16; ++i) {                /* FP16 anchors */
        int64_t page = slots16[i] >> 4;
        int off = slots16[i] & 15;
        if (slots16[i] < 0 || page_class(c, page) != ORC_FP16) return ORC_ECLASS;
        for (int32_t h = 0; h < H; ++h) {
            uint8_t *blk = block_ptr(c, page, h);
            load_row(kr, k, dtype, rows16[i], row_stride, head_stride, h);
            load_row(vr, v, dtype, rows16[i], row_stride, head_stride, h);
            if (c->anchor_fp8) {
                uint16_t ks, vs;
                orc_fp8_row(kr, D, blk + F8_K + off * 128, &ks);
                orc_fp8_row(vr, D, blk + F8_V + off * 128, &vs);
                put_u16(blk + F8_KS + off * 2, ks);
                put_u16(blk + F8_VS + off * 2, vs);
                continue;
            }
            for (int ch = 0; ch < D; ++ch) {
                put_u16(blk + F16_K + off * 256 + ch * 2, orc_f16_nearest(kr[ch]));
                put_u16(blk + F16_V + off * 256 + ch * 2, orc_f16_nearest(vr[ch]));
            }
        }
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Page-table reorder (phase 1)                                              */
/* ------------------------------------------------------------------------ */

int orc_reorder(const orc_cache *c, int32_t *tables, int32_t n_tables,
                int32_t max_entries, const int32_t *n_entries,
                int32_t *class_counts)
{
    if (!c || !tables || !n_entries || n_tables < 0 || max_entries < 0) return ORC_EARG;
    int32_t *tmp = (int32_t *)malloc(sizeof(int32_t) * (size_t)(max_entries > 0 ? max_entries : 1));
    int rc = ORC_OK;
    for (int32_t t = 0; t < n_tables && rc == ORC_OK; ++t) {
        int32_t n = n_entries[t];
        int32_t *row = tables + (int64_t)t * max_entries;
        if (n < 0 || n > max_entries) { rc = ORC_EARG; break; }
        int32_t cnt[3] = { 0, 0, 0 }, w = 0;
        for (int32_t cls = 0; cls < 3; ++cls)          /* stable: keep order within a class */
            for (int32_t e = 0; e < n; ++e) {
                int32_t pc = page_class(c, row[e]);
                if (pc < 0) { rc = ORC_ECLASS; break; }
                if (pc == cls) { tmp[w++] = row[e]; ++cnt[cls]; }
            }
        if (rc != ORC_OK) break;
        memcpy(row, tmp, sizeof(int32_t) * (size_t)n);
        for (int32_t e = 0; e < cnt[0]; e += 2)         /* INT2 entries are aligned pairs */
            if (e + 1 >= cnt[0] || (row[e] & 1) || row[e + 1] != row[e] + 1) { rc = ORC_EPAIR; break; }
        if (class_counts)
            for (int cls = 0; cls < 3; ++cls) class_counts[t * 3 + cls] = cnt[cls];
    }
    free(tmp);
    return rc;
}

/* ------------------------------------------------------------------------ */
/* Slot-map compaction                                                       */
/* ------------------------------------------------------------------------ */

int orc_compact_slots(const orc_cache *c, int32_t *tables, int32_t n_tables,
                      int32_t max_entries, const int32_t *n_entries,
                      const int32_t *head_tokens, int32_t heads,
                      int32_t *live_tokens)
{
    if (!c || !tables || !n_entries || !head_tokens || !live_tokens || n_tables < 0 ||
        max_entries < 0 || heads <= 0)
        return ORC_EARG;
    const int32_t dead = c->sentinel_slot;
    for (int32_t t = 0; t < n_tables; ++t) {
        int32_t n = n_entries[t];
        int32_t *row = tables + (int64_t)t * max_entries;
        if (n < 0 || n > max_entries) return ORC_EARG;
        for (int32_t h = 0; h < heads; ++h) {     /* live entries among the head's prefix */
            int32_t m = head_tokens[t * heads + h], live = 0;
            if (m < 0 || m > n) return ORC_ERANGE;
            for (int32_t e = 0; e < m; ++e)
                if (row[e] != dead) ++live;
            live_tokens[t * heads + h] = live;
        }
        int32_t w = 0;                             /* stable: live entries in their order */
        for (int32_t e = 0; e < n; ++e)
            if (row[e] != dead) row[w++] = row[e];
        for (int32_t e = w; e < n; ++e) row[e] = dead;
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Vertical-line selection (HyQuant Algorithm 1) and FREEZE routing (Alg. 4) */
/* ------------------------------------------------------------------------ */

static const double *g_sort_scores;  /* qsort has no context argument */

static int by_score_then_index(const void *a, const void *b)
{
    int32_t i = *(const int32_t *)a, j = *(const int32_t *)b;
    double si = g_sort_scores[i], sj = g_sort_scores[j];
    if (si > sj) return -1;
    if (si < sj) return 1;
    return (i > j) - (i < j);
}

int orc_select_vl(const float *k, const float *q_tail, int32_t batch,
                  int32_t max_tokens, int32_t hkv, int32_t hq, int32_t max_tail,
                  const int32_t *n_tokens, const int32_t *n_tail, int32_t window,
                  double rho, double *scores, uint8_t *cls, int32_t *n_vl)
{
    if (!k || !q_tail || !n_tokens || !n_tail || !scores || !cls || !n_vl || batch < 0 ||
        max_tokens < 0 || hkv <= 0 || hq <= 0 || hq % hkv || max_tail <= 0 || window < 0 ||
        !(rho >= 0.0 && rho <= 1.0))
        return ORC_EARG;
    const int32_t g = hq / hkv;
    int32_t *order = (int32_t *)malloc(sizeof(int32_t) * (size_t)(max_tokens > 0 ? max_tokens : 1));
    for (int32_t b = 0; b < batch; ++b) {
        const int32_t n = n_tokens[b], nt = n_tail[b];
        if (n < 0 || n > max_tokens || nt < 0 || nt > max_tail) { free(order); return ORC_ERANGE; }
        for (int32_t h = 0; h < hkv; ++h) {
            double u[D];                              /* tail-query proxy of the group */
            for (int c = 0; c < D; ++c) {
                double sum = 0.0;
                for (int32_t j = 0; j < g; ++j)
                    for (int32_t i = 0; i < nt; ++i)
                        sum += q_tail[(((int64_t)b * max_tail + i) * hq + h * g + j) * D + c];
                u[c] = nt > 0 ? sum / nt : 0.0;
            }
            const int64_t row = ((int64_t)b * hkv + h) * max_tokens;
            for (int32_t t = 0; t < max_tokens; ++t) {
                double s = 0.0;
                if (t < n)
                    for (int c = 0; c < D; ++c)
                        s += u[c] * k[(((int64_t)b * max_tokens + t) * hkv + h) * D + c];
                scores[row + t] = s;
                cls[row + t] = (t < n && t >= n - window) ? 2 : 0;
            }
            const int32_t n_pre = n - window > 0 ? n - window : 0;
            const int32_t m = (int32_t)floor(rho * n_pre + 0.5);
            for (int32_t t = 0; t < n_pre; ++t) order[t] = t;
            g_sort_scores = scores + row;
            qsort(order, (size_t)n_pre, sizeof(int32_t), by_score_then_index);
            for (int32_t r = 0; r < m; ++r) cls[row + order[r]] = 1;
            n_vl[b * hkv + h] = m;
        }
    }
    free(order);
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Prefill attention with an INT8 prefix (HyQuant: the fused operator of the */
/* core method, and Algorithm 2)                                             */
/* ------------------------------------------------------------------------ */

#define QTILE 64

/* Symmetric INT8 scale of a tile: fp32 max |x| / c_B with c_B = 127 (no contraction:
 * -ffp-contract=off). */
static float int8_scale(float amax)
{
    volatile float q = amax / 127.0f;
    return q;
}

static int8_t int8_code(float x, float s)
{
    if (s == 0.0f) return 0;
    volatile float r = x / s;
    float c = rintf(r);
    if (c > 127.0f) c = 127.0f;
    if (c < -127.0f) c = -127.0f;
    return (int8_t)c;
}

#define QI(b, t, j, c) ((((int64_t)(b) * n_max + (t)) * hq + (j)) * D + (c))
#define KI(b, t, h, c) ((((int64_t)(b) * n_max + (t)) * hkv + (h)) * D + (c))

/* The quantized prefix of one tensor (K or V): per request, 64-position tile and KV
 * head, the tile scale over the live positions that are not vertical lines, and every
 * live position's codes (vertical lines too, clamped; they are never read through
 * INT8).  Positions at or past the request's length get code 0. */
static void prefill_quantize(const float *x, int32_t batch, int32_t n_max, int32_t hkv,
                             const int32_t *n_tokens, const uint8_t *cls, int8_t *codes, float *scales)
{
    const int32_t tiles = (n_max + QTILE - 1) / QTILE;
    for (int32_t b = 0; b < batch; ++b) {
        const int32_t n = n_tokens[b];
        for (int32_t tile = 0; tile < tiles; ++tile) {
            const int32_t t0 = tile * QTILE, t1 = t0 + QTILE < n ? t0 + QTILE : n;
            for (int32_t h = 0; h < hkv; ++h) {
                const uint8_t *vl = cls ? cls + ((int64_t)b * hkv + h) * n_max : NULL;
                float amax = 0.0f;
                for (int32_t t = t0; t < t1; ++t)
                    if (!(vl && vl[t] == 1))
                        for (int c = 0; c < D; ++c) amax = fmaxf(amax, fabsf(x[KI(b, t, h, c)]));
                const float s = int8_scale(amax);
                scales[((int64_t)b * hkv + h) * tiles + tile] = s;
                for (int32_t t = t0; t < t0 + QTILE && t < n_max; ++t)
                    for (int c = 0; c < D; ++c)
                        codes[KI(b, t, h, c)] = t < n ? int8_code(x[KI(b, t, h, c)], s) : 0;
            }
        }
    }
}

/* One output row (request b, position t < n, query head j): one softmax over the keys
 * kk <= t.  A key that is a vertical line of the head or lies in the window
 * kk > t - window is read in full precision (K and V as given); every other key is
 * read through its tile's INT8 codes, K-hat = s_K code_K and V-hat = s_V code_V.  The
 * query is used as given.  x: scratch of t + 1 doubles. */
static void prefill_row(const float *q, const float *k, const float *v, int32_t n_max, int32_t hq, int32_t hkv,
                        const uint8_t *cls, int32_t window, const int8_t *k_codes, const float *k_scales,
                        const int8_t *v_codes, const float *v_scales, int32_t b, int32_t t, int32_t j, double *x,
                        double *o)
{
    const int32_t g = hq / hkv, h = j / g, tiles = (n_max + QTILE - 1) / QTILE;
    const uint8_t *vl = cls ? cls + ((int64_t)b * hkv + h) * n_max : NULL;
    const double inv_sqrt_d = 1.0 / sqrt((double)D);
    double mx = -INFINITY;
    for (int c = 0; c < D; ++c) o[c] = 0.0;
    for (int32_t kk = 0; kk <= t; ++kk) {
        const int full = (vl && vl[kk] == 1) || kk > t - window;
        const double sk = k_scales[((int64_t)b * hkv + h) * tiles + kk / QTILE];
        double dot = 0.0;
        for (int c = 0; c < D; ++c) {
            const double kv = full ? (double)k[KI(b, kk, h, c)] : sk * (double)k_codes[KI(b, kk, h, c)];
            dot += (double)q[QI(b, t, j, c)] * kv;
        }
        x[kk] = dot * inv_sqrt_d;
        if (x[kk] > mx) mx = x[kk];
    }
    double den = 0.0;
    for (int32_t kk = 0; kk <= t; ++kk) den += exp(x[kk] - mx);
    for (int32_t kk = 0; kk <= t; ++kk) {
        const int full = (vl && vl[kk] == 1) || kk > t - window;
        const double sv = v_scales[((int64_t)b * hkv + h) * tiles + kk / QTILE];
        const double p = exp(x[kk] - mx) / den;
        for (int c = 0; c < D; ++c) {
            const double vv = full ? (double)v[KI(b, kk, h, c)] : sv * (double)v_codes[KI(b, kk, h, c)];
            o[c] += p * vv;
        }
    }
}

static int prefill_args_ok(const float *q, const float *k, const float *v, int32_t batch, int32_t n_max,
                           int32_t hq, int32_t hkv, const int32_t *n_tokens, int32_t window)
{
    if (!q || !k || !v || !n_tokens || batch < 0 || n_max < 0 || hq <= 0 || hkv <= 0 || hq % hkv || window < 0)
        return ORC_EARG;
    for (int32_t b = 0; b < batch; ++b)
        if (n_tokens[b] < 0 || n_tokens[b] > n_max) return ORC_ERANGE;
    return ORC_OK;
}

int orc_prefill_attend(const float *q, const float *k, const float *v,
                       int32_t batch, int32_t n_max, int32_t hq, int32_t hkv,
                       const int32_t *n_tokens, const uint8_t *cls, int32_t window,
                       double *out, int8_t *k_codes, float *k_scales,
                       int8_t *v_codes, float *v_scales)
{
    int rc = prefill_args_ok(q, k, v, batch, n_max, hq, hkv, n_tokens, window);
    if (rc != ORC_OK) return rc;
    if (!out || !k_codes || !k_scales || !v_codes || !v_scales) return ORC_EARG;
    prefill_quantize(k, batch, n_max, hkv, n_tokens, cls, k_codes, k_scales);
    prefill_quantize(v, batch, n_max, hkv, n_tokens, cls, v_codes, v_scales);
    double *x = (double *)malloc(sizeof(double) * (size_t)(n_max > 0 ? n_max : 1));
    for (int32_t b = 0; b < batch; ++b)
        for (int32_t t = 0; t < n_max; ++t)
            for (int32_t j = 0; j < hq; ++j) {
                double *o = out + QI(b, t, j, 0);
                if (t >= n_tokens[b]) {
                    for (int c = 0; c < D; ++c) o[c] = 0.0;
                    continue;
                }
                prefill_row(q, k, v, n_max, hq, hkv, cls, window, k_codes, k_scales, v_codes, v_scales, b, t, j, x, o);
            }
    free(x);
    return ORC_OK;
}

int orc_prefill_attend_rows(const float *q, const float *k, const float *v,
                            int32_t batch, int32_t n_max, int32_t hq, int32_t hkv,
                            const int32_t *n_tokens, const uint8_t *cls, int32_t window,
                            int32_t n_rows, const int32_t *row_b, const int32_t *row_t, double *out_rows,
                            int8_t *k_codes, float *k_scales, int8_t *v_codes, float *v_scales)
{
    int rc = prefill_args_ok(q, k, v, batch, n_max, hq, hkv, n_tokens, window);
    if (rc != ORC_OK) return rc;
    if (n_rows < 0 || (n_rows > 0 && (!row_b || !row_t || !out_rows)) || !k_codes || !k_scales || !v_codes ||
        !v_scales)
        return ORC_EARG;
    for (int32_t r = 0; r < n_rows; ++r)
        if (row_b[r] < 0 || row_b[r] >= batch || row_t[r] < 0 || row_t[r] >= n_tokens[row_b[r]]) return ORC_ERANGE;
    prefill_quantize(k, batch, n_max, hkv, n_tokens, cls, k_codes, k_scales);
    prefill_quantize(v, batch, n_max, hkv, n_tokens, cls, v_codes, v_scales);
#pragma omp parallel for schedule(dynamic)
    for (int32_t r = 0; r < n_rows; ++r) {
        double *x = (double *)malloc(sizeof(double) * (size_t)(row_t[r] + 1));
        for (int32_t j = 0; j < hq; ++j)
            prefill_row(q, k, v, n_max, hq, hkv, cls, window, k_codes, k_scales, v_codes, v_scales, row_b[r],
                        row_t[r], j, x, out_rows + ((int64_t)r * hq + j) * D);
        free(x);
    }
    return ORC_OK;
}
#undef QI
#undef KI

/* ------------------------------------------------------------------------ */
/* Dequantization of one token (fp64, exact)                                 */
/* ------------------------------------------------------------------------ */

static double deq(uint16_t s, uint16_t z, int code)
{
    return orc_f16_value(z) + code * orc_f16_value(s);
}

int orc_token(const orc_cache *c, int32_t page, int32_t off, int32_t head,
              double *k, double *v)
{
    int32_t cls = page_class(c, page);
    if (cls < 0 || off < 0 || off >= PAGE || head < 0 || head >= c->heads_per_page)
        return ORC_ERANGE;
    const uint8_t *blk = block_ptr(c, page, head);
    for (int ch = 0; ch < D; ++ch) {
        int g = ch / GRP;
        if (cls == ORC_INT4) {
            const uint8_t *km = blk + I4_KM + (off * 4 + g) * 4;
            const uint8_t *vm = blk + I4_VM + (g * PAGE + off) * 4;
            k[ch] = deq(get_u16(km), get_u16(km + 2), get_code(blk + I4_KC + off * 64, ch, 4));
            v[ch] = deq(get_u16(vm), get_u16(vm + 2), get_code(blk + I4_VC + off * 64, ch, 4));
        } else if (cls == ORC_INT2) {
            int32_t even = page & ~1;               /* INT2 ids start at 0 */
            const uint8_t *mblk = block_ptr(c, even + ch / 64, head);
            const uint8_t *vs = blk + I2_VM + g * 64 + off * 2;   /* the zero 32 bytes on */
            k[ch] = deq(get_u16(mblk + I2_KS + (ch % 64) * 2), get_u16(mblk + I2_KZ + (ch % 64) * 2),
                        get_code(blk + I2_KC + off * 32, ch, 2));
            v[ch] = deq(get_u16(vs), get_u16(vs + 32), get_code(blk + I2_VC + off * 32, ch, 2));
        } else if (c->anchor_fp8) {
            k[ch] = orc_e4m3_value(blk[F8_K + off * 128 + ch]) * orc_f16_value(get_u16(blk + F8_KS + off * 2));
            v[ch] = orc_e4m3_value(blk[F8_V + off * 128 + ch]) * orc_f16_value(get_u16(blk + F8_VS + off * 2));
        } else {
            k[ch] = orc_f16_value(get_u16(blk + F16_K + off * 256 + ch * 2));
            v[ch] = orc_f16_value(get_u16(blk + F16_V + off * 256 + ch * 2));
        }
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Attention by definition (HyQuant background: softmax(q k^T / sqrt(d)) v)  */
/* ------------------------------------------------------------------------ */

typedef struct { const orc_cache *c; const int32_t *row; int32_t max_entries, kind, head; } src_t;

/* Resolve token t of a range: 1 = live (page, off), 0 = dead, <0 = error. */
static int resolve(const src_t *s, int32_t cls, int32_t t, int32_t *page, int32_t *off)
{
    int32_t id;
    if (s->kind == ORC_PAGES) {
        if (t < 0 || (t >> 4) >= s->max_entries) return ORC_ERANGE;
        *page = s->row[t >> 4];
        *off = t & 15;
    } else {
        if (t < 0 || t >= s->max_entries) return ORC_ERANGE;
        id = s->row[t];
        if (s->c->sentinel_slot >= 0 && id == s->c->sentinel_slot) return 0;
        if (id < 0) return ORC_ERANGE;
        *page = id >> 4;
        *off = id & 15;
    }
    if (page_class(s->c, *page) != cls) return ORC_ECLASS;
    return 1;
}

/* g queries (fp64 [g][128]) over the live tokens of ranges rs[0..nr-1]. */
static int attend_core(const src_t *s, const double *q, int g,
                       const orc_range *const *rs, int nr,
                       double *out, double *lse)
{
    const double inv_sqrt_d = 1.0 / sqrt((double)D);
    int64_t n_tok = 0;
    for (int r = 0; r < nr; ++r) n_tok += rs[r]->tok_end - rs[r]->tok_begin;
    double *x = (double *)malloc(sizeof(double) * (size_t)(n_tok > 0 ? n_tok : 1) * (size_t)g);
    double *m = (double *)malloc(sizeof(double) * (size_t)g);
    double *sum = (double *)calloc((size_t)g, sizeof(double));
    double kk[D], vv[D];
    int rc = ORC_OK;
    for (int j = 0; j < g; ++j) m[j] = -INFINITY;
    memset(out, 0, sizeof(double) * (size_t)g * D);

    int64_t live = 0;                      /* pass 1: logits and their max */
    for (int r = 0; r < nr && rc == ORC_OK; ++r)
        for (int32_t t = rs[r]->tok_begin; t < rs[r]->tok_end; ++t) {
            int32_t page, off;
            int st = resolve(s, rs[r]->cls, t, &page, &off);
            if (st < 0) { rc = st; break; }
            if (st == 0) continue;
            orc_token(s->c, page, off, s->head, kk, vv);
            for (int j = 0; j < g; ++j) {
                double dot = 0.0;
                for (int ch = 0; ch < D; ++ch) dot += q[j * D + ch] * kk[ch];
                double xj = dot * inv_sqrt_d;
                x[live * g + j] = xj;
                if (xj > m[j]) m[j] = xj;
            }
            ++live;
        }

    live = 0;                              /* pass 2: weights and weighted values */
    for (int r = 0; r < nr && rc == ORC_OK; ++r)
        for (int32_t t = rs[r]->tok_begin; t < rs[r]->tok_end; ++t) {
            int32_t page, off;
            int st = resolve(s, rs[r]->cls, t, &page, &off);
            if (st <= 0) continue;
            orc_token(s->c, page, off, s->head, kk, vv);
            for (int j = 0; j < g; ++j) {
                double w = exp(x[live * g + j] - m[j]);
                sum[j] += w;
                for (int ch = 0; ch < D; ++ch) out[j * D + ch] += w * vv[ch];
            }
            ++live;
        }

    for (int j = 0; j < g; ++j) {
        if (live == 0 || rc != ORC_OK) {
            for (int ch = 0; ch < D; ++ch) out[j * D + ch] = 0.0;
            lse[j] = -INFINITY;
        } else {
            for (int ch = 0; ch < D; ++ch) out[j * D + ch] /= sum[j];
            lse[j] = m[j] + log(sum[j]);
        }
    }
    free(x);
    free(m);
    free(sum);
    return rc;
}

typedef struct { int32_t table, head, first, count; } key_t_;

/* Sort helper without qsort_r portability concerns: insertion of indices. */
static void sort_ranges(const orc_range *r, int32_t n, int32_t *idx)
{
    for (int32_t i = 0; i < n; ++i) idx[i] = i;
    /* stable insertion sort by (table, head); range lists are short */
    for (int32_t i = 1; i < n; ++i) {
        int32_t v = idx[i], j = i - 1;
        while (j >= 0) {
            const orc_range *a = &r[idx[j]], *b = &r[v];
            if (a->table < b->table || (a->table == b->table && a->head <= b->head)) break;
            idx[j + 1] = idx[j];
            --j;
        }
        idx[j + 1] = v;
    }
}

static int check_shape(const orc_cache *c, int32_t batch, int32_t hq, int32_t hkv,
                       int32_t n_tables)
{
    int32_t H = c ? c->heads_per_page : 0;
    if (!c || batch < 0 || hq <= 0 || hkv <= 0 || hq % hkv || H <= 0 || hkv % H) return ORC_EARG;
    if (n_tables != batch * (hkv / H)) return ORC_EARG;
    return ORC_OK;
}

int orc_attend(const orc_cache *c, const float *q, int32_t batch, int32_t hq,
               int32_t hkv, const int32_t *tables, int32_t n_tables,
               int32_t max_entries, int32_t kind, const orc_range *ranges,
               int32_t n_ranges, double *out, double *lse, int32_t n_threads)
{
    int rc = check_shape(c, batch, hq, hkv, n_tables);
    if (rc) return rc;
    const int32_t H = c->heads_per_page, g = hq / hkv, tpr = hkv / H;
    for (int64_t i = 0; i < (int64_t)batch * hq; ++i) {
        lse[i] = -INFINITY;
        for (int ch = 0; ch < D; ++ch) out[i * D + ch] = 0.0;
    }
    int32_t *idx = (int32_t *)malloc(sizeof(int32_t) * (size_t)(n_ranges > 0 ? n_ranges : 1));
    key_t_ *keys = (key_t_ *)malloc(sizeof(key_t_) * (size_t)(n_ranges > 0 ? n_ranges : 1));
    sort_ranges(ranges, n_ranges, idx);
    int32_t nk = 0;
    for (int32_t i = 0; i < n_ranges; ++i) {
        const orc_range *r = &ranges[idx[i]];
        if (r->table < 0 || r->table >= n_tables || r->head < 0 || r->head >= H) { rc = ORC_EARG; break; }
        if (nk > 0 && keys[nk - 1].table == r->table && keys[nk - 1].head == r->head) keys[nk - 1].count++;
        else keys[nk++] = (key_t_){ r->table, r->head, i, 1 };
    }
    int err = rc;
    if (!err) {
#pragma omp parallel for schedule(dynamic, 1) num_threads(n_threads > 0 ? n_threads : 1)
        for (int32_t kI = 0; kI < nk; ++kI) {
            const key_t_ *key = &keys[kI];
            int32_t b = key->table / tpr, kvh = (key->table % tpr) * H + key->head;
            double qd[16 * D];
            double o[16 * D], l[16];
            const orc_range *rs[4096];
            int nr = key->count > 4096 ? 4096 : key->count;
            for (int r = 0; r < nr; ++r) rs[r] = &ranges[idx[key->first + r]];
            for (int j = 0; j < g && j < 16; ++j)
                for (int ch = 0; ch < D; ++ch)
                    qd[j * D + ch] = (double)q[((int64_t)b * hq + kvh * g + j) * D + ch];
            src_t s = { c, tables + (int64_t)key->table * max_entries, max_entries, kind, key->head };
            int st = (g > 16 || key->count > 4096) ? ORC_EARG : attend_core(&s, qd, g, rs, nr, o, l);
            if (st) {
#pragma omp atomic write
                err = st;
            }
            for (int j = 0; j < g && j < 16; ++j) {
                int64_t row = (int64_t)b * hq + kvh * g + j;
                lse[row] = l[j];
                for (int ch = 0; ch < D; ++ch) out[row * D + ch] = o[j * D + ch];
            }
        }
    }
    free(idx);
    free(keys);
    return err;
}

int orc_attend_ranges(const orc_cache *c, const float *q, int32_t batch,
                      int32_t hq, int32_t hkv, const int32_t *tables,
                      int32_t n_tables, int32_t max_entries, int32_t kind,
                      const orc_range *ranges, int32_t n_ranges,
                      double *part_out, double *part_lse, int32_t n_threads)
{
    int rc = check_shape(c, batch, hq, hkv, n_tables);
    if (rc) return rc;
    const int32_t H = c->heads_per_page, g = hq / hkv, tpr = hkv / H;
    if (g > 16) return ORC_EARG;
    int err = ORC_OK;
#pragma omp parallel for schedule(dynamic, 1) num_threads(n_threads > 0 ? n_threads : 1)
    for (int32_t i = 0; i < n_ranges; ++i) {
        const orc_range *r = &ranges[i];
        if (r->table < 0 || r->table >= n_tables || r->head < 0 || r->head >= H) {
#pragma omp atomic write
            err = ORC_EARG;
            continue;
        }
        int32_t b = r->table / tpr, kvh = (r->table % tpr) * H + r->head;
        double qd[16 * D];
        for (int j = 0; j < g; ++j)
            for (int ch = 0; ch < D; ++ch)
                qd[j * D + ch] = (double)q[((int64_t)b * hq + kvh * g + j) * D + ch];
        src_t s = { c, tables + (int64_t)r->table * max_entries, max_entries, kind, r->head };
        const orc_range *rs[1] = { r };
        int st = attend_core(&s, qd, g, rs, 1, part_out + (int64_t)i * g * D, part_lse + (int64_t)i * g);
        if (st) {
#pragma omp atomic write
            err = st;
        }
    }
    return err;
}

/* ------------------------------------------------------------------------ */
/* Log-sum-exp merge (TriAxialKV key design 4; HyQuant Algorithm 3)          */
/* ------------------------------------------------------------------------ */

int orc_merge(const double *part_out, const double *part_lse,
              const int32_t *offsets, int32_t batch, int32_t hq, int32_t hkv,
              double *out, double *lse)
{
    if (batch < 0 || hq <= 0 || hkv <= 0 || hq % hkv) return ORC_EARG;
    const int32_t g = hq / hkv;
    for (int32_t b = 0; b < batch; ++b)
        for (int32_t kvh = 0; kvh < hkv; ++kvh) {
            int32_t s0 = offsets[b * hkv + kvh], s1 = offsets[b * hkv + kvh + 1];
            if (s1 < s0) return ORC_EARG;
            for (int32_t j = 0; j < g; ++j) {
                int64_t row = (int64_t)b * hq + kvh * g + j;
                double mx = -INFINITY;
                for (int32_t s = s0; s < s1; ++s) {
                    double l = part_lse[(int64_t)s * g + j];
                    if (l > mx) mx = l;
                }
                for (int ch = 0; ch < D; ++ch) out[row * D + ch] = 0.0;
                if (mx == -INFINITY) { lse[row] = -INFINITY; continue; }
                double tot = 0.0;
                for (int32_t s = s0; s < s1; ++s) tot += exp(part_lse[(int64_t)s * g + j] - mx);
                double L = mx + log(tot);
                for (int32_t s = s0; s < s1; ++s) {
                    double w = exp(part_lse[(int64_t)s * g + j] - L);
                    for (int ch = 0; ch < D; ++ch)
                        out[row * D + ch] += w * part_out[((int64_t)s * g + j) * D + ch];
                }
                lse[row] = L;
            }
        }
    return ORC_OK;
}
