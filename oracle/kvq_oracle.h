/*
 * kvq_oracle.h -- plain, slow CPU oracle for decode attention over a
 * mixed-precision (INT2 / INT4 / FP16) paged KV cache.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no source,
 * header, table or helper with the GPU library; the byte layout is a written
 * specification that both sides implement independently.
 *
 * Sources (titles of the pages and the part of each page followed):
 *   [TriAxialKV] "TriAxialKV: Toward Extreme Low-Precision KV-Cache
 *       Quantization for Agentic Inference Tasks", key designs 3 and 4
 *       (G = 32 asymmetric groups; INT4 K/V per-token, INT2 K per-channel,
 *       INT2 V per-token; residual < 32 tokens routed to INT4; INT2-first
 *       page-table reorder; pure-precision Flash-Decoding splits; global
 *       log-sum-exp merge; new tokens appended as INT4).
 *   [HyQuant] "HyQuant: Hybrid-Precision Quantization for LLM Attention",
 *       background (softmax(QK^T/sqrt(d)), online softmax m / l / acc, GQA
 *       stacking of g = Hq/Hkv query heads), method (key partition into
 *       quantized / vertical-line / window sets; FP16 anchors), Algorithm 3;
 *       Algorithm 1 (vertical lines: window W excluded, tail-query proxy,
 *       GQA column scores, top rho of the prefix) and Algorithm 4 (FREEZE:
 *       vertical lines and window stay full precision, the rest is quantized);
 *       the core method's fused prefill operator (the query as given; the
 *       quantized prefix's keys and values both through their quantized
 *       forms, vertical lines and window in full precision, one softmax over
 *       the concatenation) and Algorithm 2 (per-tile symmetric scale
 *       max|X_T| / c_B, c_B = 127 for INT8).
 *   [IntentKV] technical summary, "layout-preserving eviction": evicted
 *       positions are redirected to one sentinel dead slot (K = -1e4, V = 0)
 *       whose attention contribution is zero.
 *   [Tangram] method steps 5-7: one page table per head group; each head
 *       reads only the entries its budget needs.
 *
 * Floating point: quantization is IEEE fp32 (round-to-nearest-even, no FMA
 * contraction: build with -ffp-contract=off); attention is fp64.
 */
#ifndef KVQ_ORACLE_H
#define KVQ_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Precision classes, decided by the page-id range (TriAxialKV key design 4:
 * one virtual address range, precision from the base offset). */
enum { ORC_INT2 = 0, ORC_INT4 = 1, ORC_FP16 = 2 };
/* Source element types. */
enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_F16 = 2 };
/* Table kinds: entries are page ids, or per-token slot ids (page*16+off). */
enum { ORC_PAGES = 0, ORC_SLOTS = 1 };

/* Return codes. */
enum { ORC_OK = 0, ORC_EARG = -1, ORC_ECLASS = -2, ORC_EPAIR = -3, ORC_ERANGE = -4 };

typedef struct {
    int32_t heads_per_page;  /* KV heads stored in every page (head-major blocks) */
    int32_t n_pages[3];      /* pages per class; ids: INT2 [0,n2), INT4 [n2,n2+n4), FP16 after */
    uint8_t *pool[3];        /* host byte pools, one per class */
    int32_t sentinel_slot;   /* slot id of the dead slot, or -1 */
    int32_t anchor_fp8;      /* 0: FP16 anchors; 1: FP8 (e4m3) anchors with a power-of-two scale */
} orc_cache;

/* A token range of one (table, head): tokens t in [tok_begin, tok_end), where
 * token t is table entry t/16, offset t%16 (page tables) or entry t (slot maps). */
typedef struct {
    int32_t table, head, cls, tok_begin, tok_end;
} orc_range;

/* --- fp16 helpers (exact; computed through fp64 scaling) --------------- */
uint16_t orc_f16_down(float x);     /* largest fp16 <= x, never -0            */
uint16_t orc_f16_up(float x);       /* smallest fp16 >= x, never -0           */
uint16_t orc_f16_nearest(float x);  /* round to nearest, ties to even          */
uint16_t orc_f16_up4(float x);      /* smallest fp16 >= x with its two lowest mantissa
                                       bits zero (INT2 key scales), never -0   */
double   orc_f16_value(uint16_t h);

/* --- FP8 (OCP e4m3: 4 exponent bits, bias 7, 3 mantissa bits, max 448) --- */
double  orc_e4m3_value(uint8_t code);   /* NaN for 0x7F / 0xFF                  */
uint8_t orc_e4m3_nearest(double y);     /* |y| <= 448; ties to the even code; 0 -> 0x00 */
/* One anchor row: scale 2^e with e the smallest integer >= -24 such that
 * max |x| <= 448 * 2^e, codes nearest to x / 2^e; *scale is 2^e as fp16 bits. */
void    orc_fp8_row(const float *x, int n, uint8_t *codes, uint16_t *scale);

/* Page head-block sizes in bytes (per class; 3 = an FP8 anchor block). */
int64_t orc_block_bytes(int32_t cls);

/* --- quantizer ------------------------------------------------------------
 * Asymmetric group quantizer Q_b over n values x[i*stride]:
 *   z = fp16 round-down(min), s = fp16 round-up(fl32(fl32(max - z) / L)),
 *   code = clamp(rint(fl32(fl32(x - z) / s)), 0, L), L = 2^bits - 1; s == 0
 *   gives all-zero codes.  Dequantization is z + code * s. */
void orc_quantize(const float *x, int32_t n, int64_t stride, int32_t bits,
                  uint8_t *codes, uint16_t *scale, uint16_t *zero);
/* The same with bits = 2 and s = orc_f16_up4(fl32(fl32(max - z) / 3)): the INT2 key
 * groups (one channel over 32 tokens).  s has at most 9 significant bits, so every
 * c s (c = 0..3) is an fp16 value. */
void orc_quantize_k2(const float *x, int32_t n, int64_t stride,
                     uint8_t *codes, uint16_t *scale, uint16_t *zero);

/* --- routing (TriAxialKV key design 3) -------------------------------------
 * flags: 0 = wants INT2, 1 = INT4, 2 = FP16 anchor.  INT2-flagged tokens, in
 * order, form groups of 32; the final < 32 of them become INT4. */
int orc_route(const uint8_t *flags, int32_t n, uint8_t *cls_out,
              int32_t *n_int2_groups, int32_t *n_int4, int32_t *n_fp16);

/* --- write path -------------------------------------------------------------
 * Rows of k / v: element (row r, head h, channel c) sits at
 * r*row_stride + h*head_stride + c (in elements of dtype).  Every head of the
 * page (heads_per_page) is written.
 *   INT4 tokens: rows4[i] -> slot slots4[i];
 *   INT2 groups: rows2[32*g .. 32*g+31] -> the page pair starting at the even
 *                INT2 page pages2[g] (tokens 0-15 even page, 16-31 odd page);
 *   FP16 tokens: rows16[i] -> slot slots16[i]. */
int orc_append(orc_cache *c, const void *k, const void *v, int32_t dtype,
               int64_t row_stride, int64_t head_stride,
               int32_t n4, const int32_t *rows4, const int32_t *slots4,
               int32_t n2g, const int32_t *rows2, const int32_t *pages2,
               int32_t n16, const int32_t *rows16, const int32_t *slots16);

/* --- page-table reorder (TriAxialKV key design 4, phase 1) -----------------
 * Stable partition of entries [0, n_entries[t]) of every table by class
 * (INT2, then INT4, then FP16); class_counts[t*3 + cls] = pages of cls. */
int orc_reorder(const orc_cache *c, int32_t *tables, int32_t n_tables,
                int32_t max_entries, const int32_t *n_entries,
                int32_t *class_counts);

/* --- slot-map compaction (Tangram dead slots carry no attention mass) -----
 * For every table t, entries [0, n_entries[t]) are stably partitioned: the
 * live entries (not the sentinel slot) keep their order at the front, the
 * dead ones follow, written as the sentinel.  Head h of table t read the first
 * head_tokens[t*heads + h] entries before; live_tokens[t*heads + h] receives
 * how many of them were live, which is the number of leading entries it reads
 * afterwards (the live entries of that prefix, in the same order). */
int orc_compact_slots(const orc_cache *c, int32_t *tables, int32_t n_tables,
                      int32_t max_entries, const int32_t *n_entries,
                      const int32_t *head_tokens, int32_t heads,
                      int32_t *live_tokens);

/* --- vertical-line selection and FREEZE routing (HyQuant Algorithms 1, 4) --
 * Per request b and KV head h, in fp64: the tail-query proxy is the mean over
 * the n_tail[b] tail queries of the sum of the g = hq/hkv query heads of h,
 * u = sum_j (1/n_tail) sum_i q[b][i][h*g + j]; the score of token k is u . K[b][k][h].
 * Tokens k >= n - window (n = n_tokens[b]) form the window; of the prefix
 * k < n - window, the n_vl = floor(rho * n_pre + 1/2) tokens of highest score
 * (ties: lower k) are the vertical lines.  cls[(b*hkv + h)*max_tokens + k] =
 * 1 (vertical line), 2 (window), 0 (quantized prefix, and k >= n); scores
 * [same index] for k < n (0 past n); n_vl[b*hkv + h].  K [batch][max_tokens]
 * [hkv][128] and q_tail [batch][max_tail][hq][128] are fp32 (bf16 sources
 * widen exactly). */
int orc_select_vl(const float *k, const float *q_tail, int32_t batch,
                  int32_t max_tokens, int32_t hkv, int32_t hq, int32_t max_tail,
                  const int32_t *n_tokens, const int32_t *n_tail, int32_t window,
                  double rho, double *scores, uint8_t *cls, int32_t *n_vl);

/* --- prefill attention with an INT8 prefix (HyQuant core method, fused
 * operator O = softmax([Q K-hat_Q^T || Q K_FP^T] / sqrt(d)) [V-hat_Q || V_FP];
 * Algorithm 2) ---------------------------------------------------------------
 * Per request b (n = n_tokens[b] prompt positions), query head j and query
 * position t, over the keys k <= t of KV head h = j / g: a key is read in full
 * precision (K and V as given) when it is a vertical line of h
 * (cls[(b*hkv + h)*n_max + k] == 1) or in the window k > t - window; every other
 * visible key is read through INT8 (K-hat = s_K code_K, V-hat = s_V code_V).  The
 * query is never quantized.  INT8 tiles are 64 positions per KV head, separately
 * for K and V, with the vertical lines left out of the tile maximum.  Tile scale
 * s = fl32(max |x| / 127) over the tile's live non-line values (0 for an empty or
 * zero tile), code = clamp(rint(fl32(x / s)), -127, 127) (0 when s = 0), all fp32.
 * Logits q . k / sqrt(128) and the softmax and its sum of V are fp64 from the
 * bf16/fp32-exact inputs.  q [batch][n_max][hq][128], k, v
 * [batch][n_max][hkv][128] fp32; out fp64 [batch][n_max][hq][128] (0 for t >= n).
 * The codes and scales are returned: k_codes, v_codes int8 like k, k_scales,
 * v_scales [batch][hkv][n_max/64 rounded up]. */
int orc_prefill_attend(const float *q, const float *k, const float *v,
                       int32_t batch, int32_t n_max, int32_t hq, int32_t hkv,
                       const int32_t *n_tokens, const uint8_t *cls, int32_t window,
                       double *out, int8_t *k_codes, float *k_scales,
                       int8_t *v_codes, float *v_scales);
/* The same for the listed rows only: out_rows [n_rows][hq][128] for (row_b[r],
 * row_t[r]), row_t[r] < n_tokens[row_b[r]]; the codes and scales in full. */
int orc_prefill_attend_rows(const float *q, const float *k, const float *v,
                            int32_t batch, int32_t n_max, int32_t hq, int32_t hkv,
                            const int32_t *n_tokens, const uint8_t *cls, int32_t window,
                            int32_t n_rows, const int32_t *row_b, const int32_t *row_t, double *out_rows,
                            int8_t *k_codes, float *k_scales, int8_t *v_codes, float *v_scales);

/* Dequantize one token of one head to fp64 (K and V, 128 channels each). */
int orc_token(const orc_cache *c, int32_t page, int32_t off, int32_t head,
              double *k, double *v);

/* --- attention ----------------------------------------------------------------
 * Exact softmax attention per (request b, query head j) over the live tokens
 * of KV head j / g: the union of the ranges given for (table, head), minus
 * sentinel slots.  Table t serves request t / (hkv/heads_per_page) and KV
 * heads (t % (hkv/heads_per_page))*heads_per_page + head.  q is fp32
 * [batch][hq][128]; out fp64 [batch][hq][128]; lse fp64 [batch][hq] (natural
 * log).  Rows with no live token: out 0, lse -inf. */
int orc_attend(const orc_cache *c, const float *q, int32_t batch, int32_t hq,
               int32_t hkv, const int32_t *tables, int32_t n_tables,
               int32_t max_entries, int32_t kind, const orc_range *ranges,
               int32_t n_ranges, double *out, double *lse, int32_t n_threads);

/* Same arithmetic per range: partial out [n_ranges][g][128] and lse
 * [n_ranges][g] of each range on its own. */
int orc_attend_ranges(const orc_cache *c, const float *q, int32_t batch,
                      int32_t hq, int32_t hkv, const int32_t *tables,
                      int32_t n_tables, int32_t max_entries, int32_t kind,
                      const orc_range *ranges, int32_t n_ranges,
                      double *part_out, double *part_lse, int32_t n_threads);

/* Log-sum-exp merge of partials: the partials of (b, kv head) are rows
 * offsets[b*hkv + kvh] .. offsets[b*hkv + kvh + 1] - 1. */
int orc_merge(const double *part_out, const double *part_lse,
              const int32_t *offsets, int32_t batch, int32_t hq, int32_t hkv,
              double *out, double *lse);

#ifdef __cplusplus
}
#endif
#endif
