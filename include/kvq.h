/*
 * kvq.h -- C ABI of libkvq: GQA decode attention read directly from a
 * mixed-precision (INT2 / INT4 / FP16) paged KV cache on AMD MI355X (gfx950).
 *
 * Pages this interface follows (title, part of the page):
 *   TriAxialKV ("TriAxialKV: Toward Extreme Low-Precision KV-Cache Quantization
 *     for Agentic Inference Tasks"), key design 3: asymmetric group quantization
 *     with G = 32 (INT4 K and V per-token; INT2 K per-channel across the 32 tokens
 *     of a group; INT2 V per-token); a residual tail of fewer than 32 tokens goes
 *     to INT4 per-token.  Key design 4: INT2 and INT4 pools in one address range
 *     with the precision decided by the base offset; before decoding, each
 *     request's page pointers are sorted so INT2 comes first (phase 1); the
 *     decode kernel splits the sequence Flash-Decoding style into splits of one
 *     precision each and merges them with a global log-sum-exp reduction
 *     (phase 2); newly generated tokens are written as INT4 at the tail.
 *   HyQuant ("HyQuant: Hybrid-Precision Quantization for LLM Attention"),
 *     background (softmax(q k^T / sqrt(d)), online softmax state m, l, acc; GQA
 *     stacks g = Hq/Hkv query heads on one KV head), method (keys partitioned into
 *     quantized, vertical-line and window sets; anchors kept FP16) and
 *     Algorithm 3 (split-K over the quantized prefix with dequantization inside
 *     attention, reduce, then the FP16 segments with the same softmax state).
 *   IntentKV (technical summary), layout-preserving eviction: evicted slot-map
 *     entries point at one sentinel dead slot (K = -1e4, V = 0) whose attention
 *     contribution is zero.
 *   Tangram, method steps 5-7: one page table per head group whose heads read
 *     only the entries their budget needs; split counts fixed ahead of time in
 *     proportion to each group's budget.
 *
 * Conventions for every call:
 *   - Pointers marked [dev] are device memory, [host] host memory.  The caller
 *     owns every buffer.  The library never allocates, frees or synchronizes.
 *   - Device calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 *     stream).  They return after enqueueing.
 *   - Argument errors the host can see are reported before anything is
 *     enqueued, as a negative kvq_status; kvq_last_error() then describes it.
 *   - Bad values inside device arrays (ids out of range, class mismatches,
 *     broken INT2 pairs) never make a kernel read or write out of bounds: the
 *     offending item is skipped (its outputs are zero / -inf) and, when
 *     dev_err is not NULL, a KVQ_DEVERR_* bit is OR-ed into *dev_err.
 *   - head_dim must be 128 and page_size 16.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    KVQ_OK = 0,
    KVQ_ERR_INVALID_ARG = -1,  /* a host-visible argument is wrong            */
    KVQ_ERR_UNSUPPORTED = -2,  /* valid but not supported (e.g. head_dim 64) */
    KVQ_ERR_CAPACITY = -3,     /* an output buffer is too small               */
    KVQ_ERR_HIP = -4,          /* a HIP runtime call failed                   */
    KVQ_ERR_NO_DEVICE = -5     /* no usable gfx950 device                     */
} kvq_status;

typedef enum { KVQ_INT2 = 0, KVQ_INT4 = 1, KVQ_FP16 = 2 } kvq_class;
typedef enum { KVQ_F32 = 0, KVQ_BF16 = 1, KVQ_F16 = 2 } kvq_dtype;
typedef enum { KVQ_TABLE_PAGES = 0, KVQ_TABLE_SLOTS = 1 } kvq_table_kind;

/* Bits OR-ed into *dev_err by kernels that meet bad device data. */
enum {
    KVQ_DEVERR_ID = 1,      /* page / slot id outside the pools or of the wrong class */
    KVQ_DEVERR_RANGE = 2,   /* token range, table or head index out of bounds         */
    KVQ_DEVERR_PAIR = 4,    /* INT2 entries that are not aligned (even, even+1) pairs */
    KVQ_DEVERR_SPLIT = 8    /* malformed split descriptor                             */
};

/*
 * Pools.  Page ids form one id space: INT2 [0, n2), INT4 [n2, n2+n4), FP16
 * [n2+n4, n2+n4+n16); the class of a page is found by comparing its id with the
 * bases.  pool[c] holds n_pages[c] pages of heads_per_page head blocks each;
 * page p's head h block starts at
 *   pool[c] + ((p - base_c) * heads_per_page + h) * kvq_block_bytes(c).
 * The three pools may be carved out of one allocation.  A slot id is
 * page * 16 + offset.  Head block layouts (little-endian, fp16 (scale, zero)).
 * A code row is a sequence of 32-bit words; with b bits per code, word w holds
 * channels w*32/b .. (w+1)*32/b - 1, the even-indexed of them in the low 16 bits
 * and the odd-indexed in the high 16 bits, ascending, b bits each.
 *   INT4 (2560 B): K codes [16 tok][64 B] @0; K meta [16 tok][4 groups][scale,
 *     zero] @1024; V codes [16 tok][64 B] @1280; V meta [4 groups][16 tok]
 *     [scale, zero] @2304.
 *   INT2 (1536 B): K codes [16 tok][32 B] @0; K per-channel meta of the page
 *     pair @512: 64 fp16 scales then 64 fp16 zeros @640 (even page: channels
 *     0-63, odd page: 64-127); V codes [16 tok][32 B] @768; V meta @1280: per
 *     group (4 x 64 B) the 16 tokens' fp16 scales, then their 16 fp16 zeros.
 *     INT2 pages are used in aligned pairs (even,
 *     even+1) holding one 32-token group; n_pages[KVQ_INT2] must be even.
 *   FP16 (8192 B): K [16 tok][128] fp16 @0; V @4096.
 */
typedef struct {
    int32_t head_dim;         /* must be 128                                  */
    int32_t page_size;        /* must be 16                                   */
    int32_t heads_per_page;   /* H_t: KV heads per page = per table, >= 1     */
    int32_t n_pages[3];       /* pages per class (INT2, INT4, FP16)           */
    void *pool[3];            /* [dev] one pool per class (NULL if 0 pages)   */
    int32_t sentinel_slot;    /* slot id of the dead slot, or -1              */
    int32_t anchor_format;    /* KVQ_ANCHOR_FP16 or KVQ_ANCHOR_FP8: the format
                                 of the FP16 class's blocks (the anchors)      */
} kvq_cache;

/* Anchor formats (HyQuant keeps its anchors in FP16 and names FP8 as the smaller
 * form).  KVQ_ANCHOR_FP8: each token's K and V rows of a head are OCP e4m3 codes
 * (max 448, nearest with ties to even) times 2^e, e the smallest integer >= -24
 * with max |x| <= 448 2^e, stored as an fp16 power of two; block of 4160 bytes =
 * kvq_block_bytes(KVQ_FP8_ANCHOR_BLOCK): K codes [16 tok][128 B] at 0, K scales
 * [16] fp16 at 2048, V codes at 2080, V scales at 4128. */
enum { KVQ_ANCHOR_FP16 = 0, KVQ_ANCHOR_FP8 = 1 };
enum { KVQ_FP8_ANCHOR_BLOCK = 3 };

/* A token range of one (table, head-in-table) in one precision class:
 * tokens t in [tok_begin, tok_end); in a page table token t is entry t/16,
 * offset t%16; in a slot map token t is entry t. */
typedef struct {
    int32_t table, head, cls, tok_begin, tok_end;
} kvq_split;

/* Bytes of one head block of a page of class cls (0 for an unknown class). */
size_t kvq_block_bytes(int32_t cls);

/*
 * Routing [host] (TriAxialKV key design 3).  flags[i]: 0 = the token wants
 * INT2, 1 = INT4, 2 = FP16 anchor.  INT2-flagged tokens, in order, are grouped
 * into groups of 32; the final fewer-than-32 of them are routed to INT4.
 * Writes cls_out[i] (a kvq_class) and the counts (each pointer may be NULL).
 * Errors: INVALID_ARG for n < 0, NULL arrays with n > 0, or a flag > 2.
 */
kvq_status kvq_route_tokens(const uint8_t *flags, int32_t n, uint8_t *cls_out,
                            int32_t *n_int2_groups, int32_t *n_int4, int32_t *n_fp16);

/*
 * Tri-axis token tags (TriAxialKV key design 1) [host].  Every token gets a tag
 * s(t) = (temporal * KVQ_N_MODAL + modal) * KVQ_N_SEMANTIC + semantic, read in one
 * pass over the token ids from the chat template's boundary tokens, named by the
 * caller in `markers` (token id -> event; each id at most once):
 *   semantic: 0 inst (system prompt, tool specs; also before any marker), 1 user,
 *     2 assistant, 3 reasoning (between THINK_BEGIN / _END), 4 tool_call (between
 *     TOOL_CALL_BEGIN / _END), 5 obs (tool or environment output), 6 delim (every
 *     marker token itself).  A role event (SYSTEM, USER, ASSISTANT, OBSERVATION)
 *     or END closes any open reasoning, tool-call or image span.
 *   modal: 1 image between IMAGE_BEGIN and IMAGE_END (markers excluded), else 0.
 *   temporal: each USER event starts a turn (tokens before the first are turn 0);
 *     with T turns in all, a token of turn u gets min(T - u, 3): 0 current,
 *     1 the turn before, 2 two before, 3 older.
 * tokens [host] int32 [n]; tags [host] uint8 [n]; *n_turns (may be NULL) = T.
 * Errors: INVALID_ARG (negative counts, NULL arrays, unknown event, an id named twice).
 */
enum { KVQ_N_TEMPORAL = 4, KVQ_N_MODAL = 2, KVQ_N_SEMANTIC = 7, KVQ_N_TAGS = 56 };
enum {
    KVQ_EV_SYSTEM = 0, KVQ_EV_USER = 1, KVQ_EV_ASSISTANT = 2, KVQ_EV_OBSERVATION = 3,
    KVQ_EV_END = 4, KVQ_EV_THINK_BEGIN = 5, KVQ_EV_THINK_END = 6,
    KVQ_EV_TOOL_CALL_BEGIN = 7, KVQ_EV_TOOL_CALL_END = 8,
    KVQ_EV_IMAGE_BEGIN = 9, KVQ_EV_IMAGE_END = 10
};
typedef struct {
    int32_t token_id;
    int32_t event;  /* KVQ_EV_* */
} kvq_tag_marker;

kvq_status kvq_tag_tokens(const int32_t *tokens, int32_t n, const kvq_tag_marker *markers,
                          int32_t n_markers, uint8_t *tags, int32_t *n_turns);

/*
 * Token counts per tag [host] (the N_k of TriAxialKV key design 2): adds the
 * histogram of tags [host] uint8 [n] into counts [host] int64 [KVQ_N_TAGS] (not
 * cleared: calls over several requests accumulate).  Errors: INVALID_ARG (a tag
 * >= KVQ_N_TAGS, NULL arrays; nothing is added then).
 */
kvq_status kvq_count_tags(const uint8_t *tags, int32_t n, int64_t *counts);

/*
 * Greedy width allocation (TriAxialKV key design 2) [host]: minimise sum_k D_k(b_k)
 * over b_k in {2, 4} subject to sum_k N_k b_k <= budget_bits * sum_k N_k.  Every tag
 * starts at 2 bits; tags with N_k > 0 are visited by decreasing
 * rho_k = (D_k(2) - D_k(4)) / (2 N_k) (ties: lower k) and upgraded to 4 bits while
 * the constraint holds; the walk stops at the first tag that would break it.
 * d2, d4 [host] double [n_tags] (the distortion table), counts [host] int64
 * [n_tags]; bits [host] uint8 [n_tags] = 2 or 4; *avg_bits (may be NULL) = the
 * resulting average width.  Errors: INVALID_ARG (budget outside [2, 4], negative
 * counts, NULL arrays).
 */
kvq_status kvq_allocate_bits(const double *d2, const double *d4, const int64_t *counts,
                             int32_t n_tags, double budget_bits, uint8_t *bits,
                             double *avg_bits);

/*
 * Per-token routing flags from tags and widths [host]: flags[i] = 0 (INT2) when
 * bits[tags[i]] is 2, 1 (INT4) when it is 4 -- the input of kvq_route_tokens.
 * Errors: INVALID_ARG (a tag >= n_tags or a width other than 2 / 4).
 */
kvq_status kvq_tag_flags(const uint8_t *tags, int32_t n, const uint8_t *bits, int32_t n_tags,
                         uint8_t *flags);

/*
 * Quantize and pack tokens into the pools (TriAxialKV key design 3; new decode
 * tokens are INT4 per key design 4; FP16 anchors per HyQuant's method).
 *   k, v [dev]: n_rows source rows; element (row r, head h, channel c) is at
 *     r*row_stride + h*head_stride + c, of type src_dtype (KVQ_F32, KVQ_BF16 or
 *     KVQ_F16).  Every one of the heads_per_page heads of a row is written; a
 *     row index outside [0, n_rows) is skipped (KVQ_DEVERR_ID).
 *   INT4:  int4_rows[i] [dev] -> slot int4_slots[i] [dev]  (i < n_int4)
 *   INT2:  the 32 rows int2_rows[32g .. 32g+31] [dev] -> the pair starting at
 *          the even INT2 page int2_pages[g] [dev] (tokens 0-15 in the even page,
 *          16-31 in the odd page)                          (g < n_int2_groups)
 *   FP16:  fp16_rows[i] [dev] -> slot fp16_slots[i] [dev]   (i < n_fp16)
 * Quantizer (bit-exact, IEEE fp32): z = largest fp16 <= min, s = smallest fp16
 * >= (max - z) / L, code = clamp(rint((x - z) / s), 0, L), L = 2^b - 1; s = 0
 * gives all-zero codes.  INT2 key groups (one channel over 32 tokens) round s up
 * once more, to the next fp16 value whose two lowest mantissa bits are zero (at
 * most 9 significant bits, so every code times s is an fp16 value).  FP16
 * anchors are rounded to nearest even.  Destinations
 * of one call must be distinct.
 * Errors: INVALID_ARG (bad cache, NULL arrays with nonzero counts, bad dtype,
 * negative counts or strides), UNSUPPORTED (head_dim != 128, page_size != 16),
 * HIP.  Device-side: KVQ_DEVERR_ID / PAIR for bad slots or pages.
 */
kvq_status kvq_quantize_append(const kvq_cache *c, const void *k, const void *v,
                               int32_t src_dtype, int64_t n_rows, int64_t row_stride,
                               int64_t head_stride,
                               int32_t n_int4, const int32_t *int4_rows, const int32_t *int4_slots,
                               int32_t n_int2_groups, const int32_t *int2_rows,
                               const int32_t *int2_pages,
                               int32_t n_fp16, const int32_t *fp16_rows, const int32_t *fp16_slots,
                               int32_t *dev_err, void *stream);

/*
 * Phase-1 page-table reorder (TriAxialKV key design 4).  tables [dev] int32
 * [n_tables][max_entries] of page ids; for every table t, entries
 * [0, n_entries[t]) ([dev]) are stably partitioned in place into INT2, then
 * INT4, then FP16 pages.  class_counts [dev] int32 [n_tables][3] receives the
 * number of pages per class (may be NULL).  The INT2 entries must form aligned
 * pairs after the partition (KVQ_DEVERR_PAIR otherwise; the table is still
 * partitioned).  Errors: INVALID_ARG, UNSUPPORTED (max_entries > 32768: 524,288
 * tokens of 16-token pages), HIP.
 */
kvq_status kvq_reorder_pages(const kvq_cache *c, int32_t *tables, int32_t n_tables,
                             int32_t max_entries, const int32_t *n_entries,
                             int32_t *class_counts, int32_t *dev_err, void *stream);

/*
 * Slot-map compaction (optional, before decoding slot maps; Tangram's sentinel
 * dead slots carry no attention mass, so the decode may skip them ahead of
 * time instead of per token).  tables [dev] int32 [n_tables][max_entries] of
 * slot ids: for every table t, entries [0, n_entries[t]) ([dev]) are stably
 * partitioned in place, live entries (not c->sentinel_slot) first in their
 * order, then the dead ones, rewritten as the sentinel.  head_tokens [dev]
 * int32 [n_tables][heads_per_page]: head h of table t reads the first
 * head_tokens[t][h] <= n_entries[t] entries; live_tokens [dev] int32
 * [n_tables][heads_per_page] receives the live entries among them, the number
 * of leading entries head h reads after the compaction (its attention is
 * unchanged).  With no sentinel slot (-1) nothing moves.  A table whose
 * n_entries or head_tokens are out of range is left as it was
 * (KVQ_DEVERR_RANGE).  Errors: INVALID_ARG, UNSUPPORTED (heads_per_page > 64),
 * HIP.
 */
kvq_status kvq_compact_slots(const kvq_cache *c, int32_t *tables, int32_t n_tables,
                             int32_t max_entries, const int32_t *n_entries,
                             const int32_t *head_tokens, int32_t *live_tokens,
                             int32_t *dev_err, void *stream);

/*
 * Vertical-line selection and FREEZE routing (HyQuant Algorithm 1 and Algorithm
 * 4), run once at the end of a prefill.  For request b < batch and KV head h:
 *   proxy[b][h][c] = (1/n_tail[b]) sum_{i < n_tail[b]} sum_{j < g} q_tail[b][i][h*g + j][c]
 *     (the tail-query proxy of the GQA group, g = hq / hkv; 0 when n_tail is 0);
 *   scores[b][h][t] = proxy[b][h] . k[b][t][h] for t < n_tokens[b] (0 beyond);
 *   token_class[b][h][t]: 2 for the window t in [n - window, n), 1 for the
 *     n_vl[b][h] = floor(rho * n_pre + 1/2) prefix tokens (t < n_pre = max(n -
 *     window, 0)) of highest score, ties to the lower t (the vertical lines),
 *     0 for the rest of the prefix and for t >= n.  FREEZE keeps classes 1 and
 *     2 in FP16 and quantizes class 0.
 *   k [dev]: [batch][max_tokens][hkv][128] of k_dtype; q_tail [dev]:
 *   [batch][max_tail][hq][128] of q_dtype (KVQ_F32 / BF16 / F16); n_tokens,
 *   n_tail [dev] int32 [batch] (n_tail <= max_tail <= 64); proxy [dev] float
 *   [batch][hkv][128]; scores [dev] float and token_class [dev] uint8
 *   [batch][hkv][max_tokens]; n_vl [dev] int32 [batch][hkv].
 * Scores are fp32 dot products; the selection is exact on them.  A request whose
 * n_tokens or n_tail is out of range is treated as empty (KVQ_DEVERR_RANGE).
 * Errors: INVALID_ARG, UNSUPPORTED (hkv other than 1, 2, 4, 8, 16), HIP.
 */
kvq_status kvq_select_vertical_lines(const void *k, int32_t k_dtype, const void *q_tail,
                                     int32_t q_dtype, int32_t batch, int32_t max_tokens,
                                     int32_t hkv, int32_t hq, int32_t max_tail,
                                     const int32_t *n_tokens, const int32_t *n_tail,
                                     int32_t window, float rho, float *proxy, float *scores,
                                     uint8_t *token_class, int32_t *n_vl, int32_t *dev_err,
                                     void *stream);

/*
 * Bytes of scratch kvq_prefill_attn needs for these sizes (0 for sizes it rejects).
 * Host only.
 */
size_t kvq_prefill_workspace_bytes(int32_t batch, int32_t n_max, int32_t hkv);

/*
 * Prefill attention with an INT8 prefix (HyQuant, core method: the fused operator
 * O = softmax([Q K-hat_Q^T || Q K_FP^T] / sqrt(d)) [V-hat_Q || V_FP]; Algorithm 2:
 * per-tile symmetric scale max|X_T| / c_B, c_B = 127 for INT8).  For request b
 * (n = n_tokens[b] <= n_max prompt positions), query head j (KV head h = j / g)
 * and query position t < n, over the keys k <= t: a key is read in full precision
 * (K and V as given) when it is a vertical line of h (token_class[b][h][k] == 1,
 * as kvq_select_vertical_lines writes it; NULL = none) or lies in the window
 * k > t - window, and through INT8 otherwise (K-hat = s_K code_K, V-hat =
 * s_V code_V); the query is used as given; one softmax over all of them,
 * out[b][t][j] = sum_k p_k v_k.  INT8: tiles of 64 positions per KV head,
 * separately for K and V (vertical lines left out of the maximum); scale
 * s = fl32(max |x| / 127), code = clamp(rint(fl32(x / s)), -127, 127) (0 when
 * s = 0, and for t >= n).
 *
 * Precision: Q . K-hat and Q . K are bf16 products with fp32 sums (the K codes
 * enter as exact integers, s_K scales the fp32 logit); V and V-hat enter P.V in
 * fp16 (V-hat = s_V code_V rounded once to fp16) with fp16 weights; the result is
 * within the 2e-3 row error of the exact operator for |v| inside fp16's normal
 * range.
 *
 * Two calls, in stream order on one workspace:
 *   kvq_prefill_prepare: the INT8 codes and tile scales of k and v, and the
 *     scratch the attention reads (the K codes as bf16, V and V-hat transposed to
 *     fp16, the keep mask, the vertical-line lists and their gathered K and V);
 *   kvq_prefill_attn: the attention, from what prepare left with the same k,
 *     n_tokens and token_class.
 *   q [dev] bf16 [batch][n_max][hq][128]; k, v [dev] bf16 [batch][n_max][hkv][128]
 *   (|v| < 65504); n_max a multiple of 64; g = hq / hkv in {1, 2, 4, 8, 16}.
 *   k_codes, v_codes [dev] int8 like k, k_scales, v_scales float
 *   [batch][hkv][n_max/64]: written by prepare; attn reads k_scales.  q, k, v and
 *   the codes 16-byte aligned.  workspace [dev]: at least
 *   kvq_prefill_workspace_bytes(batch, n_max, hkv) bytes, 256-byte aligned, owned
 *   by the caller.  out [dev] float [batch][n_max][hq][128] (0 for t >= n).
 * Errors: INVALID_ARG, UNSUPPORTED (dtype other than KVQ_BF16, another g, sizes
 * past 32-bit offsets), CAPACITY (workspace too small), HIP; a request whose
 * n_tokens is out of range is treated as empty (KVQ_DEVERR_RANGE).
 */
kvq_status kvq_prefill_prepare(const void *k, const void *v, int32_t dtype, int32_t batch,
                               int32_t n_max, int32_t hkv, const int32_t *n_tokens,
                               const uint8_t *token_class, int8_t *k_codes, float *k_scales,
                               int8_t *v_codes, float *v_scales, void *workspace,
                               size_t workspace_bytes, int32_t *dev_err, void *stream);
kvq_status kvq_prefill_attn(const void *q, const void *k, int32_t dtype, int32_t batch,
                            int32_t n_max, int32_t hq, int32_t hkv, const int32_t *n_tokens,
                            const uint8_t *token_class, int32_t window, const float *k_scales,
                            const void *workspace, size_t workspace_bytes, float *out,
                            int32_t *dev_err, void *stream);

/*
 * Split-K decode attention (TriAxialKV key design 4, phase 2; HyQuant
 * Algorithm 3).  One work item per split.  Split s = splits[s] [dev] covers
 * tokens [tok_begin, tok_end) of (table, head) in class cls; table t serves
 * request b = t / (hkv / heads_per_page) and KV head
 * kvh = (t % (hkv / heads_per_page)) * heads_per_page + head, whose query heads
 * are kvh*g .. kvh*g + g - 1 (g = hq / hkv; 1 <= g <= 16).
 *   q [dev]: [batch][hq][128] of q_dtype (KVQ_F32 / KVQ_BF16 / KVQ_F16), finite.
 *     Each query head's row enters the products as fp16 after an exact scaling
 *     by a power of two that puts its largest magnitude in [2^14, 2^15): any
 *     finite magnitude fits, BF16 and F16 rows are carried exactly (bf16's 8
 *     significant bits fit fp16's 11), F32 rows are rounded to 11 significant
 *     bits, and channels far below the row's largest keep only their share of
 *     those bits.
 *   tables [dev]: int32 [n_tables][max_entries]: page ids (KVQ_TABLE_PAGES) or
 *     slot ids (KVQ_TABLE_SLOTS); a slot equal to c->sentinel_slot is dead and
 *     excluded from the softmax.  n_tables must equal batch * hkv / heads_per_page.
 *   Every page a split touches must be of the split's class; INT2 splits must
 *   start and end on multiples of 32 tokens and use page tables.
 *   part_o [dev]: float [n_splits][g][128] = sum_t p_t v_t / sum_t p_t;
 *   part_lse [dev]: float [n_splits][g] = natural-log log-sum-exp of the
 *   logits q.k / sqrt(128) over the split's live tokens.  A split with no
 *   live token gives part_o = 0 and part_lse = -inf.
 * Errors: INVALID_ARG, UNSUPPORTED, HIP; device-side KVQ_DEVERR_*.
 */
kvq_status kvq_decode_attn(const kvq_cache *c, const void *q, int32_t q_dtype,
                           int32_t batch, int32_t hq, int32_t hkv,
                           const int32_t *tables, int32_t n_tables, int32_t max_entries,
                           int32_t table_kind, const kvq_split *splits, int32_t n_splits,
                           float *part_o, float *part_lse, int32_t *dev_err, void *stream);

/*
 * Split-K decode attention with shared windows: the same computation as
 * kvq_decode_attn, but the work items are workers that share the 32-token
 * windows of their group (the XCDs of one MI355X stream at rates that differ by a
 * few percent from launch to launch, so a fixed cut leaves the faster ones idle
 * at the end; shared windows let them take more).  Worker s = workers[s] [dev]
 * belongs to group worker_group[s] [dev] (0 <= group < n_groups); the workers of
 * a group carry the same entry (table, head, cls, tok_begin, tok_end): the
 * group's token range, whose windows start at tok_begin rounded down to a page,
 * 32 tokens apart.  Each worker takes windows from the group's counter in blocks
 * (2 windows for INT4, 3 for INT2) and writes the softmax partial of the windows
 * it took: part_o / part_lse row s, as kvq_decode_attn writes a split's (O = 0,
 * lse = -inf if it took none), so kvq_lse_merge combines them unchanged (the
 * workers of a (request, KV head) adjacent).  Page tables only; INT2 and INT4
 * groups are shared; an FP16 group must have one worker (its kernel reads the
 * range whole).  g <= 8.
 *   work [dev]: kvq_decode_work_bytes(n_groups) bytes, all 0 before the first
 *     call (the caller zeroes it once); every call leaves it 0 again when it
 *     completes.  Calls that may overlap must not share it.
 * kvq_plan_workers writes such a plan.  Workers start in a spread order (not in
 * index order) and n_workers must stay below 2^31 - 1.
 * Errors: INVALID_ARG, UNSUPPORTED (slot maps, g > 8), HIP; device-side
 * KVQ_DEVERR_* (a worker whose group is out of range: KVQ_DEVERR_SPLIT).
 */
kvq_status kvq_decode_attn_shared(const kvq_cache *c, const void *q, int32_t q_dtype,
                                  int32_t batch, int32_t hq, int32_t hkv,
                                  const int32_t *tables, int32_t n_tables, int32_t max_entries,
                                  int32_t table_kind, const kvq_split *workers,
                                  const int32_t *worker_group, int32_t n_workers, int32_t n_groups,
                                  int32_t *work, float *part_o, float *part_lse, int32_t *dev_err,
                                  void *stream);

/*
 * kvq_decode_attn_shared for callers that cannot allocate (code under graph
 * capture, tight serving loops, harnesses that forbid allocation): the same call
 * without the work argument; the counters live in a file-scope device array of
 * the library (one per GPU, held until the process ends, about 64 KB), cleared
 * by a small kernel on the stream at every call.  No allocation, no memset.  At
 * most 16384 groups (KVQ_ERR_CAPACITY beyond).  Every call on one GPU uses that
 * GPU's array: calls that may overlap on one GPU (several streams, several
 * threads) race.  Errors as kvq_decode_attn_shared, plus CAPACITY, NO_DEVICE.
 */
kvq_status kvq_decode_attn_shared_noalloc(const kvq_cache *c, const void *q, int32_t q_dtype,
                                          int32_t batch, int32_t hq, int32_t hkv,
                                          const int32_t *tables, int32_t n_tables,
                                          int32_t max_entries, int32_t table_kind,
                                          const kvq_split *workers, const int32_t *worker_group,
                                          int32_t n_workers, int32_t n_groups, float *part_o,
                                          float *part_lse, int32_t *dev_err, void *stream);

/* Bytes of the work counters of kvq_decode_attn_shared for n_groups groups (0 if
 * n_groups < 1).  Host only. */
size_t kvq_decode_work_bytes(int32_t n_groups);

/*
 * Log-sum-exp merge of split partials (TriAxialKV key design 4: global online
 * log-sum-exp reduction; HyQuant Algorithm 3: ReduceSoftmax).  The partials of
 * (request b, KV head kvh) are rows split_offsets[b*hkv + kvh] ..
 * split_offsets[b*hkv + kvh + 1] - 1 of part_o / part_lse ([dev], n_splits rows;
 * offsets are clamped to [0, n_splits]).  For each
 * query head: LSE = log sum_s exp(lse_s), O = sum_s exp(lse_s - LSE) O_s;
 * partials with lse = -inf drop out; no partial gives O = 0, LSE = -inf.
 *   split_offsets [dev]: int32 [batch*hkv + 1], non-decreasing.
 *   out [dev]: [batch][hq][128] of out_dtype; out_lse [dev]: float [batch][hq]
 *   (may be NULL).
 * Errors: INVALID_ARG, HIP.
 */
kvq_status kvq_lse_merge(const float *part_o, const float *part_lse, int32_t n_splits,
                         const int32_t *split_offsets, int32_t batch, int32_t hq,
                         int32_t hkv, void *out, int32_t out_dtype, float *out_lse,
                         void *stream);

/*
 * Split plan [host] (TriAxialKV key design 4: splits of one precision each;
 * Tangram steps 6-7: counts fixed ahead of time).  ranges [host]: the live token
 * ranges of every (table, head), one class each, sorted by (table, head); INT2
 * ranges on 32-token boundaries.  Each range is cut into near-equal pieces
 * (INT2 pieces on 32-token boundaries); the number of pieces is, in order of
 * precedence:
 *   splits_per_head [host, may be NULL]: int32 [n_tables*heads_per_page]
 *     pieces per (table, head), shared among its non-empty ranges in proportion
 *     to their decode cost, tokens x class_cost[cls] (class_cost [host, may be
 *     NULL]: float [3] per INT2 / INT4 / FP16 token-head, all > 0; NULL =
 *     1.0 / 1.0 / 6.0: FP16 splits run in their own kernel after the INT2 /
 *     INT4 one, one wave per SIMD, and the weight gives them about one round
 *     of that kernel at the hybrid-anchor shape), at
 *     least one each, largest remainders first, so a head gets exactly its count
 *     whenever that is at least its number of non-empty ranges;
 *   tokens_per_split[cls] > 0 [host, may be NULL]: ceil(tokens / that);
 *   otherwise max(1, round(range bytes / target_bytes)) with 96 / 160 / 512
 *     bytes per INT2 / INT4 / FP16 token-head.
 * Writes out[0 .. *n_out) [host] sorted by (table, head) and split_offsets
 * [host] int32 [batch*hkv + 1] for kvq_lse_merge.
 * Errors: INVALID_ARG (unsorted or malformed ranges, non-positive costs),
 * CAPACITY (max_out).
 */
kvq_status kvq_plan_splits(const kvq_split *ranges, int32_t n_ranges, int32_t batch,
                           int32_t hkv, int32_t heads_per_page,
                           const int32_t *splits_per_head, const float *class_cost,
                           const int32_t *tokens_per_split, int64_t target_bytes,
                           kvq_split *out, int32_t max_out, int32_t *n_out,
                           int32_t *split_offsets);

/*
 * Split plan per decode kernel [host] (TriAxialKV key design 4; Tangram steps 6-7):
 * the splits of a page-table launch run in two kernels, INT2 / INT4 splits in one
 * and FP16 splits in the other, each best sized to one resident round of its own
 * (kvq_decode_occupancy, kvq_decode_fp16_occupancy).  ranges, outputs and errors
 * as for kvq_plan_splits; per (table, head) i:
 *   int_splits [host] int32 [n_tables*heads_per_page]: pieces shared among its
 *     INT2 / INT4 ranges in proportion to tokens x class_cost[cls];
 *   fp16_splits [host] int32 [n_tables*heads_per_page]: pieces shared among its
 *     FP16 ranges in proportion to tokens;
 * at least one piece per non-empty range, largest remainders first.
 * class_cost [host, may be NULL]: as for kvq_plan_splits.
 */
kvq_status kvq_plan_splits_per_kernel(const kvq_split *ranges, int32_t n_ranges,
                                      int32_t batch, int32_t hkv, int32_t heads_per_page,
                                      const int32_t *int_splits, const int32_t *fp16_splits,
                                      const float *class_cost, kvq_split *out,
                                      int32_t max_out, int32_t *n_out,
                                      int32_t *split_offsets);

/*
 * Shared-work plan [host] for kvq_decode_attn_shared.  ranges as for
 * kvq_plan_splits; every non-empty range is a group.  workers_per_head [host]
 * int32 [n_tables*heads_per_page] is shared among a (table, head)'s non-empty
 * ranges in proportion to tokens x class_cost[cls] (NULL = the kvq_plan_splits
 * default) with at least one worker per range, largest remainders first, at
 * most one worker per window of the range, and one worker for an FP16 range.
 * Writes out[0 .. *n_out) [host] (each worker carries its group's range, sorted
 * by (table, head)), out_group [host] int32 [*n_out], *n_groups, and
 * split_offsets [host] int32 [batch*hkv + 1] for kvq_lse_merge.
 * Errors: INVALID_ARG, CAPACITY (max_out).
 */
kvq_status kvq_plan_workers(const kvq_split *ranges, int32_t n_ranges, int32_t batch,
                            int32_t hkv, int32_t heads_per_page, const int32_t *workers_per_head,
                            const float *class_cost, kvq_split *out, int32_t *out_group,
                            int32_t max_out, int32_t *n_out, int32_t *n_groups,
                            int32_t *split_offsets);

/*
 * Ahead-of-time split counts [host] (Tangram steps 6-7: a partition factor per
 * head group in proportion to its aggregate budget; invariant to context
 * length).  budgets [host] float [hkv]: retained fraction per KV head (> 0).
 * out [host] int32 [batch * hkv]: per (table, head-in-table) in table order,
 * max(1, round(C * budget)) with C = total_work / (batch * sum(budgets)).
 * Errors: INVALID_ARG.
 */
kvq_status kvq_aot_split_counts(const float *budgets, int32_t hkv, int32_t batch,
                                int32_t total_work, int32_t *out);

/*
 * Balanced split counts [host]: the smallest cap c >= 1 on the work of one piece
 * such that sum_i ceil(work[i] / c) over the non-empty entries fits total_work
 * work groups, and out[i] = ceil(work[i] / c) (0 for work[i] == 0).  Every piece
 * of a range cut into out[i] near-equal pieces then holds at most c, so one
 * round of resident work groups ends with no piece much longer than the
 * average (the AOT rule above fixes counts from budgets alone and lets long
 * requests straggle).  work [host] int64 [n] >= 0: e.g. live tokens per (table,
 * head), or tokens x class cost; out [host] int32 [n].  With more non-empty
 * entries than total_work, every non-empty entry gets 1.  Errors: INVALID_ARG.
 */
kvq_status kvq_balanced_split_counts(const int64_t *work, int32_t n, int32_t total_work, int32_t *out);

/*
 * Balanced split plan [host] (TriAxialKV key design 4: splits of one precision each;
 * Tangram steps 6-7: split counts fixed ahead of the decode by each head's work).
 * ranges, out, max_out, n_out and split_offsets as for kvq_plan_splits.  The work
 * of a (table, head) is the sum over its ranges of tokens x class_cost[cls]
 * (class_cost [host, may be NULL]: float [3], all > 0; NULL = the default for g:
 * 1.0 / 1.0 / 6.0 per INT2 / INT4 / FP16 token-head, and 1.0 / 0.82 / 6.0 for
 * 4 < g <= 8, where a wave computes two query tiles and an INT4 window costs less
 * than an INT2 one).  The heads' split counts are kvq_balanced_split_counts of
 * those works over total_splits work groups (so requests of different lengths end
 * together instead of the longest straggling), each shared among the head's ranges
 * as kvq_plan_splits shares splits_per_head.  g [in]: query heads per KV head (the
 * default costs only).  splits_per_head [host, may be NULL]: int32
 * [n_tables*heads_per_page] receives the counts.
 * Errors: INVALID_ARG (as kvq_plan_splits; g or total_splits not positive),
 * CAPACITY (max_out).
 */
kvq_status kvq_plan_balanced(const kvq_split *ranges, int32_t n_ranges, int32_t batch,
                             int32_t hkv, int32_t heads_per_page, int32_t g,
                             int32_t total_splits, const float *class_cost, kvq_split *out,
                             int32_t max_out, int32_t *n_out, int32_t *split_offsets,
                             int32_t *splits_per_head);

/*
 * Head groups of ragged tables and their memory [host] (Tangram: the KV heads of one
 * group share a slot-map table, sized for the group's largest budget, and each head
 * reads its own prefix of it).  budgets [host] float [hkv], 0 < r_h <= 1;
 * heads_per_group H divides hkv.  Heads are grouped by budget: order [host] int32
 * [hkv] receives the head ids by decreasing budget (ties: lower id first), and group
 * i holds order[i H .. i H + H - 1] (consecutive in that order, which minimises the
 * summed table lengths).  For a request of n_tokens, head h keeps ceil(r_h n)
 * tokens and group i's table has table_slots[i] = max over its heads (int32
 * [hkv / H]).  bytes [host] int64 [3], for the cache class cls (KVQ_INT2 / INT4 /
 * FP16; kvq_block_bytes(cls) per head-page of 16 slots):
 *   [0] grouped tables: sum_i ceil(table_slots[i] / 16) H block + 4 table_slots[i];
 *   [1] a table per head: sum_h ceil(ceil(r_h n) / 16) block + 4 ceil(r_h n);
 *   [2] no eviction: hkv ceil(n / 16) (block + 4).
 * Errors: INVALID_ARG.
 */
kvq_status kvq_head_group_plan(const float *budgets, int32_t hkv, int32_t heads_per_group,
                               int64_t n_tokens, int32_t cls, int32_t *order,
                               int32_t *table_slots, int64_t *bytes);

/*
 * Per-wave timeline [profiling builds only] for measuring where a decode launch's
 * time goes (not part of the method).  In a build compiled with KVQ_WAVE_TIMELINE
 * (libkvq_timeline.so), every later fixed-split page-table decode launch on the current
 * device writes, for split s, 8 uint64 words at buffer[8 s ..] [dev, caller-owned,
 * at least 64 B per split]: the wave's start, the landing of its first window and its
 * end (s_memrealtime, 100 MHz), the shader clock (s_memtime) at its start and end, the
 * hardware XCC_ID and HW_ID registers, and its window count.  NULL stops the
 * recording.  Launches that overlap on one device write the same buffer.  Other builds
 * return UNSUPPORTED.  Errors: UNSUPPORTED, HIP.
 */
kvq_status kvq_wave_timeline(void *buffer);

/*
 * Work groups (one wavefront each) of the decode kernel that fit on the current
 * device at once: *per_cu from the HIP occupancy API, *n_cu the compute-unit
 * count.  g (query heads per KV head) and table_kind select the kernel: page
 * tables -> the kernel of INT2 / INT4 splits, slot maps -> the slot-map kernel.
 * A plan with per_cu * n_cu splits runs as one round of waves (Tangram step 6:
 * the total work-group count from the occupancy API).
 * Errors: INVALID_ARG, NO_DEVICE, HIP.
 */
kvq_status kvq_decode_occupancy(int32_t g, int32_t table_kind, int32_t *per_cu, int32_t *n_cu);

/*
 * Work groups of the kernel that runs the FP16 splits of a page-table
 * kvq_decode_attn on the current device (as kvq_decode_occupancy): g and the
 * cache's anchor_format (KVQ_ANCHOR_FP16 / KVQ_ANCHOR_FP8) select it.
 * Errors: INVALID_ARG, NO_DEVICE, HIP.
 */
kvq_status kvq_decode_fp16_occupancy(int32_t g, int32_t anchor_format, int32_t *per_cu,
                                     int32_t *n_cu);

/* Text of a status code, and a description of this thread's last error. */
const char *kvq_status_string(int32_t status);
const char *kvq_last_error(void);

#ifdef __cplusplus
}
#endif
#endif
