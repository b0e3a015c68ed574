// Host-only parts of libkvq: status text, argument checks, token routing and
// split planning.  No device code and no HIP calls here.
#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <utility>
#include <vector>

#include "kvq_internal.h"

namespace kvq {

static thread_local char g_last_error[512] = "";

kvq_status fail(kvq_status st, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

kvq_status check_cache(const kvq_cache *c) {
  if (!c) return fail(KVQ_ERR_INVALID_ARG, "cache descriptor is NULL");
  if (c->head_dim != kHeadDim)
    return fail(KVQ_ERR_UNSUPPORTED, "head_dim %d is not supported (only 128)", c->head_dim);
  if (c->page_size != kPage)
    return fail(KVQ_ERR_UNSUPPORTED, "page_size %d is not supported (only 16)", c->page_size);
  if (c->heads_per_page < 1) return fail(KVQ_ERR_INVALID_ARG, "heads_per_page must be >= 1");
  if (c->anchor_format != KVQ_ANCHOR_FP16 && c->anchor_format != KVQ_ANCHOR_FP8)
    return fail(KVQ_ERR_INVALID_ARG, "unknown anchor format %d", c->anchor_format);
  int64_t total = 0;
  for (int i = 0; i < 3; ++i) {
    if (c->n_pages[i] < 0) return fail(KVQ_ERR_INVALID_ARG, "n_pages[%d] is negative", i);
    if (c->n_pages[i] > 0 && !c->pool[i])
      return fail(KVQ_ERR_INVALID_ARG, "pool[%d] is NULL but holds %d pages", i, c->n_pages[i]);
    total += c->n_pages[i];
  }
  if (c->n_pages[KVQ_INT2] % 2)
    return fail(KVQ_ERR_INVALID_ARG, "the INT2 pool must hold whole page pairs");
  if (total * kPage > INT32_MAX) return fail(KVQ_ERR_UNSUPPORTED, "too many pages for int32 slot ids");
  if (c->sentinel_slot < -1 || c->sentinel_slot >= total * kPage)
    return fail(KVQ_ERR_INVALID_ARG, "sentinel_slot %d is outside the pools", c->sentinel_slot);
  return KVQ_OK;
}

static int64_t token_bytes(int cls) { return cls == KVQ_INT2 ? 96 : cls == KVQ_INT4 ? 160 : 512; }

// Default relative decode time of one token-head per class on MI355X, used to share a
// head's split count among its ranges.  INT2 windows are bound by dequantization work
// and INT4 ones by their bytes, which takes about as long per token (measured: a
// weight of 1.0 for INT4 beat 0.8 and 1.15-1.8); FP16 windows move 512 B per token and
// run in their own kernel after the others, one wave per SIMD (measured on the
// hybrid-anchor decode at 12 splits per head: 6.0 gave 557 us per layer against 575 us
// for 8.0 and 606 us for 12.0: four FP16 splits per head, one resident round).
static const float kDefaultTokenCost[3] = {1.0f, 1.0f, 6.0f};
// With two query tiles per wave (g = 5 .. 8) an INT2 window costs more than an INT4 one:
// its key build and the two tiles' zero terms take more dequantization work, while the
// INT4 window's extra bytes hide behind it.  Measured on the Qwen3-VL-32B-shaped decode
// (g = 8): INT4 splits given the same tokens x cost as INT2 splits of their head took
// 0.82 of their time (per-split timestamps, 136 against 167 us).
static const float kTwoTileTokenCost[3] = {1.0f, 0.82f, 6.0f};

static const float *default_token_cost(int32_t g) { return g > 4 && g <= 8 ? kTwoTileTokenCost : kDefaultTokenCost; }

}  // namespace kvq

using namespace kvq;

namespace {

// Checks a plan's ranges: well formed, INT2 ranges on 32-token boundaries, sorted by
// (table, head).
kvq_status check_ranges(const kvq_split *ranges, int32_t n_ranges, int32_t n_tables, int32_t heads_per_page) {
  for (int32_t i = 0; i < n_ranges; ++i) {
    const kvq_split &r = ranges[i];
    if (r.table < 0 || r.table >= n_tables || r.head < 0 || r.head >= heads_per_page || r.cls < 0 ||
        r.cls > 2 || r.tok_begin < 0 || r.tok_end < r.tok_begin)
      return fail(KVQ_ERR_INVALID_ARG, "malformed range %d", i);
    if (r.cls == KVQ_INT2 && (r.tok_begin % kGroup || r.tok_end % kGroup))
      return fail(KVQ_ERR_INVALID_ARG, "INT2 range %d is not on 32-token boundaries", i);
    if (i > 0) {
      const kvq_split &p = ranges[i - 1];
      if (p.table > r.table || (p.table == r.table && p.head > r.head))
        return fail(KVQ_ERR_INVALID_ARG, "ranges are not sorted by (table, head) at %d", i);
    }
  }
  return KVQ_OK;
}

// Shares `total` pieces among the non-empty ranges i0 .. i1 - 1 that `take` accepts, in
// proportion to tokens x cost[cls]: one piece each, the rest by largest remainders, so
// the shares add up to `total` whenever it is at least the number of ranges.
template <typename Take>
void share_pieces(const kvq_split *ranges, int32_t i0, int32_t i1, int64_t total, const float *cost, Take take,
                  std::vector<int64_t> &pieces) {
  double cost_sum = 0.0;
  int32_t n_live = 0;
  for (int32_t i = i0; i < i1; ++i) {
    const int64_t toks = ranges[i].tok_end - ranges[i].tok_begin;
    if (toks == 0 || !take(ranges[i])) continue;
    ++n_live;
    cost_sum += (double)toks * (double)cost[ranges[i].cls];
  }
  if (n_live == 0) return;
  const int64_t spare = std::max<int64_t>(0, total - n_live);  // beyond one piece each
  std::vector<std::pair<double, int32_t>> frac;
  int64_t given = 0;
  for (int32_t i = i0; i < i1; ++i) {
    const int64_t toks = ranges[i].tok_end - ranges[i].tok_begin;
    if (toks == 0 || !take(ranges[i])) continue;
    const double share = (double)spare * (double)toks * (double)cost[ranges[i].cls] / cost_sum;
    const int64_t whole = (int64_t)std::floor(share);
    pieces[i] = 1 + whole;
    given += whole;
    frac.push_back({share - (double)whole, i});
  }
  std::stable_sort(frac.begin(), frac.end(),
                   [](const std::pair<double, int32_t> &x, const std::pair<double, int32_t> &y) {
                     return x.first > y.first;
                   });
  for (size_t k = 0; given < spare && k < frac.size(); ++k, ++given) ++pieces[frac[k].second];
}

// Cuts every range into its number of near-equal pieces (INT2 pieces on 32-token
// boundaries) and writes the splits and the merge offsets.
kvq_status emit_plan(const kvq_split *ranges, int32_t n_ranges, int32_t batch, int32_t hkv, int32_t heads_per_page,
                     const std::vector<int64_t> &pieces, kvq_split *out, int32_t max_out, int32_t *n_out,
                     int32_t *split_offsets) {
  const int32_t tpr = hkv / heads_per_page;
  int32_t w = 0;
  int32_t next_pair = 0;  // next (b*hkv + kvh) whose offset is still unset
  for (int32_t i = 0; i < n_ranges; ++i) {
    const kvq_split &r = ranges[i];
    const int32_t pair = (r.table / tpr) * hkv + (r.table % tpr) * heads_per_page + r.head;
    while (next_pair <= pair) split_offsets[next_pair++] = w;
    const int32_t unit = r.cls == KVQ_INT2 ? kGroup : 1;
    const int64_t units = (r.tok_end - r.tok_begin) / unit;
    if (units == 0) continue;
    const int64_t n = std::min(pieces[i], units);
    for (int64_t p = 0; p < n; ++p) {
      if (w >= max_out) return fail(KVQ_ERR_CAPACITY, "more than %d splits", max_out);
      const int64_t a = units * p / n, b = units * (p + 1) / n;
      out[w++] = kvq_split{r.table, r.head, r.cls, (int32_t)(r.tok_begin + a * unit),
                           p + 1 == n ? r.tok_end : (int32_t)(r.tok_begin + b * unit)};
    }
  }
  while (next_pair <= batch * hkv) split_offsets[next_pair++] = w;
  *n_out = w;
  return KVQ_OK;
}

// The smallest cap c >= 1 on one piece's work such that sum_i ceil(work[i] / c) fits
// total (the largest work when nothing fits).
int64_t balanced_cap(const int64_t *work, int32_t n, int64_t total) {
  int64_t lo = 1, hi = 1;
  for (int32_t i = 0; i < n; ++i) hi = std::max(hi, work[i]);
  auto pieces = [&](int64_t cap) {  // non-increasing in cap; at cap = max work, one per entry
    int64_t sum = 0;
    for (int32_t i = 0; i < n; ++i) sum += (work[i] + cap - 1) / cap;
    return sum;
  };
  while (lo < hi) {
    const int64_t mid = lo + (hi - lo) / 2;
    if (pieces(mid) <= total) hi = mid;
    else lo = mid + 1;
  }
  return lo;
}

// The ranges of one (table, head): i0 .. i1 - 1.
int32_t head_end(const kvq_split *ranges, int32_t n_ranges, int32_t i0) {
  int32_t i1 = i0 + 1;
  while (i1 < n_ranges && ranges[i1].table == ranges[i0].table && ranges[i1].head == ranges[i0].head) ++i1;
  return i1;
}

}  // namespace

extern "C" {

size_t kvq_block_bytes(int32_t cls) {
  return cls == KVQ_INT2 ? kI2Bytes : cls == KVQ_INT4 ? kI4Bytes : cls == KVQ_FP16 ? kF16Bytes
       : cls == KVQ_FP8_ANCHOR_BLOCK ? kF8Bytes : 0;
}

const char *kvq_status_string(int32_t st) {
  switch (st) {
    case KVQ_OK: return "ok";
    case KVQ_ERR_INVALID_ARG: return "invalid argument";
    case KVQ_ERR_UNSUPPORTED: return "unsupported";
    case KVQ_ERR_CAPACITY: return "output capacity too small";
    case KVQ_ERR_HIP: return "HIP runtime error";
    case KVQ_ERR_NO_DEVICE: return "no usable device";
    default: return "unknown status";
  }
}

const char *kvq_last_error(void) { return g_last_error; }

kvq_status kvq_route_tokens(const uint8_t *flags, int32_t n, uint8_t *cls_out, int32_t *n_int2_groups,
                            int32_t *n_int4, int32_t *n_fp16) {
  if (n < 0) return fail(KVQ_ERR_INVALID_ARG, "negative token count");
  if (n > 0 && (!flags || !cls_out)) return fail(KVQ_ERR_INVALID_ARG, "NULL flags or output");
  // First pass: how many INT2-flagged tokens fill whole groups of 32.
  int32_t wants_int2 = 0;
  for (int32_t i = 0; i < n; ++i) {
    if (flags[i] > 2) return fail(KVQ_ERR_INVALID_ARG, "flag %u at %d is not 0, 1 or 2", flags[i], i);
    wants_int2 += flags[i] == 0;
  }
  const int32_t grouped = wants_int2 - wants_int2 % kGroup;
  int32_t seen = 0, c4 = 0, c16 = 0;
  for (int32_t i = 0; i < n; ++i) {
    uint8_t cls;
    if (flags[i] == 0) cls = seen++ < grouped ? KVQ_INT2 : KVQ_INT4;  // residual tail -> INT4
    else cls = flags[i] == 1 ? KVQ_INT4 : KVQ_FP16;
    c4 += cls == KVQ_INT4;
    c16 += cls == KVQ_FP16;
    cls_out[i] = cls;
  }
  if (n_int2_groups) *n_int2_groups = grouped / kGroup;
  if (n_int4) *n_int4 = c4;
  if (n_fp16) *n_fp16 = c16;
  return KVQ_OK;
}

kvq_status kvq_plan_splits(const kvq_split *ranges, int32_t n_ranges, int32_t batch, int32_t hkv,
                           int32_t heads_per_page, const int32_t *splits_per_head,
                           const float *class_cost, const int32_t *tokens_per_split, int64_t target_bytes,
                           kvq_split *out, int32_t max_out, int32_t *n_out, int32_t *split_offsets) {
  const float *cost = class_cost ? class_cost : kDefaultTokenCost;
  for (int c = 0; c < 3; ++c)
    if (!(cost[c] > 0.0f)) return fail(KVQ_ERR_INVALID_ARG, "class cost %d is not positive", c);
  if (n_ranges < 0 || batch < 0 || hkv <= 0 || heads_per_page <= 0 || hkv % heads_per_page)
    return fail(KVQ_ERR_INVALID_ARG, "bad plan shape");
  if ((n_ranges > 0 && !ranges) || !n_out || !split_offsets || (max_out > 0 && !out))
    return fail(KVQ_ERR_INVALID_ARG, "NULL plan array");
  const int32_t n_tables = batch * (hkv / heads_per_page);
  kvq_status st = check_ranges(ranges, n_ranges, n_tables, heads_per_page);
  if (st != KVQ_OK) return st;
  // Pieces per range.
  std::vector<int64_t> pieces((size_t)n_ranges, 0);
  for (int32_t i0 = 0, i1; i0 < n_ranges; i0 = i1) {
    i1 = head_end(ranges, n_ranges, i0);
    if (splits_per_head) {
      share_pieces(ranges, i0, i1, splits_per_head[(size_t)ranges[i0].table * heads_per_page + ranges[i0].head],
                   cost, [](const kvq_split &) { return true; }, pieces);
    } else {
      for (int32_t i = i0; i < i1; ++i) {
        const kvq_split &r = ranges[i];
        const int64_t toks = r.tok_end - r.tok_begin;
        if (toks == 0) continue;
        if (tokens_per_split && tokens_per_split[r.cls] > 0)
          pieces[i] = (toks + tokens_per_split[r.cls] - 1) / tokens_per_split[r.cls];
        else if (target_bytes > 0)
          pieces[i] = std::max<int64_t>(1, std::llround((double)(toks * token_bytes(r.cls)) / (double)target_bytes));
        else
          pieces[i] = 1;
      }
    }
  }
  return emit_plan(ranges, n_ranges, batch, hkv, heads_per_page, pieces, out, max_out, n_out, split_offsets);
}

kvq_status kvq_plan_splits_per_kernel(const kvq_split *ranges, int32_t n_ranges, int32_t batch, int32_t hkv,
                                      int32_t heads_per_page, const int32_t *int_splits,
                                      const int32_t *fp16_splits, const float *class_cost, kvq_split *out,
                                      int32_t max_out, int32_t *n_out, int32_t *split_offsets) {
  const float *cost = class_cost ? class_cost : kDefaultTokenCost;
  for (int c = 0; c < 3; ++c)
    if (!(cost[c] > 0.0f)) return fail(KVQ_ERR_INVALID_ARG, "class cost %d is not positive", c);
  if (n_ranges < 0 || batch < 0 || hkv <= 0 || heads_per_page <= 0 || hkv % heads_per_page)
    return fail(KVQ_ERR_INVALID_ARG, "bad plan shape");
  if ((n_ranges > 0 && (!ranges || !int_splits || !fp16_splits)) || !n_out || !split_offsets ||
      (max_out > 0 && !out))
    return fail(KVQ_ERR_INVALID_ARG, "NULL plan array");
  const int32_t n_tables = batch * (hkv / heads_per_page);
  kvq_status st = check_ranges(ranges, n_ranges, n_tables, heads_per_page);
  if (st != KVQ_OK) return st;
  std::vector<int64_t> pieces((size_t)n_ranges, 0);
  for (int32_t i0 = 0, i1; i0 < n_ranges; i0 = i1) {
    i1 = head_end(ranges, n_ranges, i0);
    const size_t h = (size_t)ranges[i0].table * heads_per_page + ranges[i0].head;
    share_pieces(ranges, i0, i1, int_splits[h], cost, [](const kvq_split &r) { return r.cls != KVQ_FP16; },
                 pieces);
    share_pieces(ranges, i0, i1, fp16_splits[h], cost, [](const kvq_split &r) { return r.cls == KVQ_FP16; },
                 pieces);
  }
  return emit_plan(ranges, n_ranges, batch, hkv, heads_per_page, pieces, out, max_out, n_out, split_offsets);
}

// Shared-work plan: every range is a group whose windows its workers share; a head's
// worker count is shared among its ranges in proportion to decode cost (largest
// remainders, at least one worker per range, at most one per 32-token window), FP16
// ranges get one worker each (their kernel does not share).
kvq_status kvq_plan_workers(const kvq_split *ranges, int32_t n_ranges, int32_t batch, int32_t hkv,
                            int32_t heads_per_page, const int32_t *workers_per_head, const float *class_cost,
                            kvq_split *out, int32_t *out_group, int32_t max_out, int32_t *n_out, int32_t *n_groups,
                            int32_t *split_offsets) {
  const float *cost = class_cost ? class_cost : kDefaultTokenCost;
  for (int c = 0; c < 3; ++c)
    if (!(cost[c] > 0.0f)) return fail(KVQ_ERR_INVALID_ARG, "class cost %d is not positive", c);
  if (n_ranges < 0 || batch < 0 || hkv <= 0 || heads_per_page <= 0 || hkv % heads_per_page)
    return fail(KVQ_ERR_INVALID_ARG, "bad plan shape");
  if ((n_ranges > 0 && (!ranges || !workers_per_head)) || !n_out || !n_groups || !split_offsets ||
      (max_out > 0 && (!out || !out_group)))
    return fail(KVQ_ERR_INVALID_ARG, "NULL plan array");
  const int32_t tpr = hkv / heads_per_page;
  const int32_t n_tables = batch * tpr;
  for (int32_t i = 0; i < n_ranges; ++i) {
    const kvq_split &r = ranges[i];
    if (r.table < 0 || r.table >= n_tables || r.head < 0 || r.head >= heads_per_page || r.cls < 0 ||
        r.cls > 2 || r.tok_begin < 0 || r.tok_end < r.tok_begin)
      return fail(KVQ_ERR_INVALID_ARG, "malformed range %d", i);
    if (r.cls == KVQ_INT2 && (r.tok_begin % kGroup || r.tok_end % kGroup))
      return fail(KVQ_ERR_INVALID_ARG, "INT2 range %d is not on 32-token boundaries", i);
    if (i > 0) {
      const kvq_split &p = ranges[i - 1];
      if (p.table > r.table || (p.table == r.table && p.head > r.head))
        return fail(KVQ_ERR_INVALID_ARG, "ranges are not sorted by (table, head) at %d", i);
    }
  }
  auto windows = [](const kvq_split &r) -> int64_t {
    return r.tok_end > r.tok_begin ? (r.tok_end - (r.tok_begin & ~(kPage - 1)) + 31) / 32 : 0;
  };
  std::vector<int64_t> workers((size_t)n_ranges, 0);
  for (int32_t i0 = 0, i1; i0 < n_ranges; i0 = i1) {
    i1 = i0 + 1;
    while (i1 < n_ranges && ranges[i1].table == ranges[i0].table && ranges[i1].head == ranges[i0].head) ++i1;
    const int64_t total = workers_per_head[(size_t)ranges[i0].table * heads_per_page + ranges[i0].head];
    if (total < 0) return fail(KVQ_ERR_INVALID_ARG, "negative worker count");
    double cost_sum = 0.0;
    int32_t n_live = 0;
    for (int32_t i = i0; i < i1; ++i) {
      if (windows(ranges[i]) == 0) continue;
      ++n_live;
      if (ranges[i].cls != KVQ_FP16)
        cost_sum += (double)(ranges[i].tok_end - ranges[i].tok_begin) * (double)cost[ranges[i].cls];
    }
    if (n_live == 0) continue;
    const int64_t spare = std::max<int64_t>(0, total - n_live);  // beyond one worker each
    std::vector<std::pair<double, int32_t>> frac;
    int64_t given = 0;
    for (int32_t i = i0; i < i1; ++i) {
      if (windows(ranges[i]) == 0) continue;
      workers[i] = 1;
      if (ranges[i].cls == KVQ_FP16 || cost_sum <= 0.0) continue;
      const double share =
          (double)spare * (double)(ranges[i].tok_end - ranges[i].tok_begin) * (double)cost[ranges[i].cls] / cost_sum;
      const int64_t whole = (int64_t)std::floor(share);
      workers[i] += whole;
      given += whole;
      frac.push_back({share - (double)whole, i});
    }
    std::stable_sort(frac.begin(), frac.end(),
                     [](const std::pair<double, int32_t> &x, const std::pair<double, int32_t> &y) {
                       return x.first > y.first;
                     });
    for (size_t k = 0; given < spare && k < frac.size(); ++k, ++given) ++workers[frac[k].second];
    for (int32_t i = i0; i < i1; ++i) workers[i] = std::min(workers[i], windows(ranges[i]));
  }
  int32_t w = 0, groups = 0;
  int32_t next_pair = 0;
  for (int32_t i = 0; i < n_ranges; ++i) {
    const kvq_split &r = ranges[i];
    const int32_t pair = (r.table / tpr) * hkv + (r.table % tpr) * heads_per_page + r.head;
    while (next_pair <= pair) split_offsets[next_pair++] = w;
    if (workers[i] == 0) continue;
    for (int64_t p = 0; p < workers[i]; ++p) {
      if (w >= max_out) return fail(KVQ_ERR_CAPACITY, "more than %d workers", max_out);
      out_group[w] = groups;
      out[w++] = r;
    }
    ++groups;
  }
  while (next_pair <= batch * hkv) split_offsets[next_pair++] = w;
  *n_out = w;
  *n_groups = groups;
  return KVQ_OK;
}

size_t kvq_decode_work_bytes(int32_t n_groups) {
  // the groups' window counters, then 64 + 1 counters of finished workers
  return n_groups > 0 ? (size_t)(n_groups + 65) * sizeof(int32_t) : 0;
}

kvq_status kvq_balanced_split_counts(const int64_t *work, int32_t n, int32_t total_work, int32_t *out) {
  if (!work || !out || n <= 0 || total_work <= 0) return fail(KVQ_ERR_INVALID_ARG, "bad balanced-count arguments");
  for (int32_t i = 0; i < n; ++i)
    if (work[i] < 0) return fail(KVQ_ERR_INVALID_ARG, "work[%d] is negative", i);
  const int64_t cap = balanced_cap(work, n, total_work);
  for (int32_t i = 0; i < n; ++i) out[i] = (int32_t)((work[i] + cap - 1) / cap);
  return KVQ_OK;
}

kvq_status kvq_plan_balanced(const kvq_split *ranges, int32_t n_ranges, int32_t batch, int32_t hkv,
                             int32_t heads_per_page, int32_t g, int32_t total_splits, const float *class_cost,
                             kvq_split *out, int32_t max_out, int32_t *n_out, int32_t *split_offsets,
                             int32_t *splits_per_head) {
  if (g <= 0 || total_splits <= 0) return fail(KVQ_ERR_INVALID_ARG, "g and total_splits must be positive");
  const float *cost = class_cost ? class_cost : default_token_cost(g);
  for (int c = 0; c < 3; ++c)
    if (!(cost[c] > 0.0f)) return fail(KVQ_ERR_INVALID_ARG, "class cost %d is not positive", c);
  if (n_ranges < 0 || batch < 0 || hkv <= 0 || heads_per_page <= 0 || hkv % heads_per_page)
    return fail(KVQ_ERR_INVALID_ARG, "bad plan shape");
  if ((n_ranges > 0 && !ranges) || !n_out || !split_offsets || (max_out > 0 && !out))
    return fail(KVQ_ERR_INVALID_ARG, "NULL plan array");
  const int32_t n_tables = batch * (hkv / heads_per_page);
  kvq_status st = check_ranges(ranges, n_ranges, n_tables, heads_per_page);
  if (st != KVQ_OK) return st;
  // Work of every (table, head): its tokens x class cost, in 1/256 token units.
  const size_t n_heads = (size_t)n_tables * heads_per_page;
  std::vector<int64_t> work(n_heads, 0);
  for (int32_t i = 0; i < n_ranges; ++i) {
    const kvq_split &r = ranges[i];
    work[(size_t)r.table * heads_per_page + r.head] +=
        std::llround(256.0 * (double)(r.tok_end - r.tok_begin) * (double)cost[r.cls]);
  }
  std::vector<int32_t> counts(n_heads, 0);
  if (n_heads > 0) {
    const int64_t cap = balanced_cap(work.data(), (int32_t)n_heads, total_splits);
    for (size_t h = 0; h < n_heads; ++h) counts[h] = (int32_t)((work[h] + cap - 1) / cap);
  }
  if (splits_per_head)
    for (size_t h = 0; h < n_heads; ++h) splits_per_head[h] = counts[h];
  std::vector<int64_t> pieces((size_t)n_ranges, 0);
  for (int32_t i0 = 0, i1; i0 < n_ranges; i0 = i1) {
    i1 = head_end(ranges, n_ranges, i0);
    share_pieces(ranges, i0, i1, counts[(size_t)ranges[i0].table * heads_per_page + ranges[i0].head], cost,
                 [](const kvq_split &) { return true; }, pieces);
  }
  return emit_plan(ranges, n_ranges, batch, hkv, heads_per_page, pieces, out, max_out, n_out, split_offsets);
}

kvq_status kvq_head_group_plan(const float *budgets, int32_t hkv, int32_t heads_per_group, int64_t n_tokens,
                               int32_t cls, int32_t *order, int32_t *table_slots, int64_t *bytes) {
  if (!budgets || !order || !table_slots || !bytes || hkv <= 0 || heads_per_group <= 0 ||
      hkv % heads_per_group || n_tokens < 0 || n_tokens > INT32_MAX)
    return fail(KVQ_ERR_INVALID_ARG, "bad head-group arguments");
  if (cls != KVQ_INT2 && cls != KVQ_INT4 && cls != KVQ_FP16) return fail(KVQ_ERR_INVALID_ARG, "unknown class %d", cls);
  std::vector<int64_t> keep((size_t)hkv);
  for (int32_t h = 0; h < hkv; ++h) {
    if (!(budgets[h] > 0.0f && budgets[h] <= 1.0f)) return fail(KVQ_ERR_INVALID_ARG, "budget of head %d outside (0, 1]", h);
    keep[(size_t)h] = (int64_t)std::ceil((double)budgets[h] * (double)n_tokens);
    order[h] = h;
  }
  // Exchange argument: for groups of a fixed size, the padded total sum_i H max_i is
  // smallest when each group takes the next H heads in decreasing order of budget.
  std::stable_sort(order, order + hkv, [&](int32_t a, int32_t b) { return budgets[a] > budgets[b]; });
  const int64_t block = (int64_t)kvq_block_bytes(cls), page = kPage;
  auto pages = [&](int64_t slots) { return (slots + page - 1) / page; };
  int64_t grouped = 0, exact = 0;
  for (int32_t i = 0; i < hkv / heads_per_group; ++i) {
    int64_t slots = 0;
    for (int32_t k = 0; k < heads_per_group; ++k) slots = std::max(slots, keep[(size_t)order[i * heads_per_group + k]]);
    table_slots[i] = (int32_t)slots;
    grouped += pages(slots) * heads_per_group * block + 4 * slots;
  }
  for (int32_t h = 0; h < hkv; ++h) exact += pages(keep[(size_t)h]) * block + 4 * keep[(size_t)h];
  bytes[0] = grouped;
  bytes[1] = exact;
  bytes[2] = (int64_t)hkv * pages(n_tokens) * (block + 4);
  return KVQ_OK;
}

kvq_status kvq_aot_split_counts(const float *budgets, int32_t hkv, int32_t batch, int32_t total_work,
                                int32_t *out) {
  if (!budgets || !out || hkv <= 0 || batch <= 0 || total_work <= 0)
    return fail(KVQ_ERR_INVALID_ARG, "bad AOT split-count arguments");
  double sum = 0.0;
  for (int32_t h = 0; h < hkv; ++h) {
    if (!(budgets[h] > 0.0f)) return fail(KVQ_ERR_INVALID_ARG, "budget of head %d is not positive", h);
    sum += budgets[h];
  }
  const double per_unit = (double)total_work / ((double)batch * sum);
  for (int32_t b = 0; b < batch; ++b)
    for (int32_t h = 0; h < hkv; ++h)
      out[(size_t)b * hkv + h] = (int32_t)std::max<long long>(1, std::llround(per_unit * budgets[h]));
  return KVQ_OK;
}

}  // extern "C"
