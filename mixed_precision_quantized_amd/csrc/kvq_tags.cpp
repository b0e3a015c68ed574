// Tri-axis token tags and greedy INT2 / INT4 width allocation (TriAxialKV key designs 1
// and 2), host code.
//
// Tags: every token gets s(t) = (temporal, modal, semantic) in a 4 x 2 x 7 space, read in
// one pass over the token ids from the chat template's boundary tokens, which the caller
// names (`kvq_tag_marker`).  Widths: every tag starts at 2 bits; tags are visited by
// decreasing rho_k = (D_k(2) - D_k(4)) / (2 N_k) and upgraded to 4 bits while the
// average width stays within the budget; the walk stops at the first tag that would
// break it.
#include <algorithm>
#include <cstdint>
#include <numeric>
#include <vector>

#include "kvq.h"
#include "kvq_internal.h"

using namespace kvq;

namespace {

constexpr int kRoleInst = 0, kRoleUser = 1, kRoleAssistant = 2, kRoleObs = 5;
constexpr int kSemReasoning = 3, kSemToolCall = 4, kSemDelim = 6;

}  // namespace

extern "C" {

kvq_status kvq_tag_tokens(const int32_t *tokens, int32_t n, const kvq_tag_marker *markers, int32_t n_markers,
                          uint8_t *tags, int32_t *n_turns) {
  if (n < 0 || n_markers < 0) return fail(KVQ_ERR_INVALID_ARG, "negative token or marker count");
  if ((n > 0 && (!tokens || !tags)) || (n_markers > 0 && !markers))
    return fail(KVQ_ERR_INVALID_ARG, "NULL tokens, tags or markers");
  std::vector<std::pair<int32_t, int32_t>> table;  // (token id, event), sorted by id
  table.reserve((size_t)n_markers);
  for (int32_t i = 0; i < n_markers; ++i) {
    if (markers[i].event < KVQ_EV_SYSTEM || markers[i].event > KVQ_EV_IMAGE_END)
      return fail(KVQ_ERR_INVALID_ARG, "marker %d has unknown event %d", i, markers[i].event);
    table.emplace_back(markers[i].token_id, markers[i].event);
  }
  std::sort(table.begin(), table.end());
  for (size_t i = 1; i < table.size(); ++i)
    if (table[i].first == table[i - 1].first)
      return fail(KVQ_ERR_INVALID_ARG, "token id %d is named by two markers", table[i].first);
  auto event_of = [&](int32_t id) {
    auto it = std::lower_bound(table.begin(), table.end(), std::make_pair(id, INT32_MIN));
    return it != table.end() && it->first == id ? it->second : -1;
  };
  // One pass: role, reasoning / tool-call spans, image spans, and the turn of every
  // token (a user turn starts a new one; tokens before the first are turn 0).  The
  // temporal axis needs the last turn, so the turn is kept in `tags` until the end.
  std::vector<int32_t> turn_of((size_t)n);
  int role = kRoleInst, turn = 0;
  bool think = false, call = false, image = false;
  for (int32_t i = 0; i < n; ++i) {
    const int ev = event_of(tokens[i]);
    int sem, modal = 0;
    if (ev >= 0) {
      switch (ev) {
        case KVQ_EV_SYSTEM: role = kRoleInst; think = call = image = false; break;
        case KVQ_EV_USER: role = kRoleUser; think = call = image = false; ++turn; break;
        case KVQ_EV_ASSISTANT: role = kRoleAssistant; think = call = image = false; break;
        case KVQ_EV_OBSERVATION: role = kRoleObs; think = call = image = false; break;
        case KVQ_EV_END: think = call = image = false; break;
        case KVQ_EV_THINK_BEGIN: think = true; break;
        case KVQ_EV_THINK_END: think = false; break;
        case KVQ_EV_TOOL_CALL_BEGIN: call = true; break;
        case KVQ_EV_TOOL_CALL_END: call = false; break;
        case KVQ_EV_IMAGE_BEGIN: image = true; break;
        default: image = false; break;  // KVQ_EV_IMAGE_END
      }
      sem = kSemDelim;  // a boundary token is a template delimiter (text)
    } else {
      sem = call ? kSemToolCall : think ? kSemReasoning : role;
      modal = image ? 1 : 0;
    }
    turn_of[(size_t)i] = turn;
    tags[i] = (uint8_t)(modal * KVQ_N_SEMANTIC + sem);  // temporal added below
  }
  for (int32_t i = 0; i < n; ++i) {
    const int temporal = std::min(turn - turn_of[(size_t)i], KVQ_N_TEMPORAL - 1);
    tags[i] = (uint8_t)(temporal * KVQ_N_MODAL * KVQ_N_SEMANTIC + tags[i]);
  }
  if (n_turns) *n_turns = turn;
  return KVQ_OK;
}

kvq_status kvq_allocate_bits(const double *d2, const double *d4, const int64_t *counts, int32_t n_tags,
                             double budget_bits, uint8_t *bits, double *avg_bits) {
  if (n_tags < 0 || !(budget_bits >= 2.0 && budget_bits <= 4.0))
    return fail(KVQ_ERR_INVALID_ARG, "negative tag count or budget outside [2, 4] bits");
  if (n_tags > 0 && (!d2 || !d4 || !counts || !bits)) return fail(KVQ_ERR_INVALID_ARG, "NULL tag arrays");
  int64_t total = 0;
  for (int32_t k = 0; k < n_tags; ++k) {
    if (counts[k] < 0) return fail(KVQ_ERR_INVALID_ARG, "count of tag %d is negative", k);
    total += counts[k];
    bits[k] = 2;
  }
  // Tags with tokens, by decreasing rho_k = (D_k(2) - D_k(4)) / (2 N_k); ties by index.
  std::vector<int32_t> order;
  for (int32_t k = 0; k < n_tags; ++k)
    if (counts[k] > 0) order.push_back(k);
  auto rho = [&](int32_t k) { return (d2[k] - d4[k]) / (2.0 * (double)counts[k]); };
  std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t b) { return rho(a) > rho(b); });
  // Upgrade while sum N_k b_k <= B sum N_k holds (in integer token-bits against the
  // budget times the token count); stop at the first tag that would break it.
  const double cap = budget_bits * (double)total;
  int64_t used = 2 * total;
  for (int32_t k : order) {
    if ((double)(used + 2 * counts[k]) > cap) break;
    used += 2 * counts[k];
    bits[k] = 4;
  }
  if (avg_bits) *avg_bits = total > 0 ? (double)used / (double)total : 2.0;
  return KVQ_OK;
}

kvq_status kvq_count_tags(const uint8_t *tags, int32_t n, int64_t *counts) {
  if (n < 0) return fail(KVQ_ERR_INVALID_ARG, "negative count");
  if (!counts || (n > 0 && !tags)) return fail(KVQ_ERR_INVALID_ARG, "NULL tags or counts");
  for (int32_t i = 0; i < n; ++i)
    if (tags[i] >= KVQ_N_TAGS) return fail(KVQ_ERR_INVALID_ARG, "tag %u at %d outside [0, %d)", tags[i], i, KVQ_N_TAGS);
  for (int32_t i = 0; i < n; ++i) ++counts[tags[i]];  // N_k, the tokens of each tag
  return KVQ_OK;
}

kvq_status kvq_tag_flags(const uint8_t *tags, int32_t n, const uint8_t *bits, int32_t n_tags, uint8_t *flags) {
  if (n < 0 || n_tags < 0) return fail(KVQ_ERR_INVALID_ARG, "negative count");
  if (n > 0 && (!tags || !bits || !flags)) return fail(KVQ_ERR_INVALID_ARG, "NULL tags, bits or flags");
  for (int32_t i = 0; i < n; ++i) {
    if (tags[i] >= n_tags) return fail(KVQ_ERR_INVALID_ARG, "tag %u at %d outside [0, %d)", tags[i], i, n_tags);
    if (bits[tags[i]] != 2 && bits[tags[i]] != 4)
      return fail(KVQ_ERR_INVALID_ARG, "tag %u has width %u", tags[i], bits[tags[i]]);
    flags[i] = bits[tags[i]] == 2 ? 0 : 1;  // the routing flags of kvq_route_tokens
  }
  return KVQ_OK;
}

}  // extern "C"
