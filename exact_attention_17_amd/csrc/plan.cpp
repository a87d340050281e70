// Host-side plans for varlen prefill and paged decode: the "plan" half of a
// plan/run split.
//
// The "FIA / FlashAttention" explainer (sec. 2, FlashInfer's decoupled plan
// and run) has a host-side plan step that sees the variable sequence lengths
// and balances the load before a run step executes the whole batch.  Here
// the unit of work is one query tile (kBlockM query rows of one sequence, all
// query heads) and its cost is the number of kBlockN-key tiles the kernel
// visits for it under the causal / sliding-window mask.  For decode (the
// page's own example is FlashInfer's batch-decode plan) the unit is one key
// split of one request, all KV heads, and its cost is the number of keys it
// reads; only splits that hold a key are listed, so no workgroup of the run
// starts only to find it has nothing to do.  Dispatching the items heaviest
// first lets the short items fill the gaps left at the end of the launch,
// instead of one long item starting last and running alone
// (longest-processing-time ordering for identical parallel machines).
//
// This file makes no HIP call: the plan is computed from host copies of the
// cumulative sequence lengths and uploaded by the caller.

#include <algorithm>
#include <cstdint>
#include <numeric>
#include <vector>

#include "fa.h"
#include "fa_internal.h"

namespace {

// Key tiles the prefill kernel visits for query rows [r0, r1] of a sequence
// with Lq queries and Lk keys (bottom-right causal alignment, inclusive
// window bounds, -1 = unbounded side).
int64_t key_tiles(int r0, int r1, int Lq, int Lk, int causal, int wl, int wr) {
  const int64_t delta = (int64_t)Lk - Lq;
  const int64_t lo = wl >= 0 ? std::max<int64_t>(0, r0 + delta - wl) : 0;
  int64_t hi = Lk;
  if (causal) hi = std::min<int64_t>(hi, r1 + delta + 1);
  if (wr >= 0) hi = std::min<int64_t>(hi, r1 + delta + wr + 1);
  if (hi <= lo) return 0;
  return (hi + fa::kBlockN - 1) / fa::kBlockN - lo / fa::kBlockN;
}

}  // namespace

extern "C" {

fa_status fa_varlen_plan(const int* cu_seqlens_q, const int* cu_seqlens_k, int B, int causal,
                         int window_left, int window_right, int* plan, int plan_capacity,
                         int* num_items) {
  if (!cu_seqlens_q || !cu_seqlens_k || !num_items || B < 1) return FA_ERR_INVALID_ARG;
  if ((causal != 0 && causal != 1) || window_left < -1 || window_right < -1)
    return FA_ERR_INVALID_ARG;
  if (cu_seqlens_q[0] != 0 || cu_seqlens_k[0] != 0) return FA_ERR_INVALID_ARG;
  int64_t count = 0;
  for (int b = 0; b < B; ++b) {
    const int lq = cu_seqlens_q[b + 1] - cu_seqlens_q[b];
    const int lk = cu_seqlens_k[b + 1] - cu_seqlens_k[b];
    if (lq < 0 || lk < 0) return FA_ERR_INVALID_ARG;
    count += (lq + fa::kBlockM - 1) / fa::kBlockM;
  }
  if (count > INT32_MAX / 2) return FA_ERR_INVALID_ARG;
  *num_items = (int)count;
  if (!plan) return FA_OK;
  if (plan_capacity < count) return FA_ERR_WORKSPACE;

  struct Item { int b, qt; int64_t cost; };
  std::vector<Item> items;
  items.reserve((size_t)count);
  for (int b = 0; b < B; ++b) {
    const int lq = cu_seqlens_q[b + 1] - cu_seqlens_q[b];
    const int lk = cu_seqlens_k[b + 1] - cu_seqlens_k[b];
    const int nt = (lq + fa::kBlockM - 1) / fa::kBlockM;
    for (int qt = nt - 1; qt >= 0; --qt) {
      const int r0 = qt * fa::kBlockM, r1 = std::min(r0 + fa::kBlockM, lq) - 1;
      items.push_back({b, qt, key_tiles(r0, r1, lq, lk, causal, window_left, window_right)});
    }
  }
  // heaviest first; equal costs keep sequence order (stable)
  std::stable_sort(items.begin(), items.end(),
                   [](const Item& a, const Item& c) { return a.cost > c.cost; });
  for (size_t i = 0; i < items.size(); ++i) {
    plan[2 * i] = items[i].b;
    plan[2 * i + 1] = items[i].qt;
  }
  return FA_OK;
}

fa_status fa_decode_plan(const int* cache_seqlens, int B, int page_size, int max_blocks_per_seq,
                         int window_left, int split_tokens, int* plan, int plan_capacity,
                         int* num_items) {
  if (!cache_seqlens || !num_items || B < 1 || page_size < 1 || max_blocks_per_seq < 1)
    return FA_ERR_INVALID_ARG;
  if (window_left < -1 || split_tokens < 0 || split_tokens % 16 != 0) return FA_ERR_INVALID_ARG;
  const int64_t cap_len = (int64_t)max_blocks_per_seq * page_size;
  const int64_t split = split_tokens == 0 ? fa::kDefaultSplit : split_tokens;
  struct Item { int b, s; int64_t cost; };
  std::vector<Item> items;
  for (int b = 0; b < B; ++b) {
    const int64_t len = cache_seqlens[b];
    if (len < 0 || len > cap_len) return FA_ERR_INVALID_ARG;
    // keys [lo, len) are visible to the new token; split s covers
    // [s * split, (s + 1) * split)
    const int64_t lo = window_left >= 0 ? std::max<int64_t>(0, len - 1 - window_left) : 0;
    for (int64_t s = lo / split; s * split < len; ++s) {
      const int64_t beg = std::max(s * split, lo), end = std::min(len, s * split + split);
      if (beg < end) items.push_back({b, (int)s, end - beg});
    }
    if (items.size() > (size_t)(INT32_MAX / 2)) return FA_ERR_INVALID_ARG;
  }
  *num_items = (int)items.size();
  if (!plan) return FA_OK;
  if (plan_capacity < (int64_t)items.size()) return FA_ERR_WORKSPACE;
  std::stable_sort(items.begin(), items.end(),
                   [](const Item& a, const Item& c) { return a.cost > c.cost; });
  for (size_t i = 0; i < items.size(); ++i) {
    plan[2 * i] = items[i].b;
    plan[2 * i + 1] = items[i].s;
  }
  return FA_OK;
}

}  // extern "C"
