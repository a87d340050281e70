// C-ABI entry points: argument validation, planning and kernel dispatch.
// Every check runs on the host before any HIP call; a failed check returns a
// status and enqueues nothing.  Debug builds (-DFA_DEBUG) then check the
// device-side preconditions with one small kernel before the real work.
#include "fa.h"
#include "fa_internal.h"

#include <math.h>
#include <stdint.h>

#include <algorithm>

static_assert(FA_DECODE_NOALLOC_MAX_BYTES == fa::kDecodeScratchBytes,
              "the header's scratch limit must match the array's size");

namespace {

constexpr int64_t kMaxElems = (int64_t)1 << 31;
constexpr int64_t kMaxBatchElems = (int64_t)1 << 30;   // bf16 elements: < 2^31 bytes
constexpr float kLog2e = 1.4426950408889634f;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// The device-side preconditions (offsets, key counts, page ids), checked on
// the device in debug builds (-DFA_DEBUG) after every host check and before
// any other work is enqueued; a violation returns FA_ERR_INVALID_ARG.
// Release builds check nothing here.
fa_status device_checks(const fa::DeviceChecks& c, void* stream) {
#ifdef FA_DEBUG
  const int r = fa::debug_check_inputs(c, static_cast<hipStream_t>(stream));
  return r < 0 ? FA_ERR_HIP : r != 0 ? FA_ERR_INVALID_ARG : FA_OK;
#else
  (void)c;
  (void)stream;
  return FA_OK;
#endif
}

fa::DeviceChecks varlen_checks(const int* cu_q, const int* cu_k, int B, int total_q, int total_k,
                               int max_q, int max_k) {
  fa::DeviceChecks c = {};
  c.cu_q = cu_q; c.cu_k = cu_k; c.B = B;
  c.total_q = total_q; c.total_k = total_k; c.max_q = max_q; c.max_k = max_k;
  return c;
}

fa::DeviceChecks paged_checks(const int* block_table, const int* seqlens, int B, int max_blocks,
                              int page_size, int num_pages, int extra_len) {
  fa::DeviceChecks c = {};
  c.block_table = block_table; c.seqlens = seqlens; c.B = B;
  c.max_blocks = max_blocks; c.page_size = page_size; c.num_pages = num_pages;
  c.extra_len = extra_len;
  return c;
}

fa_status check_common(int Hq, int Hkv, int d, float scale, int causal, int wl, int wr) {
  if (Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return FA_ERR_INVALID_ARG;
  if (d < 1) return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (!(scale > 0.f) || !isfinite(scale)) return FA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
  if (wl < -1 || wr < -1) return FA_ERR_INVALID_ARG;
  return FA_OK;
}

fa_status check_tensors(const void* q, const void* k, const void* v, const void* o, const float* lse) {
  if (!q || !k || !v || !o) return FA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16)) return FA_ERR_INVALID_ARG;
  if (lse && !aligned(lse, 4)) return FA_ERR_INVALID_ARG;
  return FA_OK;
}

// softcap >= 0 (0: off); ALiBi slopes NULL or float32 with batch stride 0 (one
// slope per query head) or Hq (one per batch and head).
fa_status check_mods(float softcap, const float* alibi, int alibi_bstride, int Hq) {
  if (!(softcap >= 0.f) || !isfinite(softcap)) return FA_ERR_INVALID_ARG;
  if (alibi && (!aligned(alibi, 4) || (alibi_bstride != 0 && alibi_bstride != Hq))) return FA_ERR_INVALID_ARG;
  return FA_OK;
}

void set_mods(fa::PrefillParams& p, float scale, float softcap, const float* alibi, int alibi_bstride) {
  p.cap_in = softcap > 0.f ? scale / softcap : 0.f;
  p.cap_out = softcap > 0.f ? softcap / scale : 0.f;
  p.alibi = alibi;
  p.alibi_bstride = alibi ? alibi_bstride : 0;
  p.alibi_scale = 1.f / scale;
}

// A window side of 2^30 or more reaches past every key (sequence lengths are
// below 2^24 at d >= 64), so it is the same as an unbounded side; normalising
// it keeps the kernels' 32-bit position sums (row + offset + window) in range.
int norm_window(int w) { return w >= (1 << 30) ? -1 : w; }

// XCD-aware mapping needs the KV-group count to split evenly over 8 XCDs.
int xcd_groups(int kv_groups) { return (kv_groups > 0 && kv_groups % 8 == 0) ? kv_groups : 0; }

int pow2_rows(int g) {
  int r = 1;
  while (r < g && r < 8) r <<= 1;
  return r;
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

extern "C" {

const char* fa_status_string(fa_status status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_INVALID_ARG: return "invalid argument";
    case FA_ERR_UNSUPPORTED: return "unsupported configuration (head_dim must be 64 or 128)";
    case FA_ERR_WORKSPACE: return "decode workspace missing, misaligned or too small";
    case FA_ERR_HIP: return "HIP kernel launch failed";
  }
  return "unknown status";
}

fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                 int B, int Lq, int Lk, int Hq, int Hkv, int d,
                 float softmax_scale, int causal, int window_left, int window_right,
                 float softcap, const float* alibi_slopes, int alibi_batch_stride,
                 void* stream) {
  fa_status st = check_common(Hq, Hkv, d, softmax_scale, causal, window_left, window_right);
  if (st != FA_OK) return st;
  if ((st = check_tensors(q, k, v, o, lse)) != FA_OK) return st;
  if ((st = check_mods(softcap, alibi_slopes, alibi_batch_stride, Hq)) != FA_OK) return st;
  if (B < 1 || Lq < 1 || Lk < 1) return FA_ERR_INVALID_ARG;
  // per-batch tensors are addressed with 32-bit byte offsets
  if ((int64_t)Lq * Hq * d >= kMaxBatchElems || (int64_t)Lk * Hkv * d >= kMaxBatchElems)
    return FA_ERR_INVALID_ARG;

  fa::PrefillParams p = {};
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.o = static_cast<uint16_t*>(o);
  p.lse = lse;
  p.B = B; p.Lq = Lq; p.Lk = Lk;
  p.Hq = Hq; p.Hkv = Hkv; p.group = Hq / Hkv;
  p.q_tok_stride = (int64_t)Hq * d;
  p.k_tok_stride = (int64_t)Hkv * d;
  p.q_batch_stride = (int64_t)Lq * Hq * d;
  p.k_batch_stride = (int64_t)Lk * Hkv * d;
  p.lse_seq_stride = Lq;
  p.scale_log2 = softmax_scale * kLog2e;
  p.causal = causal; p.win_left = norm_window(window_left); p.win_right = norm_window(window_right);
  set_mods(p, softmax_scale, softcap, alibi_slopes, alibi_batch_stride);
  // Long sequences at head_dim 128 take the wide-tile kernel (256 query rows,
  // one workgroup per CU): its steady state is faster, but a workgroup's fixed
  // start and end cost is not hidden by a second workgroup on the CU, which
  // outweighs that below a few thousand query rows.  Everything else takes the
  // narrow kernel (128 rows; two workgroups per CU at head_dim 128, three at 64).
  const bool wide = d == 128 && Lq >= fa::kWideMinRows;
  // A wide workgroup takes 4 query heads of one KV group when the group size
  // allows (64 rows each: its waves share every K/V tile and meet the causal
  // diagonal in one step instead of four), else 2 heads of 128 rows or one of 256.
  p.wide_heads = !wide ? 1 : p.group % 4 == 0 ? 4 : p.group % 2 == 0 ? 2 : 1;
  const int rows = wide ? fa::kWideRows / p.wide_heads : fa::kBlockM;
  const int slots = wide ? fa::kWideSlotsPerXcd : fa::kPrefillSlotsPerXcd;
  p.num_q_tiles = (int)cdiv(Lq, rows);
  p.xcd_groups = xcd_groups(B * Hkv);
  // KV groups per XCD chunk: about one XCD's worth of resident workgroups
  p.chunk_groups = (int)std::max<int64_t>(
      1, slots / ((int64_t)(p.group / p.wide_heads) * p.num_q_tiles));
  if ((int64_t)p.num_q_tiles * B * (Hq / p.wide_heads) >= kMaxElems) return FA_ERR_INVALID_ARG;
  hipError_t e = wide ? fa::launch_prefill_wide(p, static_cast<hipStream_t>(stream))
                      : fa::launch_prefill(p, d, 0, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // extern "C"

namespace {

// fa_fwd_varlen and fa_fwd_varlen_run: plan = NULL walks the tiles in
// sequence order, else the kernel takes its items from the plan.
fa_status varlen_impl(const void* q, const void* k, const void* v, void* o, float* lse,
                      const int* cu_seqlens_q, const int* cu_seqlens_k, const int* plan,
                      int num_items, int B, int max_seqlen_q, int max_seqlen_k, int total_q,
                      int total_k, int Hq, int Hkv, int d, float softmax_scale, int causal,
                      int window_left, int window_right, float softcap,
                      const float* alibi_slopes, int alibi_batch_stride, void* stream) {
  fa_status st = check_common(Hq, Hkv, d, softmax_scale, causal, window_left, window_right);
  if (st != FA_OK) return st;
  if ((st = check_tensors(q, k, v, o, lse)) != FA_OK) return st;
  if ((st = check_mods(softcap, alibi_slopes, alibi_batch_stride, Hq)) != FA_OK) return st;
  if (!cu_seqlens_q || !cu_seqlens_k || !aligned(cu_seqlens_q, 4) || !aligned(cu_seqlens_k, 4))
    return FA_ERR_INVALID_ARG;
  if (B < 1 || total_q < 0 || total_k < 0 || max_seqlen_q < 0 || max_seqlen_k < 0)
    return FA_ERR_INVALID_ARG;
  if (max_seqlen_q > total_q || max_seqlen_k > total_k) return FA_ERR_INVALID_ARG;
  if (total_q > 0 && max_seqlen_q < 1) return FA_ERR_INVALID_ARG;
  if ((int64_t)total_q * Hq * d >= kMaxBatchElems || (int64_t)total_k * Hkv * d >= kMaxBatchElems)
    return FA_ERR_INVALID_ARG;
  if (total_q == 0) return FA_OK;

  fa::PrefillParams p = {};
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.o = static_cast<uint16_t*>(o);
  p.lse = lse;
  p.cu_q = cu_seqlens_q;
  p.cu_k = cu_seqlens_k;
  p.B = B; p.Lq = max_seqlen_q; p.Lk = max_seqlen_k;
  p.Hq = Hq; p.Hkv = Hkv; p.group = Hq / Hkv;
  p.q_tok_stride = (int64_t)Hq * d;
  p.k_tok_stride = (int64_t)Hkv * d;
  p.lse_seq_stride = total_q;
  p.scale_log2 = softmax_scale * kLog2e;
  p.causal = causal; p.win_left = norm_window(window_left); p.win_right = norm_window(window_right);
  set_mods(p, softmax_scale, softcap, alibi_slopes, alibi_batch_stride);
  if (plan) {
    p.plan = plan;
    p.num_q_tiles = num_items;
  } else {
    // tile slots: sequence b owns [cu_q[b]/128 + b, cu_q[b+1]/128 + b + 1)
    p.num_q_tiles = total_q / fa::kBlockM + B;
  }
  p.xcd_groups = xcd_groups(Hkv);
  if ((int64_t)p.num_q_tiles * Hq >= kMaxElems) return FA_ERR_INVALID_ARG;
  if (p.num_q_tiles == 0) return FA_OK;
  st = device_checks(varlen_checks(cu_seqlens_q, cu_seqlens_k, B, total_q, total_k, max_seqlen_q,
                                   max_seqlen_k), stream);
  if (st != FA_OK) return st;
  hipError_t e = fa::launch_prefill(p, d, 1, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // namespace

extern "C" {

fa_status fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                        const int* cu_seqlens_q, const int* cu_seqlens_k, int B,
                        int max_seqlen_q, int max_seqlen_k, int total_q, int total_k,
                        int Hq, int Hkv, int d, float softmax_scale, int causal,
                        int window_left, int window_right, float softcap,
                        const float* alibi_slopes, int alibi_batch_stride, void* stream) {
  return varlen_impl(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, nullptr, 0, B, max_seqlen_q,
                     max_seqlen_k, total_q, total_k, Hq, Hkv, d, softmax_scale, causal,
                     window_left, window_right, softcap, alibi_slopes, alibi_batch_stride, stream);
}

fa_status fa_fwd_varlen_run(const void* q, const void* k, const void* v, void* o, float* lse,
                            const int* cu_seqlens_q, const int* cu_seqlens_k, const int* plan,
                            int num_items, int B, int max_seqlen_q, int max_seqlen_k,
                            int total_q, int total_k, int Hq, int Hkv, int d,
                            float softmax_scale, int causal, int window_left, int window_right,
                            float softcap, const float* alibi_slopes, int alibi_batch_stride,
                            void* stream) {
  if (num_items < 0 || (num_items > 0 && (!plan || !aligned(plan, 8)))) return FA_ERR_INVALID_ARG;
  // one item per query tile: a plan for these lengths has between 1 (when
  // total_q > 0) and total_q / 128 + B items; an empty plan may be NULL
  if ((int64_t)num_items > (int64_t)total_q / fa::kBlockM + B) return FA_ERR_INVALID_ARG;
  if (total_q > 0 && num_items == 0) return FA_ERR_INVALID_ARG;
  return varlen_impl(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, plan, num_items, B,
                     max_seqlen_q, max_seqlen_k, total_q, total_k, Hq, Hkv, d, softmax_scale,
                     causal, window_left, window_right, softcap, alibi_slopes,
                     alibi_batch_stride, stream);
}

fa_status fa_fwd_kvcache(const void* q, void* k_cache, void* v_cache,
                         const void* k_new, const void* v_new,
                         const int* block_table, const int* cache_seqlens,
                         void* o, float* lse, int B, int Lq, int Hq, int Hkv, int d,
                         int num_pages, int page_size, int max_blocks_per_seq,
                         float softmax_scale, int causal, int window_left, int window_right,
                         float softcap, const float* alibi_slopes, int alibi_batch_stride,
                         void* stream) {
  fa_status st = check_common(Hq, Hkv, d, softmax_scale, causal, window_left, window_right);
  if (st != FA_OK) return st;
  if ((st = check_tensors(q, k_cache, v_cache, o, lse)) != FA_OK) return st;
  if ((st = check_mods(softcap, alibi_slopes, alibi_batch_stride, Hq)) != FA_OK) return st;
  if ((k_new == nullptr) != (v_new == nullptr)) return FA_ERR_INVALID_ARG;
  if (k_new && (!aligned(k_new, 16) || !aligned(v_new, 16))) return FA_ERR_INVALID_ARG;
  if (!block_table || !cache_seqlens || !aligned(block_table, 4) || !aligned(cache_seqlens, 4))
    return FA_ERR_INVALID_ARG;
  if (B < 1 || Lq < 0 || num_pages < 1 || max_blocks_per_seq < 1 || page_size < 1)
    return FA_ERR_INVALID_ARG;
  if (page_size % 16 != 0) return FA_ERR_UNSUPPORTED;
  // one page of one KV head is addressed with 32-bit byte offsets, with room
  // for the out-of-range marker; queries per request likewise
  if ((int64_t)page_size * Hkv * d * 2 >= ((int64_t)1 << 30)) return FA_ERR_INVALID_ARG;
  if ((int64_t)Lq * Hq * d >= kMaxBatchElems) return FA_ERR_INVALID_ARG;
  if ((int64_t)max_blocks_per_seq * page_size >= ((int64_t)1 << 30)) return FA_ERR_INVALID_ARG;
  if (cdiv(Lq, fa::kBlockM) * B * Hq >= kMaxElems) return FA_ERR_INVALID_ARG;
  if (k_new && B > 65535) return FA_ERR_INVALID_ARG;   // append grid (Lq, B)
  if (Lq == 0) return FA_OK;
  st = device_checks(paged_checks(block_table, cache_seqlens, B, max_blocks_per_seq, page_size,
                                  num_pages, k_new ? Lq : 0), stream);
  if (st != FA_OK) return st;

  hipStream_t s = static_cast<hipStream_t>(stream);
  if (k_new) {
    fa::AppendParams a = {};
    a.k_new = static_cast<const uint16_t*>(k_new);
    a.v_new = static_cast<const uint16_t*>(v_new);
    a.k_cache = static_cast<uint16_t*>(k_cache);
    a.v_cache = static_cast<uint16_t*>(v_cache);
    a.block_table = block_table;
    a.cache_seqlens = cache_seqlens;
    a.B = B; a.L_new = Lq; a.Hkv = Hkv; a.d = d;
    a.page_size = page_size; a.max_blocks = max_blocks_per_seq;
    if (fa::launch_append(a, s) != hipSuccess) return FA_ERR_HIP;
  }

  fa::PrefillParams p = {};
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k_cache);
  p.v = static_cast<const uint16_t*>(v_cache);
  p.o = static_cast<uint16_t*>(o);
  p.lse = lse;
  p.B = B; p.Lq = Lq; p.Lk = 0;   // per request: cache_seqlens[b] + append_len
  p.Hq = Hq; p.Hkv = Hkv; p.group = Hq / Hkv;
  p.q_tok_stride = (int64_t)Hq * d;
  p.k_tok_stride = (int64_t)Hkv * d;
  p.q_batch_stride = (int64_t)Lq * Hq * d;
  p.k_batch_stride = 0;
  p.lse_seq_stride = Lq;
  p.scale_log2 = softmax_scale * kLog2e;
  p.causal = causal; p.win_left = norm_window(window_left); p.win_right = norm_window(window_right);
  set_mods(p, softmax_scale, softcap, alibi_slopes, alibi_batch_stride);
  p.num_q_tiles = (int)cdiv(Lq, fa::kBlockM);
  p.xcd_groups = xcd_groups(B * Hkv);
  p.chunk_groups = (int)std::max<int64_t>(1, fa::kPrefillSlotsPerXcd / ((int64_t)p.group * p.num_q_tiles));
  p.block_table = block_table;
  p.cache_seqlens = cache_seqlens;
  p.page_size = page_size;
  p.max_blocks = max_blocks_per_seq;
  p.append_len = k_new ? Lq : 0;
  p.page_shift = -1;
  for (int sh = 0; sh < 31; ++sh)
    if ((1 << sh) == page_size) p.page_shift = sh;
  hipError_t e = fa::launch_prefill(p, d, 2, s);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

static int effective_split(int split_tokens) { return split_tokens == 0 ? fa::kDefaultSplit : split_tokens; }

static bool decode_sizes_ok(int B, int Hq, int d, int max_blocks, int page_size, int split_tokens) {
  if (B < 1 || Hq < 1 || max_blocks < 1 || page_size < 1) return false;
  if (d != 64 && d != 128) return false;
  if (split_tokens < 0 || split_tokens % 16 != 0) return false;
  if ((int64_t)max_blocks * page_size >= kMaxElems) return false;
  return true;
}

static size_t part_o_bytes(int B, int Hq, int d, int max_splits) {
  const size_t n = (size_t)B * Hq * max_splits * d * sizeof(float);
  return (n + 255) & ~(size_t)255;
}

// the unplanned call's device-made item list: (request, split) per slot
static size_t order_bytes(int B, int max_splits) {
  const size_t n = (size_t)B * max_splits * 2 * sizeof(int);
  return (n + 255) & ~(size_t)255;
}

size_t fa_decode_paged_workspace_size(int B, int Hq, int d, int max_blocks_per_seq,
                                      int page_size, int split_tokens) {
  if (!decode_sizes_ok(B, Hq, d, max_blocks_per_seq, page_size, split_tokens)) return 0;
  const int split = effective_split(split_tokens);
  const int max_splits = (int)cdiv((int64_t)max_blocks_per_seq * page_size, split);
  const size_t lse_bytes = ((size_t)B * Hq * max_splits * sizeof(float) + 255) & ~(size_t)255;
  return part_o_bytes(B, Hq, d, max_splits) + lse_bytes + order_bytes(B, max_splits);
}

}  // extern "C"

namespace {

// fa_decode_paged and fa_decode_paged_run: plan = NULL launches every
// (request, split) slot, else only the plan's items.
fa_status decode_impl(const void* q, const void* k_cache, const void* v_cache,
                      const int* block_table, const int* cache_seqlens, bool planned,
                      const int* plan, int num_items, void* o, float* lse, int B, int Hq, int Hkv, int d,
                      int num_pages, int page_size, int max_blocks_per_seq,
                      float softmax_scale, int window_left, float softcap,
                      const float* alibi_slopes, int alibi_batch_stride, int split_tokens,
                      void* workspace, size_t workspace_bytes, void* stream) {
  fa_status st = check_common(Hq, Hkv, d, softmax_scale, 0, window_left, -1);
  if (st != FA_OK) return st;
  if ((st = check_mods(softcap, alibi_slopes, alibi_batch_stride, Hq)) != FA_OK) return st;
  if ((st = check_tensors(q, k_cache, v_cache, o, lse)) != FA_OK) return st;
  if (!block_table || !cache_seqlens || !aligned(block_table, 4) || !aligned(cache_seqlens, 4))
    return FA_ERR_INVALID_ARG;
  if (num_pages < 1) return FA_ERR_INVALID_ARG;
  if (!decode_sizes_ok(B, Hq, d, max_blocks_per_seq, page_size, split_tokens)) return FA_ERR_INVALID_ARG;
  // launch grid: (Hkv * head subgroups, splits, B); the merge grid is (Hq, B)
  if (B > 65535 || cdiv((int64_t)max_blocks_per_seq * page_size, effective_split(split_tokens)) > 65535)
    return FA_ERR_INVALID_ARG;
  if ((int64_t)num_pages * page_size * Hkv * d >= ((int64_t)1 << 40)) return FA_ERR_INVALID_ARG;
  const int split = effective_split(split_tokens);
  const int max_splits = (int)cdiv((int64_t)max_blocks_per_seq * page_size, split);
  const int rows = pow2_rows(Hq / Hkv);
  const int sub_groups = (int)cdiv(Hq / Hkv, rows);
  if (planned) {
    // planned grid: one 1-D launch of num_items * Hkv * sub_groups workgroups;
    // an empty plan (every request empty) may be NULL
    if (num_items < 0 || (int64_t)num_items > (int64_t)B * max_splits) return FA_ERR_INVALID_ARG;
    if (num_items > 0 && (!plan || !aligned(plan, 8))) return FA_ERR_INVALID_ARG;
    if ((int64_t)num_items * Hkv * sub_groups * fa::kDecodeThreads >= ((int64_t)1 << 32))
      return FA_ERR_INVALID_ARG;
  }
  const size_t need = fa_decode_paged_workspace_size(B, Hq, d, max_blocks_per_seq, page_size, split_tokens);
  if (!workspace || !aligned(workspace, 256) || workspace_bytes < need) return FA_ERR_WORKSPACE;

  fa::DecodeParams p = {};
  p.q = static_cast<const uint16_t*>(q);
  p.k_cache = static_cast<const uint16_t*>(k_cache);
  p.v_cache = static_cast<const uint16_t*>(v_cache);
  p.block_table = block_table;
  p.seqlens = cache_seqlens;
  p.o = static_cast<uint16_t*>(o);
  p.lse = lse;
  p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.group = Hq / Hkv;
  p.sub_groups = sub_groups;
  p.page_size = page_size;
  p.max_blocks = max_blocks_per_seq;
  p.split_tokens = split;
  p.max_splits = max_splits;
  p.part_o = static_cast<float*>(workspace);
  p.part_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) + part_o_bytes(B, Hq, d, p.max_splits));
  p.order = reinterpret_cast<int*>(static_cast<char*>(workspace) + part_o_bytes(B, Hq, d, p.max_splits) +
                                   ((((size_t)B * Hq * max_splits * sizeof(float)) + 255) & ~(size_t)255));
  p.scale_log2 = softmax_scale * kLog2e;
  p.win_left = norm_window(window_left);
  p.planned = planned;
  p.plan = plan;
  p.num_items = num_items;
  p.cap_in = softcap > 0.f ? softmax_scale / softcap : 0.f;
  p.cap_out = softcap > 0.f ? softcap / softmax_scale : 0.f;
  p.alibi = alibi_slopes;
  p.alibi_bstride = alibi_slopes ? alibi_batch_stride : 0;
  p.alibi_scale = 1.f / softmax_scale;
  st = device_checks(paged_checks(block_table, cache_seqlens, B, max_blocks_per_seq, page_size,
                                  num_pages, 0), stream);
  if (st != FA_OK) return st;
  hipError_t e = fa::launch_decode(p, d, rows, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // namespace

extern "C" {

fa_status fa_decode_paged(const void* q, const void* k_cache, const void* v_cache,
                          const int* block_table, const int* cache_seqlens,
                          void* o, float* lse, int B, int Hq, int Hkv, int d,
                          int num_pages, int page_size, int max_blocks_per_seq,
                          float softmax_scale, int window_left, float softcap,
                          const float* alibi_slopes, int alibi_batch_stride, int split_tokens,
                          void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(q, k_cache, v_cache, block_table, cache_seqlens, false, nullptr, 0, o, lse, B, Hq,
                     Hkv, d, num_pages, page_size, max_blocks_per_seq, softmax_scale,
                     window_left, softcap, alibi_slopes, alibi_batch_stride, split_tokens,
                     workspace, workspace_bytes, stream);
}

fa_status fa_decode_paged_run(const void* q, const void* k_cache, const void* v_cache,
                              const int* block_table, const int* cache_seqlens, const int* plan,
                              int num_items, void* o, float* lse, int B, int Hq, int Hkv, int d,
                              int num_pages, int page_size, int max_blocks_per_seq,
                              float softmax_scale, int window_left, float softcap,
                              const float* alibi_slopes, int alibi_batch_stride,
                              int split_tokens, void* workspace, size_t workspace_bytes,
                              void* stream) {
  return decode_impl(q, k_cache, v_cache, block_table, cache_seqlens, true, plan, num_items, o, lse, B,
                     Hq, Hkv, d, num_pages, page_size, max_blocks_per_seq, softmax_scale,
                     window_left, softcap, alibi_slopes, alibi_batch_stride, split_tokens,
                     workspace, workspace_bytes, stream);
}

fa_status fa_decode_paged_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                  const int* block_table, const int* cache_seqlens,
                                  void* o, float* lse, int B, int Hq, int Hkv, int d,
                                  int num_pages, int page_size, int max_blocks_per_seq,
                                  float softmax_scale, int window_left, float softcap,
                                  const float* alibi_slopes, int alibi_batch_stride,
                                  int split_tokens, void* stream) {
  // every argument check of fa_decode_paged, without a workspace: it reports
  // the missing workspace only when all else is valid (no HIP call is made)
  fa_status st = decode_impl(q, k_cache, v_cache, block_table, cache_seqlens, false, nullptr, 0, o,
                             lse, B, Hq, Hkv, d, num_pages, page_size, max_blocks_per_seq,
                             softmax_scale, window_left, softcap, alibi_slopes, alibi_batch_stride,
                             split_tokens, nullptr, 0, stream);
  if (st != FA_ERR_WORKSPACE) return st;
  const size_t need = fa_decode_paged_workspace_size(B, Hq, d, max_blocks_per_seq, page_size,
                                                     split_tokens);
  if (need > fa::kDecodeScratchBytes) return FA_ERR_WORKSPACE;
  hipError_t e = hipSuccess;
  void* scratch = fa::decode_scratch(&e);
  if (!scratch) return FA_ERR_HIP;
  return decode_impl(q, k_cache, v_cache, block_table, cache_seqlens, false, nullptr, 0, o, lse, B,
                     Hq, Hkv, d, num_pages, page_size, max_blocks_per_seq, softmax_scale,
                     window_left, softcap, alibi_slopes, alibi_batch_stride, split_tokens,
                     scratch, fa::kDecodeScratchBytes, stream);
}

size_t fa_bwd_workspace_size(int B, int Hq, int Lq) {
  if (B < 1 || Hq < 1 || Lq < 1) return 0;
  const int64_t lq_pad = cdiv(Lq, fa::kBlockM) * fa::kBlockM;
  const int64_t bytes = (int64_t)B * Hq * lq_pad * 2 * (int64_t)sizeof(float);
  if (bytes >= ((int64_t)1 << 31)) return 0;
  return (size_t)bytes;
}

fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                 const void* dout, void* dq, void* dk, void* dv, int B, int Lq, int Lk, int Hq,
                 int Hkv, int d, float softmax_scale, int causal, int window_left,
                 int window_right, void* workspace, size_t workspace_bytes, void* stream) {
  fa_status st = check_common(Hq, Hkv, d, softmax_scale, causal, window_left, window_right);
  if (st != FA_OK) return st;
  if ((st = check_tensors(q, k, v, o, lse)) != FA_OK) return st;
  if (!lse || !dout || !dq || !dk || !dv) return FA_ERR_INVALID_ARG;
  if (!aligned(dout, 16) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16))
    return FA_ERR_INVALID_ARG;
  if (B < 1 || Lq < 1 || Lk < 1) return FA_ERR_INVALID_ARG;
  if ((int64_t)Lq * Hq * d >= kMaxBatchElems || (int64_t)Lk * Hkv * d >= kMaxBatchElems)
    return FA_ERR_INVALID_ARG;
  const size_t need = fa_bwd_workspace_size(B, Hq, Lq);
  if (need == 0) return FA_ERR_INVALID_ARG;
  if (!workspace || !aligned(workspace, 256) || workspace_bytes < need) return FA_ERR_WORKSPACE;

  fa::BwdParams p = {};
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.o = static_cast<const uint16_t*>(o);
  p.dout = static_cast<const uint16_t*>(dout);
  p.lse = lse;
  p.dq = static_cast<uint16_t*>(dq);
  p.dk = static_cast<uint16_t*>(dk);
  p.dv = static_cast<uint16_t*>(dv);
  p.stat = static_cast<float*>(workspace);
  p.lse_seq_stride = Lq;
  p.B = B; p.Lq = Lq; p.Lk = Lk;
  p.Hq = Hq; p.Hkv = Hkv; p.group = Hq / Hkv;
  p.Lq_pad = (int)(cdiv(Lq, fa::kBlockM) * fa::kBlockM);
  p.q_tok_stride = (int64_t)Hq * d;
  p.k_tok_stride = (int64_t)Hkv * d;
  p.q_batch_stride = (int64_t)Lq * Hq * d;
  p.k_batch_stride = (int64_t)Lk * Hkv * d;
  p.scale_log2 = softmax_scale * kLog2e;
  p.scale = softmax_scale;
  p.causal = causal; p.win_left = norm_window(window_left); p.win_right = norm_window(window_right);
  p.num_q_tiles = (int)cdiv(Lq, fa::kBlockM);
  p.num_k_tiles = (int)cdiv(Lk, fa::kBwdKeys);
  p.xcd_groups = xcd_groups(B * Hkv);
  p.chunk_groups = (int)std::max<int64_t>(1, fa::kPrefillSlotsPerXcd / ((int64_t)p.group * p.num_q_tiles));
  if ((int64_t)p.num_q_tiles * B * Hq >= kMaxElems || (int64_t)p.num_k_tiles * B * Hkv >= kMaxElems)
    return FA_ERR_INVALID_ARG;
  if ((int64_t)B * p.Lq_pad * Hq * (d / 8) >= ((int64_t)1 << 40)) return FA_ERR_INVALID_ARG;
  hipError_t e = fa::launch_bwd(p, d, false, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

size_t fa_bwd_varlen_workspace_size(int B, int Hq, int total_q) {
  if (B < 1 || Hq < 1 || total_q < 0) return 0;
  // tile slots: sequence b owns [cu_q[b]/128 + b, cu_q[b+1]/128 + b + 1)
  const int64_t rows = ((int64_t)total_q / fa::kBlockM + B) * fa::kBlockM;
  const int64_t bytes = (int64_t)Hq * rows * 2 * (int64_t)sizeof(float);
  if (bytes >= ((int64_t)1 << 31)) return 0;
  return (size_t)bytes;
}

fa_status fa_bwd_varlen(const void* q, const void* k, const void* v, const void* o,
                        const float* lse, const void* dout, void* dq, void* dk, void* dv,
                        const int* cu_seqlens_q, const int* cu_seqlens_k, int B,
                        int max_seqlen_q, int max_seqlen_k, int total_q, int total_k, int Hq,
                        int Hkv, int d, float softmax_scale, int causal, int window_left,
                        int window_right, void* workspace, size_t workspace_bytes,
                        void* stream) {
  fa_status st = check_common(Hq, Hkv, d, softmax_scale, causal, window_left, window_right);
  if (st != FA_OK) return st;
  if ((st = check_tensors(q, k, v, o, lse)) != FA_OK) return st;
  if (!lse || !dout || !dq || !dk || !dv) return FA_ERR_INVALID_ARG;
  if (!aligned(dout, 16) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16))
    return FA_ERR_INVALID_ARG;
  if (!cu_seqlens_q || !cu_seqlens_k || !aligned(cu_seqlens_q, 4) || !aligned(cu_seqlens_k, 4))
    return FA_ERR_INVALID_ARG;
  if (B < 1 || total_q < 0 || total_k < 0 || max_seqlen_q < 0 || max_seqlen_k < 0)
    return FA_ERR_INVALID_ARG;
  if (max_seqlen_q > total_q || max_seqlen_k > total_k) return FA_ERR_INVALID_ARG;
  if ((int64_t)total_q * Hq * d >= kMaxBatchElems || (int64_t)total_k * Hkv * d >= kMaxBatchElems)
    return FA_ERR_INVALID_ARG;
  const size_t need = fa_bwd_varlen_workspace_size(B, Hq, total_q);
  if (need == 0) return FA_ERR_INVALID_ARG;
  if (!workspace || !aligned(workspace, 256) || workspace_bytes < need) return FA_ERR_WORKSPACE;
  if (total_q == 0 && total_k == 0) return FA_OK;

  fa::BwdParams p = {};
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.o = static_cast<const uint16_t*>(o);
  p.dout = static_cast<const uint16_t*>(dout);
  p.lse = lse;
  p.dq = static_cast<uint16_t*>(dq);
  p.dk = static_cast<uint16_t*>(dk);
  p.dv = static_cast<uint16_t*>(dv);
  p.stat = static_cast<float*>(workspace);
  p.cu_q = cu_seqlens_q;
  p.cu_k = cu_seqlens_k;
  p.lse_seq_stride = total_q;
  p.B = B; p.Lq = max_seqlen_q; p.Lk = max_seqlen_k;
  p.Hq = Hq; p.Hkv = Hkv; p.group = Hq / Hkv;
  p.q_tok_stride = (int64_t)Hq * d;
  p.k_tok_stride = (int64_t)Hkv * d;
  p.scale_log2 = softmax_scale * kLog2e;
  p.scale = softmax_scale;
  p.causal = causal; p.win_left = norm_window(window_left); p.win_right = norm_window(window_right);
  // tile slots, as for the forward: sequence b's start at floor(cu[b] / tile) + b
  p.num_q_tiles = total_q / fa::kBlockM + B;
  p.num_k_tiles = total_k / fa::kBwdKeys + B;
  p.stat_rows = p.num_q_tiles * fa::kBlockM;
  p.xcd_groups = xcd_groups(Hkv);
  if ((int64_t)p.num_q_tiles * Hq >= kMaxElems || (int64_t)p.num_k_tiles * Hkv >= kMaxElems)
    return FA_ERR_INVALID_ARG;
  st = device_checks(varlen_checks(cu_seqlens_q, cu_seqlens_k, B, total_q, total_k, max_seqlen_q,
                                   max_seqlen_k), stream);
  if (st != FA_OK) return st;
  hipError_t e = fa::launch_bwd(p, d, true, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // extern "C"
