// Internal interface between the C-ABI layer (fa_api.cpp) and the HIP kernels.
// Everything here is validated by the caller before a launcher runs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// Prefill tile shape: one workgroup = 4 waves = 128 query rows (32 per wave),
// iterating over 64-key tiles.
constexpr int kPrefillThreads = 256;
constexpr int kBlockM = 128;
constexpr int kBlockN = 64;

// Decode split kernel: one workgroup = 4 waves per (request, KV head, split).
constexpr int kDecodeThreads = 256;
constexpr int kDecodeChunk = 64;     // keys per wave iteration
constexpr int kDefaultSplit = 512;
// Prefill workgroups resident per XCD (32 CUs x 2), used to size work chunks.
constexpr int kPrefillSlotsPerXcd = 64;
// Wide-tile prefill (head_dim 128, dense): 256 (query row, head) pairs per
// workgroup -- 64 rows of 4 heads of one KV group, 128 rows of 2, or 256 rows
// of one -- one workgroup per CU.
constexpr int kWideRows = 256;
constexpr int kWideSlotsPerXcd = 32;
constexpr int kWideMinRows = 4096;   // query rows from which fa_fwd takes it

struct PrefillParams {
  const uint16_t* q;       // bf16 bits
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;              // may be null
  const int* cu_q;         // varlen only
  const int* cu_k;
  const int* plan;         // varlen only, may be null: (b, query tile) pairs in run order
  int B, Lq, Lk;           // dense: lengths; varlen: Lq/Lk unused
  int Hq, Hkv, group;      // group = Hq / Hkv
  int64_t q_tok_stride;    // elements between consecutive tokens = H*d
  int64_t k_tok_stride;
  int64_t q_batch_stride;  // dense only: Lq*Hq*d
  int64_t k_batch_stride;  // dense only: Lk*Hkv*d
  int lse_seq_stride;      // dense: Lq (lse is (B, Hq, Lq)); varlen: total_q
  float scale_log2;        // softmax_scale * log2(e)
  int causal, win_left, win_right;
  int num_q_tiles;         // dense: ceil(Lq / kBlockM); varlen: tile slots or plan items
  int xcd_groups;          // >0: XCD-aware work mapping with this many KV groups
  int chunk_groups;        // KV groups an XCD works on together (dense mapping)
  int wide_heads;          // wide kernel: query heads of one KV group per workgroup (1, 2, 4)
  // paged KV cache (chunked prefill): k/v are the page pools
  // [num_pages][page_size][Hkv][d]; request b has cache_seqlens[b] + append_len keys
  const int* block_table;  // [B][max_blocks]
  const int* cache_seqlens;
  int page_size, max_blocks, append_len;
  int page_shift;          // log2(page_size) when a power of two, else -1
  // score modifiers, in units of the raw dot product q.k (logit = scale * q.k)
  float cap_in, cap_out;   // softcap c: q.k -> cap_out * tanh(cap_in * q.k); cap_in = 0: off
  const float* alibi;      // slopes, NULL: off; slope of (b, h) = alibi[b * alibi_bstride + h]
  int alibi_bstride;
  float alibi_scale;       // 1 / softmax_scale
};

// Copy new tokens' K/V rows into a paged cache (see fa_fwd_kvcache).
struct AppendParams {
  const uint16_t* k_new;   // (B, L_new, Hkv, d)
  const uint16_t* v_new;
  uint16_t* k_cache;       // [num_pages][page_size][Hkv][d]
  uint16_t* v_cache;
  const int* block_table;
  const int* cache_seqlens;
  int B, L_new, Hkv, d, page_size, max_blocks;
};

// Backward pass (dense layout).  Row statistics live in a caller workspace,
// per (batch, query head) in blocks of 64 rows: [lse2 x 64][delta x 64] floats,
// rows padded to a multiple of kBlockM (padded rows: lse2 = +inf, delta = 0).
constexpr int kBwdStatRows = 64;
struct BwdParams {
  const uint16_t* q;       // (B, Lq, Hq, d) bf16 bits; varlen: (total_q, Hq, d)
  const uint16_t* k;       // (B, Lk, Hkv, d)
  const uint16_t* v;
  const uint16_t* o;       // forward output (B, Lq, Hq, d)
  const uint16_t* dout;    // upstream gradient (B, Lq, Hq, d)
  const float* lse;        // forward LSE (B, Hq, Lq), natural log
  uint16_t* dq;            // (B, Lq, Hq, d)
  uint16_t* dk;            // (B, Lk, Hkv, d)
  uint16_t* dv;
  float* stat;             // workspace: lse2 = lse * log2(e) (+inf for rows with no key), delta = dO . O
  const int* cu_q;         // varlen: cumulative sequence offsets (device), else null
  const int* cu_k;
  const int* plan;         // always null (the shared varlen work map takes a plan)
  int B, Lq, Lk, Hq, Hkv, group;   // varlen: Lq, Lk unused
  int Lq_pad;              // dense: ceil(Lq / kBlockM) * kBlockM
  // Statistics rows: dense, (batch b, head h) owns rows from (b * Hq + h) *
  // Lq_pad; varlen, head h owns stat_rows = num_q_tiles * kBlockM rows from
  // h * stat_rows, sequence b's starting (cu_q[b] / kBlockM + b) * kBlockM later.
  int stat_rows;
  int lse_seq_stride;      // dense Lq (lse (B, Hq, Lq)); varlen total_q (lse (Hq, total_q))
  int64_t q_tok_stride, k_tok_stride, q_batch_stride, k_batch_stride;
  float scale_log2;        // softmax_scale * log2(e)
  float scale;
  int causal, win_left, win_right;
  int num_q_tiles;         // dense ceil(Lq / kBlockM) per (batch, head); varlen total tile slots
  int num_k_tiles;         // dense ceil(Lk / kBwdKeys) per (batch, KV head); varlen total slots
  int xcd_groups, chunk_groups;
};
constexpr int kBwdKeys = 128;    // keys per dK/dV workgroup (4 waves x 32)

struct DecodeParams {
  const uint16_t* q;
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  const int* block_table;
  const int* seqlens;
  uint16_t* o;
  float* lse;              // may be null
  float* part_o;           // [B][Hq][max_splits][d]
  float* part_lse;         // [B][Hq][max_splits]  (log2 units)
  int B, Hq, Hkv, group, sub_groups;
  int page_size, max_blocks, split_tokens, max_splits;
  float scale_log2;
  int win_left;
  bool planned;            // false: grid over every (split, request) slot
  const int* plan;         // planned: (request, split) pairs, one per item
  int num_items;
  int* order;              // workspace: the unplanned call's item list, made on the device
  bool self_order;         // unplanned, head-set kernel: each workgroup finds its own item
  // score modifiers, as in PrefillParams (cap_in = 0 and alibi = NULL: off)
  float cap_in, cap_out;
  const float* alibi;
  int alibi_bstride;
  float alibi_scale;
};

// mode: 0 dense, 1 varlen, 2 paged KV cache
hipError_t launch_prefill(const PrefillParams& p, int d, int mode, hipStream_t stream);
// dense, head_dim 128; p.num_q_tiles and p.chunk_groups sized for
// kWideRows / p.wide_heads rows of p.wide_heads query heads per workgroup
hipError_t launch_prefill_wide(const PrefillParams& p, hipStream_t stream);
hipError_t launch_append(const AppendParams& a, hipStream_t stream);
hipError_t launch_decode(const DecodeParams& p, int d, int rows, hipStream_t stream);
// Size of the device scratch array behind fa_decode_paged_noalloc, and its
// address on the current device (looked up once per device); NULL and *err set
// if the lookup fails.
constexpr size_t kDecodeScratchBytes = (size_t)32 << 20;
void* decode_scratch(hipError_t* err);
// row statistics, then dK/dV, then dQ, in stream order
hipError_t launch_bwd(const BwdParams& p, int d, bool varlen, hipStream_t stream);

// Device-side preconditions that the host cannot see (debug builds only,
// -DFA_DEBUG).  Varlen: cu_q / cu_k (B + 1 entries) start at 0, never
// decrease, end at total_q / total_k, and no sequence is longer than
// max_q / max_k.  Paged: each request's key count n_b = seqlens[b] +
// extra_len lies in [extra_len, max_blocks * page_size] and the first
// ceil(n_b / page_size) entries of its block-table row lie in
// [0, num_pages).  A null cu_q (block_table) skips the varlen (paged) part.
struct DeviceChecks {
  const int* cu_q; const int* cu_k;
  int total_q, total_k, max_q, max_k;
  const int* block_table; const int* seqlens;
  int max_blocks, page_size, num_pages, extra_len;
  int B;
};
// Runs the checks on `stream` and waits for them: 0 when they hold, a
// non-zero mask of the violated groups (1 varlen offsets, 2 key counts,
// 4 page ids) otherwise, -1 if a HIP call failed.  Allocates nothing (the
// result goes through a device word of the library); it waits for the
// stream, so it is not for code under graph capture.
int debug_check_inputs(const DeviceChecks& c, hipStream_t stream);

}  // namespace fa
