/*
 * fa.h -- C ABI of an MI355X (gfx950) library for fused exact attention.
 *
 * The library computes O = softmax(scale * Q K^T + mask) V together with the
 * per-row log-sum-exp, tile by tile with an online softmax, so the score
 * matrix never reaches device memory.  Sources, cited by page title and
 * section:
 *   - "FlashAttention-3 vs naive attention: inference comparison (FA3)",
 *     sec. 1.1 (the definition), 1.2 (no materialised S or P), 2.1/2.2
 *     (prefill vs decode), 4.2 (one fused kernel);
 *   - "FIA / FlashAttention" explainer, sec. 1 (tiling, online softmax with a
 *     running max m and normaliser l) and sec. 2 (flash-decoding with an
 *     online-softmax reduction over a paged KV cache);
 *   - "flash-attention" configuration skill page, sec. 3.1-3.5 and the
 *     appendix (argument names and shapes, causal, window_size, cu_seqlens,
 *     block_table, split-KV, GQA broadcast).
 *
 * Conventions shared by every entry point
 *   - Element type of q, k, v, o, caches: bfloat16, row-major, contiguous,
 *     last dimension (head_dim) has stride 1.  lse: float32, natural log.
 *   - All pointers except `stream` and those of fa_varlen_plan (host memory)
 *     are DEVICE pointers owned by the caller;
 *     the library never allocates, frees, synchronises or keeps a pointer
 *     after the call returns.  q/k/v/o/cache pointers must be 16-byte
 *     aligned.  `lse` may be NULL (then no LSE is written).
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *     on it and the call returns at once.
 *   - head_dim d is 64 or 128.  Hkv must divide Hq; query head h reads KV head
 *     h / (Hq / Hkv) (GQA/MQA broadcast with no copy of K/V).
 *   - softmax_scale must be finite and > 0 (callers use 1/sqrt(d) by default).
 *   - Masking: causal attention is aligned bottom-right, i.e. query row i of a
 *     sequence with Lq queries and Lk keys sits at key position i + Lk - Lq
 *     and sees keys j <= i + Lk - Lq.  window_left / window_right >= 0 limit
 *     the keys to [i + Lk - Lq - left, i + Lk - Lq + right] inclusive;
 *     -1 leaves that side unbounded.  A row with no visible key gets O = 0
 *     and LSE = -inf.
 *   - Score modifiers of the attention entry points (fa_fwd, fa_fwd_varlen,
 *     fa_fwd_kvcache, fa_decode_paged; skill page sec. 3.3): softcap > 0 replaces each logit
 *     x = softmax_scale * q.k by softcap * tanh(x / softcap) (0 = off; must
 *     be finite and >= 0).  alibi_slopes (device float32, or NULL = off) adds
 *     -slope * |i + Lk - Lq - j| to the logit of query row i and key j, after
 *     the softcap and before the mask; the slope of (batch b, query head h)
 *     is alibi_slopes[b * alibi_batch_stride + h], with alibi_batch_stride 0
 *     (slopes of shape (Hq,)) or Hq (shape (B, Hq); for varlen, b is the
 *     sequence index).  In paged decode the one query row of request b sits
 *     at position cache_seqlens[b] - 1.  The backward takes neither.
 *   - Errors: every argument is validated on the host before any HIP call.
 *     On a non-zero status nothing has been enqueued and no output has been
 *     touched.  FA_ERR_HIP reports a failed kernel launch.  Device-side
 *     preconditions that cannot be checked without reading device memory
 *     (monotone cu_seqlens ending at total, block_table entries in
 *     [0, num_pages) for the pages a request uses, cache_seqlens[b] <=
 *     max_blocks_per_seq * page_size) are the caller's responsibility.  The
 *     debug build of this library (compiled with -DFA_DEBUG) checks them on
 *     the device, after the host checks and before any other work is
 *     enqueued, and returns FA_ERR_INVALID_ARG when one fails; its calls
 *     wait for their stream, so they cannot be captured in a graph.
 *   - Calls are reentrant and thread-safe: the library has no global state,
 *     except the per-GPU scratch array of fa_decode_paged_noalloc (see there).
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fa_status {
  FA_OK = 0,
  FA_ERR_INVALID_ARG = 1,   /* null/misaligned pointer, bad size or flag      */
  FA_ERR_UNSUPPORTED = 2,   /* valid but not built: head_dim not in {64,128}  */
  FA_ERR_WORKSPACE = 3,     /* decode workspace missing or too small          */
  FA_ERR_HIP = 4            /* a HIP launch failed                            */
} fa_status;

/* Static English text for a status code.  Never NULL. */
const char* fa_status_string(fa_status status);

/*
 * Dense prefill forward (skill page sec. 3.1/3.2, flash_attn_func;
 * "FlashAttention-3 vs naive attention" sec. 2.1).
 *   q, o : (B, Lq, Hq, d)      k, v : (B, Lk, Hkv, d)
 *   lse  : (B, Hq, Lq) float32, or NULL
 * B, Lq, Lk >= 1 (B*Hq*Lq and B*Hkv*Lk*d must fit in 2^31).  causal is 0/1.
 */
fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                 int B, int Lq, int Lk, int Hq, int Hkv, int d,
                 float softmax_scale, int causal, int window_left, int window_right,
                 float softcap, const float* alibi_slopes, int alibi_batch_stride,
                 void* stream);

/*
 * Packed variable-length prefill (skill page sec. 3.4 and the appendix on
 * continuous batching, flash_attn_varlen_func): sequences are concatenated
 * with no padding and never attend across each other.
 *   q, o : (total_q, Hq, d)    k, v : (total_k, Hkv, d)
 *   cu_seqlens_q, cu_seqlens_k : device int32 arrays of B+1 cumulative
 *       offsets, cu[0] = 0, cu[B] = total (e.g. lengths [100,200,150] give
 *       [0,100,300,450]);
 *   max_seqlen_q / max_seqlen_k : host upper bounds of the per-sequence
 *       lengths (only used for validation and planning);
 *   lse  : (Hq, total_q) float32, or NULL.
 * Masks apply per sequence with that sequence's own Lq_b and Lk_b.
 */
fa_status fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                        const int* cu_seqlens_q, const int* cu_seqlens_k, int B,
                        int max_seqlen_q, int max_seqlen_k, int total_q, int total_k,
                        int Hq, int Hkv, int d, float softmax_scale, int causal,
                        int window_left, int window_right, float softcap,
                        const float* alibi_slopes, int alibi_batch_stride, void* stream);

/*
 * Plan / run split for varlen prefill ("FIA / FlashAttention" explainer,
 * sec. 2: FlashInfer's plan step balances the load of variable-length
 * batches on the host, then a run step executes the batch).
 *
 * fa_varlen_plan is pure host code (no HIP call).  From HOST copies of the
 * cumulative lengths it lists the work items of fa_fwd_varlen_run -- one per
 * query tile of 128 rows, (sequence b, tile index) as two int32 -- ordered
 * by the number of key tiles each one visits under the given causal flag and
 * window, heaviest first (ties keep sequence order), so that long items start
 * early and short ones fill the end of the launch.
 *   cu_seqlens_q, cu_seqlens_k : host int32 arrays of B+1 offsets, as for
 *       fa_fwd_varlen (non-decreasing, cu[0] = 0; checked here).
 *   plan : host int32 array of 2 * plan_capacity, or NULL to only count.
 *   num_items : out, the number of items (sum over b of ceil(Lq_b / 128)).
 * Returns FA_ERR_WORKSPACE if plan_capacity < *num_items (then *num_items
 * is still set and plan is untouched), FA_ERR_INVALID_ARG for bad lengths.
 *
 * fa_fwd_varlen_run computes exactly what fa_fwd_varlen computes (bit for
 * bit: every tile runs the same code) in the order of a plan uploaded by the
 * caller to device memory.  Arguments are those of fa_fwd_varlen plus
 *   plan : device int32 array of 2 * num_items, 8-byte aligned, made by
 *       fa_varlen_plan for these cu_seqlens, causal flag and window (may be
 *       NULL when num_items is 0);
 *   num_items : its item count (1 .. total_q / 128 + B when total_q > 0;
 *       0 when total_q is 0).
 * The run computes only the listed tiles: rows of a tile missing from the
 * plan are not written; an item naming a sequence or tile that does not
 * exist is skipped.  A plan can be reused for every call with the same
 * lengths, mask and window.
 */
fa_status fa_varlen_plan(const int* cu_seqlens_q, const int* cu_seqlens_k, int B, int causal,
                         int window_left, int window_right, int* plan, int plan_capacity,
                         int* num_items);

fa_status fa_fwd_varlen_run(const void* q, const void* k, const void* v, void* o, float* lse,
                            const int* cu_seqlens_q, const int* cu_seqlens_k, const int* plan,
                            int num_items, int B, int max_seqlen_q, int max_seqlen_k,
                            int total_q, int total_k, int Hq, int Hkv, int d,
                            float softmax_scale, int causal, int window_left, int window_right,
                            float softcap, const float* alibi_slopes, int alibi_batch_stride,
                            void* stream);

/*
 * Bytes of device workspace fa_decode_paged needs for these sizes (split
 * partials: one float32 row of d values plus one float32 LSE per request,
 * query head and split; and two int32 per (request, split) for the work
 * order the call makes on the device).  split_tokens = 0 selects the
 * default of 512.  Returns 0 if the sizes are invalid.
 */
size_t fa_decode_paged_workspace_size(int B, int Hq, int d, int max_blocks_per_seq,
                                      int page_size, int split_tokens);

/*
 * One decode step over a paged KV cache with split-KV flash-decoding
 * (skill page appendix: PagedAttention, FlashDecoding / Split-KV;
 * "FIA / FlashAttention" explainer sec. 2).  Each request's one query row
 * attends to its cache_seqlens[b] cached tokens; the keys are cut into
 * chunks of split_tokens, each chunk yields a partial (LSE, O) and a second
 * kernel merges the partials by their log-sum-exp.  A one-workgroup kernel
 * first lists, on the device, the splits that hold keys (full splits first),
 * and the split kernel follows that list; the result is bit for bit that of
 * fa_decode_paged_run with any plan.
 *   q, o     : (B, 1, Hq, d)
 *   k_cache, v_cache : [num_pages, page_size, Hkv, d]
 *   block_table : device int32 [B, max_blocks_per_seq]; token j of request b
 *       is in page block_table[b][j / page_size], slot j % page_size.  Only
 *       the first ceil(cache_seqlens[b] / page_size) entries of a row are read.
 *   cache_seqlens : device int32 [B], 0 <= len <= max_blocks_per_seq*page_size.
 *       A request with len 0 gets O = 0, LSE = -inf.
 *   lse      : (B, Hq) float32, or NULL
 *   window_left : -1 for none, else only the last window_left + 1 tokens count.
 *   softcap, alibi_slopes, alibi_batch_stride : the score modifiers above.
 *   split_tokens : 0 (= 512) or a positive multiple of 16.
 *   workspace : device buffer of at least fa_decode_paged_workspace_size(...)
 *       bytes, 256-byte aligned; its contents on entry do not matter.
 * Cache contents of unused pages and of slots at or past a request's length
 * never influence the result (they may hold NaN).
 */
fa_status fa_decode_paged(const void* q, const void* k_cache, const void* v_cache,
                          const int* block_table, const int* cache_seqlens,
                          void* o, float* lse, int B, int Hq, int Hkv, int d,
                          int num_pages, int page_size, int max_blocks_per_seq,
                          float softmax_scale, int window_left, float softcap,
                          const float* alibi_slopes, int alibi_batch_stride, int split_tokens,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * Plan / run split for paged decode ("FIA / FlashAttention" explainer,
 * sec. 2 and its batch-decode example: a plan object is made on the host,
 * then the batched decode runs with it).
 *
 * fa_decode_plan is pure host code (no HIP call).  From a HOST copy of
 * cache_seqlens it lists the (request b, split s) pairs that hold at least
 * one visible key -- split s covers keys [s * split_tokens, (s+1) *
 * split_tokens), and with window_left >= 0 only the last window_left + 1
 * keys are visible -- as two int32 each, ordered by the number of keys they
 * read, heaviest first (ties keep request order).  Arguments as for
 * fa_decode_paged; it also checks 0 <= cache_seqlens[b] <=
 * max_blocks_per_seq * page_size on the host.
 *   plan : host int32 array of 2 * plan_capacity, or NULL to only count.
 *   num_items : out, the number of items.
 * Returns FA_ERR_WORKSPACE if plan_capacity < *num_items (then *num_items
 * is still set and plan is untouched), FA_ERR_INVALID_ARG for bad sizes.
 *
 * fa_decode_paged_run computes what fa_decode_paged computes (bit for bit:
 * every split runs the same code and the merge is the same kernel) but
 * launches one workgroup per plan item and KV head (group) instead of one
 * per (request, split slot), so no workgroup starts without keys to read.
 * Arguments are those of fa_decode_paged plus
 *   plan : device int32 array of 2 * num_items, 8-byte aligned, made by
 *       fa_decode_plan for the same cache_seqlens, page_size,
 *       max_blocks_per_seq, window_left and split_tokens (may be NULL when
 *       num_items is 0);
 *   num_items : its item count (0 .. B * number of split slots).
 * The plan must be complete: the merge reads the partial result of every
 * split that holds a visible key, and a split missing from the plan leaves
 * its workspace slot as it was (the output is then undefined, though no
 * memory outside the buffers is touched).  Items naming a request or split
 * that does not exist are skipped.
 */
fa_status fa_decode_plan(const int* cache_seqlens, int B, int page_size, int max_blocks_per_seq,
                         int window_left, int split_tokens, int* plan, int plan_capacity,
                         int* num_items);

fa_status fa_decode_paged_run(const void* q, const void* k_cache, const void* v_cache,
                              const int* block_table, const int* cache_seqlens, const int* plan,
                              int num_items, void* o, float* lse, int B, int Hq, int Hkv, int d,
                              int num_pages, int page_size, int max_blocks_per_seq,
                              float softmax_scale, int window_left, float softcap,
                              const float* alibi_slopes, int alibi_batch_stride,
                              int split_tokens, void* workspace, size_t workspace_bytes,
                              void* stream);

/*
 * fa_decode_paged without a workspace, for callers that cannot allocate
 * device memory: code being captured into a HIP graph, tight serving loops,
 * harnesses that forbid allocation.  It computes exactly what
 * fa_decode_paged computes (same kernels, bit for bit) and takes the same
 * arguments minus workspace and workspace_bytes.  The split partials and the
 * work order live instead in a device array of FA_DECODE_NOALLOC_MAX_BYTES
 * (32 MiB) inside the library, one per GPU, reserved when the library is
 * loaded on that GPU and held until the process ends; the call makes no
 * allocation of any kind.
 *   - A call needing more than that, i.e. fa_decode_paged_workspace_size(B,
 *     Hq, d, max_blocks_per_seq, page_size, split_tokens) >
 *     FA_DECODE_NOALLOC_MAX_BYTES, returns FA_ERR_WORKSPACE and enqueues
 *     nothing (for example 64 requests x 32 query heads x d 128 x 8192-token
 *     tables with 512-token splits need about 17 MiB).
 *   - The first call on each GPU (with that GPU current) looks up the array's
 *     device address (hipGetSymbolAddress); a failed lookup returns
 *     FA_ERR_HIP.  Nothing in the array needs to start zeroed: every byte a
 *     call reads, the same call wrote first.
 *   - Every call on one GPU shares that GPU's array: calls that can overlap
 *     on one GPU (different streams, or host threads) race and must be
 *     ordered by the caller, e.g. by issuing them on one stream.  This is the
 *     library's only global state.
 */
#define FA_DECODE_NOALLOC_MAX_BYTES ((size_t)32 << 20)
fa_status fa_decode_paged_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                  const int* block_table, const int* cache_seqlens,
                                  void* o, float* lse, int B, int Hq, int Hkv, int d,
                                  int num_pages, int page_size, int max_blocks_per_seq,
                                  float softmax_scale, int window_left, float softcap,
                                  const float* alibi_slopes, int alibi_batch_stride,
                                  int split_tokens, void* stream);

/*
 * Attention of Lq new query tokens per request over a paged KV cache
 * (chunked prefill), with an optional append of their K/V rows first
 * (skill page sec. 3.5: k_new / v_new and cache_seqlens; appendix on
 * PagedAttention for the cache layout).
 *   q, o     : (B, Lq, Hq, d) bf16
 *   k_cache, v_cache : [num_pages, page_size, Hkv, d] bf16; page_size must be
 *       a positive multiple of 16 (else FA_ERR_UNSUPPORTED) and one page of
 *       one cache must be < 2^30 bytes.
 *   k_new, v_new : (B, Lq, Hkv, d) bf16, both NULL or both set.  When set,
 *       new token i of request b is first written to sequence position
 *       cache_seqlens[b] + i (page block_table[b][pos / page_size], slot
 *       pos % page_size); the caches are modified in place and
 *       cache_seqlens is not updated (the caller advances it).
 *   block_table : device int32 [B, max_blocks_per_seq].
 *   cache_seqlens : device int32 [B]: keys already in the cache.  Request b
 *       attends to n_b = cache_seqlens[b] (+ Lq when appending) keys, with
 *       n_b <= max_blocks_per_seq * page_size and the first ceil(n_b /
 *       page_size) table entries valid (checked only by the debug build).
 *   lse      : (B, Hq, Lq) float32, or NULL.
 *   causal, window_left, window_right : as fa_fwd, with query row i at key
 *       position i + n_b - Lq (bottom-right).
 * Cache contents at or past a request's n_b never influence the result.
 * The append (when requested) and the attention are enqueued on `stream` in
 * that order.
 */
fa_status fa_fwd_kvcache(const void* q, void* k_cache, void* v_cache,
                         const void* k_new, const void* v_new,
                         const int* block_table, const int* cache_seqlens,
                         void* o, float* lse, int B, int Lq, int Hq, int Hkv, int d,
                         int num_pages, int page_size, int max_blocks_per_seq,
                         float softmax_scale, int causal, int window_left, int window_right,
                         float softcap, const float* alibi_slopes, int alibi_batch_stride,
                         void* stream);

/*
 * Backward pass of dense attention: dQ, dK, dV for an
 * upstream gradient dO.  The score blocks are recomputed from the forward's
 * LSE instead of being stored ("FlashAttention" concept page, recomputation;
 * "FIA / FlashAttention" explainer, sec. 1); the values are the derivative of
 * fa_fwd's definition:
 *   P = exp(scale * Q K^T - LSE) (masked),  dV = P^T dO,
 *   dS = P * (dO V^T - rowsum(dO * O)),  dQ = scale * dS K,  dK = scale * dS^T Q,
 * with dK, dV of a KV head summed over its Hq / Hkv query heads (GQA).
 *   q, o, dout, dq : (B, Lq, Hq, d) bf16     k, v, dk, dv : (B, Lk, Hkv, d) bf16
 *   lse  : (B, Hq, Lq) float32, the LSE fa_fwd returned for these q, k, v and
 *          mask (required); o: fa_fwd's output.
 *   causal, window_left, window_right, softmax_scale: as given to fa_fwd.
 *   workspace : device buffer of at least fa_bwd_workspace_size(B, Hq, Lq)
 *       bytes, 256-byte aligned (per-row statistics); contents on entry do
 *       not matter.
 * Softcap and ALiBi are not supported here (forward only).  Every output
 * element is summed in a fixed order by one wave, without atomics: results
 * are bitwise identical from run to run (the deterministic mode of the
 * skill page, sec. 3.3, is the only mode).  Keys no query row sees get
 * dK = dV = 0; rows that see no key get dQ = 0.
 */
size_t fa_bwd_workspace_size(int B, int Hq, int Lq);

fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                 const void* dout, void* dq, void* dk, void* dv, int B, int Lq, int Lk, int Hq,
                 int Hkv, int d, float softmax_scale, int causal, int window_left,
                 int window_right, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward of fa_fwd_varlen (packed sequences, skill page sec. 3.4): as
 * fa_bwd, per sequence, with the layouts of fa_fwd_varlen:
 *   q, o, dout, dq : (total_q, Hq, d)    k, v, dk, dv : (total_k, Hkv, d)
 *   lse : (Hq, total_q) float32 from fa_fwd_varlen
 *   cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, total_q,
 *   total_k : as for fa_fwd_varlen (device offsets; the same device-side
 *       preconditions)
 *   workspace : at least fa_bwd_varlen_workspace_size(B, Hq, total_q) bytes,
 *       256-byte aligned.
 * Rows of a sequence without keys get dQ = 0; keys of a sequence without
 * rows (or that no row sees) get dK = dV = 0.  Deterministic, as fa_bwd.
 */
size_t fa_bwd_varlen_workspace_size(int B, int Hq, int total_q);

fa_status fa_bwd_varlen(const void* q, const void* k, const void* v, const void* o,
                        const float* lse, const void* dout, void* dq, void* dk, void* dv,
                        const int* cu_seqlens_q, const int* cu_seqlens_k, int B,
                        int max_seqlen_q, int max_seqlen_k, int total_q, int total_k, int Hq,
                        int Hkv, int d, float softmax_scale, int causal, int window_left,
                        int window_right, void* workspace, size_t workspace_bytes,
                        void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
