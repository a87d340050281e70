// Split-KV flash-decoding over a paged KV cache for gfx950.
//
// What it computes (cited by page title and section):
//   one query row per request attends to that request's cached keys, read in
//   place from fixed-size pages through a block table, without copying them
//   into a contiguous tensor ("FIA / FlashAttention" explainer, sec. 2;
//   configuration skill page, appendix on PagedAttention).  Because one query
//   row per (request, head) gives too little parallelism, the keys are also
//   split along the sequence: several workgroups take different key ranges of
//   the same head and a final reduction merges their partial results (skill
//   page appendix, FlashDecoding / Split-KV).  The merge is the online-softmax
//   reduction by log-sum-exp (explainer, sec. 2).  All query heads of a GQA
//   group are served by one read of their KV head (explainer, sec. 2,
//   head-query fusion; skill page GQA appendix).
//
// Mapping onto CDNA4 (our design):
//   * decode_split: one workgroup (4 wave64s) per (request, KV head, split of
//     split_tokens keys).  Each wave takes 64-key chunks of the split.
//     Scores for the group's query heads come from v_mfma_f32_16x16x32_bf16
//     with the (zero-padded) query heads as the 16-row A operand and K rows
//     as the B operand.  K and V rows are both read so that each 16-lane
//     group covers one full 256-byte row; K then goes through a per-wave LDS
//     tile into the MFMA operand order.  P goes through a small
//     per-wave LDS buffer; P*V runs on the fp32 VALU with V read in fully
//     coalesced 256-byte rows.  The four waves merge in LDS and write one
//     partial (O_s normalised, LSE_s) per query head.
//   * decode_split_heads<D, NH> (page sizes that are multiples of 16; NH = 4
//     for at most four query heads per KV head, NH = 2 for more, taken in
//     subgroups of eight):
//     one workgroup per (request, split, NH adjacent KV heads), so every load
//     instruction reads 1 KB of whole NH-head segments of contiguous cache
//     memory (one to four tokens' rows of the NH heads) instead of row pieces
//     of separate slots; the general kernel above serves the other shapes.
//   * decode_merge: one wave per (request, query head) combines the
//     partials by their LSE and writes bf16 O and fp32 LSE.
//   * Keys at or past a request's length (and before its window) never reach
//     the result: they read a safe in-bounds cache row (never an unused
//     block-table entry), their scores are set to -inf and their V rows to
//     zero, so NaN or stale cache contents cannot leak in.  When page_size is
//     a multiple of 16 the page id of each 16-key block is wave-uniform and
//     comes from one scalar load.
#include "fa_internal.h"
#include "gfx950.h"

#include <math.h>

#include <mutex>

namespace fa {

// Request b's key count, clamped to [0, max_blocks * page_size] (the block
// table's capacity); every decode kernel reads lengths through this.
FA_DEV int clamp_len(const DecodeParams& p, int b) {
  return (int)min((int64_t)max(p.seqlens[b], 0), (int64_t)p.max_blocks * p.page_size);
}

namespace {
constexpr float kRescaleTau = 8.0f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLog2eF = 1.4426950408889634f;

// Score modifiers on a raw dot product s = q.k, softcap then ALiBi, as in the
// prefill kernel: the capped logit c * tanh(scale * s / c) is kept in
// dot-product units as cap_out * tanh(cap_in * s), with tanh(y) = 1 - 2 /
// (e^{2y} + 1), and ALiBi subtracts (slope / scale) * |query pos - key pos|
// (slope already divided by the scale).
__device__ __forceinline__ float modify_score(const DecodeParams& p, float s, float slope, int dist) {
  if (p.cap_in > 0.f)
    s = p.cap_out * (1.f - 2.f * __builtin_amdgcn_rcpf(exp2_fast(s * (2.f * kLog2eF * p.cap_in)) + 1.f));
  return s - slope * (float)dist;
}

// ---- the unplanned call's work order ---------------------------------------
// Work items are the (request, split) pairs that hold a visible key: first
// the full splits (split_tokens keys), request by request, then the partial
// ones (a request's first split under a window, its last split), by size,
// largest first, in 64 size buckets.  Small splits go last, so the launch's
// tail is short.  Either one workgroup writes the whole list
// (decode_order_kernel) or, for batches of at most kSelfOrderMaxB requests,
// every workgroup of the head-set kernel finds its own slot's item
// (self_order_item); there, within a bucket, partial splits are taken in
// (request, split) order.  Results do not depend on the order.
constexpr int kOrderBuckets = 64;
constexpr int kSelfOrderMaxB = 256;

FA_DEV int size_bucket(int keys, int S) { return (int)(((int64_t)keys * kOrderBuckets - 1) / S); }

// Splits s0..s1 hold request b's visible keys [lo, len).  pf / pl: the size
// bucket of its first / last split if that split is partial, else -1 (a
// single partial split is its first); its full splits are ff..ff+nf-1.
struct RequestSplits {
  int s0, s1, ff, nf, pf, pl;
};
FA_DEV RequestSplits request_splits(const DecodeParams& p, int b) {
  const int S = p.split_tokens;
  const int len = clamp_len(p, b);
  const int lo = p.win_left >= 0 ? max(0, len - 1 - p.win_left) : 0;
  RequestSplits r;
  r.s0 = lo / S;
  r.s1 = len > 0 ? (len - 1) / S : r.s0 - 1;
  r.ff = r.s0;
  r.nf = 0;
  r.pf = r.pl = -1;
  if (r.s1 < r.s0) return r;
  const int kf = min(len, r.s0 * S + S) - max(r.s0 * S, lo);
  if (kf < S) {
    r.pf = size_bucket(kf, S);
    r.ff = r.s0 + 1;
  }
  if (r.s1 > r.s0 && len - r.s1 * S < S) r.pl = size_bucket(len - r.s1 * S, S);
  r.nf = r.s1 - r.ff + 1 - (r.pl >= 0 ? 1 : 0);
  return r;
}

// Inclusive prefix sum over the 64 lanes of a wave.
FA_DEV int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int t = __shfl_up(v, off, 64);
    if (lane >= off) v += t;
  }
  return v;
}

// Item `item` of the order above, computed by one wave (every wave of a
// workgroup gets the same answer): false if the slot holds no item.  hist:
// 64 ints of the wave's own LDS.  Lanes take requests 64 at a time: full
// splits by a prefix sum of their counts; a partial one by a histogram of the
// buckets (lane j holds bucket 63 - j, so the prefix sum runs largest first),
// then by a prefix sum over the requests of its bucket.
FA_DEV bool self_order_item(const DecodeParams& p, int item, int* hist, int& b_out, int& s_out) {
  const int lane = threadIdx.x & 63;
  int base = 0, parts = 0;
  for (int c = 0; c < p.B; c += 64) {
    RequestSplits r{0, -1, 0, 0, -1, -1};
    if (c + lane < p.B) r = request_splits(p, c + lane);
    const int incl = wave_incl_scan(r.nf);
    const int tot = __shfl(incl, 63, 64);
    parts += __shfl(wave_incl_scan((r.pf >= 0) + (r.pl >= 0)), 63, 64);
    if (item < base + tot) {
      const int rel = item - base;
      const uint64_t hit = __builtin_amdgcn_ballot_w64(rel >= incl - r.nf && rel < incl);
      const int src = (int)__builtin_ctzll(hit);
      b_out = c + src;
      s_out = __shfl(r.ff + rel - (incl - r.nf), src, 64);
      return true;
    }
    base += tot;
  }
  int rank = item - base;            // among the partial splits
  if (rank >= parts) return false;
  hist[lane] = 0;
  for (int c = 0; c < p.B; c += 64) {
    if (c + lane < p.B) {
      const RequestSplits r = request_splits(p, c + lane);
      if (r.pf >= 0) atomicAdd(&hist[r.pf], 1);
      if (r.pl >= 0) atomicAdd(&hist[r.pl], 1);
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  __builtin_amdgcn_wave_barrier();
  const int cnt = hist[63 - lane];
  const int incl_b = wave_incl_scan(cnt);
  const uint64_t hit_b = __builtin_amdgcn_ballot_w64(rank >= incl_b - cnt && rank < incl_b);
  const int j = (int)__builtin_ctzll(hit_b);
  const int kb = 63 - j;
  rank -= __shfl(incl_b - cnt, j, 64);
  base = 0;
  for (int c = 0; c < p.B; c += 64) {
    RequestSplits r{0, -1, 0, 0, -1, -1};
    if (c + lane < p.B) r = request_splits(p, c + lane);
    const int m = (r.pf == kb) + (r.pl == kb);
    const int incl = wave_incl_scan(m);
    const int tot = __shfl(incl, 63, 64);
    if (rank < base + tot) {
      const int rel = rank - base;
      const uint64_t hit = __builtin_amdgcn_ballot_w64(rel >= incl - m && rel < incl);
      const int src = (int)__builtin_ctzll(hit);
      const int sv = (rel == incl - m && r.pf == kb) ? r.s0 : r.s1;
      b_out = c + src;
      s_out = __shfl(sv, src, 64);
      return true;
    }
    base += tot;
  }
  return false;
}
}  // namespace

// GR = padded number of query heads handled per workgroup (1, 2, 4 or 8).
// PAGE16: page_size is a multiple of 16, so every 16-key block lies in one page.
template <int D, int GR, bool PAGE16>
__global__ __launch_bounds__(kDecodeThreads, 2)
void decode_split_kernel(DecodeParams p) {
  constexpr int KT = D / 32;              // MFMA k-steps over d
  constexpr int VCH = D / 8;              // 16-byte chunks per V row
  constexpr int VKEYS = 64 / VCH;         // keys covered by one V load instruction
  constexpr int VLOADS = kDecodeChunk / VKEYS;
  constexpr int PST = GR < 4 ? 4 : GR;    // P row stride in the LDS buffer (floats)

  constexpr int KST = D + 8;               // padded K row in the per-wave staging tile
  static_assert(GR * D * 4 <= kDecodeChunk * KST * 2, "wave partial must fit its K tile");
  __shared__ __attribute__((aligned(16))) float p_lds[4][kDecodeChunk][PST];
  __shared__ float a_lds[4][16];
  __shared__ float m_lds[4][GR], l_lds[4][GR];
  // Per-wave K tile [64 keys][D + 8]; after a wave's last chunk its region
  // holds that wave's partial O (GR x D floats) for the workgroup merge.
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[4][kDecodeChunk * KST];
  auto o_part = [&](int w_) { return reinterpret_cast<float*>(&k_lds[w_][0]); };   // [GR][D]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // grid = (KV head x head subgroup, split, request): the workgroups of all KV
  // heads of one split are dispatched together, so the heads interleaved in
  // each cache page are read at the same time (DRAM row locality).  With a
  // host plan the grid is 1-D, (KV head x head subgroup) fastest, and the
  // plan's item names the (request, split).
  int s, b, gx;
  if (p.planned) {
    const int per = p.Hkv * p.sub_groups;
    const int item = blockIdx.x / per;
    gx = blockIdx.x - item * per;
    const __attribute__((address_space(4))) int* pc =
        (const __attribute__((address_space(4))) int*)p.plan;
    b = pc[2 * item];
    s = pc[2 * item + 1];
    if (b < 0 || b >= p.B || s < 0 || s >= p.max_splits) return;   // not an item of this batch
  } else {
    s = blockIdx.y;
    b = blockIdx.z;
    gx = blockIdx.x;
  }
  const int kvh = gx / p.sub_groups, sub = gx % p.sub_groups;
  const int h0 = kvh * p.group + sub * GR;
  const int nrow = min(GR, p.group - sub * GR);

  // lengths past the block table's capacity are out of contract; clamped as in
  // the order kernel and the host plan, so no read leaves the table or the partials
  const int len = clamp_len(p, b);
  const int lo = p.win_left >= 0 ? max(0, len - 1 - p.win_left) : 0;
  const int split_base = s * p.split_tokens;
  const int k_beg = max(split_base, lo);
  const int k_end = min(len, split_base + p.split_tokens);
  if (k_beg >= k_end) return;

  const int* bt = p.block_table + (int64_t)b * p.max_blocks;
  const int64_t tok_stride = (int64_t)p.Hkv * D;    // elements between cache slots
  const uint16_t* kcache = p.k_cache + (int64_t)kvh * D;
  const uint16_t* vcache = p.v_cache + (int64_t)kvh * D;

  // Q heads as the A operand: lane row i = lane % 16, d = 32t + 8*(lane/16) + 0..7
  const int qi = lane & 15, qg = lane >> 4;
  u32x4 qa[KT];
  {
    const bool ok = qi < nrow;
    const uint16_t* qrow = p.q + ((int64_t)b * p.Hq + h0 + qi) * D + 8 * qg;
#pragma unroll
    for (int t = 0; t < KT; ++t)
      qa[t] = ok ? *reinterpret_cast<const u32x4*>(qrow + 32 * t) : u32x4{0, 0, 0, 0};
  }

  // S layout: lane (key n = lane%16, row group g = lane/16) holds rows 4g..4g+3.
  const int sn = lane & 15, sg = lane >> 4;
  float m_ref[4], l_part[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) { m_ref[r] = -INFINITY; l_part[r] = 0.f; }
  // PV layout: lane (key j = lane / VCH, d chunk vc = lane % VCH)
  const int vj = lane / VCH, vc = lane % VCH;
  float oacc[GR][8];
#pragma unroll
  for (int r = 0; r < GR; ++r)
#pragma unroll
    for (int e = 0; e < 8; ++e) oacc[r][e] = 0.f;

  // score modifiers (the query sits at position len - 1); the slope of S row
  // 4*sg + r (0 for padding rows) is read where it is used, so that nothing
  // extra stays live through the loop
  const bool mods = p.cap_in > 0.f || p.alibi != nullptr;
  auto slope_of = [&](int r) {
    return p.alibi && 4 * sg + r < nrow
               ? p.alibi[(int64_t)b * p.alibi_bstride + h0 + 4 * sg + r] * p.alibi_scale : 0.f;
  };

  const float c = p.scale_log2;
  const int nchunks = (k_end - split_base + kDecodeChunk - 1) / kDecodeChunk;
  const int c0 = (k_beg - split_base) / kDecodeChunk;

  for (int ch = c0 + wave; ch < nchunks; ch += 4) {
    const int kc = split_base + ch * kDecodeChunk;
    // ---- loads: K in MFMA B layout, V in coalesced rows -------------------
    // Keys outside [k_beg, k_end) read a safe in-bounds row (page 0 when their
    // page is not in use); their scores are masked and their V rows zeroed.
    const bool partial = kc < k_beg || kc + kDecodeChunk > k_end;   // wave-uniform
    int pid16[4];
    if (PAGE16) {
#pragma unroll
      for (int blk = 0; blk < 4; ++blk) {
        const int key0 = kc + 16 * blk;
        pid16[blk] = key0 < k_end ? __builtin_amdgcn_readfirstlane(bt[key0 / p.page_size]) : 0;
      }
    }
    auto row_of = [&](int key, int blk) -> int64_t {   // cache slot index of a key
      if (PAGE16) return (int64_t)pid16[blk] * p.page_size + key % p.page_size;
      const bool ok = key >= 0 && key < k_end;
      const int pid = ok ? bt[key / p.page_size] : 0;
      return (int64_t)pid * p.page_size + (ok ? key % p.page_size : 0);
    };
    // K rows are read like V rows (a 16-lane group covers 256 contiguous bytes),
    // then re-laid out through the wave's LDS tile into the MFMA operand order.
    u32x4 kr[4][KT];
#pragma unroll
    for (int i = 0; i < VLOADS; ++i) {
      const int key = kc + VKEYS * i + vj;
      const uint16_t* src = kcache + row_of(key, (VKEYS * i) / 16) * tok_stride + 8 * vc;
      kr[i / KT][i % KT] = *reinterpret_cast<const u32x4*>(src);
    }
    u32x4 vr[VLOADS];
#pragma unroll
    for (int i = 0; i < VLOADS; ++i) {
      const int key = kc + VKEYS * i + vj;
      const uint16_t* src = vcache + row_of(key, (VKEYS * i) / 16) * tok_stride + 8 * vc;
      vr[i] = *reinterpret_cast<const u32x4*>(src);
    }
    if (partial) {
#pragma unroll
      for (int i = 0; i < VLOADS; ++i) {
        const int key = kc + VKEYS * i + vj;
        if (!(key >= k_beg && key < k_end)) vr[i] = u32x4{0, 0, 0, 0};
      }
    }
    {
      uint16_t* kt = k_lds[wave];
#pragma unroll
      for (int i = 0; i < VLOADS; ++i)
        *reinterpret_cast<u32x4*>(kt + (VKEYS * i + vj) * KST + 8 * vc) = kr[i / KT][i % KT];
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int blk = 0; blk < 4; ++blk)
#pragma unroll
        for (int t = 0; t < KT; ++t)
          kr[blk][t] = *reinterpret_cast<const u32x4*>(kt + (16 * blk + sn) * KST + 32 * t + 8 * sg);
      __builtin_amdgcn_wave_barrier();
    }
    // ---- scores S = Q K^T (rows = query heads, columns = 16 keys per block)
    f32x4 sacc[4];
#pragma unroll
    for (int blk = 0; blk < 4; ++blk) {
      sacc[blk] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < KT; ++t) sacc[blk] = mfma16x16x32(qa[t], kr[blk][t], sacc[blk]);
      const int key = kc + 16 * blk + sn;
      if (mods) {
#pragma unroll
        for (int r = 0; r < 4; ++r) sacc[blk][r] = modify_score(p, sacc[blk][r], slope_of(r), abs(len - 1 - key));
      }
      if (partial && !(key >= k_beg && key < k_end))
        sacc[blk] = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    }
    // ---- online softmax per query row ------------------------------------
    bool any_up = false;
    float tmax[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float mx = fmaxf(fmaxf(sacc[0][r], sacc[1][r]), fmaxf(sacc[2][r], sacc[3][r]));
      tmax[r] = row16_max(mx) * c;
      any_up |= tmax[r] > m_ref[r] + kRescaleTau;
    }
    if (wave_any(any_up)) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool up = tmax[r] > m_ref[r] + kRescaleTau;
        const float m_new = up ? tmax[r] : m_ref[r];
        const float alpha = up ? exp2_fast(m_ref[r] - m_new) : 1.f;
        l_part[r] *= alpha;
        m_ref[r] = m_new;
        if (sn == 0 && 4 * sg + r < 16) a_lds[wave][4 * sg + r] = alpha;
      }
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int r = 0; r < GR; ++r) {
        const float alpha = a_lds[wave][r];
#pragma unroll
        for (int e = 0; e < 8; ++e) oacc[r][e] *= alpha;
      }
      __builtin_amdgcn_wave_barrier();
    }
#pragma unroll
    for (int blk = 0; blk < 4; ++blk) {
      float pv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float mb = m_ref[r] == -INFINITY ? 0.f : m_ref[r];
        pv[r] = exp2_fast(fmaf(sacc[blk][r], c, -mb));
        l_part[r] += pv[r];
      }
      if (4 * sg < GR) {
        float* dst = &p_lds[wave][16 * blk + sn][4 * sg];
        if (GR >= 4) {
          *reinterpret_cast<f32x4*>(dst) = f32x4{pv[0], pv[1], pv[2], pv[3]};
        } else {
#pragma unroll
          for (int r = 0; r < GR; ++r) dst[r] = pv[r];
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
    // ---- O += P V on the VALU (fp32) -------------------------------------
#pragma unroll
    for (int i = 0; i < VLOADS; ++i) {
      const int kl = VKEYS * i + vj;
      float pr[GR];
      if (GR >= 4) {
#pragma unroll
        for (int r4 = 0; r4 < GR; r4 += 4) {
          const f32x4 t4 = *reinterpret_cast<const f32x4*>(&p_lds[wave][kl][r4]);
          pr[r4] = t4[0]; pr[r4 + 1] = t4[1]; pr[r4 + 2] = t4[2]; pr[r4 + 3] = t4[3];
        }
      } else {
#pragma unroll
        for (int r = 0; r < GR; ++r) pr[r] = p_lds[wave][kl][r];
      }
      float vf[8];
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        vf[2 * e2] = bf16lo(vr[i][e2]);
        vf[2 * e2 + 1] = bf16hi(vr[i][e2]);
      }
#pragma unroll
      for (int r = 0; r < GR; ++r)
#pragma unroll
        for (int e = 0; e < 8; ++e) oacc[r][e] = fmaf(pr[r], vf[e], oacc[r][e]);
    }
    __builtin_amdgcn_wave_barrier();
  }

  // ---- per-wave totals: l over the 16 key lanes, O over the key groups -----
#pragma unroll
  for (int r = 0; r < 4; ++r) l_part[r] = row16_sum(l_part[r]);
#pragma unroll
  for (int r = 0; r < GR; ++r) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float x = oacc[r][e];
#pragma unroll
      for (int off = VCH; off < 64; off <<= 1)
        x += __int_as_float(__builtin_amdgcn_ds_bpermute((lane ^ off) << 2, __float_as_int(x)));
      oacc[r][e] = x;
    }
  }
  if (sn == 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (4 * sg + r < GR) {
        m_lds[wave][4 * sg + r] = m_ref[r];
        l_lds[wave][4 * sg + r] = l_part[r];
      }
    }
  }
  if (vj == 0) {
#pragma unroll
    for (int r = 0; r < GR; ++r) {
      *reinterpret_cast<f32x4*>(o_part(wave) + r * D + 8 * vc) =
          f32x4{oacc[r][0], oacc[r][1], oacc[r][2], oacc[r][3]};
      *reinterpret_cast<f32x4*>(o_part(wave) + r * D + 8 * vc + 4) =
          f32x4{oacc[r][4], oacc[r][5], oacc[r][6], oacc[r][7]};
    }
  }
  __syncthreads();

  // ---- merge the four waves; write the split's partial -------------------
  for (int idx = tid; idx < GR * D; idx += kDecodeThreads) {
    const int r = idx / D, d = idx % D;
    if (r >= nrow) continue;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, m_lds[w][r]);
    float lsum = 0.f, osum = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float f = m_lds[w][r] == -INFINITY ? 0.f : exp2_fast(m_lds[w][r] - M);
      lsum += f * l_lds[w][r];
      osum += f * o_part(w)[r * D + d];
    }
    const int64_t slot = ((int64_t)b * p.Hq + h0 + r) * p.max_splits + s;
    p.part_o[slot * D + d] = osum / lsum;
    if (d == 0) p.part_lse[slot] = M + log2_fast(lsum);
  }
}

// NH KV heads per workgroup (page_size a multiple of 16): NH = 4 for at most
// four query heads per KV head, NH = 2 for more (eight per workgroup and KV
// head; the rest in further subgroups that read the same keys).  The cache holds a
// token's rows of all KV heads side by side, so heads NH*x..NH*x+NH-1 of one
// token are NH * 2d bytes of contiguous memory, and each load instruction
// reads 1 KB of whole such segments (TPL = 1, 2 or 4 tokens; 16 bytes per
// lane) instead of rows of one head in separate slots.  A wave takes 16-token chunks; the 16 tokens lie in one
// page, so their page id is one scalar load.  Scores: the A operand holds 16
// query rows, GM = 16 / NH per KV head (row GM*h + j is query j of KV head h,
// zero when j >= group), and one v_mfma_f32_16x16x32_bf16 chain per KV head h
// multiplies them with that head's K rows; the lanes whose four result rows
// belong to head h keep that chain's result.  P*V on the VALU: a lane holds
// d = 8c..8c+7 of one KV head for the tokens it loaded, so it accumulates
// GM x 8 outputs of that head with no cross-lane sum (TPL > 1: the tokens of
// a load go to lanes l, l + 64/TPL, ..., added once at the end).
constexpr int kQuadChunk = 16;   // tokens per wave iteration

// NT: one query subgroup, so every cache row is read by one workgroup only.
template <int D, int NH, bool NT>
__global__ __launch_bounds__(kDecodeThreads, 2)
void decode_split_heads_kernel(DecodeParams p) {
  static_assert(NH == 4 || NH == 2, "four or two KV heads per workgroup");
  static_assert(D == 128 || D == 64, "head dim");
  constexpr int CH = kQuadChunk, KT = D / 32;
  constexpr int DC = D / 8;          // 16-byte pieces of one head's row
  constexpr int GM = 16 / NH;        // query rows per KV head (zero-padded)
  constexpr int SEG = NH * D;        // elements of a token's NH-head segment
  constexpr int LPT = SEG / 8;       // lanes per token in one load (16 bytes each)
  constexpr int TPL = 64 / LPT;      // tokens per load instruction
  constexpr int LPC = CH / TPL;      // load instructions per chunk and operand
  constexpr int KST = SEG + 8;       // padded row of the per-wave K staging tile
  static_assert(16 * D * 4 <= CH * KST * 2, "wave partial must fit its K tile");
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[4][CH * KST];
  __shared__ __attribute__((aligned(16))) float p_lds[4][CH][16];
  __shared__ float a_lds[4][16];
  __shared__ float m_lds[4][16], l_lds[4][16];
  auto o_part = [&](int w_) { return reinterpret_cast<float*>(&k_lds[w_][0]); };   // [16][D]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // grid = (head set x query subgroup, split, request), or 1-D over (work
  // item, head set x query subgroup) with the workgroups of one item
  // adjacent, the item taken from the plan or found by self_order_item.  More
  // than GM query heads per KV head (NH = 2 only): subgroup sub takes queries
  // GM*sub..GM*sub+GM-1 of each KV head of the set.
  const int per = (p.Hkv / NH) * p.sub_groups;
  int s, b, hsub;
  if (p.self_order) {
    const int item = blockIdx.x / per;
    hsub = blockIdx.x - item * per;
    if (!self_order_item(p, item, reinterpret_cast<int*>(&p_lds[wave][0][0]), b, s)) return;
    b = __builtin_amdgcn_readfirstlane(b);
    s = __builtin_amdgcn_readfirstlane(s);
  } else if (p.planned) {
    const int item = blockIdx.x / per;
    hsub = blockIdx.x - item * per;
    const __attribute__((address_space(4))) int* pc =
        (const __attribute__((address_space(4))) int*)p.plan;
    b = pc[2 * item];
    s = pc[2 * item + 1];
    if (b < 0 || b >= p.B || s < 0 || s >= p.max_splits) return;   // not an item of this batch
  } else {
    hsub = blockIdx.x;
    s = blockIdx.y;
    b = blockIdx.z;
  }
  const int hs = hsub / p.sub_groups, q0 = (hsub - hs * p.sub_groups) * GM;
  const int G = p.group;

  // lengths past the block table's capacity are out of contract; clamped as in
  // the order kernel and the host plan, so no read leaves the table or the partials
  const int len = clamp_len(p, b);
  const int lo = p.win_left >= 0 ? max(0, len - 1 - p.win_left) : 0;
  const int split_base = s * p.split_tokens;
  const int k_beg = max(split_base, lo);
  const int k_end = min(len, split_base + p.split_tokens);
  if (k_beg >= k_end) return;

  const int* bt = p.block_table + (int64_t)b * p.max_blocks;
  const int64_t tok_stride = (int64_t)p.Hkv * D;    // elements between cache slots
  // load layout: lane (token tl of the load, 16-byte piece el of the segment)
  const int tl = lane / LPT, el = lane % LPT;
  const uint16_t* kcache = p.k_cache + (int64_t)hs * SEG + 8 * el;
  const uint16_t* vcache = p.v_cache + (int64_t)hs * SEG + 8 * el;

  // A operand: lane row i = lane % 16 (KV head i / GM, query i % GM), d = 32t + 8*(lane/16)
  u32x4 qa[KT];
  {
    const int qi = lane & 15, qg = lane >> 4;
    const bool ok = q0 + qi % GM < G;
    const int qh = (hs * NH + qi / GM) * G + q0 + qi % GM;
    const uint16_t* qrow = p.q + ((int64_t)b * p.Hq + qh) * D + 8 * qg;
#pragma unroll
    for (int t = 0; t < KT; ++t)
      qa[t] = ok ? *reinterpret_cast<const u32x4*>(qrow + 32 * t) : u32x4{0, 0, 0, 0};
  }

  // S layout: lane (key n = lane%16, g = lane/16) holds rows 4g..4g+3, all of
  // KV head 4g / GM.  PV layout: the load layout, i.e. KV head hv = el / DC
  // (rows GM*hv..GM*hv+GM-1) and d chunk dc = el % DC.
  const int sn = lane & 15, sg = lane >> 4;
  const int hv = el / DC, dc = el % DC;
  float m_ref[4], l_part[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) { m_ref[r] = -INFINITY; l_part[r] = 0.f; }
  float oacc[GM][8];
#pragma unroll
  for (int r = 0; r < GM; ++r)
#pragma unroll
    for (int e = 0; e < 8; ++e) oacc[r][e] = 0.f;

  // score modifiers (the query sits at position len - 1); the slope of S row
  // i = 4*sg + r (0 for padding rows) is read where it is used, so that
  // nothing extra stays live through the loop
  const bool mods = p.cap_in > 0.f || p.alibi != nullptr;
  auto slope_of = [&](int r) {
    const int i = 4 * sg + r;
    return p.alibi && q0 + i % GM < G
               ? p.alibi[(int64_t)b * p.alibi_bstride + (hs * NH + i / GM) * G + q0 + i % GM] * p.alibi_scale
               : 0.f;
  };

  const float c = p.scale_log2;
  const int nchunks = (k_end - split_base + CH - 1) / CH;
  const int c0 = (k_beg - split_base) / CH;
  uint16_t* kt = k_lds[wave];

  for (int ch = c0 + wave; ch < nchunks; ch += 4) {
    const int kc = split_base + ch * CH;               // kc < k_end <= len
    const bool partial = kc < k_beg || kc + CH > k_end;   // wave-uniform
    // the chunk's 16 tokens share one page (kc and page_size are multiples
    // of 16); tokens outside [k_beg, k_end) are read but masked below
    const int pid = __builtin_amdgcn_readfirstlane(bt[kc / p.page_size]);
    const int64_t slot0 = (int64_t)pid * p.page_size + kc % p.page_size + tl;
    // With one query subgroup each cache row is read once per step, and the
    // loads are non-temporal so that they displace nothing in L2; further
    // subgroups read the same rows again, from L2.
    u32x4 kr[LPC], vr[LPC];
    if constexpr (NT) {
#pragma unroll
      for (int i = 0; i < LPC; ++i)
        kr[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kcache + (slot0 + TPL * i) * tok_stride));
#pragma unroll
      for (int i = 0; i < LPC; ++i)
        vr[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vcache + (slot0 + TPL * i) * tok_stride));
    } else {
#pragma unroll
      for (int i = 0; i < LPC; ++i)
        kr[i] = *reinterpret_cast<const u32x4*>(kcache + (slot0 + TPL * i) * tok_stride);
#pragma unroll
      for (int i = 0; i < LPC; ++i)
        vr[i] = *reinterpret_cast<const u32x4*>(vcache + (slot0 + TPL * i) * tok_stride);
    }
    if (partial) {
#pragma unroll
      for (int i = 0; i < LPC; ++i) {
        const int key = kc + TPL * i + tl;
        if (!(key >= k_beg && key < k_end)) vr[i] = u32x4{0, 0, 0, 0};
      }
    }
    // K through the wave's LDS tile into the B operand order
#pragma unroll
    for (int i = 0; i < LPC; ++i) *reinterpret_cast<u32x4*>(kt + (TPL * i + tl) * KST + 8 * el) = kr[i];
    __builtin_amdgcn_wave_barrier();
    f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < KT; ++t)
        acc = mfma16x16x32(qa[t], *reinterpret_cast<const u32x4*>(kt + sn * KST + h * D + 32 * t + 8 * sg), acc);
      if ((4 * sg) / GM == h) sacc = acc;
    }
    __builtin_amdgcn_wave_barrier();
    if (mods) {
#pragma unroll
      for (int r = 0; r < 4; ++r) sacc[r] = modify_score(p, sacc[r], slope_of(r), abs(len - 1 - (kc + sn)));
    }
    if (partial && !(kc + sn >= k_beg && kc + sn < k_end))
      sacc = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    // ---- online softmax per query row ------------------------------------
    bool any_up = false;
    float tmax[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      tmax[r] = row16_max(sacc[r]) * c;
      any_up |= tmax[r] > m_ref[r] + kRescaleTau;
    }
    if (wave_any(any_up)) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool up = tmax[r] > m_ref[r] + kRescaleTau;
        const float m_new = up ? tmax[r] : m_ref[r];
        const float alpha = up ? exp2_fast(m_ref[r] - m_new) : 1.f;
        l_part[r] *= alpha;
        m_ref[r] = m_new;
        if (sn == 0) a_lds[wave][4 * sg + r] = alpha;
      }
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int r = 0; r < GM; ++r) {
        const float alpha = a_lds[wave][GM * hv + r];
#pragma unroll
        for (int e = 0; e < 8; ++e) oacc[r][e] *= alpha;
      }
      __builtin_amdgcn_wave_barrier();
    }
    {
      float pv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float mb = m_ref[r] == -INFINITY ? 0.f : m_ref[r];
        pv[r] = exp2_fast(fmaf(sacc[r], c, -mb));
        l_part[r] += pv[r];
      }
      *reinterpret_cast<f32x4*>(&p_lds[wave][sn][4 * sg]) = f32x4{pv[0], pv[1], pv[2], pv[3]};
    }
    __builtin_amdgcn_wave_barrier();
    // ---- O += P V on the VALU (fp32) -------------------------------------
#pragma unroll
    for (int i = 0; i < LPC; ++i) {
      float pr[GM];
#pragma unroll
      for (int r4 = 0; r4 < GM; r4 += 4) {
        const f32x4 q4 = *reinterpret_cast<const f32x4*>(&p_lds[wave][TPL * i + tl][GM * hv + r4]);
#pragma unroll
        for (int k = 0; k < 4; ++k) pr[r4 + k] = q4[k];
      }
      float vf[8];
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        vf[2 * e2] = bf16lo(vr[i][e2]);
        vf[2 * e2 + 1] = bf16hi(vr[i][e2]);
      }
#pragma unroll
      for (int r = 0; r < GM; ++r)
#pragma unroll
        for (int e = 0; e < 8; ++e) oacc[r][e] = fmaf(pr[r], vf[e], oacc[r][e]);
    }
    __builtin_amdgcn_wave_barrier();
  }
  // lanes l, l + 64/TPL, ... summed different tokens of the same outputs
  if constexpr (TPL >= 2) {
#pragma unroll
    for (int r = 0; r < GM; ++r)
#pragma unroll
      for (int e = 0; e < 8; ++e) oacc[r][e] += xor32(oacc[r][e]);
  }
  if constexpr (TPL == 4) {
#pragma unroll
    for (int r = 0; r < GM; ++r)
#pragma unroll
      for (int e = 0; e < 8; ++e) oacc[r][e] += xor16(oacc[r][e]);
  }

  // ---- per-wave totals, then the merge of the four waves -------------------
#pragma unroll
  for (int r = 0; r < 4; ++r) l_part[r] = row16_sum(l_part[r]);
  if (sn == 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      m_lds[wave][4 * sg + r] = m_ref[r];
      l_lds[wave][4 * sg + r] = l_part[r];
    }
  }
  if (tl == 0) {
    float* op = o_part(wave);
#pragma unroll
    for (int r = 0; r < GM; ++r) {
      *reinterpret_cast<f32x4*>(op + (GM * hv + r) * D + 8 * dc) =
          f32x4{oacc[r][0], oacc[r][1], oacc[r][2], oacc[r][3]};
      *reinterpret_cast<f32x4*>(op + (GM * hv + r) * D + 8 * dc + 4) =
          f32x4{oacc[r][4], oacc[r][5], oacc[r][6], oacc[r][7]};
    }
  }
  __syncthreads();
  for (int idx = tid; idx < 16 * D; idx += kDecodeThreads) {
    const int r = idx / D, d = idx % D;
    if (q0 + r % GM >= G) continue;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, m_lds[w][r]);
    float lsum = 0.f, osum = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float f = m_lds[w][r] == -INFINITY ? 0.f : exp2_fast(m_lds[w][r] - M);
      lsum += f * l_lds[w][r];
      osum += f * o_part(w)[r * D + d];
    }
    const int qh = (hs * NH + r / GM) * G + q0 + r % GM;
    const int64_t slot = ((int64_t)b * p.Hq + qh) * p.max_splits + s;
    p.part_o[slot * D + d] = osum / lsum;
    if (d == 0) p.part_lse[slot] = M + log2_fast(lsum);
  }
}

// One wave per (request, query head).  Lanes first take one split each to find
// the largest partial LSE and the total weight; then every lane owns d/64
// output columns and sums the weighted partials with all loads of a group of
// splits issued before their use.
template <int D>
__global__ __launch_bounds__(64)
void decode_merge_kernel(DecodeParams p) {
  constexpr int PER = D / 64;
  const int h = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
  // lengths past the block table's capacity are out of contract; clamped as in
  // the order kernel and the host plan, so no read leaves the table or the partials
  const int len = clamp_len(p, b);
  const int lo = p.win_left >= 0 ? max(0, len - 1 - p.win_left) : 0;
  const int s_beg = lo / p.split_tokens;
  const int s_end = (len + p.split_tokens - 1) / p.split_tokens;
  const int64_t row = (int64_t)b * p.Hq + h;
  const float* plse = p.part_lse + row * p.max_splits;
  const float* po = p.part_o + row * p.max_splits * D;

  float M = -INFINITY;
  for (int s = s_beg + lane; s < s_end; s += 64) M = fmaxf(M, plse[s]);
  for (int off = 32; off > 0; off >>= 1)
    M = fmaxf(M, __int_as_float(__builtin_amdgcn_ds_bpermute((lane ^ off) << 2, __float_as_int(M))));
  float wsum = 0.f;
  for (int s = s_beg + lane; s < s_end; s += 64) wsum += exp2_fast(plse[s] - M);
  for (int off = 32; off > 0; off >>= 1)
    wsum += __int_as_float(__builtin_amdgcn_ds_bpermute((lane ^ off) << 2, __float_as_int(wsum)));

  float acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.f;
  for (int s0 = s_beg; s0 < s_end; s0 += 8) {
    float wv[8], ov[8][PER];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int s = min(s0 + u, s_end - 1);
      wv[u] = plse[s];
#pragma unroll
      for (int e = 0; e < PER; ++e) ov[u][e] = po[(int64_t)s * D + lane + 64 * e];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float wgt = (s0 + u < s_end) ? exp2_fast(wv[u] - M) : 0.f;
#pragma unroll
      for (int e = 0; e < PER; ++e) acc[e] = fmaf(wgt, ov[u][e], acc[e]);
    }
  }
  const bool empty = s_end <= s_beg;
  const float inv = empty ? 0.f : 1.f / wsum;
#pragma unroll
  for (int e = 0; e < PER; ++e)
    p.o[row * D + lane + 64 * e] = (uint16_t)(pack_bf16x2(acc[e] * inv, 0.f) & 0xffffu);
  if (p.lse && lane == 0) p.lse[row] = empty ? -INFINITY : (M + log2_fast(wsum)) * kLn2;
}

template <int D, bool PAGE16>
static void launch_split(const DecodeParams& p, int rows, hipStream_t stream) {
  const dim3 grid = p.planned ? dim3(p.num_items * p.Hkv * p.sub_groups)
                           : dim3(p.Hkv * p.sub_groups, p.max_splits, p.B);
  const dim3 block(kDecodeThreads);
  switch (rows) {
    case 1: hipLaunchKernelGGL((decode_split_kernel<D, 1, PAGE16>), grid, block, 0, stream, p); break;
    case 2: hipLaunchKernelGGL((decode_split_kernel<D, 2, PAGE16>), grid, block, 0, stream, p); break;
    case 4: hipLaunchKernelGGL((decode_split_kernel<D, 4, PAGE16>), grid, block, 0, stream, p); break;
    default: hipLaunchKernelGGL((decode_split_kernel<D, 8, PAGE16>), grid, block, 0, stream, p); break;
  }
}

// The unplanned call's work order (see above), written by one workgroup for
// the kernels that do not find their own items, then -1 for the remaining
// slots of the B x max_splits list, which the split kernel skips; within a
// bucket the order is whatever the LDS counters give.
constexpr int kOrderThreads = 1024;

__global__ __launch_bounds__(kOrderThreads)
void decode_order_kernel(DecodeParams p) {
  __shared__ int scan_f[kOrderThreads];
  __shared__ int bucket_n[kOrderBuckets], bucket_at[kOrderBuckets];
  __shared__ int total_items;
  const int tid = threadIdx.x;
  const int S = p.split_tokens;
  // visible keys [lo, len) of request b lie in splits s0..s1
  auto range = [&](int b, int& s0, int& s1, int& lo, int& len) {
    len = clamp_len(p, b);
    lo = p.win_left >= 0 ? max(0, len - 1 - p.win_left) : 0;
    s0 = lo / S;
    s1 = len > 0 ? (len - 1) / S : s0 - 1;
  };
  auto keys_in = [&](int s, int lo, int len) { return min(len, s * S + S) - max(s * S, lo); };
  auto bucket = [&](int keys) { return size_bucket(keys, S); };   // 0..63
  // exclusive scan of one value per thread over the workgroup (Hillis-Steele)
  auto scan = [&](int* a, int v) {
    a[tid] = v;
    __syncthreads();
    for (int off = 1; off < kOrderThreads; off <<= 1) {
      const int add = tid >= off ? a[tid - off] : 0;
      __syncthreads();
      a[tid] += add;
      __syncthreads();
    }
    const int incl = a[tid], total = a[kOrderThreads - 1];
    __syncthreads();
    return make_int2(incl - v, total);
  };
  if (tid < kOrderBuckets) bucket_n[tid] = 0;
  __syncthreads();
  // pass 1: full splits per thread, partial splits per size bucket
  int mine = 0;
  for (int b = tid; b < p.B; b += kOrderThreads) {
    int s0, s1, lo, len;
    range(b, s0, s1, lo, len);
    for (int s = s0; s <= s1; ++s) {
      const int k = keys_in(s, lo, len);
      if (k == S) ++mine;
      else atomicAdd(&bucket_n[bucket(k)], 1);
    }
  }
  const int2 tf = scan(scan_f, mine);
  if (tid == 0) {
    int at = tf.y;                      // partial splits follow the full ones, largest first
    for (int k = kOrderBuckets - 1; k >= 0; --k) {
      bucket_at[k] = at;
      at += bucket_n[k];
    }
    total_items = at;
  }
  __syncthreads();
  // pass 2: full splits in request order (scan offsets), partial ones by bucket
  int base_f = 0;
  for (int b0 = 0; b0 < p.B; b0 += kOrderThreads) {
    const int b = b0 + tid;
    int s0 = 0, s1 = -1, lo = 0, len = 0, nf = 0;
    if (b < p.B) {
      range(b, s0, s1, lo, len);
      for (int s = s0; s <= s1; ++s) nf += keys_in(s, lo, len) == S;
    }
    const int2 ef = scan(scan_f, nf);
    int wf = base_f + ef.x;
    for (int s = s0; s <= s1; ++s) {
      const int k = keys_in(s, lo, len);
      const int at = k == S ? wf++ : atomicAdd(&bucket_at[bucket(k)], 1);
      p.order[2 * at] = b;
      p.order[2 * at + 1] = s;
    }
    base_f += ef.y;
  }
  const int n_slots = p.B * p.max_splits;
  for (int i = total_items + tid; i < n_slots; i += kOrderThreads) {
    p.order[2 * i] = -1;
    p.order[2 * i + 1] = -1;
  }
}

// KV heads per workgroup of the head-set kernel, or 0 for the general one
// (the head-set kernel's 16-token chunks start at multiples of 16 and must
// not cross a page)
// (more than 8 query heads per KV head: NH = 2 with subgroups of 8, the
// host's head subgroups)
static int head_set(const DecodeParams& p) {
  if (p.page_size % 16 != 0 || p.split_tokens % 16 != 0) return 0;
  if (p.group <= 4 && p.Hkv % 4 == 0) return 4;
  if (p.group > 4 && p.Hkv % 2 == 0 && p.sub_groups == (p.group + 7) / 8) return 2;
  return 0;
}

template <int D>
static hipError_t launch_decode_d(const DecodeParams& p_in, int rows, hipStream_t stream) {
  DecodeParams p = p_in;
  // Without a host plan the split grid takes the device-made order when the
  // 1-D grid over every slot fits: found by each workgroup of the head-set
  // kernel for small batches, else written by the order kernel; otherwise one
  // workgroup per (request, split) slot.
  const int nh = head_set(p);
  const int64_t per = nh > 0 ? (int64_t)p.Hkv / nh * p.sub_groups : (int64_t)p.Hkv * p.sub_groups;
  const bool fits = (int64_t)p.B * p.max_splits * per * kDecodeThreads < ((int64_t)1 << 32);
  if (!p.planned && fits && nh > 0 && p.B <= kSelfOrderMaxB) {
    p.self_order = true;
    p.num_items = p.B * p.max_splits;
  } else if (!p.planned && fits) {
    hipLaunchKernelGGL(decode_order_kernel, dim3(1), dim3(kOrderThreads), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    p.planned = true;
    p.plan = p.order;
    p.num_items = p.B * p.max_splits;
  }
  // an empty plan (every request has length 0): the merge alone writes O = 0
  if (!p.planned || p.num_items > 0) {
    if (nh > 0) {
      const dim3 grid = p.planned || p.self_order ? dim3((unsigned)(p.num_items * per))
                                                  : dim3((unsigned)per, p.max_splits, p.B);
      const bool nt = p.sub_groups == 1;
      if (nh == 4) hipLaunchKernelGGL((decode_split_heads_kernel<D, 4, true>), grid, dim3(kDecodeThreads), 0, stream, p);
      else if (nt) hipLaunchKernelGGL((decode_split_heads_kernel<D, 2, true>), grid, dim3(kDecodeThreads), 0, stream, p);
      else hipLaunchKernelGGL((decode_split_heads_kernel<D, 2, false>), grid, dim3(kDecodeThreads), 0, stream, p);
    } else if (p.page_size % 16 == 0) {
      launch_split<D, true>(p, rows, stream);
    } else {
      launch_split<D, false>(p, rows, stream);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const dim3 grid2(p.Hq, p.B), block2(64);
  hipLaunchKernelGGL((decode_merge_kernel<D>), grid2, block2, 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeParams& p, int d, int rows, hipStream_t stream) {
  return d == 128 ? launch_decode_d<128>(p, rows, stream) : launch_decode_d<64>(p, rows, stream);
}

// Device memory of the allocation-free decode call (fa_decode_paged_noalloc):
// the split partials and the work order live here instead of in a caller's
// workspace.  Each GPU the library runs on holds one copy for the life of the
// process; host code reaches it only through the address hipGetSymbolAddress
// returns for the current device (the array's own name is not a device
// address in host code).
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

void* decode_scratch(hipError_t* err) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* ptrs[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *err = e != hipSuccess ? e : hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (!ptrs[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      *err = e != hipSuccess ? e : hipErrorInvalidSymbol;
      return nullptr;
    }
    ptrs[dev] = p;
  }
  *err = hipSuccess;
  return ptrs[dev];
}

}  // namespace fa
