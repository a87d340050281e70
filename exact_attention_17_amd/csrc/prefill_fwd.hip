// Fused exact-attention prefill forward for gfx950 (dense and varlen).
//
// What it computes (cited by page title and section):
//   O = softmax(scale * Q K^T + mask) V and LSE = m + ln(l) per query row
//   ("FlashAttention-3 vs naive attention: inference comparison", sec. 1.1),
//   tile by tile with an online softmax that keeps a running row max m and a
//   normaliser l and rescales the partial output when m grows ("FIA /
//   FlashAttention" explainer, sec. 1), with QK^T, masking, softmax and PV
//   fused in one kernel so S and P never reach HBM (the FA3 inference page,
//   sec. 1.2 and 4.2).  Q is split into row blocks and K/V into column blocks
//   held on chip (the "FlashAttention" concept page, tiling strategy).
//   Causal and sliding-window masks, GQA broadcast and packed varlen batches
//   follow the configuration skill page (sec. 3.2-3.4, GQA appendix).
//
// Mapping onto CDNA4 (our design, not the pages'):
//   * A workgroup is 4 wave64s and owns 128 query rows of one (batch, head);
//     each wave owns 32 rows.  The loop walks 64-key tiles of K and V.
//   * Scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_bf16: K rows are the A operand (from LDS), the
//     wave's Q rows are the B operand and stay in registers for the whole
//     loop.  In the accumulator each lane then holds ONE query (column) and
//     16 keys per 32x32 tile, so the row max is an in-lane max plus one
//     exchange between the two wave halves, and the row sum needs no
//     cross-lane work until the epilogue.
//   * The same accumulator registers, rounded to bf16, are exactly the B
//     operand of the PV product computed as O^T = V^T P^T: no LDS round trip
//     for P.  The A operand V^T needs 4 consecutive keys per lane at a fixed
//     d, so V is transposed while it is staged into LDS (register shuffles
//     with v_perm_b32 and 8-byte LDS writes).
//   * Softmax runs in base 2 with scale*log2(e) folded into one FMA per score.
//     The reference max used in the exponent is only raised when a row's max
//     exceeds it by more than 2^8 (wave-uniform branch), so the output
//     rescale is skipped on almost every tile; P stays <= 256 and the final
//     division by l makes the result exact either way.
//   * K/V tiles are double-buffered in LDS: the buffer loads of tile j+1 are
//     issued before tile j is computed and written to the other buffer after
//     it.  Rows past a sequence end come back as zeros from the buffer range
//     check.  LDS rows are padded so MFMA operand reads and the staging
//     writes avoid bank conflicts with affine addresses.
//   * Workgroup order: heavy causal tiles first; when the KV-group count is a
//     multiple of 8, all query heads of a KV group land on one XCD (blocks are
//     dealt to the 8 XCDs round-robin), so its K/V stays in one L2.
#include "fa_internal.h"
#include "gfx950.h"

#include <float.h>
#include <math.h>

namespace fa {

namespace {

constexpr float kRescaleTau = 8.0f;   // log2 units: rescale only if max grows > 2^8
constexpr float kLn2 = 0.6931471805599453f;

// LDS tile layouts (element units are bf16).  Rows are padded so that the
// MFMA operand reads of 32 different rows hit different banks while every
// address stays affine (one base register plus immediate offsets).
//   K tile   [64 keys][D + 8]: a 16-byte read per lane, 8 lanes per bank cycle.
//   V^T tile [D rows][64 + 4]: 4 keys (8 bytes) per lane, 16 lanes per cycle.
template <int D> struct Lds {
  static constexpr int kStride = D + 8;
  static constexpr int vStride = kBlockN + 4;
  static constexpr int kTile = kBlockN * kStride;
  static constexpr int vTile = D * vStride;
  static constexpr int stage = kTile + vTile;
};

struct WorkItem {
  int b, h, qt;
  int q_base, k_base;   // first token of the sequence (varlen) or 0
  int Lq, Lk;
  bool valid;
};

__device__ __forceinline__ WorkItem map_work_dense(const PrefillParams& p, int id) {
  WorkItem w;
  if (p.xcd_groups > 0) {
    const int x = id & 7, s = id >> 3;
    const int per = (p.xcd_groups >> 3) * p.group;      // query heads per XCD
    const int qrev = s / per, r = s - qrev * per;
    const int gl = r / p.group, gq = r - gl * p.group;
    const int kvg = x + 8 * gl;
    w.b = kvg / p.Hkv;
    w.h = (kvg - w.b * p.Hkv) * p.group + gq;
    w.qt = p.num_q_tiles - 1 - qrev;
  } else {
    const int NH = p.B * p.Hq;
    const int qrev = id / NH, r = id - qrev * NH;
    w.b = r / p.Hq;
    w.h = r - w.b * p.Hq;
    w.qt = p.num_q_tiles - 1 - qrev;
  }
  w.q_base = 0;
  w.k_base = 0;
  w.Lq = p.Lq;
  w.Lk = p.Lk;
  w.valid = true;
  return w;
}

// Varlen: tile slots of sequence b start at T_b = floor(cu_q[b] / 128) + b,
// which leaves room for its ceil(len_b / 128) tiles before T_{b+1}.
__device__ __forceinline__ WorkItem map_work_varlen(const PrefillParams& p, int id) {
  WorkItem w;
  const int r = id % p.Hq, t = id / p.Hq;
  if (p.xcd_groups > 0) {
    const int x = r & 7, i = r >> 3;
    const int kvh = x + 8 * (i / p.group);
    w.h = kvh * p.group + (i % p.group);
  } else {
    w.h = r;
  }
  int lo = 0, hi = p.B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (p.cu_q[mid] / kBlockM + mid <= t) lo = mid; else hi = mid - 1;
  }
  w.b = lo;
  w.q_base = p.cu_q[lo];
  w.Lq = p.cu_q[lo + 1] - w.q_base;
  w.k_base = p.cu_k[lo];
  w.Lk = p.cu_k[lo + 1] - w.k_base;
  const int lt = t - (w.q_base / kBlockM + lo);
  const int ntiles = (w.Lq + kBlockM - 1) / kBlockM;
  w.valid = lt < ntiles;
  w.qt = ntiles - 1 - lt;
  return w;
}

}  // namespace

template <int D, bool VARLEN>
__global__ __launch_bounds__(kPrefillThreads, 2)
void prefill_fwd_kernel(PrefillParams p) {
  constexpr int KSTEPS = D / 16;                 // QK^T MFMA steps over d
  constexpr int DBLK = D / 32;                   // 32-row blocks of O^T
  constexpr int KCH = D / 8;                     // 16-byte chunks per row
  constexpr int K_LOADS = kBlockN * KCH / kPrefillThreads;
  constexpr int K_ROWS_PER_PASS = kPrefillThreads / KCH;
  constexpr int V_ITEMS = (kBlockN / 4) * KCH;   // 4 keys x 8 d per item
  constexpr int STAGE = Lds<D>::stage;           // K tile + V^T tile (bf16 elements)
  constexpr int KS = Lds<D>::kStride, VS = Lds<D>::vStride;

  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, hi = lane >> 5;

  const WorkItem w = VARLEN ? map_work_varlen(p, blockIdx.x) : map_work_dense(p, blockIdx.x);
  if (!w.valid) return;
  const int Lq = w.Lq, Lk = w.Lk;
  const int kvh = w.h / p.group;
  const int delta = Lk - Lq;

  const uint16_t* qg;
  const uint16_t* kg;
  const uint16_t* vg;
  uint16_t* og;
  float* lseg = nullptr;
  if (VARLEN) {
    qg = p.q + (int64_t)w.q_base * p.q_tok_stride + (int64_t)w.h * D;
    og = p.o + (int64_t)w.q_base * p.q_tok_stride + (int64_t)w.h * D;
    kg = p.k + (int64_t)w.k_base * p.k_tok_stride + (int64_t)kvh * D;
    vg = p.v + (int64_t)w.k_base * p.k_tok_stride + (int64_t)kvh * D;
    if (p.lse) lseg = p.lse + (int64_t)w.h * p.lse_seq_stride + w.q_base;
  } else {
    qg = p.q + (int64_t)w.b * p.q_batch_stride + (int64_t)w.h * D;
    og = p.o + (int64_t)w.b * p.q_batch_stride + (int64_t)w.h * D;
    kg = p.k + (int64_t)w.b * p.k_batch_stride + (int64_t)kvh * D;
    vg = p.v + (int64_t)w.b * p.k_batch_stride + (int64_t)kvh * D;
    if (p.lse) lseg = p.lse + ((int64_t)w.b * p.Hq + w.h) * p.lse_seq_stride;
  }

  // ---- key range of the workgroup and of this wave ------------------------
  const int q0 = w.qt * kBlockM;
  const int r_first = q0, r_last = min(q0 + kBlockM, Lq) - 1;
  auto key_lo = [&](int row) { return p.win_left >= 0 ? max(0, row + delta - p.win_left) : 0; };
  auto key_hi = [&](int row) {    // exclusive
    int e = Lk;
    if (p.causal) e = min(e, row + delta + 1);
    if (p.win_right >= 0) e = min(e, row + delta + p.win_right + 1);
    return e;
  };
  const int kv_lo = key_lo(r_first);
  const int kv_hi = key_hi(r_last);
  const int kt_begin = kv_lo / kBlockN;
  const int kt_end = kv_hi > kv_lo ? (kv_hi + kBlockN - 1) / kBlockN : kt_begin;
  const int ntiles = kt_end - kt_begin;

  const int qw0 = q0 + 32 * wave;
  const bool wave_rows = qw0 < Lq;
  const int rw0 = qw0, rw1 = min(qw0 + 31, Lq - 1);
  const int wlo_first = key_lo(rw0), wlo_last = key_lo(rw1);
  const int whi_first = key_hi(rw0), whi_last = key_hi(rw1);
  const int row = qw0 + n;                       // this lane's query row
  const int my_lo = key_lo(row), my_hi = key_hi(row);

  // ---- Q fragments (B operand), resident for the whole loop --------------
  const uint32_t q_bytes = (uint32_t)(((int64_t)(Lq - 1) * p.q_tok_stride + D) * 2);
  const uint32_t k_bytes = Lk > 0 ? (uint32_t)(((int64_t)(Lk - 1) * p.k_tok_stride + D) * 2) : 0u;
  const uint32_t k_row_bytes = (uint32_t)(p.k_tok_stride * 2);
  u32x4 qf[KSTEPS];
  {
    const __amdgpu_buffer_rsrc_t qr = make_rsrc(qg, q_bytes);
    const uint32_t off = row < Lq ? (uint32_t)(row * p.q_tok_stride + 8 * hi) * 2u : kOob;
#pragma unroll
    for (int t = 0; t < KSTEPS; ++t) qf[t] = buf_load16(qr, off + 32u * t);
  }

  // ---- staging of one K/V tile: global -> registers -> LDS ----------------
  u32x4 kreg[K_LOADS];
  u32x4 vreg[4];
  const int kc = tid % KCH, kr0 = tid / KCH;
  // V items (4 keys x 8 d): 16 lanes of one LDS write phase take 8 key groups x
  // 2 d-chunks, so (d + key group) mod 16 -- the bank pair -- is distinct.
  const int vkg = (tid & 7) | (((tid >> 4) & 1) << 3);
  const int vdc = ((tid >> 3) & 1) | ((tid >> 5) << 1);
  const bool v_active = tid < V_ITEMS;

  const __amdgpu_buffer_rsrc_t krs = make_rsrc(kg, k_bytes);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vg, k_bytes);
  auto load_tile = [&](int kb) {
#pragma unroll
    for (int i = 0; i < K_LOADS; ++i) {
      const int key = kb + kr0 + i * K_ROWS_PER_PASS;
      const uint32_t off = key < Lk ? (uint32_t)key * k_row_bytes + kc * 16u : kOob;
      kreg[i] = buf_load16(krs, off);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = kb + 4 * vkg + i;
      const uint32_t off = (v_active && key < Lk) ? (uint32_t)key * k_row_bytes + vdc * 16u : kOob;
      vreg[i] = buf_load16(vrs, off);
    }
  };
  auto store_tile = [&](int stage) {
    uint16_t* ks = smem + stage * STAGE;
    uint16_t* vs = ks + Lds<D>::kTile;
#pragma unroll
    for (int i = 0; i < K_LOADS; ++i) {
      const int r = kr0 + i * K_ROWS_PER_PASS;
      *reinterpret_cast<u32x4*>(ks + r * KS + kc * 8) = kreg[i];
    }
    if (v_active) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
        const uint32_t w0 = __builtin_amdgcn_perm(vreg[1][e >> 1], vreg[0][e >> 1], sel);
        const uint32_t w1 = __builtin_amdgcn_perm(vreg[3][e >> 1], vreg[2][e >> 1], sel);
        *reinterpret_cast<u32x2*>(vs + (vdc * 8 + e) * VS + vkg * 4) = u32x2{w0, w1};
      }
    }
  };

  // ---- running state ------------------------------------------------------
  f32x16 oacc[DBLK];
#pragma unroll
  for (int i = 0; i < DBLK; ++i) oacc[i] = f32x16{};
  float m_ref = -INFINITY;   // reference max, log2 units
  float l_sum = 0.f;         // partial row sum over this lane's half of the keys
  const float c = p.scale_log2;

  if (ntiles > 0) {
    load_tile(kt_begin * kBlockN);
    store_tile(0);
  }
  __syncthreads();

  for (int it = 0; it < ntiles; ++it) {
    const int stage = it & 1;
    const int kb = (kt_begin + it) * kBlockN;
    if (it + 1 < ntiles) load_tile(kb + kBlockN);

    const bool active = wave_rows && kb < whi_last && kb + kBlockN > wlo_first;
    if (active) {
      const uint16_t* ks = smem + stage * STAGE;
      const uint16_t* vs = ks + Lds<D>::kTile;
      // S^T = K Q^T for two 32-key halves of the tile
      f32x16 sacc[2];
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
        sacc[kb2] = f32x16{};
        const int key = 32 * kb2 + n;
#pragma unroll
        for (int t = 0; t < KSTEPS; ++t) {
          const u32x4 a = *reinterpret_cast<const u32x4*>(ks + key * KS + (2 * t + hi) * 8);
          sacc[kb2] = mfma32x32x16(a, qf[t], sacc[kb2]);
        }
      }
      // mask only on tiles that cut through some row's visible band
      const bool full = kb >= wlo_last && kb + kBlockN <= whi_first;
      if (!full) {
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kb + 32 * kb2 + 8 * (r >> 2) + 4 * hi + (r & 3);
            sacc[kb2][r] = (key >= my_lo && key < my_hi) ? sacc[kb2][r] : -INFINITY;
          }
        }
      }
      // row max over the tile: in-lane, then across the two wave halves
      float mx = sacc[0][0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sacc[0][r]);
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[1][r]);
      mx = fmaxf(mx, xor32(mx));
      const float tmax = mx * c;
      const bool up = tmax > m_ref + kRescaleTau;
      if (wave_any(up)) {
        const float m_new = up ? tmax : m_ref;
        const float alpha = up ? exp2_fast(m_ref - m_new) : 1.f;
        l_sum *= alpha;
#pragma unroll
        for (int i = 0; i < DBLK; ++i) oacc[i] *= alpha;
        m_ref = m_new;
      }
      const float mb = (m_ref == -INFINITY) ? 0.f : m_ref;
      // P = 2^(S*c - m): fp32 exponentials, bf16 fragments for the PV MFMA
      u32x4 pf[4];
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
        float pv[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          pv[r] = exp2_fast(fmaf(sacc[kb2][r], c, -mb));
          l_sum += pv[r];
        }
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          pf[2 * kb2 + hh] = u32x4{pack_bf16x2(pv[8 * hh + 0], pv[8 * hh + 1]),
                                   pack_bf16x2(pv[8 * hh + 2], pv[8 * hh + 3]),
                                   pack_bf16x2(pv[8 * hh + 4], pv[8 * hh + 5]),
                                   pack_bf16x2(pv[8 * hh + 6], pv[8 * hh + 7])};
        }
      }
      // O^T += V^T P^T, 16 keys per MFMA
#pragma unroll
      for (int db = 0; db < DBLK; ++db) {
        const int d = 32 * db + n;
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
          const u32x2 lo = *reinterpret_cast<const u32x2*>(vs + d * VS + (4 * cc + hi) * 4);
          const u32x2 hi2 = *reinterpret_cast<const u32x2*>(vs + d * VS + (4 * cc + 2 + hi) * 4);
          const u32x4 a = u32x4{lo[0], lo[1], hi2[0], hi2[1]};
          oacc[db] = mfma32x32x16(a, pf[cc], oacc[db]);
        }
      }
    }

    if (it + 1 < ntiles) store_tile(stage ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O = acc / l (bf16), LSE = (m + log2 l) * ln 2 ------------
  const float lt = l_sum + xor32(l_sum);
  if (row < Lq) {
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    uint16_t* orow = og + (int64_t)row * p.q_tok_stride;
#pragma unroll
    for (int db = 0; db < DBLK; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = 32 * db + 8 * g + 4 * hi;
        const u32x2 val = u32x2{pack_bf16x2(oacc[db][4 * g + 0] * inv, oacc[db][4 * g + 1] * inv),
                                pack_bf16x2(oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv)};
        *reinterpret_cast<u32x2*>(orow + d) = val;
      }
    }
    if (lseg && hi == 0) lseg[row] = lt > 0.f ? (m_ref + log2_fast(lt)) * kLn2 : -INFINITY;
  }
}

hipError_t launch_prefill(const PrefillParams& p, int d, bool varlen, hipStream_t stream) {
  const int64_t nblocks = varlen ? (int64_t)p.num_q_tiles * p.Hq
                                 : (int64_t)p.num_q_tiles * p.B * p.Hq;
  if (nblocks <= 0) return hipSuccess;
  const dim3 grid((unsigned)nblocks), block(kPrefillThreads);
  if (d == 128) {
    if (varlen) hipLaunchKernelGGL((prefill_fwd_kernel<128, true>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((prefill_fwd_kernel<128, false>), grid, block, 0, stream, p);
  } else {
    if (varlen) hipLaunchKernelGGL((prefill_fwd_kernel<64, true>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((prefill_fwd_kernel<64, false>), grid, block, 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace fa
