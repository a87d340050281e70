// Backward pass of fused exact attention for gfx950 (dense layout).
//
// What it computes: dQ, dK, dV of O = softmax(scale * Q K^T + mask) V (the
// forward of prefill_fwd.hip) for an upstream gradient dO, by the chain rule
// of that definition:
//   P = exp(scale * Q K^T - LSE)       recomputed from the saved LSE
//   dV = P^T dO,  dP = dO V^T,  delta_i = dO_i . O_i,  dS = P * (dP - delta)
//   dQ = scale * dS K,  dK = scale * dS^T Q
// with the dK, dV of a KV head summed over the query heads of its group.  The
// pages' backward keeps no score matrix from the forward and recomputes the
// blocks it needs from the saved row statistics ("FlashAttention" concept
// page, recomputation; "FIA / FlashAttention" explainer, sec. 1).
//
// Mapping onto CDNA4 (our design, not the pages'):
//   * bwd_prep_kernel: delta = dO . O and lse2 = LSE * log2(e) per query row,
//     one coalesced pass over dO and O, into a caller workspace.
//   * bwd_dkdv_kernel: a workgroup owns 128 keys of one (batch, KV head) and
//     has 8 waves, two per 32-key block: one keeps K resident (MFMA B
//     operand) and accumulates dV^T, its partner keeps V resident and
//     accumulates dK^T, over every query row of every query head of the
//     group, streamed through LDS in 64-row tiles.  Per 32-row half,
//     S = Q K^T and dP = dO V^T take Q and dO rows from LDS as the A operand;
//     the accumulator gives each lane one key and 16 query rows, which
//     rounded to bf16 are exactly the B operand of dV^T += dO^T P and
//     dK^T += Q^T dS (A = dO^T and Q^T by transpose reads).  P goes to the
//     partner through LDS (fp32).
//   * bwd_dq_kernel: a workgroup owns 128 query rows of one (batch, head), 32
//     per wave, as in the forward; the wave's Q and dO rows stay in registers
//     as B operands while K and V stream through LDS in 64-key tiles:
//     S^T = K Q^T, dP^T = V dO^T, then dQ^T += K^T dS^T (K^T by transpose
//     reads).  Each lane holds one query row, so its lse2 and delta are two
//     registers.
//   * No atomics: every gradient element is summed by one wave in a fixed
//     order, so the result is bitwise reproducible run to run.
//   * Tiles go global -> LDS directly (buffer loads with the lds flag),
//     double-buffered; one XOR swizzle serves both the row reads and the
//     transpose reads of the same tile.
#include "fa_internal.h"
#include "gfx950.h"
#include "work_map.h"

#include <math.h>

#include <type_traits>

namespace fa {

namespace {

constexpr float kLog2eF = 1.4426950408889634f;

// [64 rows][D] bf16 tiles, row-major and unpadded (each direct-to-LDS load
// instruction writes 1 KB contiguously).  16-byte chunk c of row r is stored
// at chunk c ^ swz(r), which depends on r & 15 only:
//   D = 128: swz = 4 (r & 3) + ((r >> 2) & 3).  The 16 rows of a 16-row block
//     get 16 distinct values, so a row read (lane n on row n, 16 bytes) puts
//     16 lanes on 16 distinct 16-byte bank groups; the 4 rows of an aligned
//     transpose-read group differ in bits 2-3, so their 4 x 4 chunks land on
//     16 distinct bank groups.
//   D = 64: swz = 4 ((r >> 1) & 1) + ((r >> 2) & 3).  Rows are 128 bytes, so
//     rows of equal parity share a bank half: the 8 even (odd) rows of a
//     16-row block get distinct values, and rows r and r + 2 of a transpose
//     group differ in bit 2.
template <int D> struct BLds {
  static constexpr int kTile = 64 * D;
  FA_DEV static int swz(int r) {
    return D == 128 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
  }
};

// Float offset of statistics row r's lse2; its delta is 64 floats further.
// Every (batch, head) or (sequence, head) starts at a multiple of 64 rows.
FA_DEV int64_t stat_offset(int64_t r) {
  return (r / kBwdStatRows) * (2 * kBwdStatRows) + (r % kBwdStatRows);
}

// First statistics row of (batch b, head h) (dense), or of sequence b of
// head h, whose tile slots start at t_b (varlen).
template <bool VARLEN>
FA_DEV int64_t stat_base(const BwdParams& p, int b, int h, int t_b) {
  return VARLEN ? (int64_t)h * p.stat_rows + (int64_t)t_b * kBlockM
                : (int64_t)(b * p.Hq + h) * p.Lq_pad;
}

// Sequence owning tile slot t when sequence b's slots start at
// floor(cu[b] / tile) + b (binary search over the cumulative offsets).
FA_DEV int slot_sequence(const int* cu, int B, int t, int tile) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu[mid] / tile + mid <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

}  // namespace

// One group of D/8 lanes per statistics row, in row order, so consecutive
// groups write consecutive statistics: delta = sum_d dO * O in fp32 (fixed
// order), lse2 = LSE * log2(e), or +inf for a row with no visible key
// (LSE = -inf) and for padding rows, so that exp2(x - lse2) = 0 there.
template <int D, bool VARLEN>
__global__ __launch_bounds__(256)
void bwd_prep_kernel(BwdParams p) {
  constexpr int KCH = D / 8;
  // all statistics rows < 2^28 (the statistics are < 2^31 bytes): 32-bit indices
  const uint32_t gid = blockIdx.x * 256u + threadIdx.x;
  const uint32_t row = gid / KCH;
  const int ch = (int)(gid % KCH);
  const uint32_t rows_per_head = VARLEN ? (uint32_t)p.stat_rows : (uint32_t)p.Lq_pad;
  if (row >= (uint32_t)(VARLEN ? p.Hq : p.B * p.Hq) * rows_per_head) return;   // whole groups exit together
  const uint32_t bh = row / rows_per_head;
  const int r = (int)(row - bh * rows_per_head);
  int b, h, i, lq;
  int64_t tok;       // token index of the row (varlen: in the packed batch)
  if (VARLEN) {
    h = (int)bh;
    b = slot_sequence(p.cu_q, p.B, r / kBlockM, kBlockM);
    i = r - (p.cu_q[b] / kBlockM + b) * kBlockM;
    lq = p.cu_q[b + 1] - p.cu_q[b];
    tok = (int64_t)p.cu_q[b] + i;
  } else {
    b = (int)(bh / (uint32_t)p.Hq);
    h = (int)(bh - (uint32_t)b * (uint32_t)p.Hq);
    i = r;
    lq = p.Lq;
    tok = (int64_t)b * p.Lq + i;
  }
  float s = 0.f;
  if (i < lq) {
    const int64_t off = tok * p.q_tok_stride + (int64_t)h * D + 8 * ch;
    const u32x4 a = *reinterpret_cast<const u32x4*>(p.dout + off);
    const u32x4 o = *reinterpret_cast<const u32x4*>(p.o + off);
#pragma unroll
    for (int e = 0; e < 4; ++e) s += bf16lo(a[e]) * bf16lo(o[e]) + bf16hi(a[e]) * bf16hi(o[e]);
  }
#pragma unroll
  for (int m = KCH / 2; m > 0; m >>= 1) s += __shfl_xor(s, m);
  if (ch == 0) {
    float l2 = INFINITY;
    if (i < lq) {
      const float l = VARLEN ? p.lse[(int64_t)h * p.lse_seq_stride + tok]
                             : p.lse[((int64_t)b * p.Hq + h) * p.lse_seq_stride + i];
      l2 = l == -INFINITY ? INFINITY : l * kLog2eF;
    }
    const int64_t so = stat_offset(row);
    p.stat[so] = l2;
    p.stat[so + kBwdStatRows] = s;
  }
}

// Split roles: 8 waves, two per 32-key block.  Wave w < 4 (the "P" wave)
// keeps K^T of keys 32w.. resident, computes S and P and accumulates dV^T;
// wave w + 4 (the "dS" wave, on the same SIMD) keeps V^T resident, computes
// dP, takes P (fp32) from its partner through LDS, forms dS and accumulates
// dK^T.  Each wave then holds one resident operand and one accumulator, and
// the MFMA work of a block splits evenly between the pair.
// At d = 64 the kernel is held to 128 VGPRs (four waves per SIMD), so two
// workgroups share a CU (2 x 66 KB of LDS) and each hides the other's
// barriers; at d = 128 it needs 234 and runs one workgroup per CU.
constexpr int kDkdvThreads = 512;

template <int D, bool VARLEN>
__global__ __attribute__((amdgpu_flat_work_group_size(kDkdvThreads, kDkdvThreads),
                          amdgpu_waves_per_eu(D == 64 ? 4 : 2)))
void bwd_dkdv_kernel(BwdParams p) {
  constexpr int KSTEPS = D / 16;                 // MFMA steps over d
  constexpr int DBLK = D / 32;                   // 32-row blocks of dK^T, dV^T
  constexpr int KCH = D / 8;                     // 16-byte chunks per row
  constexpr int RPI = 64 / KCH;                  // rows per 1 KB load instruction
  constexpr int TILE_BYTES = BLds<D>::kTile * 2;
  constexpr int LOADS = TILE_BYTES / 1024 / 8;   // load instructions per wave per tile
  static_assert(LOADS >= 1, "tile smaller than one load per wave");

  __shared__ __attribute__((aligned(1024))) uint16_t q_lds[2 * BLds<D>::kTile];
  __shared__ __attribute__((aligned(1024))) uint16_t do_lds[2 * BLds<D>::kTile];
  __shared__ __attribute__((aligned(1024))) float st_lds[2 * 256];   // per buffer: lse2[64], delta[64]
  // P of a 32-row half, per key block: [half][block][j][lane][4] floats
  __shared__ __attribute__((aligned(16))) float x_lds[2][4][4][64][4];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int blk = wave & 3, role = wave >> 2;    // role 0: S, P, dV; role 1: dP, dS, dK
  const int n = lane & 31, hi = lane >> 5;
  const int i16 = lane & 15, g16 = lane >> 4;

  // ---- work item: (batch b, KV head g, key tile kt), early key tiles (which
  // the most causal rows see) first; with the XCD-aware order all key tiles
  // of a KV group run on one XCD, so its Q and dO stay in that L2.  Varlen:
  // key tile slots of sequence b start at floor(cu_k[b] / 128) + b.
  int b, g, kt;
  int Lq = p.Lq, Lk = p.Lk;
  int64_t q_tok0 = 0, k_tok0 = 0;   // first token of the sequence (varlen)
  int t_b = 0;                      // first query tile slot of the sequence (varlen)
  if (VARLEN) {
    const int id = blockIdx.x;
    g = id % p.Hkv;
    const int t = id / p.Hkv;
    b = slot_sequence(p.cu_k, p.B, t, kBwdKeys);
    kt = t - (p.cu_k[b] / kBwdKeys + b);
    q_tok0 = p.cu_q[b];
    k_tok0 = p.cu_k[b];
    Lq = p.cu_q[b + 1] - p.cu_q[b];
    Lk = p.cu_k[b + 1] - p.cu_k[b];
    t_b = p.cu_q[b] / kBlockM + b;
    if (kt * kBwdKeys >= Lk) return;   // a spare slot: no keys (uniform per workgroup)
  } else {
    const int id = blockIdx.x;
    if (p.xcd_groups > 0) {
      const int x = id & 7, s = id >> 3;
      const int grp = x + 8 * (s / p.num_k_tiles);
      kt = s % p.num_k_tiles;
      b = grp / p.Hkv;
      g = grp - b * p.Hkv;
    } else {
      const int NG = p.B * p.Hkv;
      kt = id / NG;
      const int r = id - kt * NG;
      b = r / p.Hkv;
      g = r - b * p.Hkv;
    }
    q_tok0 = (int64_t)b * p.Lq;
    k_tok0 = (int64_t)b * p.Lk;
  }
  const int delta = Lk - Lq;
  const int k0 = kt * kBwdKeys;
  const int kw0 = k0 + 32 * blk;
  const int key = kw0 + n;
  const int kend = min(k0 + kBwdKeys, Lk);

  // ---- resident operand (B): K^T (role 0) or V^T (role 1); lane (key n,
  // half hi) holds d = 16t + 8hi + 0..7 of its key; keys past Lk read zeros.
  const int64_t kv_off = k_tok0 * p.k_tok_stride + (int64_t)g * D;
  u32x4 rf[KSTEPS];
  {
    const uint32_t kbytes = (uint32_t)(((int64_t)(Lk - 1) * p.k_tok_stride + D) * 2);   // Lk >= 1 here
    const __amdgpu_buffer_rsrc_t rr = make_rsrc((role == 0 ? p.k : p.v) + kv_off, kbytes);
    const uint32_t off = key < Lk ? (uint32_t)((int64_t)key * p.k_tok_stride + 8 * hi) * 2u : kOob;
#pragma unroll
    for (int t = 0; t < KSTEPS; ++t) rf[t] = buf_load16(rr, off + 32u * t);
#pragma unroll
    for (int t = 0; t < KSTEPS; ++t) await_value(rf[t]);   // not inside the loop
  }

  // ---- query rows that see any key of the workgroup -----------------------
  // key_lo(i) and key_hi(i) grow with i: row i sees a key in [k0, kend) iff
  // key_hi(i) > k0 and key_lo(i) < kend.
  auto key_lo = [&](int row) { return p.win_left >= 0 ? max(0, row + delta - p.win_left) : 0; };
  auto key_hi = [&](int row) {    // exclusive
    int e = Lk;
    if (p.causal) e = min(e, row + delta + 1);
    if (p.win_right >= 0) e = min(e, row + delta + p.win_right + 1);
    return e;
  };
  int64_t i_lo = 0, i_hi = Lq - 1;
  if (p.causal) i_lo = max(i_lo, (int64_t)k0 - delta);
  if (p.win_right >= 0) i_lo = max(i_lo, (int64_t)k0 - delta - p.win_right);
  if (p.win_left >= 0) i_hi = min(i_hi, (int64_t)kend - 1 - delta + p.win_left);
  // Rows that see this lane's key: qmin <= i <= qmax (the key is visible to
  // row i iff key_lo(i) <= key < key_hi(i)); keys past Lk only feed their
  // own, unwritten, columns.
  int64_t qmin = -((int64_t)1 << 40), qmax = (int64_t)1 << 40;
  if (p.causal) qmin = max(qmin, (int64_t)key - delta);
  if (p.win_right >= 0) qmin = max(qmin, (int64_t)key - delta - p.win_right);
  if (p.win_left >= 0) qmax = (int64_t)key - delta + p.win_left;
  const int qmin_c = (int)max(qmin, (int64_t)-1), qmax_c = (int)min(qmax, (int64_t)Lq);
  const int qt_begin = (int)(i_lo / 64);
  const int nq = i_hi >= i_lo ? (int)(i_hi / 64) - qt_begin + 1 : 0;
  const int nsteps = p.group * nq;               // (query head, 64-row tile), head-major

  // ---- staging: global -> LDS directly --------------------------------------
  // Load instruction i of wave w fills tile bytes [(8i + w) KB, +1 KB): rows
  // (8i + w) * RPI + lane / KCH, stored chunk lane % KCH holding logical chunk
  // (lane % KCH) ^ swz(row); swz depends on row & 15, which i does not
  // change, so each lane keeps one byte offset and the tile row goes in the
  // scalar offset.  Rows at or past Lq fall outside the buffer and load as
  // zeros.  Wave 0 also loads the tile's 64 lse2 and 64 delta values (512
  // contiguous bytes of the statistics; lanes 32-63 load zeros).
  const uint32_t q_row_bytes = (uint32_t)(p.q_tok_stride * 2);
  const uint32_t q_bytes = Lq > 0 ? (uint32_t)(((int64_t)(Lq - 1) * p.q_tok_stride + D) * 2) : 0u;
  uint32_t src;
  {
    const int r = wave * RPI + lane / KCH, slot = lane % KCH;
    src = (uint32_t)r * q_row_bytes + (uint32_t)((slot ^ BLds<D>::swz(r)) * 16);
  }
  const uint32_t q_lds_addr = lds_address(q_lds), do_lds_addr = lds_address(do_lds);
  const uint32_t st_lds_addr = lds_address(st_lds);
  const uint32_t wave_lds = (uint32_t)__builtin_amdgcn_readfirstlane(wave * 1024);
  const uint16_t* qb = p.q + q_tok0 * p.q_tok_stride;
  const uint16_t* dob = p.dout + q_tok0 * p.q_tok_stride;
  const uint32_t stat_bytes = (uint32_t)((int64_t)(VARLEN ? p.Hq : p.B * p.Hq) *
                                         (VARLEN ? p.stat_rows : p.Lq_pad) * 2 * 4);
  const __amdgpu_buffer_rsrc_t srs = make_rsrc(p.stat, stat_bytes);
  const uint32_t st_src = lane < 32 ? 16u * lane : kOob;
  auto fetch = [&](int s, int buf) {
    const int hh = g * p.group + s / nq;
    const int qt = qt_begin + s % nq;
    const __amdgpu_buffer_rsrc_t qr = make_rsrc(qb + (int64_t)hh * D, q_bytes);
    const __amdgpu_buffer_rsrc_t dr = make_rsrc(dob + (int64_t)hh * D, q_bytes);
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const uint32_t soff =
          (uint32_t)__builtin_amdgcn_readfirstlane((int)((uint32_t)(qt * 64 + 8 * i * RPI) * q_row_bytes));
      lds_load16(qr, src, soff, q_lds_addr + buf * TILE_BYTES + wave_lds + 8192u * i);
      lds_load16(dr, src, soff, do_lds_addr + buf * TILE_BYTES + wave_lds + 8192u * i);
    }
    if (wave == 0) {
      const int64_t sr = stat_base<VARLEN>(p, b, hh, t_b) + qt * 64;
      const uint32_t so = (uint32_t)__builtin_amdgcn_readfirstlane((int)(stat_offset(sr) * 4));
      lds_load16(srs, st_src, so, st_lds_addr + buf * 1024u);
    }
  };

  // ---- LDS reads ----------------------------------------------------------
  // Row reads (A operand of S = Q K^T and dP = dO V^T): lane (row n, half hi)
  // reads logical chunk 2t + hi of row 32qh + n; the stored chunk's byte
  // address is a per-lane base XOR 32t.
  const uint32_t row_base = (uint32_t)(n * 2 * D) | ((16u * hi) ^ (16u * BLds<D>::swz(n)));
  auto row_frag = [&](const char* tile, int qh, int t) {
    return *reinterpret_cast<const u32x4*>(tile + 64 * qh * D + (row_base ^ (32u * t)));
  };
  // Transpose reads (A operand of dV^T = dO^T P and dK^T = Q^T dS): lane i of
  // 16-lane group g addresses row 16cc + 8j + 4hi + i/4 and the 8-byte unit
  // 8db + 4(g&1) + (i&3) of it, i.e. half i&1 of logical chunk
  // 4db + 2(g&1) + (i&3)/2; the row's swizzle depends on j, hi and i/4, and
  // db enters the stored chunk's byte address as XOR 64db.
  uint32_t tr_base[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int r = 8 * j + 4 * hi + (i16 >> 2);
    tr_base[j] = (uint32_t)(r * 2 * D) |
                 ((((32u * (g16 & 1)) | (16u * ((i16 & 3) >> 1))) ^ (16u * BLds<D>::swz(r))) |
                  (8u * (i16 & 1)));
  }
  auto tr_frag = [&](const char* tile, int cc, int db) {
    const char* a = tile + 16 * cc * 2 * D;
    const u32x2 lo = tr_read_b64(reinterpret_cast<const uint16_t*>(a + (tr_base[0] ^ (64u * db))));
    const u32x2 hi2 = tr_read_b64(reinterpret_cast<const uint16_t*>(a + (tr_base[1] ^ (64u * db))));
    return u32x4{lo[0], lo[1], hi2[0], hi2[1]};
  };
  f32x16 acc[DBLK];
#pragma unroll
  for (int db = 0; db < DBLK; ++db) acc[db] = f32x16{};
  const float c = p.scale_log2;

  // S = Q K^T (role 0) or dP = dO V^T (role 1) of the tile's 32-row half qh.
  // Lane (key n, half hi) holds rows 32qh + 8j + 4hi + e of the tile in
  // element 4j + e.
  auto product = [&](const char* rt, int qh) {
    f32x16 S = f32x16{};
#pragma unroll
    for (int t = 0; t < KSTEPS; ++t) S = mfma32x32x16(row_frag(rt, qh, t), rf[t], S);
    return S;
  };
  // Role 0: P = 2^(S c - lse2), masked to the rows that see the lane's key
  // (offsets rlo .. rlo + rcount - 1 from row 4hi of the tile); written to the
  // partner as fp32 and packed as the bf16 B operand of dV^T += dO^T P.
  auto make_p = [&](auto masked, const f32x16& S, const float* st, int qh, int rlo,
                    uint32_t rcount, u32x4 (&ops)[2]) {
    float (*xs)[64][4] = x_lds[qh][blk];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4 l2 = *reinterpret_cast<const f32x4*>(st + 32 * qh + 8 * j + 4 * hi);
      f32x4 pv;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float pe = exp2_fast(fmaf(S[4 * j + e], c, -l2[e]));
        if constexpr (decltype(masked)::value) {
          const uint32_t off = (uint32_t)(32 * qh + 8 * j + e);
          pe = (off - (uint32_t)rlo) < rcount ? pe : 0.f;
        }
        pv[e] = pe;
      }
      *reinterpret_cast<f32x4*>(xs[j][lane]) = pv;
      ops[j >> 1][2 * (j & 1)] = pack_bf16x2(pv[0], pv[1]);
      ops[j >> 1][2 * (j & 1) + 1] = pack_bf16x2(pv[2], pv[3]);
    }
  };
  // Role 1: dS = P (dP - delta), with P from the partner and dP in S.
  auto make_ds = [&](const f32x16& S, const float* st, int qh, u32x4 (&ops)[2]) {
    float (*xs)[64][4] = x_lds[qh][blk];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4 dl = *reinterpret_cast<const f32x4*>(st + 64 + 32 * qh + 8 * j + 4 * hi);
      const f32x4 pv = *reinterpret_cast<const f32x4*>(xs[j][lane]);
      float dv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) dv[e] = pv[e] * (S[4 * j + e] - dl[e]);
      ops[j >> 1][2 * (j & 1)] = pack_bf16x2(dv[0], dv[1]);
      ops[j >> 1][2 * (j & 1) + 1] = pack_bf16x2(dv[2], dv[3]);
    }
  };
  // role 0: dV^T += dO^T P; role 1: dK^T += Q^T dS, for half qh
  auto grad = [&](const char* tt, int qh, const u32x4 (&ops)[2]) {
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2) {
#pragma unroll
      for (int db = 0; db < DBLK; ++db)
        acc[db] = mfma32x32x16(tr_frag(tt, 2 * qh + c2, db), ops[c2], acc[db]);
    }
  };
  // Order of a role-0 block: each MFMA, then a few VALU ops of the P
  // computation and the next LDS read, so the exponentials run under the
  // matrix core.
  auto interleave = [](auto n_mfma) {
#pragma unroll
    for (int i = 0; i < decltype(n_mfma)::value; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
  };

  // One step: the 64-row tile s (in buffer `cur`) against the pair's 32 keys,
  // in three phases separated by barriers, so that each wave always has
  // matrix work beside its vector work:
  //   1. S, dP of both halves; role 0 forms P of half 0 under the MFMAs of half 1;
  //   2. role 0: dV with P of half 0, forming P of half 1 under it;
  //      role 1: dS of half 0 (P from the partner), dK with it;
  //   3. dV with P of half 1; role 1: dS of half 1, dK with it.
  // (the role, the buffer parity and whether the tile needs the mask are
  // compile-time constants of each instance, so no accumulator has to be
  // merged across a branch)
  auto step = [&](auto parity, auto role_c, auto masked, int s, int i0) {
    constexpr int cur = decltype(parity)::value;
    constexpr int ROLE = decltype(role_c)::value;
    if (s + 1 < nsteps) fetch(s + 1, cur ^ 1);
    const int rlo = qmin_c - i0 - 4 * hi;
    const uint32_t rcount = (uint32_t)max(qmax_c - qmin_c + 1, 0);
    const char* rt = reinterpret_cast<const char*>(ROLE == 0 ? q_lds : do_lds) + cur * TILE_BYTES;
    const char* tt = reinterpret_cast<const char*>(ROLE == 0 ? do_lds : q_lds) + cur * TILE_BYTES;
    const float* st = st_lds + cur * 256;
    using Eight = std::integral_constant<int, 8>;
    const f32x16 S0 = product(rt, 0);
    __builtin_amdgcn_sched_barrier(0);   // half 1's MFMAs go with P of half 0 (below)
    u32x4 ops0[2], ops1[2];
    const f32x16 S1 = product(rt, 1);
    if constexpr (ROLE == 0) {
      make_p(masked, S0, st, 0, rlo, rcount, ops0);
      interleave(Eight{});
    }
    __syncthreads();   // P of half 0 is in x_lds
    if constexpr (ROLE == 0) {
      grad(tt, 0, ops0);
      make_p(masked, S1, st, 1, rlo, rcount, ops1);
      interleave(Eight{});
    } else {
      make_ds(S0, st, 0, ops0);
      grad(tt, 0, ops0);
    }
    __syncthreads();   // P of half 1 is in x_lds
    if constexpr (ROLE == 1) make_ds(S1, st, 1, ops1);
    grad(tt, 1, ops1);
    lds_load_wait();
    __syncthreads();
  };
  // one step of this wave's role; P needs the mask unless every row of the
  // tile sees all 32 keys of the pair (the dS wave multiplies by P, already
  // masked, so it needs no variant)
  auto role_step = [&](auto parity, auto role_c, int s) {
    const int i0 = (qt_begin + s % nq) * 64;
    const int i_last = min(i0 + 63, Lq - 1);
    const bool full = key_lo(i_last) <= kw0 && key_hi(i0) >= kw0 + 32;
    if (decltype(role_c)::value == 0 && !full)
      step(parity, role_c, std::true_type{}, s, i0);
    else
      step(parity, role_c, std::false_type{}, s, i0);
  };
  auto run = [&](auto role_c) {
    for (int s = 0; s < nsteps; s += 2) {
      role_step(std::integral_constant<int, 0>{}, role_c, s);
      if (s + 1 < nsteps) role_step(std::integral_constant<int, 1>{}, role_c, s + 1);
    }
  };

  if (nsteps > 0) fetch(0, 0);
  lds_load_wait();
  __syncthreads();
  // both roles pass the same barriers in the same order (three per step)
  if (role == 0) run(std::integral_constant<int, 0>{});
  else run(std::integral_constant<int, 1>{});

  // ---- epilogue: role 0 writes dV = dV^T, role 1 dK = scale * dK^T --------
  // Staged through the Q (dV) and dO (dK) tiles, unused from here on: each
  // wave writes its 32 key rows there (16-byte chunk c of row r at
  // c ^ (r % chunks per row)), reads them back as 16-byte chunks and stores
  // whole contiguous rows.
  {
    constexpr int RB = 2 * D;                 // bytes per output row
    constexpr int ORPI = 1024 / RB;           // rows per 1 KB store instruction
    char* stage = reinterpret_cast<char*>(role == 0 ? q_lds : do_lds);   // 128 rows of RB bytes
    uint16_t* out = (role == 0 ? p.dv : p.dk) + kv_off;
    const float f = role == 0 ? 1.f : p.scale;
    const int rl = 32 * blk + n;              // the lane's key within the workgroup
#pragma unroll
    for (int db = 0; db < DBLK; ++db) {
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int cidx = 4 * db + gq;         // chunk of d = 32db + 8gq .. +7; this lane has half hi
        *reinterpret_cast<u32x2*>(stage + rl * RB + ((cidx ^ (rl & (KCH - 1))) * 16) + 8 * hi) =
            u32x2{pack_bf16x2(acc[db][4 * gq] * f, acc[db][4 * gq + 1] * f),
                  pack_bf16x2(acc[db][4 * gq + 2] * f, acc[db][4 * gq + 3] * f)};
      }
    }
#pragma unroll
    for (int i = 0; i < 32 / ORPI; ++i) {
      const int r = 32 * blk + i * ORPI + lane / KCH, cc = lane % KCH;
      const u32x4 val = *reinterpret_cast<const u32x4*>(stage + r * RB + ((cc ^ (r & (KCH - 1))) * 16));
      if (k0 + r < Lk)   // non-temporal: written once
        __builtin_nontemporal_store(val, reinterpret_cast<u32x4*>(out + (int64_t)(k0 + r) * p.k_tok_stride + 8 * cc));
    }
  }
}

template <int D, bool VARLEN>
__global__ __launch_bounds__(kPrefillThreads, 2)
void bwd_dq_kernel(BwdParams p) {
  constexpr int KSTEPS = D / 16;
  constexpr int DBLK = D / 32;
  constexpr int KCH = D / 8;
  constexpr int RPI = 64 / KCH;
  constexpr int LOADS = kBlockN / RPI / 4;
  constexpr int TILE_BYTES = BLds<D>::kTile * 2;

  __shared__ __attribute__((aligned(1024))) uint16_t k_lds[2 * BLds<D>::kTile];
  __shared__ __attribute__((aligned(1024))) uint16_t v_lds[2 * BLds<D>::kTile];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, hi = lane >> 5;
  const int i16 = lane & 15, g16 = lane >> 4;

  const WorkItem w = VARLEN ? map_work_varlen(p, blockIdx.x) : map_work_dense(p, blockIdx.x);
  if (!w.valid) return;    // a spare varlen slot (uniform per workgroup)
  const int Lq = w.Lq, Lk = w.Lk, delta = Lk - Lq;
  const int kvh = w.h / p.group;
  const int64_t q_tok0 = VARLEN ? (int64_t)w.q_base : (int64_t)w.b * p.Lq;
  const int64_t k_tok0 = VARLEN ? (int64_t)w.k_base : (int64_t)w.b * p.Lk;
  const int64_t q_off = q_tok0 * p.q_tok_stride + (int64_t)w.h * D;
  const int64_t kv_off = k_tok0 * p.k_tok_stride + (int64_t)kvh * D;

  // ---- key range of the workgroup and of this wave (as in the forward) ----
  const int q0 = w.qt * kBlockM;
  const int r_first = q0, r_last = min(q0 + kBlockM, Lq) - 1;
  auto key_lo = [&](int row) { return p.win_left >= 0 ? max(0, row + delta - p.win_left) : 0; };
  auto key_hi = [&](int row) {
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
  const int rw0 = min(qw0, Lq - 1), rw1 = min(qw0 + 31, Lq - 1);
  const int wlo_last = key_lo(rw1), whi_first = key_hi(rw0);
  const int wlo_first = key_lo(rw0), whi_last = key_hi(rw1);
  const int row = qw0 + n;
  const int my_lo = key_lo(row), my_hi = key_hi(row);

  // ---- resident Q^T and dO^T (B operand), the row's lse2 and delta --------
  u32x4 qf[KSTEPS], dof[KSTEPS];
  {
    const uint32_t qbytes = (uint32_t)(((int64_t)(Lq - 1) * p.q_tok_stride + D) * 2);   // Lq >= 1 here
    const __amdgpu_buffer_rsrc_t qr = make_rsrc(p.q + q_off, qbytes);
    const __amdgpu_buffer_rsrc_t dr = make_rsrc(p.dout + q_off, qbytes);
    const uint32_t off = row < Lq ? (uint32_t)(row * p.q_tok_stride + 8 * hi) * 2u : kOob;
#pragma unroll
    for (int t = 0; t < KSTEPS; ++t) {
      qf[t] = buf_load16(qr, off + 32u * t);
      dof[t] = buf_load16(dr, off + 32u * t);
    }
  }
  // the tile's rows lie in the sequence's padded statistics
  const int64_t so = stat_offset(stat_base<VARLEN>(p, w.b, w.h, VARLEN ? w.q_base / kBlockM + w.b : 0) + row);
  const float lse2 = p.stat[so], dlt = p.stat[so + kBwdStatRows];
  // all ordinary loads complete before the loop, whose direct-to-LDS loads
  // the compiler's waits would otherwise count
#pragma unroll
  for (int t = 0; t < KSTEPS; ++t) {
    await_value(qf[t]);
    await_value(dof[t]);
  }
  await_value(lse2);
  await_value(dlt);

  // ---- staging of K/V tiles (as in the forward, one swizzle for both) -----
  const uint32_t k_row_bytes = (uint32_t)(p.k_tok_stride * 2);
  const uint32_t k_bytes = Lk > 0 ? (uint32_t)(((int64_t)(Lk - 1) * p.k_tok_stride + D) * 2) : 0u;
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(p.k + kv_off, k_bytes);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(p.v + kv_off, k_bytes);
  uint32_t src;
  {
    const int r = wave * RPI + lane / KCH, slot = lane % KCH;
    src = (uint32_t)r * k_row_bytes + (uint32_t)((slot ^ BLds<D>::swz(r)) * 16);
  }
  const uint32_t k_lds_addr = lds_address(k_lds), v_lds_addr = lds_address(v_lds);
  const uint32_t wave_lds = (uint32_t)__builtin_amdgcn_readfirstlane(wave * 1024);
  auto fetch = [&](int kb, int buf) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const uint32_t soff =
          (uint32_t)__builtin_amdgcn_readfirstlane((int)((uint32_t)(kb + 4 * i * RPI) * k_row_bytes));
      lds_load16(krs, src, soff, k_lds_addr + buf * TILE_BYTES + wave_lds + 4096u * i);
      lds_load16(vrs, src, soff, v_lds_addr + buf * TILE_BYTES + wave_lds + 4096u * i);
    }
  };

  const uint32_t row_base = (uint32_t)(n * 2 * D) | ((16u * hi) ^ (16u * BLds<D>::swz(n)));
  const char* k_lds_b = reinterpret_cast<const char*>(k_lds);
  const char* v_lds_b = reinterpret_cast<const char*>(v_lds);
  auto row_frag = [&](const char* tile, int kh, int t) {
    return *reinterpret_cast<const u32x4*>(tile + 64 * kh * D + (row_base ^ (32u * t)));
  };
  uint32_t tr_base[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int r = 8 * j + 4 * hi + (i16 >> 2);
    tr_base[j] = (uint32_t)(r * 2 * D) |
                 ((((32u * (g16 & 1)) | (16u * ((i16 & 3) >> 1))) ^ (16u * BLds<D>::swz(r))) |
                  (8u * (i16 & 1)));
  }
  auto tr_frag = [&](const char* tile, int cc, int db) {
    const char* a = tile + 16 * cc * 2 * D;
    const u32x2 lo = tr_read_b64(reinterpret_cast<const uint16_t*>(a + (tr_base[0] ^ (64u * db))));
    const u32x2 hi2 = tr_read_b64(reinterpret_cast<const uint16_t*>(a + (tr_base[1] ^ (64u * db))));
    return u32x4{lo[0], lo[1], hi2[0], hi2[1]};
  };

  f32x16 dqa[DBLK];
#pragma unroll
  for (int db = 0; db < DBLK; ++db) dqa[db] = f32x16{};
  const float c = p.scale_log2;
  const int kb0 = kt_begin * kBlockN;

  auto step = [&](auto parity, int j) {
    constexpr int cur = decltype(parity)::value;
    const int kb = kb0 + j * kBlockN;
    if (j + 1 < ntiles) fetch(kb + kBlockN, cur ^ 1);
    const char* kt_b = k_lds_b + cur * TILE_BYTES;
    const char* vt_b = v_lds_b + cur * TILE_BYTES;
    // a tile none of whose keys any row of this wave sees adds nothing to
    // its dQ (on the causal diagonal, the workgroup's first rows): the wave
    // only takes part in the tile's loads and barrier
    const bool none = kb >= whi_last || kb + kBlockN <= wlo_first;
    const bool full = kb >= wlo_last && kb + kBlockN <= whi_first;
    const int klo = my_lo - kb - 4 * hi, kspan = max(my_hi - my_lo, 0);
    if (!none) {
    u32x4 dsf[4];
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      f32x16 S = f32x16{}, dP = f32x16{};
#pragma unroll
      for (int t = 0; t < KSTEPS; ++t) {
        S = mfma32x32x16(row_frag(kt_b, kh, t), qf[t], S);
        dP = mfma32x32x16(row_frag(vt_b, kh, t), dof[t], dP);
      }
      // lane (row n, half hi) holds keys kb + 32kh + 8(r/4) + 4hi + r%4 in element r
#pragma unroll
      for (int r2 = 0; r2 < 8; ++r2) {
        float ds[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int r = 2 * r2 + u;
          float pe = exp2_fast(fmaf(S[r], c, -lse2));
          if (!full) {
            // key kb + 4hi + off visible iff my_lo <= key < my_hi
            const uint32_t off = (uint32_t)(32 * kh + 8 * (r >> 2) + (r & 3));
            pe = (off - (uint32_t)klo) < (uint32_t)kspan ? pe : 0.f;
          }
          ds[u] = pe * (dP[r] - dlt);
        }
        dsf[2 * kh + (r2 >> 2)][r2 & 3] = pack_bf16x2(ds[0], ds[1]);
      }
    }
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
#pragma unroll
      for (int db = 0; db < DBLK; ++db) dqa[db] = mfma32x32x16(tr_frag(kt_b, cc, db), dsf[cc], dqa[db]);
    }
    }
    lds_load_wait();
    __syncthreads();
  };

  if (ntiles > 0) fetch(kb0, 0);
  lds_load_wait();
  __syncthreads();
  for (int j = 0; j < ntiles; j += 2) {
    step(std::integral_constant<int, 0>{}, j);
    if (j + 1 < ntiles) step(std::integral_constant<int, 1>{}, j + 1);
  }

  // ---- epilogue: dQ = scale * dQ^T, row-major ------------------------------
  // Staged through the K tiles, unused from here on (the last step's barrier
  // ended their reads), so that stores write whole contiguous rows, as in the
  // forward kernel.
  {
    constexpr int RB = 2 * D;                 // bytes per dQ row
    constexpr int ORPI = 1024 / RB;           // rows per 1 KB store instruction
    char* stage = reinterpret_cast<char*>(k_lds);   // 128 rows of RB bytes
    const int rl = 32 * wave + n;             // the lane's row within the tile
#pragma unroll
    for (int db = 0; db < DBLK; ++db) {
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int cidx = 4 * db + gq;
        *reinterpret_cast<u32x2*>(stage + rl * RB + ((cidx ^ (rl & (KCH - 1))) * 16) + 8 * hi) =
            u32x2{pack_bf16x2(dqa[db][4 * gq] * p.scale, dqa[db][4 * gq + 1] * p.scale),
                  pack_bf16x2(dqa[db][4 * gq + 2] * p.scale, dqa[db][4 * gq + 3] * p.scale)};
      }
    }
#pragma unroll
    for (int i = 0; i < 32 / ORPI; ++i) {
      const int r = 32 * wave + i * ORPI + lane / KCH, cc = lane % KCH;
      const u32x4 val = *reinterpret_cast<const u32x4*>(stage + r * RB + ((cc ^ (r & (KCH - 1))) * 16));
      if (q0 + r < Lq)   // non-temporal: written once
        __builtin_nontemporal_store(val, reinterpret_cast<u32x4*>(p.dq + q_off + (int64_t)(q0 + r) * p.q_tok_stride + 8 * cc));
    }
  }
}

template <int D, bool VARLEN>
static hipError_t launch_bwd_d(const BwdParams& p, hipStream_t stream) {
  const int64_t stat_rows = VARLEN ? (int64_t)p.Hq * p.stat_rows : (int64_t)p.B * p.Hq * p.Lq_pad;
  const int64_t prep_threads = stat_rows * (D / 8);
  hipLaunchKernelGGL((bwd_prep_kernel<D, VARLEN>), dim3((unsigned)((prep_threads + 255) / 256)),
                     dim3(256), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t kv_blocks = (int64_t)(VARLEN ? 1 : p.B) * p.Hkv * p.num_k_tiles;
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, VARLEN>), dim3((unsigned)kv_blocks), dim3(kDkdvThreads), 0,
                     stream, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int64_t q_blocks = (int64_t)(VARLEN ? 1 : p.B) * p.Hq * p.num_q_tiles;
  hipLaunchKernelGGL((bwd_dq_kernel<D, VARLEN>), dim3((unsigned)q_blocks), dim3(kPrefillThreads), 0,
                     stream, p);
  return hipGetLastError();
}

hipError_t launch_bwd(const BwdParams& p, int d, bool varlen, hipStream_t stream) {
  if (varlen) return d == 128 ? launch_bwd_d<128, true>(p, stream) : launch_bwd_d<64, true>(p, stream);
  return d == 128 ? launch_bwd_d<128, false>(p, stream) : launch_bwd_d<64, false>(p, stream);
}

}  // namespace fa
