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
//   follow the configuration skill page (sec. 3.2-3.4, GQA appendix).  The
//   paged mode reads K/V of several new query rows per request from a paged
//   KV cache through its block table (skill page sec. 3.5 and the appendix on
//   PagedAttention), after an optional append of the new rows.
//
// Mapping onto CDNA4 (our design, not the pages'):
//   * A workgroup is 4 wave64s and owns 128 query rows of one (batch, head);
//     each wave owns 32 rows.  Two workgroups share a CU (two waves per SIMD),
//     so one wave's MFMAs overlap the other's softmax.  The loop walks
//     64-key tiles of K and V.
//   * Scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_bf16: K rows are the A operand (from LDS), the
//     wave's Q rows are the B operand and stay in registers for the whole
//     loop.  In the accumulator each lane holds ONE query (column) and 16 keys per
//     32x32 tile, so the row max is an in-lane max plus one exchange between
//     the two wave halves, and the row sum needs no cross-lane work until the
//     epilogue.
//   * The same accumulator registers, rounded to bf16, are exactly the B
//     operand of the PV product computed as O^T = V^T P^T: no LDS round trip
//     for P.  V stays row-major in LDS; its A operand (4 consecutive keys per
//     lane at a fixed d) comes from ds_read_b64_tr_b16 transpose reads.
//   * Software pipeline across tiles: step j issues the MFMAs of S^T for tile
//     j+1 and of P_{j-1} V_{j-1} while the softmax of tile j runs on the VALU,
//     interleaved instruction by instruction (a wave64 MFMA 32x32x16 keeps
//     the matrix core busy for 32 cycles, enough to issue about 5 independent
//     VALU ops beside it).  K runs one tile ahead and V one tile behind.
//   * Softmax runs in base 2 with scale*log2(e) folded into one FMA per score.
//     The reference max used in the exponent is only raised when a row's max
//     exceeds it by more than 2^8 (wave-uniform branch), so the output
//     rescale is skipped on almost every tile; P stays <= 256 and the final
//     division by l makes the result exact either way.
//   * K/V tiles are double-buffered in LDS and filled by buffer loads that
//     write LDS directly (no VGPR staging, no ds_write): the loads of K(j+2)
//     and V(j) are issued at the start of tile j and awaited at its end.  The
//     Q tile arrives the same way (into the V buffers, before the first V
//     tile) and each wave reads its fragments from there.
//     Rows past a sequence end come back as zeros from the buffer range
//     check.  16-byte chunks are XOR-swizzled within each row so the MFMA
//     operand reads and the transpose reads avoid LDS bank conflicts.
//   * O leaves through the idle K buffers: each wave writes its normalised
//     rows there and stores whole 256-byte rows, instead of 8-byte pieces of
//     32 rows per store instruction.
//   * Workgroup order: when the KV-group count is a multiple of 8, all query
//     heads of a KV group land on one XCD (blocks are dealt to the 8 XCDs
//     round-robin), a few KV groups at a time so their K/V stays in that L2;
//     within such a chunk heavy causal tiles go first.
#include "fa_internal.h"
#include "gfx950.h"
#include "work_map.h"

#include <float.h>
#include <math.h>

#include <type_traits>

namespace fa {

namespace {

constexpr float kRescaleTau = 8.0f;   // log2 units: rescale only if max grows > 2^8
constexpr float kLn2 = 0.6931471805599453f;

// LDS tile layouts: K and V tiles are [64 keys][D] bf16, row-major and
// unpadded, because the direct-to-LDS loads write 1 KB contiguous blocks.  The
// 16-byte chunk c of row r is stored at chunk c ^ swz(r):
//   K (D=128): swz = r & 15 -- an MFMA operand read (16 bytes per lane, lane n
//     on row n) puts 16 consecutive rows on 16 distinct 16-byte bank groups;
//   K (D=64):  swz = (r & 7) ^ ((r >> 3) & 1) -- rows are 128 bytes, so row
//     parity also picks the bank half;
//   V (D=128): swz = {0, 6, 12, 10}[r & 3] and V (D=64): swz = 2 (r & 3) -- a
//     transpose read touches 4 rows x 4 chunks per 32 lanes; these put them on
//     16 distinct bank groups (and any 16 lanes on 8).
template <int D> struct Lds {
  static constexpr int kTile = kBlockN * D;   // bf16 elements per K or V tile
  FA_DEV static int kswz(int r) { return D == 128 ? (r & 15) : ((r & 7) ^ ((r >> 3) & 1)); }
  FA_DEV static int vswz(int r) { return D == 128 ? ((r & 1) * 6) ^ (((r >> 1) & 1) * 12) : 2 * (r & 3); }
};


}  // namespace

// MODE 0: dense (B, L, H, d); 1: packed varlen; 2: queries dense (B, Lq, Hq, d),
// keys from a paged KV cache.
// MODS: softcap and/or ALiBi requested (a separate instance, so the plain
// kernel carries none of their registers).
// Occupancy: two workgroups per CU at d = 128 (235 VGPRs); three at d = 64
// (164 VGPRs, within the 168 that three workgroups allow).
template <int D, int MODE, bool MODS>
__global__ __launch_bounds__(kPrefillThreads, D == 64 ? 3 : 2)
void prefill_fwd_kernel(PrefillParams p) {
  constexpr bool VARLEN = MODE == 1, PAGED = MODE == 2;
  constexpr int KSTEPS = D / 16;                 // QK^T MFMA steps over d
  constexpr int DBLK = D / 32;                   // 32-row blocks of O^T
  constexpr int KCH = D / 8;                     // 16-byte chunks per row
  constexpr int RPI = 64 / KCH;                  // rows per 1 KB load instruction
  constexpr int LOADS = kBlockN / RPI / 4;       // load instructions per wave per tile
  constexpr int TILE_BYTES = Lds<D>::kTile * 2;

  __shared__ __attribute__((aligned(1024))) uint16_t k_lds[2 * Lds<D>::kTile];
  __shared__ __attribute__((aligned(1024))) uint16_t v_lds[2 * Lds<D>::kTile];

  const int tid = threadIdx.x;
  // the wave index is the same in all lanes: keep it (and everything derived
  // from it, such as load offsets) in scalar registers
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, hi = lane >> 5;
  const int i16 = lane & 15, g16 = lane >> 4;

  WorkItem w = VARLEN ? map_work_varlen(p, blockIdx.x) : map_work_dense(p, blockIdx.x);
  if (PAGED) w.Lk = p.cache_seqlens[w.b] + p.append_len;
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
    // paged: the pools, offset to this KV head; rows are addressed per page
    const int64_t kb_off = PAGED ? 0 : (int64_t)w.b * p.k_batch_stride;
    kg = p.k + kb_off + (int64_t)kvh * D;
    vg = p.v + kb_off + (int64_t)kvh * D;
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
  // the loop runs the tiles in pairs: an odd count gets one more tile, past
  // every row's last key (masked for all rows; rows at or past Lk load zeros)
  const int ntiles = (kt_end - kt_begin + 1) & ~1;

  const int qw0 = q0 + 32 * wave;
  const int rw0 = min(qw0, Lq - 1), rw1 = min(qw0 + 31, Lq - 1);
  const int wlo_last = key_lo(rw1), whi_first = key_hi(rw0);
  const int row = qw0 + n;
  const int my_lo = key_lo(row), my_hi = key_hi(row);

  // ---- sizes of the Q, K, V buffers; Q fragments (B operand) stay in ------
  // registers for the whole loop (the tile is staged through LDS below)
  const uint32_t q_bytes = (uint32_t)(((int64_t)(Lq - 1) * p.q_tok_stride + D) * 2);
  const uint32_t k_bytes = Lk > 0 ? (uint32_t)(((int64_t)(Lk - 1) * p.k_tok_stride + D) * 2) : 0u;
  const uint32_t k_row_bytes = (uint32_t)(p.k_tok_stride * 2);
  u32x4 qf[KSTEPS];
  const __amdgpu_buffer_rsrc_t qrs = make_rsrc(qg, q_bytes);

  // ---- staging of K/V tiles: global -> LDS directly ------------------------
  // Load instruction i of wave w fills tile bytes [(4i + w) KB, +1 KB): rows
  // (4i + w) * RPI + lane / KCH, stored chunk lane % KCH, which holds logical
  // chunk (lane % KCH) ^ swz(row).  swz(row) does not depend on i, so each lane
  // keeps one byte offset per tensor and the uniform part (tile and i) goes in
  // the scalar offset.  The range check covers both, so rows at or past Lk
  // fall outside the buffer (k_bytes) and load as zeros.  Offsets stay below
  // 2^32: per-batch tensors are < 2^31 bytes and a tile adds < 2^24.
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(kg, k_bytes);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vg, k_bytes);
  uint32_t k_src, v_src;
  {
    const int r = wave * RPI + lane / KCH, slot = lane % KCH;
    k_src = (uint32_t)r * k_row_bytes + (uint32_t)((slot ^ Lds<D>::kswz(r)) * 16);
    v_src = (uint32_t)r * k_row_bytes + (uint32_t)((slot ^ Lds<D>::vswz(r)) * 16);
  }
  const uint32_t k_lds_addr = lds_address(k_lds), v_lds_addr = lds_address(v_lds);
  const uint32_t wave_lds = (uint32_t)__builtin_amdgcn_readfirstlane(wave * 1024);
  // Paged mode: the 4 * RPI rows of load instruction i lie in one page (page
  // sizes are multiples of 16), whose id is one scalar load; the descriptor
  // spans that page's rows of this KV head, so the scalar offset is the row in
  // the page.  Keys at or past Lk get an out-of-range lane offset and load as
  // zeros; a key past the last used page reads page 0's range, never an
  // unused block-table entry.
  const int* bt_row = PAGED ? p.block_table + (int64_t)w.b * p.max_blocks : nullptr;
  const int64_t page_elems = PAGED ? (int64_t)p.page_size * p.k_tok_stride : 0;
  const uint32_t page_bytes = PAGED ? (uint32_t)((p.page_size - 1) * k_row_bytes + D * 2) : 0u;
  const uint32_t lane_row = (uint32_t)(lane / KCH);
  const uint32_t k_src_pg = k_src - (uint32_t)(wave * RPI) * k_row_bytes;   // row part of the lane
  const uint32_t v_src_pg = v_src - (uint32_t)(wave * RPI) * k_row_bytes;
  // Page ids of the LOADS row groups this wave loads for the tile at kb, read
  // together (scalar loads) ahead of the loads that need them.  The index is
  // clamped to the last used page: rows past Lk load as zeros in any case.
  const int last_pidx = PAGED && Lk > 0 ? (Lk - 1) / p.page_size : 0;
  // read through the constant address space: scalar loads (the table is not
  // written by this kernel), counted apart from the direct-to-LDS loads
  const __attribute__((address_space(4))) int* bt_const = (const __attribute__((address_space(4))) int*)bt_row;
  struct PageIds { int pg[LOADS]; };
  auto page_ids = [&](int kb) {
    PageIds r;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      if (PAGED) {
        const int key0 = kb + (4 * i + wave) * RPI;
        const int pidx = p.page_shift >= 0 ? key0 >> p.page_shift : key0 / p.page_size;
        r.pg[i] = bt_const[min(pidx, last_pidx)];
      } else {
        r.pg[i] = 0;
      }
    }
    return r;
  };
  // src / src_pg: the lane's byte offset for K or V; gbase: that tensor's base.
  auto fetch = [&](const __amdgpu_buffer_rsrc_t& rs, uint32_t src, uint32_t src_pg,
                   const uint16_t* gbase, uint32_t dst, int kb, const PageIds& ids) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      if (!PAGED) {
        const uint32_t soff = (uint32_t)(kb + 4 * i * RPI) * k_row_bytes;
        lds_load16(rs, src, (uint32_t)__builtin_amdgcn_readfirstlane(soff), dst + wave_lds + 4096u * i);
      } else {
        const int key0 = kb + (4 * i + wave) * RPI;                  // wave-uniform
        const int pidx = p.page_shift >= 0 ? key0 >> p.page_shift : key0 / p.page_size;
        const int prow = key0 - pidx * p.page_size;
        const uint16_t* base = gbase + (int64_t)ids.pg[i] * page_elems;
        const uint32_t soff = (uint32_t)prow * k_row_bytes;
        const uint32_t off = src_pg | ((uint32_t)key0 + lane_row >= (uint32_t)Lk ? kOob : 0u);
        lds_load16(make_rsrc(base, page_bytes), off, (uint32_t)__builtin_amdgcn_readfirstlane(soff),
                   dst + wave_lds + 4096u * i);
      }
    }
  };

  // ---- the per-tile phases ---------------------------------------------------
  // S^T = K Q^T for the two 32-key halves of a tile.  Lane (key n, half hi)
  // reads logical chunk 2t + hi of rows n and 32 + n (same swizzle).  The
  // stored chunk is (2t + hi) ^ swz(n), so its byte address is a per-lane base
  // XOR 32t: one address register serves all t.
  const uint32_t k_base = (uint32_t)(n * 2 * D) | ((16u * hi) ^ (16u * Lds<D>::kswz(n)));
  const char* k_lds_b = reinterpret_cast<const char*>(k_lds);
  auto k_frag = [&](int buf, int kh, int t) {
    return *reinterpret_cast<const u32x4*>(k_lds_b + buf * TILE_BYTES + 64 * kh * D + (k_base ^ (32u * t)));
  };
  auto qk = [&](int buf, f32x16 (&S)[2]) {
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      S[kh] = f32x16{};
#pragma unroll
      for (int t = 0; t < KSTEPS; ++t) S[kh] = mfma32x32x16(k_frag(buf, kh, t), qf[t], S[kh]);
    }
  };
  // Score modifiers (skill page sec. 3.3), on the raw dot products before the
  // mask: softcap replaces the logit x = scale*s by c*tanh(x/c), i.e. s by
  // (c/scale)*tanh((scale/c)*s), with tanh(y) = 1 - 2/(e^{2y} + 1); the ALiBi
  // bias -slope*|pos - key| of the logit is -(slope/scale)*|pos - key| on s.
  const float alibi_s = MODS && p.alibi ? p.alibi[(int64_t)w.b * p.alibi_bstride + w.h] * p.alibi_scale : 0.f;
  await_value(alibi_s);   // not inside the loop, whose direct-to-LDS loads a wait there would count
  auto modify = [&](f32x16 (&S)[2], int kb) {
    if (!MODS) return;
    const float two_log2e = 2.f * 1.4426950408889634f * p.cap_in;
    const int pos = row + delta;
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x = S[kh][r];
        if (p.cap_in > 0.f)
          x = p.cap_out * (1.f - 2.f * __builtin_amdgcn_rcpf(exp2_fast(x * two_log2e) + 1.f));
        const int key = kb + 32 * kh + 8 * (r >> 2) + 4 * hi + (r & 3);
        x -= alibi_s * (float)abs(pos - key);
        S[kh][r] = x;
      }
  };
  // mask only on tiles that cut through some row's visible band; key k is
  // visible iff (unsigned)(k - my_lo) < my_hi - my_lo, one compare per score
  const uint32_t my_span = (uint32_t)max(my_hi - my_lo, 0);
  auto mask_tile = [&](f32x16 (&S)[2], int kb) {
    if (kb >= wlo_last && kb + kBlockN <= whi_first) return;
    const uint32_t base = (uint32_t)(kb + 4 * hi - my_lo);
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const uint32_t off = (uint32_t)(32 * kh + 8 * (r >> 2) + (r & 3));
        S[kh][r] = base + off < my_span ? S[kh][r] : -INFINITY;
      }
  };
  // P = 2^(S*c - m) as packed bf16 MFMA fragments; l sums the unrounded fp32
  // P (two chains), which keeps LSE to fp32 accuracy.
  float m_ref = -INFINITY;
  float l_a = 0.f, l_b = 0.f;
  const float c = p.scale_log2;
  f32x16 oacc[DBLK];
#pragma unroll
  for (int db = 0; db < DBLK; ++db) oacc[db] = f32x16{};
  // Row max of the tile (log2 units); raise the reference max only when it
  // grows by more than 2^8 and rescale O and l then (rare: wave-uniform branch).
  // flush() first adds the pending P V product, which is relative to the old
  // reference max.
  auto update_max = [&](const f32x16 (&S)[2], auto&& flush) {
    float mx = S[0][0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, S[0][r]);
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, S[1][r]);
    mx = fmaxf(mx, xor32(mx)) * c;
    const bool up = mx > m_ref + kRescaleTau;
    // a row that has seen no key yet has O = 0 and l = 0: nothing to rescale
    if (wave_any(up && m_ref != -INFINITY)) {
      flush();   // pending P V products are relative to the old max
      const float alpha = up ? exp2_fast(m_ref - mx) : 1.f;
      l_a *= alpha;
      l_b *= alpha;
#pragma unroll
      for (int db = 0; db < DBLK; ++db) oacc[db] *= alpha;
    }
    if (up) m_ref = mx;
  };
  auto softmax = [&](const f32x16 (&S)[2], u32x4 (&P)[4]) {
    const float mb = (m_ref == -INFINITY) ? 0.f : m_ref;
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
#pragma unroll
      for (int r2 = 0; r2 < 8; ++r2) {
        const float p0 = exp2_fast(fmaf(S[kh][2 * r2], c, -mb));
        const float p1 = exp2_fast(fmaf(S[kh][2 * r2 + 1], c, -mb));
        l_a += p0;
        l_b += p1;
        P[2 * kh + (r2 >> 2)][r2 & 3] = pack_bf16x2(p0, p1);
      }
    }
  };
  // O^T += V^T P^T: V^T fragments from transpose reads of the row-major tile.
  // Lane i of a 16-lane group g addresses key row 16cc + 8j + 4hi + i/4 and
  // the 8-byte unit 8db + 4(g&1) + (i&3) of it, i.e. half i&1 of logical
  // chunk 4db + 2(g&1) + (i&3)/2; the row's swizzle depends on i/4 only, and
  // db enters the stored chunk's byte address as XOR 64db.
  const uint32_t v_base = (uint32_t)((4 * hi + (i16 >> 2)) * 2 * D) |
                          (((32u * (g16 & 1)) | (16u * ((i16 & 3) >> 1))) ^ (16u * Lds<D>::vswz(i16 >> 2))) |
                          (8u * (i16 & 1));
  const char* v_lds_b = reinterpret_cast<const char*>(v_lds);
  auto pv = [&](int buf, const u32x4 (&P)[4]) {
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
#pragma unroll
      for (int db = 0; db < DBLK; ++db) {
        const char* a = v_lds_b + buf * TILE_BYTES + 16 * cc * 2 * D + (v_base ^ (64u * db));
        const u32x2 lo = tr_read_b64(reinterpret_cast<const uint16_t*>(a));
        const u32x2 hi2 = tr_read_b64(reinterpret_cast<const uint16_t*>(a + 16 * D));
        oacc[db] = mfma32x32x16(u32x4{lo[0], lo[1], hi2[0], hi2[1]}, P[cc], oacc[db]);
      }
    }
  };

  // Instruction order of the step's main block: a few K fragment reads first,
  // then each MFMA followed by some softmax VALU ops and the next LDS reads,
  // so reads stay a few MFMAs ahead and the VALU work hides under the MFMAs.
  auto interleave_hint = [](auto with_qk, auto with_pv) {
    // fixed schedule: K fragment reads issued up front, then per S^T MFMA
    // 4 VALU ops and 1 read, per P V MFMA 3 VALU ops and 2 reads
    constexpr int kReadsUp = 3, kValuQk = 4, kReadsQk = 1, kValuPv = 3, kReadsPv = 2;
    __builtin_amdgcn_sched_group_barrier(0x100, kReadsUp, 0);
    if constexpr (decltype(with_qk)::value) {
#pragma unroll
      for (int i = 0; i < 2 * KSTEPS; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, kValuQk, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, kReadsQk, 0);
      }
    }
    if constexpr (decltype(with_pv)::value) {
#pragma unroll
      for (int i = 0; i < 4 * DBLK; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, kValuPv, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, kReadsPv, 0);
      }
    }
    __builtin_amdgcn_sched_group_barrier(0x002, 64, 0);
  };

  // ---- prologue: Q, K(0), K(1) into LDS; S^T(0) ----------------------------
  const int kb0 = kt_begin * kBlockN;
  // page ids of step 0's loads (paged mode; read one step ahead from then on)
  PageIds ids_k = page_ids(kb0 + 2 * kBlockN), ids_v = page_ids(kb0);
  {
    // the Q tile (128 rows) into the two V buffers, K swizzle
    const uint32_t q_row_bytes = (uint32_t)(p.q_tok_stride * 2);
    const int r = wave * RPI + lane / KCH;
    const uint32_t q_src = (uint32_t)r * q_row_bytes + (uint32_t)(((lane % KCH) ^ Lds<D>::kswz(r)) * 16);
#pragma unroll
    for (int i = 0; i < 2 * LOADS; ++i) {
      const uint32_t soff = (uint32_t)(q0 + 4 * i * RPI) * q_row_bytes;
      lds_load16(qrs, q_src, (uint32_t)__builtin_amdgcn_readfirstlane(soff), v_lds_addr + wave_lds + 4096u * i);
    }
  }
  if (ntiles > 0) {   // then ntiles >= 2
    const PageIds i0 = page_ids(kb0), i1 = page_ids(kb0 + kBlockN);
    fetch(krs, k_src, k_src_pg, kg, k_lds_addr, kb0, i0);
    fetch(krs, k_src, k_src_pg, kg, k_lds_addr + TILE_BYTES, kb0 + kBlockN, i1);
  }
  // S^T(0) needs Q and K(0) only: K(1) may still be in flight (its LOADS
  // loads were issued last) until the barrier before step 0
  if (ntiles > 0) lds_load_wait_n<LOADS>(); else lds_load_wait();
  __syncthreads();
  {
    const int rl = 32 * wave + n;
    const char* qt = reinterpret_cast<const char*>(v_lds) + rl * 2 * D;
#pragma unroll
    for (int t = 0; t < KSTEPS; ++t)
      qf[t] = *reinterpret_cast<const u32x4*>(qt + (((2 * t + hi) ^ Lds<D>::kswz(rl)) * 16));
  }
  f32x16 s0[2], s1[2];
  u32x4 p0[4], p1[4];
  qk(0, s0);
  // step 0 reads K(1), loads K(2) into K buffer 0 and V(0) over Q: every wave
  // must have its share of K(1) in LDS and be done reading K(0) and its Q rows
  lds_load_wait();
  __syncthreads();

  // ---- main loop: two tiles per trip, ping-pong S and P registers ---------
  // Step j: S^T(j) and P_{j-1} are ready.  K(j+2) and V(j) are loaded into the
  // buffers of K(j) and V(j-2), whose last reads finished before the barrier
  // that ended step j-1.  Then one basic block holds the MFMAs of S^T(j+1)
  // and of P_{j-1} V_{j-1} and the softmax of tile j (P_j), interleaved.
  // While some row has seen no key, the max is taken before the block; when
  // it must be raised then, P_{j-1} V_{j-1} is added first, O is rescaled and
  // P_{j-1} cleared, so the block adds zeros.  Afterwards the max is taken
  // only when the tile shows a probability above 2^8 (rare).
  // Step 0 has no P_{-1}: its block holds only S^T(1) and the softmax of tile 0.
  // The last step has no tile j+1: its block holds only P_{j-1} V_{j-1} (if
  // any) and the softmax of tile j.
  // (the parity of j, and so every LDS buffer offset, is a compile-time constant)
  auto step = [&](auto parity, auto first, auto last, int j, f32x16 (&Scur)[2], f32x16 (&Snxt)[2],
                  u32x4 (&Pprev)[4], u32x4 (&Pcur)[4]) {
    constexpr int cur = decltype(parity)::value, nxt = cur ^ 1;
    constexpr bool FIRST = decltype(first)::value;   // no P_{j-1} V_{j-1} before tile 0
    constexpr bool LAST = decltype(last)::value;     // no S^T(j+1) after the last tile
    const int kb = kb0 + j * kBlockN;
    modify(Scur, kb);
    mask_tile(Scur, kb);
    // A row that has seen no key yet needs its max up front (its scores can
    // lie anywhere).  Otherwise the max is only needed when a probability of
    // the tile exceeds 2^8, which the growth of the row sum shows afterwards.
    const bool exact = wave_any(m_ref == -INFINITY);
    if (exact) {
      update_max(Scur, [&] {
        if constexpr (!FIRST) {
          pv(nxt, Pprev);
#pragma unroll
          for (int i = 0; i < 4; ++i) Pprev[i] = u32x4{0u, 0u, 0u, 0u};
        }
      });
    }
    // page ids of this step's loads were read one step ahead (paged mode)
    if (j + 2 < ntiles) fetch(krs, k_src, k_src_pg, kg, k_lds_addr + cur * TILE_BYTES, kb + 2 * kBlockN, ids_k);
    fetch(vrs, v_src, v_src_pg, vg, v_lds_addr + cur * TILE_BYTES, kb, ids_v);
    ids_k = page_ids(kb + 3 * kBlockN);
    ids_v = page_ids(kb + kBlockN);
    const float la0 = l_a, lb0 = l_b;
    if constexpr (!LAST) qk(nxt, Snxt);
    if constexpr (!FIRST) pv(nxt, Pprev);
    softmax(Scur, Pcur);
    interleave_hint(std::integral_constant<bool, !LAST>{}, std::integral_constant<bool, !FIRST>{});
    // this lane's share of the tile's row sum bounds each of its probabilities
    // (also catches inf/NaN): above 2^8, take back the tile, raise the max and
    // rescale (P_{j-1} V_{j-1} is already in O, relative to the old max), and
    // redo P_j (rare: wave-uniform branch)
    if (!exact && wave_any(!((l_a - la0) + (l_b - lb0) <= 256.f))) {
      l_a = la0;
      l_b = lb0;
      update_max(Scur, [] {});
      softmax(Scur, Pcur);
    }
    lds_load_wait();
    __syncthreads();
  };
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  using T = std::true_type;
  using F = std::false_type;
  // ntiles is even: step 0, pairs of steps, and the last step (odd parity)
  if (ntiles > 0) {
    step(P0{}, T{}, F{}, 0, s0, s1, p1, p0);
    for (int j = 1; j + 1 < ntiles; j += 2) {
      step(P1{}, F{}, F{}, j, s1, s0, p0, p1);
      step(P0{}, F{}, F{}, j + 1, s0, s1, p1, p0);
    }
    step(P1{}, F{}, T{}, ntiles - 1, s1, s0, p0, p1);
    // the last tile's P V, unless no row of this wave sees a key of that
    // tile (its P is zero: the causal diagonal of the wave's earlier rows, or
    // the extra tile of an odd count)
    const int kb_last = kb0 + (ntiles - 1) * kBlockN;
    if (kb_last < key_hi(rw1) && kb_last + kBlockN > key_lo(rw0)) pv(1, p1);
  }

  // ---- epilogue: O = acc / l (bf16), LSE = (m + log2 l) * ln 2 ------------
  // O goes out through the K tiles, unused from here on (the last step's
  // barrier ended their reads): each lane holds 4-element pieces of one row,
  // which stored directly would touch 32 rows per instruction.  Every wave
  // writes its own 32 rows into the staging area (16-byte chunk c of row r at
  // c ^ (r % chunks per row)), reads them back as 16-byte chunks, and stores
  // whole contiguous rows.
  const float lpart = l_a + l_b;
  const float lt = lpart + xor32(lpart);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  {
    constexpr int RB = 2 * D;                 // bytes per O row
    constexpr int ORPI = 1024 / RB;           // rows per 1 KB store instruction
    char* stage = reinterpret_cast<char*>(k_lds);   // 128 rows of RB bytes
    const int rl = 32 * wave + n;             // the lane's row within the tile
#pragma unroll
    for (int db = 0; db < DBLK; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c = 4 * db + g;             // chunk of d = 32db + 8g .. +7; this lane has half hi
        *reinterpret_cast<u32x2*>(stage + rl * RB + ((c ^ (rl & (KCH - 1))) * 16) + 8 * hi) =
            u32x2{pack_bf16x2(oacc[db][4 * g + 0] * inv, oacc[db][4 * g + 1] * inv),
                  pack_bf16x2(oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv)};
      }
    }
#pragma unroll
    for (int i = 0; i < 32 / ORPI; ++i) {
      const int r = 32 * wave + i * ORPI + lane / KCH, cc = lane % KCH;
      const u32x4 val = *reinterpret_cast<const u32x4*>(stage + r * RB + ((cc ^ (r & (KCH - 1))) * 16));
      // non-temporal: O is written once, so it need not displace K/V tiles
      // that other workgroups of the head still read from L2
      if (q0 + r < Lq)
        __builtin_nontemporal_store(val, reinterpret_cast<u32x4*>(og + (int64_t)(q0 + r) * p.q_tok_stride + 8 * cc));
    }
  }
  if (row < Lq && lseg && hi == 0) lseg[row] = lt > 0.f ? (m_ref + log2_fast(lt)) * kLn2 : -INFINITY;
}

hipError_t launch_prefill(const PrefillParams& p, int d, int mode, hipStream_t stream) {
  const int64_t nblocks = mode == 1 ? (int64_t)p.num_q_tiles * p.Hq
                                    : (int64_t)p.num_q_tiles * p.B * p.Hq;
  if (nblocks <= 0) return hipSuccess;
  const dim3 grid((unsigned)nblocks), block(kPrefillThreads);
  const bool mods = p.cap_in > 0.f || p.alibi != nullptr;
#define FA_PREFILL(DD, MM)                                                                  \
  do {                                                                                      \
    if (mods) hipLaunchKernelGGL((prefill_fwd_kernel<DD, MM, true>), grid, block, 0, stream, p); \
    else hipLaunchKernelGGL((prefill_fwd_kernel<DD, MM, false>), grid, block, 0, stream, p);     \
  } while (0)
  if (d == 128) {
    if (mode == 0) FA_PREFILL(128, 0); else if (mode == 1) FA_PREFILL(128, 1); else FA_PREFILL(128, 2);
  } else {
    if (mode == 0) FA_PREFILL(64, 0); else if (mode == 1) FA_PREFILL(64, 1); else FA_PREFILL(64, 2);
  }
#undef FA_PREFILL
  return hipGetLastError();
}

// One workgroup per (new token i, request b): 16-byte copies of the token's
// K and V rows (all KV heads) into cache position cache_seqlens[b] + i.
__global__ __launch_bounds__(256)
void kvcache_append_kernel(AppendParams a) {
  const int i = blockIdx.x, b = blockIdx.y;
  const int pos = a.cache_seqlens[b] + i;
  const int pg = a.block_table[(int64_t)b * a.max_blocks + pos / a.page_size];
  const int64_t row = (int64_t)a.Hkv * a.d;                  // elements per token
  const int64_t dst = ((int64_t)pg * a.page_size + pos % a.page_size) * row;
  const int64_t src = ((int64_t)b * a.L_new + i) * row;
  const int chunks = (int)(row / 8);
  for (int c = threadIdx.x; c < 2 * chunks; c += blockDim.x) {
    const bool is_v = c >= chunks;
    const int cc = is_v ? c - chunks : c;
    const u32x4 val = *reinterpret_cast<const u32x4*>((is_v ? a.v_new : a.k_new) + src + 8 * cc);
    *reinterpret_cast<u32x4*>((is_v ? a.v_cache : a.k_cache) + dst + 8 * cc) = val;
  }
}

hipError_t launch_append(const AppendParams& a, hipStream_t stream) {
  if (a.B <= 0 || a.L_new <= 0) return hipSuccess;
  hipLaunchKernelGGL(kvcache_append_kernel, dim3(a.L_new, a.B), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace fa
