// Fused exact-attention prefill forward for gfx950, head_dim 128, dense
// layout: the wide-tile kernel.
//
// What it computes is exactly what prefill_fwd.hip computes (the definition
// of the "FlashAttention-3 vs naive attention" page, sec. 1.1, with the
// online softmax of the "FIA / FlashAttention" explainer, sec. 1, and the
// masks, GQA broadcast and score modifiers of the configuration skill page,
// sec. 3.2-3.3 and its GQA appendix); only the mapping onto the chip differs.
//
// Mapping onto CDNA4:
//   * One workgroup = 4 wave64s = 256 (query row, head) pairs of one batch
//     and KV group: 64 rows of each of 4 query heads when the GQA group size
//     is a multiple of 4 (all waves then reach the causal diagonal in the
//     same step), 128 rows of 2 heads when it is even, else 256 rows of one
//     head.  Each wave owns 64 rows of one head as two 32-row blocks, and one
//     workgroup fills a CU (one wave per SIMD, 512 registers per lane).  Every
//     K or V operand fragment read from LDS then feeds two MFMAs, one per row
//     block, which halves LDS read bytes per MFMA against 32 rows per wave;
//     the per-CU K/V tile loads (direct-to-LDS) halve too, since a tile
//     serves 256 query rows.
//   * Scores are computed transposed, S^T = K Q^T (v_mfma_f32_32x32x16_bf16):
//     K rows are the A operand from LDS, Q rows the B operand, so each lane
//     holds one query row of a 32x32 tile and the row sum needs no cross-lane
//     work.  The scores rounded to bf16 are the B operand of O^T = V^T P^T;
//     V^T comes from ds_read_b64_tr_b16 transpose reads of the row-major tile.
//   * Register classes are fixed by hand: the O accumulators (128 per lane)
//     and the Q fragments (64) live in AGPRs, the MFMAs take them there
//     directly (inline assembly), and the VGPRs hold the double-buffered
//     scores (128), P (64) and the fragments in flight.  All MFMAs are inline
//     assembly, so the hazards the compiler would otherwise track are
//     covered by explicit wait states (mfma_drain) wherever a VALU
//     instruction reads or writes an MFMA result register.
//   * One wave per SIMD means no other wave hides this wave's VALU work, so
//     each step is one hand-ordered sequence: 64 MFMA slots (S^T of tile j+1
//     and P V of tile j-1, alternating), the softmax of tile j spread over
//     them one score element per slot in three pipelined stages (scale,
//     exponential, row sum and pack), so that no VALU instruction waits on
//     one of its own slot, each LDS fragment read issued one fragment ahead
//     of its MFMAs, and the step's eight direct-to-LDS tile loads one every
//     four slots of the first half.  Scheduling barriers keep that order.
//     The VALU, LDS and load instructions of a step then take about as many
//     issue cycles as its 64 MFMAs run, which is what bounds this kernel.
//   * Base-2 softmax with the lazy 2^8 rescale of the narrow kernel; the rare
//     rescale reads and writes the AGPR accumulators in a cold branch.
#include "fa_internal.h"
#include "gfx950.h"
#include "work_map.h"

#include <math.h>

#include <type_traits>

namespace fa {

namespace {

constexpr float kWideTau = 8.0f;   // log2 units: rescale only if a max grows > 2^8
constexpr float kWideLn2 = 0.6931471805599453f;

// S (VGPR) = A * B with B from AGPRs; the accumulator starts at zero.
FA_DEV void mma_s_first(f32x16& d, const u32x4& a, const u32x4& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "a"(b));
}
// S (VGPR) += A * B with B from AGPRs.
FA_DEV void mma_s(f32x16& d, const u32x4& a, const u32x4& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "a"(b));
}
// O += A * B: a compiler builtin, so the compiler tracks this MFMA's hazards
// and register moves; at one wave per SIMD it keeps the accumulators in AGPRs.
FA_DEV void mma_o(f32x16& d, const u32x4& a, const u32x4& b) { d = mfma32x32x16(a, b, d); }
// Wait states that let every MFMA issued before it finish writing its result
// before a VALU instruction reads it (or writes one of its operands): 26 cycles
// of the issuing wave, more than the 8-pass MFMA's requirement.
FA_DEV void mfma_drain() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 1" ::: "memory"); }
// lds_load16 with one wait state (for the M0 write just before) instead of
// five: the kernel's load offsets and descriptors come from scalar
// arithmetic, not from VALU writes of SGPRs (checked in the compiled code by
// isa_check.check_lds_loads).
FA_DEV void lds_load16_m0(__amdgpu_buffer_rsrc_t r, uint32_t voffset, uint32_t soffset, uint32_t lds_base) {
  lds_poison16(lds_base);
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
               :: "v"(voffset), "s"(r), "s"(soffset), "{m0}"(lds_base) : "memory");
}
// M0 <- base + OFF for a later lds_load16_after_m0 (the value stays live in
// M0).  The sum is formed in M0 itself, so no SGPR holds the eight
// destinations of a step.
template <uint32_t OFF>
FA_DEV uint32_t set_m0(uint32_t base) {
  uint32_t m;
  asm volatile("s_add_u32 m0, %1, %2" : "={m0}"(m) : "s"(base), "n"(OFF));
  return m;
}
// Direct-to-LDS load whose M0 was written by set_m0 at least one instruction
// earlier, so it needs no wait state of its own.
FA_DEV void lds_load16_after_m0(__amdgpu_buffer_rsrc_t r, uint32_t voffset, uint32_t soffset, uint32_t m) {
  lds_poison16(m);
  asm volatile("buffer_load_dwordx4 %0, %1, %2 offen lds"
               :: "v"(voffset), "s"(r), "s"(soffset), "{m0}"(m) : "memory");
}
// No instruction may be scheduled across this point.
FA_DEV void sched_fence() { __builtin_amdgcn_sched_barrier(0); }
// Pins a value in AGPRs at this point: copies into it (v_accvgpr_write) must
// be issued before, and reads of it (v_accvgpr_read) after.  Each pin also
// adds two wait states, so a run of pins separates VALU writes of AGPRs from
// the MFMAs that read them.
FA_DEV void pin_agpr(f32x16& x) { asm volatile("s_nop 1" : "+a"(x)); }
FA_DEV void pin_agpr(u32x4& x) { asm volatile("s_nop 1" : "+a"(x)); }

// x, hidden from the optimiser: values derived from it are recomputed where
// they are used instead of being hoisted out of the loop and held in registers.
FA_DEV int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// f(integral_constant<int, I>) for I = B..E-1, unrolled at compile time, so
// every register-array index in f is a constant.
template <int B, int E, class F>
FA_DEV void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

}  // namespace

// LDS: K and V tiles [64 keys][128] bf16, double-buffered (64 KB), with the
// narrow kernel's 16-byte chunk swizzles: K chunk c of row r at c ^ (r & 15),
// V chunk c at c ^ {0, 6, 12, 10}[r & 3].
template <bool MODS>
__global__ __launch_bounds__(kPrefillThreads, 1)
void prefill_fwd_wide_kernel(PrefillParams p) {
  constexpr int D = 128;
  constexpr int KSTEPS = 8;     // QK^T MFMA steps over d
  constexpr int DBLK = 4;       // 32-row blocks of O^T
  constexpr int KCH = 16;       // 16-byte chunks per row
  constexpr int RPI = 4;        // rows per 1 KB load instruction
  constexpr int LOADS = 4;      // load instructions per wave per tile and tensor
  constexpr int TILE = kBlockN * D;
  constexpr int TILE_BYTES = TILE * 2;
  constexpr int QB = 2;         // 32-row blocks per wave

  __shared__ __attribute__((aligned(1024))) uint16_t k_lds[2 * TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t v_lds[2 * TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, hi = lane >> 5;
  const int i16 = lane & 15, g16 = lane >> 4;

  // The workgroup owns GW query heads of one KV group (a "head set") and RW
  // rows of each; wave w takes head w % GW and the 64-row block w / GW.  The
  // dense work order runs over head sets as if they were heads.
  const int GW = p.wide_heads;
  const int RW = kWideRows / GW;
  struct HeadSetView { int B, Hq, Hkv, group, num_q_tiles, xcd_groups, chunk_groups, Lq, Lk; };
  const HeadSetView hs = {p.B, p.Hq / GW, p.Hkv, p.group / GW, p.num_q_tiles, p.xcd_groups,
                          p.chunk_groups, p.Lq, p.Lk};
  WorkItem w = map_work_dense(hs, blockIdx.x);
  // the work item is the same in every lane: keep it in scalar registers so
  // every buffer descriptor built from it is an SGPR operand
  w.b = __builtin_amdgcn_readfirstlane(w.b);
  w.h = __builtin_amdgcn_readfirstlane(w.h * GW + wave % GW);   // this wave's head
  w.qt = __builtin_amdgcn_readfirstlane(w.qt);
  const int rblk = wave / GW;
  const int Lq = __builtin_amdgcn_readfirstlane(w.Lq), Lk = __builtin_amdgcn_readfirstlane(w.Lk);
  const int kvh = w.h / p.group;
  const int delta = Lk - Lq;
  const uint16_t* qg = p.q + (int64_t)w.b * p.q_batch_stride + (int64_t)w.h * D;
  uint16_t* og = p.o + (int64_t)w.b * p.q_batch_stride + (int64_t)w.h * D;
  const uint16_t* kg = p.k + (int64_t)w.b * p.k_batch_stride + (int64_t)kvh * D;
  const uint16_t* vg = p.v + (int64_t)w.b * p.k_batch_stride + (int64_t)kvh * D;
  float* lseg = p.lse ? p.lse + ((int64_t)w.b * p.Hq + w.h) * p.lse_seq_stride : nullptr;

  // ---- key ranges: workgroup, wave, and each of the lane's two rows -------
  const int q0 = w.qt * RW;
  auto key_lo = [&](int row) __attribute__((always_inline)) { return p.win_left >= 0 ? max(0, row + delta - p.win_left) : 0; };
  auto key_hi = [&](int row) __attribute__((always_inline)) {    // exclusive
    int e = Lk;
    if (p.causal) e = min(e, row + delta + 1);
    if (p.win_right >= 0) e = min(e, row + delta + p.win_right + 1);
    return e;
  };
  const int kv_lo = key_lo(q0);
  const int kv_hi = key_hi(min(q0 + RW, Lq) - 1);
  const int kt_begin = kv_lo / kBlockN;
  const int kt_end = kv_hi > kv_lo ? (kv_hi + kBlockN - 1) / kBlockN : kt_begin;
  const int ntiles = kt_end - kt_begin;
  const int qw0 = q0 + 64 * rblk;
  const int rw0 = min(qw0, Lq - 1), rw1 = min(qw0 + 63, Lq - 1);
  const int wlo_last = key_lo(rw1), whi_first = key_hi(rw0);
  // the lane's query row in block qb; the masks recompute their bounds from
  // it on the tiles that need them rather than hold them in registers
  auto row_of = [&](int qb) __attribute__((always_inline)) { return qw0 + 32 * qb + (opaque(lane) & 31); };

  // ---- buffers -----------------------------------------------------------
  const uint32_t q_row_bytes = (uint32_t)(p.q_tok_stride * 2);
  const uint32_t k_row_bytes = (uint32_t)(p.k_tok_stride * 2);
  const uint32_t q_bytes = (uint32_t)(((int64_t)(Lq - 1) * p.q_tok_stride + D) * 2);
  const uint32_t k_bytes = (uint32_t)(((int64_t)(Lk - 1) * p.k_tok_stride + D) * 2);
  const __amdgpu_buffer_rsrc_t qrs = make_rsrc(qg, q_bytes);
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(kg, k_bytes);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vg, k_bytes);

  // Direct-to-LDS staging: load instruction i of wave w fills tile bytes
  // [(4i + w) KB, +1 KB) = rows (4i + w) * 4 + lane / 16, stored chunk lane % 16
  // (holding logical chunk (lane % 16) ^ swz(row)).  Rows at or past Lk fall
  // outside the buffer and load as zeros.
  uint32_t k_src, v_src;
  {
    const int r = wave * RPI + lane / KCH, slot = lane % KCH;
    k_src = (uint32_t)r * k_row_bytes + (uint32_t)((slot ^ (r & 15)) * 16);
    v_src = (uint32_t)r * k_row_bytes + (uint32_t)((slot ^ (((r & 1) * 6) ^ (((r >> 1) & 1) * 12))) * 16);
  }
  const uint32_t k_lds_addr = lds_address(k_lds), v_lds_addr = lds_address(v_lds);
  const uint32_t wave_lds = (uint32_t)__builtin_amdgcn_readfirstlane(wave * 1024);
  auto fetch = [&](const __amdgpu_buffer_rsrc_t& rs, uint32_t src, uint32_t dst, int kb) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const uint32_t soff = (uint32_t)(kb + 4 * i * RPI) * k_row_bytes;
      lds_load16_m0(rs, src, (uint32_t)__builtin_amdgcn_readfirstlane(soff), dst + wave_lds + 4096u * i);
    }
  };

  // Fragment reads.  K: lane (key n, half hi) reads logical chunk 2t + hi of
  // rows n and 32 + n; V^T: transpose reads as in the narrow kernel.
  const uint32_t k_base = (uint32_t)(n * 2 * D) | ((16u * hi) ^ (16u * (n & 15)));
  const uint32_t v_base = (uint32_t)((4 * hi + (i16 >> 2)) * 2 * D) |
                          (((32u * (g16 & 1)) | (16u * ((i16 & 3) >> 1))) ^
                           (16u * (((i16 >> 2) & 1) * 6 ^ (((i16 >> 3) & 1) * 12)))) |
                          (8u * (i16 & 1));
  const char* k_lds_b = reinterpret_cast<const char*>(k_lds);
  const char* v_lds_b = reinterpret_cast<const char*>(v_lds);
  auto k_frag = [&](int buf, int g) __attribute__((always_inline)) {     // g = 8 kh + t
    const int kh = g >> 3, t = g & 7;
    return *reinterpret_cast<const u32x4*>(k_lds_b + buf * TILE_BYTES + 64 * kh * D + (k_base ^ (32u * t)));
  };
  auto v_frag = [&](int buf, int f) __attribute__((always_inline)) {     // f = 4 cc + db
    const int cc = f >> 2, db = f & 3;
    const char* a = v_lds_b + buf * TILE_BYTES + 16 * cc * 2 * D + (v_base ^ (64u * db));
    const u32x2 lo = tr_read_b64(reinterpret_cast<const uint16_t*>(a));
    const u32x2 hi2 = tr_read_b64(reinterpret_cast<const uint16_t*>(a + 16 * D));
    return u32x4{lo[0], lo[1], hi2[0], hi2[1]};
  };

  // ---- state ---------------------------------------------------------------
  u32x4 qf[QB][KSTEPS];          // AGPRs (only ever MFMA B operands)
  f32x16 oacc[QB][DBLK];         // AGPRs (only ever MFMA accumulators)
  f32x16 S[2][QB][2];            // scores of two tiles (VGPRs)
  u32x4 P[2][QB][4];             // bf16 probabilities of two tiles (VGPRs)
  float m_ref[QB], l_a[QB], l_b[QB];
  const float c = p.scale_log2;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_ref[qb] = -INFINITY;
    l_a[qb] = 0.f;
    l_b[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < DBLK; ++db) oacc[qb][db] = f32x16{};
  }

  // Score modifiers (skill page sec. 3.3) on the raw dot products, as in the
  // narrow kernel: softcap s -> (c/scale) tanh((scale/c) s), then ALiBi
  // -(slope/scale)|pos - key|.
  const float alibi_s = MODS && p.alibi ? p.alibi[(int64_t)w.b * p.alibi_bstride + w.h] * p.alibi_scale : 0.f;
  await_value(alibi_s);
  auto modify = [&](f32x16 (&Sq)[2], int qb, int kb) __attribute__((always_inline)) {
    if (!MODS) return;
    const float two_log2e = 2.f * 1.4426950408889634f * p.cap_in;
    const int pos = row_of(qb) + delta;
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x = Sq[kh][r];
        if (p.cap_in > 0.f)
          x = p.cap_out * (1.f - 2.f * __builtin_amdgcn_rcpf(exp2_fast(x * two_log2e) + 1.f));
        const int key = kb + 32 * kh + 8 * (r >> 2) + 4 * hi + (r & 3);
        x -= alibi_s * (float)abs(pos - key);
        Sq[kh][r] = x;
      }
  };
  // mask only tiles that cut through some row's visible band of this wave
  auto mask_tile = [&](f32x16 (&Sq)[2], int qb, int kb) __attribute__((always_inline)) {
    const int rq = row_of(qb);
    const int my_lo = key_lo(rq);
    const uint32_t my_span = (uint32_t)max(key_hi(rq) - my_lo, 0);
    const uint32_t base = (uint32_t)(kb + 4 * hi - my_lo);
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const uint32_t off = (uint32_t)(32 * kh + 8 * (r >> 2) + (r & 3));
        Sq[kh][r] = base + off < my_span ? Sq[kh][r] : -INFINITY;
      }
  };
  // Raise the reference max of block qb if its tile max exceeds it by > 2^8.
  // Returns whether O and l of the block must be rescaled (by alpha): only
  // when a finite max was raised (a row that has seen no key has O = l = 0).
  auto raise_max = [&](const f32x16 (&Sq)[2], int qb, float& alpha) __attribute__((always_inline)) {
    float mx = Sq[0][0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, Sq[0][r]);
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, Sq[1][r]);
    mx = fmaxf(mx, xor32(mx)) * c;
    const bool up = mx > m_ref[qb] + kWideTau;
    const bool need = up && m_ref[qb] != -INFINITY;
    alpha = need ? exp2_fast(m_ref[qb] - mx) : 1.f;
    if (up) m_ref[qb] = mx;
    return need;
  };
  // O and l of block qb times alpha.  The accumulators are read after the
  // MFMAs that wrote them have drained and pinned back into AGPRs, with wait
  // states, before any MFMA reads them again.
  auto rescale = [&](int qb, float alpha) __attribute__((always_inline)) {
    l_a[qb] *= alpha;
    l_b[qb] *= alpha;
#pragma unroll
    for (int db = 0; db < DBLK; ++db) oacc[qb][db] *= alpha;
  };
  auto pin_o = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int db = 0; db < DBLK; ++db) pin_agpr(oacc[qb][db]);
  };
  // P V of a whole tile outside the interleaved block (prologue of a rescale
  // and the last tile)
  auto pv_all = [&](int buf, const u32x4 (&Pp)[QB][4]) __attribute__((always_inline)) {
#pragma unroll
    for (int f = 0; f < 16; ++f) {
      const u32x4 vf = v_frag(buf, f);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) mma_o(oacc[qb][f & 3], vf, Pp[qb][f >> 2]);
    }
  };
  // S^T of a whole tile (prologue)
  auto s_all = [&](int buf, f32x16 (&Sd)[QB][2]) __attribute__((always_inline)) {
#pragma unroll
    for (int g = 0; g < 16; ++g) {
      const u32x4 kf = k_frag(buf, g);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        if ((g & 7) == 0) mma_s_first(Sd[qb][g >> 3], kf, qf[qb][g & 7]);
        else mma_s(Sd[qb][g >> 3], kf, qf[qb][g & 7]);
      }
    }
  };
  // score pair i (0..31) of the tile: block (qb, kh) = i / 8 in the order
  // (0,0) (1,0) (0,1) (1,1), elements 2 r2 and 2 r2 + 1 with r2 = i % 8 (the
  // redo path; the block uses the pipelined stages below)
  float mb[QB];
  auto sm_pair = [&](const f32x16 (&Sc)[QB][2], u32x4 (&Pc)[QB][4], auto ic) __attribute__((always_inline)) {
    constexpr int i = decltype(ic)::value;
    constexpr int blk = i >> 3, r2 = i & 7;
    constexpr int qb = blk & 1, kh = blk >> 1;
    const float p0 = exp2_fast(fmaf(Sc[qb][kh][2 * r2], c, -mb[qb]));
    const float p1 = exp2_fast(fmaf(Sc[qb][kh][2 * r2 + 1], c, -mb[qb]));
    l_a[qb] += p0;
    l_b[qb] += p1;
    Pc[qb][2 * kh + (r2 >> 2)][r2 & 3] = pack_bf16x2(p0, p1);
  };

  // Softmax of one score element per MFMA slot, software-pipelined: element e
  // (0..63) is score 2 r2 + (e & 1) of pair i = e / 2 (block (qb, kh) = i / 8 in
  // the order (0,0) (1,0) (0,1) (1,1), r2 = i % 8).  Slot s finishes element s
  // (row-sum add; the pack of the pair on odd e), takes the exponential of
  // element s + 3 and scales element s + 4, so no instruction waits for
  // another of its own slot and each exponential has three slots to finish.
  auto el_a = [&](const f32x16 (&Sc)[QB][2], float (&xs)[64], auto ec) __attribute__((always_inline)) {
    constexpr int e = decltype(ec)::value;
    if constexpr (e < 64) {
      constexpr int i = e >> 1, blk = i >> 3, r2 = i & 7, qb = blk & 1, kh = blk >> 1;
      xs[e] = fmaf(Sc[qb][kh][2 * r2 + (e & 1)], c, -mb[qb]);
    }
  };
  auto el_b = [&](const float (&xs)[64], float (&ps)[64], auto ec) __attribute__((always_inline)) {
    constexpr int e = decltype(ec)::value;
    if constexpr (e < 64) ps[e] = exp2_fast(xs[e]);
  };
  auto el_c = [&](const float (&ps)[64], u32x4 (&Pc)[QB][4], auto ec) __attribute__((always_inline)) {
    constexpr int e = decltype(ec)::value;
    constexpr int i = e >> 1, blk = i >> 3, r2 = i & 7, qb = blk & 1, kh = blk >> 1;
    if constexpr ((e & 1) == 0) {
      l_a[qb] += ps[e];
    } else {
      l_b[qb] += ps[e];
      Pc[qb][2 * kh + (r2 >> 2)][r2 & 3] = pack_bf16x2(ps[e - 1], ps[e]);
    }
  };

  // ---- prologue: Q fragments (global -> AGPR), K(0), K(1) -> LDS; S^T(0) -----
  const int kb0 = kt_begin * kBlockN;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int t = 0; t < KSTEPS; ++t)
      qf[qb][t] = buf_load16(qrs, (uint32_t)(qw0 + 32 * qb + n) * q_row_bytes + (uint32_t)((2 * t + hi) * 16));
  if (ntiles > 0) {
    fetch(krs, k_src, k_lds_addr, kb0);
    if (ntiles > 1) fetch(krs, k_src, k_lds_addr + TILE_BYTES, kb0 + kBlockN);
  }
  lds_load_wait();
  __syncthreads();
  // the Q fragments go to AGPRs here; the pins' wait states separate those
  // writes from the MFMAs that read them
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int t = 0; t < KSTEPS; ++t) pin_agpr(qf[qb][t]);
  if (ntiles > 0) s_all(0, S[0]);
  mfma_drain();
  // step 0 loads K(2) into K buffer 0: every wave must be done reading K(0)
  __syncthreads();

  // ---- main loop -------------------------------------------------------------
  // Step j: S^T(j) is in S[j&1], P_{j-1} in P[(j+1)&1].  K(j+2) and V(j) are
  // loaded into the buffers of K(j) and V(j-2).  Then one block of 64 MFMA
  // slots: even slots S^T(j+1) (K fragment g = slot/4, row block slot/2 & 1),
  // odd slots P_{j-1} V_{j-1} (V fragment f = slot/4); softmax pair i of tile
  // j rides in slot 2i.  Step 0 has no P_{-1}: its odd slots are empty.
  auto step = [&](auto parity, auto first, int j) __attribute__((always_inline)) {
    constexpr int cur = decltype(parity)::value, nxt = cur ^ 1;
    constexpr bool FIRST = decltype(first)::value;
    f32x16 (&Sc)[QB][2] = S[cur];
    f32x16 (&Sn)[QB][2] = S[nxt];
    u32x4 (&Pc)[QB][4] = P[cur];
    u32x4 (&Pp)[QB][4] = P[nxt];
    const int kb = kb0 + j * kBlockN;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) modify(Sc[qb], qb, kb);
    if (!(kb >= wlo_last && kb + kBlockN <= whi_first)) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) mask_tile(Sc[qb], qb, kb);
    }
    // A row that has seen no key yet needs its max up front; a raise then
    // first adds the pending P V (relative to the old max) and clears it.
    // Past the first key of the wave's last row every row with a visible key
    // has a finite max, so the vote is skipped from there on.
    const bool exact = kb <= wlo_last && wave_any(m_ref[0] == -INFINITY || m_ref[1] == -INFINITY);
    if (exact) {
      float al[QB];
      bool need[QB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) need[qb] = raise_max(Sc[qb], qb, al[qb]);
      if (wave_any(need[0] || need[1])) {
        if constexpr (!FIRST) {
          pv_all(nxt, Pp);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int i = 0; i < 4; ++i) Pp[qb][i] = u32x4{0u, 0u, 0u, 0u};
        }
        mfma_drain();
        pin_o();
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) rescale(qb, al[qb]);
        pin_o();
        mfma_drain();
      }
    }
    const float la0[QB] = {l_a[0], l_a[1]}, lb0[QB] = {l_b[0], l_b[1]};
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) mb[qb] = m_ref[qb] == -INFINITY ? 0.f : m_ref[qb];

    // the interleaved block
    // V fragments are read before K ones: the wait for a K fragment before an
    // S^T MFMA then also covers the V fragment of the P V MFMA after it, so
    // a slot pair needs one LDS wait instead of two
    u32x4 kf[2], vf[2];
    if constexpr (!FIRST) vf[0] = v_frag(nxt, 0);
    kf[0] = k_frag(nxt, 0);
    float xs[64], ps[64];
    el_a(Sc, xs, std::integral_constant<int, 0>{});
    el_a(Sc, xs, std::integral_constant<int, 1>{});
    el_a(Sc, xs, std::integral_constant<int, 2>{});
    el_a(Sc, xs, std::integral_constant<int, 3>{});
    el_b(xs, ps, std::integral_constant<int, 0>{});
    el_b(xs, ps, std::integral_constant<int, 1>{});
    el_b(xs, ps, std::integral_constant<int, 2>{});
    sched_fence();
    static_for<0, 64>([&](auto slot) __attribute__((always_inline)) {
      constexpr int s = decltype(slot)::value;
      constexpr int g = s >> 2;   // fragment index of this slot's MFMA
      constexpr int qb = (s >> 1) & 1;
      uint32_t m0v = 0;
      if constexpr ((s & 3) == 2 && s < 32) {
        constexpr int i = s >> 2;
        if constexpr (i < LOADS)
          m0v = set_m0<cur * TILE_BYTES + 4096u * i>(k_lds_addr + wave_lds);
        else
          m0v = set_m0<cur * TILE_BYTES + 4096u * (i - LOADS)>(v_lds_addr + wave_lds);
      }
      if constexpr ((s & 1) == 0) {
        if constexpr ((g & 7) == 0) mma_s_first(Sn[qb][g >> 3], kf[g & 1], qf[qb][g & 7]);
        else mma_s(Sn[qb][g >> 3], kf[g & 1], qf[qb][g & 7]);
      } else if constexpr (!FIRST) {
        mma_o(oacc[qb][g & 3], vf[g & 1], Pp[qb][g >> 2]);
      }
      el_c(ps, Pc, std::integral_constant<int, s>{});
      el_b(xs, ps, std::integral_constant<int, s + 3>{});
      el_a(Sc, xs, std::integral_constant<int, s + 4>{});
      // The step's tile loads ride in the first half of the block, one 1 KB
      // load every 4 slots: K(j+2) into the buffer of K(j) and V(j) into that
      // of V(j-2), both last read in step j-1.  Spread this way their issue
      // overlaps the MFMAs (a burst of eight before the block took about 300
      // cycles of the step).  K(j+2) is loaded even past the last tile: rows
      // beyond the causal range are harmless, rows at or past Lk load zeros,
      // and such a buffer is only read by the discarded S^T of the last step.
      if constexpr ((s & 3) == 2 && s < 32) {
        constexpr int i = s >> 2;
        if constexpr (i < LOADS) {
          const uint32_t soff = (uint32_t)(kb + 2 * kBlockN + 4 * i * RPI) * k_row_bytes;
          lds_load16_after_m0(krs, k_src, (uint32_t)__builtin_amdgcn_readfirstlane(soff), m0v);
        } else {
          const uint32_t soff = (uint32_t)(kb + 4 * (i - LOADS) * RPI) * k_row_bytes;
          lds_load16_after_m0(vrs, v_src, (uint32_t)__builtin_amdgcn_readfirstlane(soff), m0v);
        }
      }
      // one fragment ahead: fragment g + 1 goes into the buffer fragment g - 1
      // left, whose last MFMA was in the previous slot group
      if constexpr ((s & 3) == 0 && g + 1 < 16) {
        if constexpr (!FIRST) vf[(g + 1) & 1] = v_frag(nxt, g + 1);
        kf[(g + 1) & 1] = k_frag(nxt, g + 1);
      }
      sched_fence();
    });
    // This lane's share of the tile's row sum bounds each of its
    // probabilities (inf and NaN included): above 2^8, take the tile back,
    // raise the max, rescale (P_{j-1} V_{j-1} is already in O) and redo P_j.
    bool redo = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) redo |= !((l_a[qb] - la0[qb]) + (l_b[qb] - lb0[qb]) <= 256.f);
    if (!exact && wave_any(redo)) {
      mfma_drain();
      pin_o();
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        l_a[qb] = la0[qb];
        l_b[qb] = lb0[qb];
        float al;
        if (raise_max(Sc[qb], qb, al)) rescale(qb, al);
        mb[qb] = m_ref[qb] == -INFINITY ? 0.f : m_ref[qb];
      }
      pin_o();
      mfma_drain();
      static_for<0, 32>([&](auto i) __attribute__((always_inline)) { sm_pair(Sc, Pc, i); });
    }
    // the next step's VALU reads S^T(j+1); the row-sum check above already
    // counts toward these wait states
    mfma_drain();
    lds_load_wait();
    __syncthreads();
  };
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  if (ntiles > 0) step(P0{}, std::true_type{}, 0);
  for (int j = 1; j < ntiles; j += 2) {
    step(P1{}, std::false_type{}, j);
    if (j + 1 < ntiles) step(P0{}, std::false_type{}, j + 1);
  }
  if (ntiles > 0) {
    if ((ntiles - 1) & 1) pv_all(1, P[1]); else pv_all(0, P[0]);
  }
  mfma_drain();
  pin_o();          // the epilogue's AGPR reads come after the drain
  // every wave is done reading V before the tiles are reused as staging
  __syncthreads();

  // ---- epilogue: O = acc / l (bf16) through LDS, LSE = (m + log2 l) ln 2 -----
  // Wave w stages its 64 rows (16 KB) in bytes [16w KB, +16 KB) of the tile
  // area (k_lds then v_lds): 16-byte chunk c of local row r at c ^ (r % 16).
  constexpr int RB = 2 * D;
  char* stage = wave < 2 ? reinterpret_cast<char*>(k_lds) + wave * 16384
                         : reinterpret_cast<char*>(v_lds) + (wave - 2) * 16384;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float lpart = l_a[qb] + l_b[qb];
    const float lt = lpart + xor32(lpart);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const int rl = 32 * qb + n;
#pragma unroll
    for (int db = 0; db < DBLK; ++db) {
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int ch = 4 * db + gq;
        *reinterpret_cast<u32x2*>(stage + rl * RB + ((ch ^ (rl & (KCH - 1))) * 16) + 8 * hi) =
            u32x2{pack_bf16x2(oacc[qb][db][4 * gq + 0] * inv, oacc[qb][db][4 * gq + 1] * inv),
                  pack_bf16x2(oacc[qb][db][4 * gq + 2] * inv, oacc[qb][db][4 * gq + 3] * inv)};
      }
    }
    const int rq = qw0 + 32 * qb + n;
    if (rq < Lq && lseg && hi == 0)
      lseg[rq] = lt > 0.f ? (m_ref[qb] + log2_fast(lt)) * kWideLn2 : -INFINITY;
  }
  // each wave reads back only its own rows: no barrier between waves needed,
  // the wave's LDS writes complete in order before its reads
#pragma unroll
  for (int i = 0; i < 64 / RPI; ++i) {
    const int r = i * RPI + lane / KCH, cc = lane % KCH;
    const u32x4 val = *reinterpret_cast<const u32x4*>(stage + r * RB + ((cc ^ (r & (KCH - 1))) * 16));
    if (qw0 + r < Lq)
      __builtin_nontemporal_store(val, reinterpret_cast<u32x4*>(og + (int64_t)(qw0 + r) * p.q_tok_stride + 8 * cc));
  }
}

hipError_t launch_prefill_wide(const PrefillParams& p, hipStream_t stream) {
  const int64_t nblocks = (int64_t)p.num_q_tiles * p.B * (p.Hq / p.wide_heads);
  if (nblocks <= 0) return hipSuccess;
  const bool mods = p.cap_in > 0.f || p.alibi != nullptr;
  if (mods)
    hipLaunchKernelGGL(prefill_fwd_wide_kernel<true>, dim3((unsigned)nblocks), dim3(kPrefillThreads), 0, stream, p);
  else
    hipLaunchKernelGGL(prefill_fwd_wide_kernel<false>, dim3((unsigned)nblocks), dim3(kPrefillThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace fa
