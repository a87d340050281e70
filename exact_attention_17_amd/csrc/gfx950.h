// Device helpers for CDNA4 / gfx950: MFMA wrappers, bf16 packing, wave64
// cross-lane reductions and the base-2 exponential.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define FA_DEV __device__ __forceinline__

// D(32x32, f32) += A(32x16, bf16) * B(16x32, bf16).  Lane l holds row/column
// l % 32 of A/B and 8 consecutive contraction elements chosen by l / 32; the
// accumulator holds column l % 32 and rows 8*(r/4) + 4*(l/32) + r%4, r < 16.
FA_DEV f32x16 mfma32x32x16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// D(16x16, f32) += A(16x32, bf16) * B(32x16, bf16).  Lane l holds row/column
// l % 16 and 8 contraction elements chosen by l / 16; the accumulator holds
// column l % 16 and rows 4*(l/16) + r, r < 4.
FA_DEV f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two fp32 -> packed bf16 pair (lo in bits 0..15), round-to-nearest-even
// (one v_cvt_pk_bf16_f32 on gfx950).
FA_DEV uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

FA_DEV float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
FA_DEV float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// 2^x on the transcendental unit (v_exp_f32); 2^-inf = 0.
FA_DEV float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

FA_DEV float log2_fast(float x) { return __builtin_amdgcn_logf(x); }

// Value from lane (lane ^ 32): swaps the two halves of a wave64.
FA_DEV float xor32(float x) {
  return __int_as_float(__builtin_amdgcn_ds_bpermute(((threadIdx.x & 63) ^ 32) << 2,
                                                     __float_as_int(x)));
}

// Value from lane (lane ^ 16).
FA_DEV float xor16(float x) {
  return __int_as_float(__builtin_amdgcn_ds_bpermute(((threadIdx.x & 63) ^ 16) << 2,
                                                     __float_as_int(x)));
}

// Butterfly max / sum over the 16 lanes of a DPP row (lanes 16k..16k+15).
// row_ror rotates within the row, quad_perm swaps within 4-lane groups.
template <int CTRL>
FA_DEV float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
constexpr int kDppRowRor8 = 0x128;
constexpr int kDppRowRor4 = 0x124;
constexpr int kDppQuadXor2 = 0x4e;   // quad_perm [2,3,0,1]
constexpr int kDppQuadXor1 = 0xb1;   // quad_perm [1,0,3,2]

FA_DEV float row16_max(float x) {
  x = fmaxf(x, dpp<kDppRowRor8>(x));
  x = fmaxf(x, dpp<kDppRowRor4>(x));
  x = fmaxf(x, dpp<kDppQuadXor2>(x));
  x = fmaxf(x, dpp<kDppQuadXor1>(x));
  return x;
}

FA_DEV float row16_sum(float x) {
  x += dpp<kDppRowRor8>(x);
  x += dpp<kDppRowRor4>(x);
  x += dpp<kDppQuadXor2>(x);
  x += dpp<kDppQuadXor1>(x);
  return x;
}

// LDS transpose read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// lane i receives 16-bit element i%4 of the 8-byte rows addressed by lanes
// i/4, 4+i/4, 8+i/4 and 12+i/4.  So if lane j addresses row r0 + j/4, column
// c0 + 4*(j%4) of a row-major matrix, lane i gets column c0 + i of rows
// r0..r0+3: a 4x16 block comes back transposed.
typedef short s16x4 __attribute__((ext_vector_type(4)));
FA_DEV u32x2 tr_read_b64(const uint16_t* lds) {
  return __builtin_bit_cast(
      u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)lds));
}

// Byte address of a __shared__ object in the workgroup's LDS window.
FA_DEV uint32_t lds_address(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p;
}

// Debug builds (-DFA_DEBUG): the 16 bytes that a lane's direct-to-LDS load
// will write are first set to bf16 NaN and the write is awaited, so a read
// that a missing wait or barrier lets through returns NaN, which the outputs
// show, instead of the previous tile's finite data.  Release builds: nothing.
#ifdef FA_DEBUG
FA_DEV void lds_poison16(uint32_t lds_base) {
  *(__attribute__((address_space(3))) u32x4*)(uintptr_t)(lds_base + 16u * (threadIdx.x & 63)) =
      u32x4{0xffffffffu, 0xffffffffu, 0xffffffffu, 0xffffffffu};
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}
#else
FA_DEV void lds_poison16(uint32_t) {}
#endif

// 16-byte buffer load that writes LDS instead of VGPRs: lane l reads bytes
// [voffset + soffset, +16) of the buffer and stores them at LDS byte
// lds_base + 16 l (soffset and lds_base must be wave-uniform; lds_base goes
// in M0).  The range check applies to voffset + soffset: out-of-range lanes
// store zeros.  The compiler does not track these loads, so lds_load_wait()
// must run before the data is read.  Nor does it see the instruction's
// hazards: an SGPR operand written by a VALU op (v_readfirstlane) needs 5 wait
// states before a VMEM read, and M0 one before an LDS-destination load, so 5
// are inserted here.
FA_DEV void lds_load16(__amdgpu_buffer_rsrc_t r, uint32_t voffset, uint32_t soffset, uint32_t lds_base) {
  lds_poison16(lds_base);
  asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
               :: "v"(voffset), "s"(r), "s"(soffset), "{m0}"(lds_base) : "memory");
}
FA_DEV void lds_load_wait() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// Waits until at most N of the wave's vector-memory loads are still in
// flight.  Loads complete in issue order, so all but the last N have landed.
template <int N>
FA_DEV void lds_load_wait_n() { asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory"); }

// Forces the wait for a value from an ordinary (compiler-tracked) load at
// this point.  A loop that also issues direct-to-LDS loads, which the compiler
// does not see, must not inherit the wait for such a value: the vmcnt it
// would place in the loop counts the invisible loads too and stalls on them.
template <class T>
FA_DEV void await_value(const T& v) { asm volatile("" ::"v"(v)); }

FA_DEV bool wave_any(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }

// Raw buffer resource over [base, base + bytes).  A load whose byte offset is
// at or past `bytes` returns zeros, so ragged tiles need no branches; offsets
// of invalid rows are set to kOob (bytes must stay below 2^31).
constexpr uint32_t kOob = 0x80000000u;
FA_DEV __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
FA_DEV u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
}

}  // namespace fa
