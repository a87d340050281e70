// Streaming-read bandwidth probe, built as its own small library for the
// benchmark: how fast this GPU's HBM delivers a large buffer to plain 16-byte
// vector loads with no arithmetic and no reuse.  It is the measured context
// beside the 8 TB/s spec for the HBM-bound paged decode; the attention
// library neither contains nor calls it.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kUnroll = 4;

// Grid-stride loop, kUnroll independent 16-byte non-temporal loads in flight
// per lane; the XOR of everything read goes to one sink word per lane so
// that no load is dead.
__global__ __launch_bounds__(kThreads) void read_kernel(const u32x4* __restrict__ src, int64_t n,
                                                        uint32_t* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kUnroll - 1) * stride < n; i += kUnroll * stride) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(src + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  sink[(int64_t)blockIdx.x * kThreads + threadIdx.x] = acc;
}

}  // namespace

extern "C" {

// Reads `bytes` of device memory at src (16-byte aligned, a multiple of 16)
// with `blocks` workgroups of 256 threads on `stream` (a hipStream_t, NULL =
// default); writes blocks * 256 uint32 to sink.  Returns 0, 1 for a bad
// argument (nothing enqueued), 2 if the launch failed.
int fa_membw_read(const void* src, size_t bytes, unsigned* sink, int blocks, void* stream) {
  if (!src || !sink || bytes == 0 || bytes % 16 != 0 || blocks < 1 || blocks > (1 << 20) ||
      (reinterpret_cast<uintptr_t>(src) & 15) != 0 || (reinterpret_cast<uintptr_t>(sink) & 3) != 0)
    return 1;
  hipLaunchKernelGGL(read_kernel, dim3((unsigned)blocks), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4*>(src),
                     (int64_t)(bytes / 16), reinterpret_cast<uint32_t*>(sink));
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
