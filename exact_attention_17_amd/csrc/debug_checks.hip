// Debug builds (-DFA_DEBUG) only: the device-side preconditions of the
// varlen and paged entry points, checked by one small kernel before any
// attention kernel is enqueued, so that a bad offset or page id becomes an
// error status instead of an out-of-range read.  Release builds compile
// this file to nothing.
#include "fa_internal.h"

#ifdef FA_DEBUG

#include <mutex>

namespace fa {

// written by every check before it is read; host code takes its address
// from hipGetSymbolAddress on the current device
static __device__ int check_result;

namespace {

constexpr int kCheckThreads = 256;

__global__ __launch_bounds__(kCheckThreads) void debug_check_kernel(DeviceChecks c, int* result) {
  __shared__ int bad;
  if (threadIdx.x == 0) bad = 0;
  __syncthreads();
  int mine = 0;
  if (c.cu_q) {
    for (int b = threadIdx.x; b <= c.B; b += kCheckThreads) {
      const int q = c.cu_q[b], k = c.cu_k[b];
      if (b == 0 && (q != 0 || k != 0)) mine |= 1;
      if (b == c.B && (q != c.total_q || k != c.total_k)) mine |= 1;
      if (b > 0) {
        const int64_t lq = (int64_t)q - c.cu_q[b - 1], lk = (int64_t)k - c.cu_k[b - 1];
        if (lq < 0 || lk < 0 || lq > c.max_q || lk > c.max_k) mine |= 1;
      }
    }
  }
  if (c.block_table) {
    const int64_t cap = (int64_t)c.max_blocks * c.page_size;
    for (int b = 0; b < c.B; ++b) {
      const int64_t n = (int64_t)c.seqlens[b] + c.extra_len;
      if (n < c.extra_len || n > cap) {   // the row is not read past its end
        mine |= 2;
        continue;
      }
      const int pages = (int)((n + c.page_size - 1) / c.page_size);
      for (int j = threadIdx.x; j < pages; j += kCheckThreads) {
        const int pg = c.block_table[(int64_t)b * c.max_blocks + j];
        if (pg < 0 || pg >= c.num_pages) mine |= 4;
      }
    }
  }
  if (mine) atomicOr(&bad, mine);
  __syncthreads();
  if (threadIdx.x == 0) *result = bad;
}

}  // namespace

int debug_check_inputs(const DeviceChecks& c, hipStream_t stream) {
  // one result word per device; the lock keeps concurrent checks from
  // sharing it (each waits for its own result before releasing the lock)
  static std::mutex lock;
  std::lock_guard<std::mutex> guard(lock);
  int* d = nullptr;
  if (hipGetSymbolAddress(reinterpret_cast<void**>(&d), HIP_SYMBOL(check_result)) != hipSuccess)
    return -1;
  int h = -1;
  hipLaunchKernelGGL(debug_check_kernel, dim3(1), dim3(kCheckThreads), 0, stream, c, d);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess) e = hipMemcpyAsync(&h, d, sizeof(int), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  return e == hipSuccess ? h : -1;
}

}  // namespace fa

#endif  // FA_DEBUG
