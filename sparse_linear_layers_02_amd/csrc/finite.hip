// The optional input check (SBN_CHECK_FINITE=1): a scan of a bf16 or fp32
// matrix for NaN / Inf (exponent field all ones).  Non-finite inputs are
// outside the contract of every entry point; with the check on, an entry point
// scans its floating-point inputs first and rejects them before launching
// anything else.  The scan reads the flag back to the host, so it synchronizes
// the stream (a diagnostic mode, not for graph capture).
#include "sbn_internal.h"

#include <algorithm>
#include <mutex>

namespace sbn {
namespace {

// One flag per device; host code reaches it through hipGetSymbolAddress.
__device__ int g_nonfinite;

__global__ void clear_flag_kernel(int* flag) {
  if (threadIdx.x == 0) flag[0] = 0;
}

// Grid-stride over the 16-byte chunks of the valid part of every row.
// ELEM: 2 (bf16) or 4 (fp32).
template <int ELEM>
__global__ __launch_bounds__(256) void nonfinite_scan_kernel(const uint8_t* __restrict__ x, int64_t rows,
                                                             int64_t cpr, int64_t ld_bytes, int* flag) {
  const int64_t total = rows * cpr;
  bool bad = false;
  for (int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x; c < total; c += (int64_t)gridDim.x * 256) {
    const int64_t r = c / cpr;
    const uint4 v = *(const uint4*)(x + r * ld_bytes + (c - r * cpr) * 16);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (ELEM == 2) {
        bad |= (w[i] & 0x7F80u) == 0x7F80u;
        bad |= (w[i] & 0x7F800000u) == 0x7F800000u;
      } else {
        bad |= (w[i] & 0x7F800000u) == 0x7F800000u;
      }
    }
  }
  if (bad) flag[0] = 1;   // every writer stores the same value
}

int* flag_ptr(hipError_t& e) {
  static std::mutex mu;
  static int* ptrs[64] = {};
  int dev = 0;
  e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= 64) {
    if (e == hipSuccess) e = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (!ptrs[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(g_nonfinite));
    if (e != hipSuccess) return nullptr;
    ptrs[dev] = (int*)p;
  }
  return ptrs[dev];
}

}  // namespace

hipError_t scan_nonfinite(const void* x, int64_t rows, int64_t cols, int64_t ld, int elem_bytes, hipStream_t st,
                          bool* found) {
  static std::mutex serial;                  // one flag per device: one scan at a time
  std::lock_guard<std::mutex> lock(serial);
  *found = false;
  hipError_t e;
  int* flag = flag_ptr(e);
  if (!flag) return e;
  const int64_t cpr = cols * elem_bytes / 16;  // cols is a multiple of 64
  const int64_t total = rows * cpr;
  const unsigned grid = (unsigned)std::min<int64_t>(cdiv(total, 256), 4096);
  hipLaunchKernelGGL(clear_flag_kernel, dim3(1), dim3(64), 0, st, flag);
  if (elem_bytes == 2)
    hipLaunchKernelGGL(nonfinite_scan_kernel<2>, dim3(grid), dim3(256), 0, st, (const uint8_t*)x, rows, cpr,
                       ld * 2, flag);
  else
    hipLaunchKernelGGL(nonfinite_scan_kernel<4>, dim3(grid), dim3(256), 0, st, (const uint8_t*)x, rows, cpr,
                       ld * 4, flag);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  int h = 0;
  e = hipMemcpyAsync(&h, flag, sizeof(int), hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return e;
  *found = h != 0;
  return hipSuccess;
}

}  // namespace sbn
