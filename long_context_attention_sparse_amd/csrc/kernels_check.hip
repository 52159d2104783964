// Pattern validation kernels and their launch wrappers (default IEEE mode; integer work).
#include "check.cuh"
#include "launch.h"

namespace bsa {

// Result words of the checks run by the attention entry points when BSA_DEBUG_CHECKS is set
// (one copy per device; concurrent debug checks on one device share it).
__device__ int32_t g_debug_result[2];

void launch_check(const CheckArgs& a, hipStream_t st) {
  const int64_t n = (int64_t)a.B * a.Ht * a.nqb;
  hipLaunchKernelGGL(check_init_kernel, dim3(1), dim3(64), 0, st, a.result);
  hipLaunchKernelGGL(check_pattern_kernel, dim3((unsigned)((n + 63) / 64)), dim3(64), 0, st, a);
}

// Runs the check into g_debug_result and waits for it: violations found, or -1 when the
// launch or the copy failed.
int debug_check(CheckArgs a, hipStream_t st) {
  int32_t* dev = nullptr;
  if (hipGetSymbolAddress(reinterpret_cast<void**>(&dev), HIP_SYMBOL(g_debug_result)) != hipSuccess) return -1;
  a.result = dev;
  launch_check(a, st);
  int32_t host[2] = {0, 0};
  if (hipMemcpyFromSymbolAsync(host, HIP_SYMBOL(g_debug_result), sizeof(host), 0, hipMemcpyDeviceToHost, st) !=
          hipSuccess ||
      hipStreamSynchronize(st) != hipSuccess)
    return -1;
  return host[0];
}

}  // namespace bsa
