// Selected attention (top-k key blocks per query token): index inversion kernels and the
// key-block-outer MFMA kernel, with their launch wrapper; compiled with the tile kernels'
// flags (no IEEE NaN quieting: masked scores are -inf, handled explicitly).
#include <algorithm>

#include "launch.h"
#include "selected.cuh"

namespace bsa {

void launch_selected(const SelArgs& a, int main_grid, hipStream_t st) {
  const int n_lists = a.B * a.Hkv * a.nkb;
  const int64_t pairs = (int64_t)a.T * a.Hkv * a.topk;
  const int zero_grid = (n_lists + 255) / 256;
  const int pair_grid = (int)((pairs + 255) / 256);
  hipLaunchKernelGGL(sel_zero_kernel, dim3(zero_grid), dim3(256), 0, st, a);
  hipLaunchKernelGGL(sel_count_kernel, dim3(pair_grid), dim3(256), 0, st, a);
  hipLaunchKernelGGL(sel_scan_kernel, dim3(1), dim3(1024), 0, st, a);
  hipLaunchKernelGGL(sel_fill_kernel, dim3(pair_grid), dim3(256), 0, st, a);
  hipLaunchKernelGGL(selected_kernel, dim3(main_grid), dim3(256), 0, st, a);
}

}  // namespace bsa
