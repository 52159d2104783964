// Selected attention (top-k key blocks per query token): index inversion kernels and the
// key-block-outer MFMA kernel, with their launch wrapper; compiled with the tile kernels'
// flags (no IEEE NaN quieting: masked scores are -inf, handled explicitly).
#include "launch.h"
#include "selected.cuh"

namespace bsa {

void launch_selected(const SelArgs& a, int main_grid, hipStream_t st) {
  const int n_lists = a.B * a.Hkv * a.nkb;
  const dim3 tiles((a.Sq + kSelTile - 1) / kSelTile, a.Hkv, a.B);
  hipLaunchKernelGGL(sel_zero_kernel, dim3((n_lists + 255) / 256), dim3(256), 0, st, a);
  hipLaunchKernelGGL(sel_count_kernel, tiles, dim3(256), 0, st, a);
  hipLaunchKernelGGL(sel_scan_kernel, dim3(1), dim3(1024), 0, st, a);
  hipLaunchKernelGGL(sel_fill_kernel, tiles, dim3(256), 0, st, a);
  hipLaunchKernelGGL(selected_kernel, dim3(main_grid), dim3(256), 0, st, a);
}

}  // namespace bsa
