// Backward of block-sparse attention: the row-dot, list-inversion, dK/dV and dQ kernels and
// their launch wrapper; compiled with the tile kernels' flags (no IEEE NaN quieting).
#include "backward.cuh"
#include "launch.h"

namespace bsa {

void launch_bwd(const BwdArgs& a, int chunk_bound, hipStream_t st) {
  const int64_t rows = (int64_t)a.B * a.Sq * a.Hq;
  const int n_lists = a.B * a.Hkv * a.nks;
  hipLaunchKernelGGL(bwd_dot_kernel, dim3((unsigned)((rows + 15) / 16)), dim3(256), 0, st, a);
  if (a.pat.kind != 0) {
    const int Ht = a.list_by_kv ? a.Hkv : a.Hq;
    const int64_t words = (int64_t)a.B * Ht * a.nkb * a.W;
    const int64_t slots = (int64_t)a.B * Ht * a.nqb * a.pat.cap;
    hipLaunchKernelGGL(bwd_bits_zero_kernel, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, st, a);
    if (slots > 0)
      hipLaunchKernelGGL(bwd_bits_set_kernel, dim3((unsigned)((slots + 255) / 256)), dim3(256), 0, st, a);
    hipLaunchKernelGGL(bwd_list_count_kernel, dim3((n_lists + 255) / 256), dim3(256), 0, st, a);
    hipLaunchKernelGGL(bwd_scan_kernel, dim3(1), dim3(1024), 0, st, a);
    hipLaunchKernelGGL(bwd_list_fill_kernel, dim3((n_lists + 3) / 4), dim3(256), 0, st, a);
  } else {
    hipLaunchKernelGGL(bwd_dense_count_kernel, dim3((n_lists + 255) / 256), dim3(256), 0, st, a);
    hipLaunchKernelGGL(bwd_scan_kernel, dim3(1), dim3(1024), 0, st, a);
  }
  const bool cap = a.cap_in != 0.f;
  if (cap) hipLaunchKernelGGL(bwd_dkdv_kernel<true>, dim3(chunk_bound), dim3(256), 0, st, a);
  else hipLaunchKernelGGL(bwd_dkdv_kernel<false>, dim3(chunk_bound), dim3(256), 0, st, a);
  hipLaunchKernelGGL(bwd_reduce_kernel, dim3(n_lists * (a.SB / kBwdReduceKeys)), dim3(256), 0, st, a);
  const unsigned dq_grid = (unsigned)((int64_t)a.B * a.Hq * a.nqb);
  if (a.BM == 128) {
    if (cap) hipLaunchKernelGGL((bwd_dq_kernel<4, true>), dim3(dq_grid), dim3(256), 0, st, a);
    else hipLaunchKernelGGL((bwd_dq_kernel<4, false>), dim3(dq_grid), dim3(256), 0, st, a);
  } else {
    if (cap) hipLaunchKernelGGL((bwd_dq_kernel<2, true>), dim3(dq_grid), dim3(128), 0, st, a);
    else hipLaunchKernelGGL((bwd_dq_kernel<2, false>), dim3(dq_grid), dim3(128), 0, st, a);
  }
}

}  // namespace bsa
