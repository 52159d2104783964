// MFMA tile kernels (prefill over patterns, BSFA gating) and their launch wrappers;
// compiled without IEEE NaN quieting (the kernels never produce NaNs), which keeps the
// softmax row maxima to plain v_max/v_max3 instructions.
#include "gated.cuh"
#include "launch.h"
#include "prefill_pipe.cuh"
#include "prefill_tile.cuh"
#include "prefill_vs_pair.cuh"

namespace bsa {

// Final outputs use the large-chunk kernel; partial outputs (whose group boundaries fall
// on list entries) the 2-stage pipelined one.
template <int NW, int KIND>
static void launch_prefill_t(const PrefillArgs& a, hipStream_t st) {
  if (a.partial)
    hipLaunchKernelGGL((prefill_pipe_kernel<KIND, NW>), dim3(a.n_items), dim3(NW * 64), 0, st, a);
  else
    hipLaunchKernelGGL((prefill_tile_kernel<KIND, NW>), dim3(a.n_items), dim3(NW * 64), 0, st, a);
}

void launch_prefill(const PrefillArgs& a, int NW, int KIND, hipStream_t st) {
  if (NW == 4) {
    if (KIND == 0) launch_prefill_t<4, 0>(a, st);
    else if (KIND == 1) launch_prefill_t<4, 1>(a, st);
    else launch_prefill_t<4, 2>(a, st);
  } else {
    if (KIND == 0) launch_prefill_t<2, 0>(a, st);
    else if (KIND == 1) launch_prefill_t<2, 1>(a, st);
    else launch_prefill_t<2, 2>(a, st);
  }
}

void launch_vs_pair(const PrefillArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((vs_pair_kernel<8>), dim3(a.n_items), dim3(256), 0, st, a);
}

void launch_gated(const GatedArgs& a, bool calib, hipStream_t st) {
  if (calib) hipLaunchKernelGGL((gated_kernel<true, false>), dim3(a.n_items), dim3(256), 0, st, a);
  else if (a.count_skipped) hipLaunchKernelGGL((gated_kernel<false, true>), dim3(a.n_items), dim3(256), 0, st, a);
  else hipLaunchKernelGGL((gated_kernel<false, false>), dim3(a.n_items), dim3(256), 0, st, a);
}

}  // namespace bsa
