// Memory-streaming kernels (split-KV decode, combine, vertical-slash conversion, threshold
// selection) and their launch wrappers; compiled with the default IEEE floating-point mode.
#include "calibrate.cuh"
#include "combine.cuh"
#include "decode.cuh"
#include "launch.h"
#include "vs_convert.cuh"

namespace bsa {

void launch_decode(const DecodeArgs& a, int D, int gx, int groups, int B, hipStream_t st) {
  if (D == 128) hipLaunchKernelGGL((decode_kernel<128>), dim3(gx, groups, B), dim3(256), 0, st, a);
  else hipLaunchKernelGGL((decode_kernel<64>), dim3(gx, groups, B), dim3(256), 0, st, a);
}

void launch_combine(const CombineArgs& c, hipStream_t st) {
  const int64_t rows = (int64_t)c.B * c.Sq * c.Hq;
  const int rows_per_block = 256 / (c.D / 4);
  const int64_t blocks = (rows + rows_per_block - 1) / rows_per_block;
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)blocks), dim3(256), 0, st, c);
}

void launch_vs_convert(const VSConvArgs& a, hipStream_t st) {
  dim3 grid((a.rows + kVSConvThreads - 1) / kVSConvThreads, a.B * a.H);
  const unsigned lds_walk = a.nnz_s <= kVSConvLdsInts ? (unsigned)a.nnz_s * sizeof(int32_t) : 0u;
  hipLaunchKernelGGL(vs_convert_kernel, grid, dim3(kVSConvThreads), lds_walk, st, a);
  const unsigned lds_cols = (unsigned)(a.nnz_s < kVSColLdsInts ? a.nnz_s : kVSColLdsInts) * sizeof(int32_t);
  hipLaunchKernelGGL(vs_columns_kernel, dim3(a.rows, a.B * a.H), dim3(64), lds_cols, st, a);
}

void launch_threshold(const ThresholdArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(threshold_kernel, dim3(a.nqb, a.Hq), dim3(256), 0, st, a);
}

}  // namespace bsa
