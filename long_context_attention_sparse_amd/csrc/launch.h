// Host-side launch wrappers, one per kernel family, defined in the translation unit that
// instantiates the kernels (kernels_stream.hip, kernels_tile.hip, kernels_select.hip,
// kernels_bwd.hip, kernels_check.hip) so that each family is compiled with its own
// code-generation flags.
#pragma once
#include <hip/hip_runtime.h>

#include "args.cuh"

namespace bsa {

// decode_kernel<D>: grid (gx, groups, B), 256 threads.  D is 64 or 128.
void launch_decode(const DecodeArgs& a, int D, int gx, int groups, int B, hipStream_t st);
// combine_kernel over B*Sq*Hq rows.
void launch_combine(const CombineArgs& a, hipStream_t st);
// vs_convert_kernel (windows): grid (cdiv(rows, kVSConvThreads), B*H), the slash list in dynamic LDS;
// then vs_columns_kernel (columns): grid (rows, B*H) of one wave, a block's windows in dynamic LDS.
void launch_vs_convert(const VSConvArgs& a, hipStream_t st);
// prefill_pipe_kernel<KIND, NW>: n_items workgroups of NW*64 threads (NW 2 or 4, KIND 0..2).
void launch_prefill(const PrefillArgs& a, int NW, int KIND, hipStream_t st);
// vs_pair_kernel: vertical-slash patterns on 64-row query blocks, final outputs; n_items =
// B * Hq * cdiv(nqb, 2) workgroups (pairs of query blocks) of 256 threads.
void launch_vs_pair(const PrefillArgs& a, hipStream_t st);
// gated_kernel<calib, count>: n_items workgroups of 256 threads (count: a.count_skipped).
void launch_gated(const GatedArgs& a, bool calib, hipStream_t st);
// threshold_kernel: grid (nqb, Hq), 256 threads; nqb <= kThreshMaxCand.
void launch_threshold(const ThresholdArgs& a, hipStream_t st);

// backward: bwd_dot, the lists (block patterns: bwd_bits_zero / bwd_bits_set / bwd_list_count /
// bwd_scan / bwd_list_fill; dense: bwd_dense_count / bwd_scan), bwd_dkdv (four waves) over
// chunk_bound workgroups (an upper bound on the chunks), bwd_reduce, bwd_dq.
void launch_bwd(const BwdArgs& a, int chunk_bound, hipStream_t st);
// selected attention: sel_zero, sel_count, sel_scan, sel_fill, then selected_kernel over
// main_grid workgroups (an upper bound on the chunks; the surplus exits at once).
void launch_selected(const SelArgs& a, int main_grid, hipStream_t st);

// pattern check: result[0] = violating lists, result[1] = the first one (flat index).
void launch_check(const CheckArgs& a, hipStream_t st);
// The same check into the library's own result words, waited for: violations or -1.
int debug_check(CheckArgs a, hipStream_t st);

}  // namespace bsa
