// Validation of key patterns: the preconditions the attention kernels rely on but do not
// check (list entries unique and in range; vertical-slash windows ascending and disjoint,
// columns ascending, unique and outside every window).  One thread per list; a violating
// list adds 1 to result[0] and lowers result[1] to its flat index (b * Ht + ht) * nqb + i.
#pragma once
#include "common.cuh"

namespace bsa {

__global__ __launch_bounds__(64) void check_init_kernel(int32_t* result) {
  if (tid_x() == 0) {
    result[0] = 0;
    result[1] = 0x7fffffff;
  }
}

__device__ __forceinline__ bool check_list(const CheckArgs& a, int b, int64_t lb) {
  const PatternArg& p = a.pat;
  const int kv_len = a.cu_k ? a.cu_k[b + 1] - a.cu_k[b] : a.Sk;
  const int n = p.count[lb];
  if (n < 0 || n > p.cap) return false;
  const int32_t* ent = p.index + lb * p.cap;
  if (p.kind == 1) {  // block ids: in range and distinct
    for (int x = 0; x < n; ++x) {
      const int j = ent[x];
      if (j < 0 || (int64_t)j * p.block_N >= kv_len) return false;
      for (int y = 0; y < x; ++y)
        if (ent[y] == j) return false;
    }
    return true;
  }
  // vertical-slash: window starts ascending, disjoint, inside the sequence
  for (int x = 0; x < n; ++x) {
    if (ent[x] < 0 || ent[x] >= kv_len) return false;
    if (x > 0 && ent[x] < ent[x - 1] + p.block_N) return false;
  }
  const int nc = p.col_count[lb];
  if (nc < 0 || nc > p.col_cap) return false;
  const int32_t* col = p.col_index + lb * p.col_cap;
  int wi = 0;
  for (int x = 0; x < nc; ++x) {
    const int c = col[x];
    if (c < 0 || c >= kv_len || (x > 0 && c <= col[x - 1])) return false;
    while (wi < n && ent[wi] + p.block_N <= c) ++wi;  // windows ending at or before c
    if (wi < n && ent[wi] <= c) return false;           // c lies in window wi
  }
  return true;
}

__global__ __launch_bounds__(64) void check_pattern_kernel(CheckArgs a) {
  const int64_t x = (int64_t)wg_x() * 64 + tid_x();
  const int64_t n = (int64_t)a.B * a.Ht * a.nqb;
  if (x >= n) return;
  const int i = (int)(x % a.nqb);
  const int64_t bh = x / a.nqb;
  const int ht = (int)(bh % a.Ht), b = (int)(bh / a.Ht);
  // varlen: lists past the sequence's own query blocks are never read
  if (a.cu_q && (int64_t)i * a.pat.block_M >= a.cu_q[b + 1] - a.cu_q[b]) return;
  const int64_t lb = (int64_t)b * a.pat.s_b + (int64_t)ht * a.pat.s_h + (int64_t)i * a.pat.s_q;
  if (!check_list(a, b, lb)) {
    atomicAdd(&a.result[0], 1);
    atomicMin(&a.result[1], (int)x);
  }
}

}  // namespace bsa
