// Vertical-slash index conversion ("Implementation: Sgl project Sglang Sparse
// Flash Attention", Description and I/O Contract: raw vertical and slash
// indices -> block_count/block_offset and column_count/column_index per query
// block).  The page defers the rule to a paper that is not among the
// sources; this is the library's own rule:
//
// For query block m of sequence b (rows r0 .. r1-1, d = kv_len - q_len), the
// slash offsets s (key = row + d - s), in the given descending order, cover
// key ranges [max(0, r0+d-s), r1-1+d-s] that move rightwards.  A frontier f
// (start -inf) places windows of block_N keys: a range [a, e] opens a window
// at a when a >= f (f = a + block_N), at f when a < f <= e (f += block_N),
// and nothing otherwise.  Vertical indices v <= r1-1+d, ascending, that no
// window contains become columns.  Rows past the sequence get counts 0.
//
// The merged-head variant takes per-head counts of valid vertical and slash
// indices (same page, Description): head h uses only the first count entries
// of its rows.
//
// One thread per query block; a workgroup takes 64 consecutive query blocks
// of one (b, h) and stages that head's slash and vertical lists in LDS.  The
// vertical list is merged with the windows as they are produced (windows are
// disjoint and ascending), so each thread makes a single pass over both lists.
#pragma once
#include "common.cuh"

namespace bsa {



__global__ __launch_bounds__(kVSConvThreads) void vs_convert_kernel(VSConvArgs a) {
  extern __shared__ int32_t lists[];
  const int bh = blockIdx.y;
  const int b = bh / a.H, h = bh % a.H;
  const int m = blockIdx.x * kVSConvThreads + threadIdx.x;
  const int32_t* sl_g = a.slash + (int64_t)bh * a.nnz_s;
  const int32_t* vt_g = a.vertical + (int64_t)bh * a.nnz_v;
  // per-head counts (the merged-head variant): only the first ns / nv entries are indices
  const int ns = a.s_count ? min(max(a.s_count[h], 0), a.nnz_s) : a.nnz_s;
  const int nv = a.v_count ? min(max(a.v_count[h], 0), a.nnz_v) : a.nnz_v;
  const bool staged = a.nnz_s + a.nnz_v <= kVSConvLdsInts;
  if (staged) {
    for (int x = threadIdx.x; x < ns; x += kVSConvThreads) lists[x] = sl_g[x];
    for (int x = threadIdx.x; x < nv; x += kVSConvThreads) lists[a.nnz_s + x] = vt_g[x];
  }
  __syncthreads();
  if (m >= a.rows) return;
  const int32_t* sl = staged ? lists : sl_g;
  const int32_t* vt = staged ? lists + a.nnz_s : vt_g;

  const int64_t item = (int64_t)bh * a.rows + m;
  const int q_len = a.q_seqlens[b];
  const int kv_len = a.kv_seqlens[b];
  const int r0 = m * a.BM;
  if (r0 >= q_len) {
    a.bc[item] = 0;
    a.cc[item] = 0;
    return;
  }
  const int r1 = min(r0 + a.BM, q_len);
  const int d = kv_len - q_len;
  const int last_visible = r1 - 1 + d;
  int32_t* bo = a.bo + item * a.nnz_s;
  int32_t* co = a.ci + item * a.nnz_v;

  int nwin = 0, ncol = 0, vi = 0;
  int frontier = 0;            // valid once nwin > 0
  int prev_end = -0x7fffffff;  // end (exclusive) of the last window
  for (int si = 0; si < ns; ++si) {
    const int s = sl[si];
    const int e = last_visible - s;
    if (e < 0) continue;
    const int lo = max(0, r0 + d - s);
    int wstart;
    if (nwin == 0 || lo >= frontier) {
      wstart = lo;
    } else if (e >= frontier) {
      wstart = frontier;
    } else {
      continue;
    }
    frontier = wstart + a.BN;
    // verticals left of this window: outside every window unless inside the previous one
    while (vi < nv) {
      const int v = vt[vi];
      if (v >= wstart || v > last_visible) break;
      if (v >= prev_end) co[ncol++] = v;
      ++vi;
    }
    bo[nwin++] = wstart;
    prev_end = frontier;
  }
  while (vi < nv) {
    const int v = vt[vi];
    if (v > last_visible) break;
    if (v >= prev_end) co[ncol++] = v;
    ++vi;
  }
  a.bc[item] = nwin;
  a.cc[item] = ncol;
}

}  // namespace bsa
