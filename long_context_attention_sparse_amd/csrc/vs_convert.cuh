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

// A thread's output row, written four entries at a time when the row is 16-byte aligned: each
// lane writes its own row, so every store is a separate L2 request, and 16-byte stores make a
// quarter as many of them.
template <bool VEC>
struct RowWriter {
  int32_t* base;
  int n = 0;
  int32_t v0 = 0, v1 = 0, v2 = 0, v3 = 0;  // the last four entries
  __device__ __forceinline__ explicit RowWriter(int32_t* p) : base(p) {}
  __device__ __forceinline__ void push(int32_t x) {
    if constexpr (VEC) {
      v0 = v1;
      v1 = v2;
      v2 = v3;
      v3 = x;
      if ((++n & 3) == 0)
        *reinterpret_cast<u32x4*>(base + n - 4) = u32x4{(uint32_t)v0, (uint32_t)v1, (uint32_t)v2, (uint32_t)v3};
    } else {
      base[n++] = x;
    }
  }
  __device__ __forceinline__ void flush() {
    if constexpr (VEC) {
      const int r = n & 3;  // entries not yet written: the last r
      if (r >= 3) base[n - 3] = v1;
      if (r >= 2) base[n - 2] = v2;
      if (r >= 1) base[n - 1] = v3;
    }
  }
};

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

  // the single pass over both lists; called once with the LDS copies and once with the global
  // lists, so that each call reads through pointers of a known address space (LDS reads, not
  // generic ones)
  auto convert = [&](const int32_t* sl, const int32_t* vt, auto wo, auto co_w) __attribute__((always_inline)) {
    int vi = 0;
    int frontier = 0;            // valid once a window exists
    int prev_end = -0x7fffffff;  // end (exclusive) of the last window
    // the next vertical index, read one step ahead so the LDS latency overlaps the compare
    int vnext = vi < nv ? vt[vi] : 0x7fffffff;
    auto slash = [&](int s) __attribute__((always_inline)) {
      const int e = last_visible - s;
      if (e < 0) return;
      const int lo = max(0, r0 + d - s);
      int wstart;
      if (wo.n == 0 || lo >= frontier) {
        wstart = lo;
      } else if (e >= frontier) {
        wstart = frontier;
      } else {
        return;
      }
      frontier = wstart + a.BN;
      // verticals left of this window: outside every window unless inside the previous one
      while (vi < nv) {
        const int v = vnext;
        if (v >= wstart || v > last_visible) break;
        ++vi;
        vnext = vi < nv ? vt[vi] : 0x7fffffff;
        if (v >= prev_end) co_w.push(v);
      }
      wo.push(wstart);
      prev_end = frontier;
    };
    // slash indices four at a time (one 16-byte read) where the list allows it
    int si = 0;
    if ((reinterpret_cast<uintptr_t>(sl) & 15) == 0) {
      for (; si + 4 <= ns; si += 4) {
        const u32x4 s4 = *reinterpret_cast<const u32x4*>(sl + si);
        slash((int)s4[0]);
        slash((int)s4[1]);
        slash((int)s4[2]);
        slash((int)s4[3]);
      }
    }
    for (; si < ns; ++si) slash(sl[si]);
    while (vi < nv) {
      const int v = vnext;
      if (v > last_visible) break;
      ++vi;
      vnext = vi < nv ? vt[vi] : 0x7fffffff;
      if (v >= prev_end) co_w.push(v);
    }
    wo.flush();
    co_w.flush();
    a.bc[item] = wo.n;
    a.cc[item] = co_w.n;
  };
  // 16-byte stores need 16-byte aligned rows (uniform over the launch)
  const bool vec = ((a.nnz_s | a.nnz_v) & 3) == 0 && ((reinterpret_cast<uintptr_t>(a.bo) |
                                                       reinterpret_cast<uintptr_t>(a.ci)) & 15) == 0;
  if (vec) {
    if (staged) convert(lists, lists + a.nnz_s, RowWriter<true>(bo), RowWriter<true>(co));
    else convert(sl_g, vt_g, RowWriter<true>(bo), RowWriter<true>(co));
  } else {
    if (staged) convert(lists, lists + a.nnz_s, RowWriter<false>(bo), RowWriter<false>(co));
    else convert(sl_g, vt_g, RowWriter<false>(bo), RowWriter<false>(co));
  }
}

}  // namespace bsa
