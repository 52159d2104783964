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
// Two kernels.  vs_convert_kernel: one thread per query block walks the slash
// list in order (the window frontier is a sequential dependence); a workgroup
// takes 64 consecutive query blocks of one (b, h) and stages that head's slash
// list in LDS.  vs_columns_kernel: one wave per query block tests 64 verticals
// per round against the block's windows (a vertical is a column iff it is at
// most the block's last visible key and no window holds it: windows are
// disjoint and ascending, so a binary search over their starts decides it) and
// writes the kept ones in order.  The one-thread merge of both lists that this
// replaces spent three quarters of its time on the verticals.
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
  // per-head counts (the merged-head variant): only the first ns entries are indices
  const int ns = a.s_count ? min(max(a.s_count[h], 0), a.nnz_s) : a.nnz_s;
  const bool staged = a.nnz_s <= kVSConvLdsInts;
  if (staged)
    for (int x = threadIdx.x; x < ns; x += kVSConvThreads) lists[x] = sl_g[x];
  __syncthreads();
  if (m >= a.rows) return;

  const int64_t item = (int64_t)bh * a.rows + m;
  const int q_len = a.q_seqlens[b];
  const int kv_len = a.kv_seqlens[b];
  const int r0 = m * a.BM;
  if (r0 >= q_len) {
    a.bc[item] = 0;
    return;
  }
  const int r1 = min(r0 + a.BM, q_len);
  const int d = kv_len - q_len;
  const int last_visible = r1 - 1 + d;
  int32_t* bo = a.bo + item * a.nnz_s;

  // the walk; called once with the LDS copy and once with the global list, so that each call
  // reads through a pointer of a known address space (LDS reads, not generic ones)
  auto convert = [&](const int32_t* sl, auto wo) __attribute__((always_inline)) {
    int frontier = 0;  // valid once a window exists
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
      wo.push(wstart);
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
    wo.flush();
    a.bc[item] = wo.n;
  };
  // 16-byte stores need 16-byte aligned rows (uniform over the launch)
  const bool vec = (a.nnz_s & 3) == 0 && (reinterpret_cast<uintptr_t>(a.bo) & 15) == 0;
  if (vec) {
    if (staged) convert(lists, RowWriter<true>(bo));
    else convert(sl_g, RowWriter<true>(bo));
  } else {
    if (staged) convert(lists, RowWriter<false>(bo));
    else convert(sl_g, RowWriter<false>(bo));
  }
}

// Columns of query block blockIdx.x of (b, h) = blockIdx.y, after vs_convert_kernel has written
// its windows: one wave, verticals in rounds of 64 (one per lane, ascending), the kept ones
// written in order through a ballot and a prefix count.  The block's windows are staged in LDS
// when they fit (kVSColLdsInts), else searched in global memory.
__global__ __launch_bounds__(64) void vs_columns_kernel(VSConvArgs a) {
  extern __shared__ int32_t wins[];
  const int m = blockIdx.x, bh = blockIdx.y;
  const int b = bh / a.H, h = bh % a.H;
  const int64_t item = (int64_t)bh * a.rows + m;
  const int l = threadIdx.x;
  const int q_len = a.q_seqlens[b];
  const int kv_len = a.kv_seqlens[b];
  const int r0 = m * a.BM;
  if (r0 >= q_len) {  // uniform: no barrier has run yet
    if (l == 0) a.cc[item] = 0;
    return;
  }
  const int last_visible = min(r0 + a.BM, q_len) - 1 + (kv_len - q_len);
  const int nv = a.v_count ? min(max(a.v_count[h], 0), a.nnz_v) : a.nnz_v;
  const int nw = a.bc[item];
  const int32_t* bo = a.bo + item * a.nnz_s;  // read only when nw > 0
  const bool staged = nw <= min(a.nnz_s, kVSColLdsInts);
  if (staged)
    for (int x = l; x < nw; x += 64) wins[x] = bo[x];
  __syncthreads();
  const int32_t* vt = a.vertical + (int64_t)bh * a.nnz_v;
  int32_t* co = a.ci + item * a.nnz_v;
  // v lies in a window iff the last window starting at or before v still holds it
  auto covered = [&](int v, const int32_t* w) __attribute__((always_inline)) {
    int lo = 0, hi = nw;  // windows with start <= v: [0, lo)
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (w[mid] <= v) lo = mid + 1;
      else hi = mid;
    }
    return lo > 0 && v < w[lo - 1] + a.BN;
  };
  int n = 0;
  for (int i0 = 0; i0 < nv; i0 += 64) {
    const int i = i0 + l;
    const int v = i < nv ? vt[i] : 0x7fffffff;
    bool keep = v <= last_visible;
    if (keep) keep = !(staged ? covered(v, wins) : covered(v, bo));
    const uint64_t bal = __ballot(keep);
    if (keep)
      co[n + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u))] = v;
    n += __popcll(bal);
    // ascending: once a vertical of this round lies past the block, so do all later ones
    if (__ballot(i < nv && v > last_visible) != 0) break;
  }
  if (l == 0) a.cc[item] = n;
}

}  // namespace bsa
