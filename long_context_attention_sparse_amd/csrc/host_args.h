// Host-side helpers of the C ABI layer: bsa.h views -> kernel argument blocks, the score
// scale and the softcap constants, launch status and row alignment.
#pragma once
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "args.cuh"
#include "bsa.h"

namespace bsa {

constexpr float kLog2e = 1.4426950408889634f;

inline bool valid_dtype(int32_t d) { return d == BSA_BF16 || d == BSA_F32; }

inline float scale_of(const bsa_problem& p) {
  return p.softmax_scale > 0.f ? p.softmax_scale : 1.0f / std::sqrt((float)p.D);
}

// softcap_score constants: cap_in = 2 scale log2(e) / c, cap_out = c / scale; (0, 0) when off.
inline void cap_consts(const bsa_problem& p, float& cap_in, float& cap_out) {
  cap_in = cap_out = 0.f;
  if (p.softcap > 0.f) {
    const float t = scale_of(p);
    cap_in = 2.f * t * kLog2e / p.softcap;
    cap_out = p.softcap / t;
  }
}

inline TensorArg targ(const bsa_tensor& t) { return TensorArg{t.ptr, t.stride_b, t.stride_s, t.stride_h}; }
inline OutArg oarg(const bsa_tensor& t) { return OutArg{t.ptr, t.stride_b, t.stride_s, t.stride_h, t.dtype == BSA_F32}; }

inline PatternArg parg(const bsa_pattern* p) {
  PatternArg a{};
  if (!p) return a;
  a.kind = p->kind;
  a.block_M = p->block_M;
  a.block_N = p->block_N;
  a.cap = p->cap;
  a.col_cap = p->col_cap;
  a.count = p->count;
  a.index = p->index;
  a.col_count = p->col_count;
  a.col_index = p->col_index;
  a.s_b = p->s_b;
  a.s_h = p->s_h;
  a.s_q = p->s_q;
  return a;
}

inline bsa_status launch_status() {
  return hipGetLastError() == hipSuccess ? BSA_OK : BSA_ERR_HIP;
}

// 16-byte alignment of every row start: base pointer and all strides must keep
// head-dim rows 16-byte aligned for the vector loads.
// Token (row) strides the kernels take: non-negative and at most 32 MB, so that the byte offsets
// of 64 rows from a block's first row fit the 32-bit offsets of buffer loads.
inline bool row_stride_ok(const bsa_tensor& t, int elem_bytes) {
  return t.stride_s >= 0 && t.stride_s * elem_bytes <= ((int64_t)1 << 25);
}

inline bool aligned_rows(const bsa_tensor& t, int elem_bytes) {
  const uintptr_t p = reinterpret_cast<uintptr_t>(t.ptr);
  auto ok = [&](int64_t s) { return ((s * elem_bytes) & 15) == 0; };
  return (p & 15) == 0 && ok(t.stride_b) && ok(t.stride_s) && ok(t.stride_h);
}

}  // namespace bsa
