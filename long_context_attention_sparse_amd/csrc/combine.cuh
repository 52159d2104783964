// Log-sum-exp combine of attention partials ("Sparse FlashAttention with
// Incremental Repair", What's in this fork and Usage 2: FA(A u B) equals
// Combine(FA(A), FA(B))).  For each (b, s, h): m = max_p lse_p; when m is
// -inf the row has no keys and the result is (0, -inf); otherwise
// w_p = exp(lse_p - m), O = sum w_p o_p / sum w_p, LSE = m + ln sum w_p.
//
// Memory bound: each thread owns four consecutive head-dim values of one row
// (D/4 threads per row, all in one wavefront), reads every partial's LSE for
// its row and streams the partial outputs with 16-byte loads.
#pragma once
#include "common.cuh"

namespace bsa {

// Partials are read once: nontemporal loads (the streaming cache policy); 2% faster on the
// selected-attention workload, whose combine reads 3.3 GB of them.
__device__ __forceinline__ f32x4 ldg128f_nt(const float* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
}

__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
  const int tpr = a.D / 4;
  const int rows_per_block = 256 / tpr;
  const int64_t row = (int64_t)blockIdx.x * rows_per_block + threadIdx.x / tpr;
  const int d = (threadIdx.x % tpr) * 4;
  const int64_t nrows = (int64_t)a.B * a.Sq * a.Hq;
  if (row >= nrows) return;
  const int h = (int)(row % a.Hq);
  const int s = (int)((row / a.Hq) % a.Sq);
  const int b = (int)(row / ((int64_t)a.Hq * a.Sq));
  const int64_t lse_stride = (int64_t)a.B * a.Hq * a.Sq;
  const int64_t lse0 = ((int64_t)b * a.Hq + h) * a.Sq + s;
  const int64_t o_stride = (int64_t)a.B * a.Sq * a.Hq * a.D;
  const int64_t o0 = row * a.D + d;  // row = (b*Sq + s)*Hq + h

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f, m = kNegInf;
  constexpr int ONE = 16;
  if (a.P <= ONE) {
    // up to 16 partials: every load in flight at once, one round trip to memory
    float lv[ONE];
    f32x4 ov[ONE];
#pragma unroll
    for (int j = 0; j < ONE; ++j) {
      const bool ok = j < a.P;
      lv[j] = ok ? a.lse_part[lse0 + j * lse_stride] : kNegInf;
      ov[j] = ok ? ldg128f_nt(a.o_part + o0 + j * o_stride) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int j = 0; j < ONE; ++j) m = fmaxf(m, lv[j]);
    if (m != kNegInf) {
#pragma unroll
      for (int j = 0; j < ONE; ++j) {
        const float wgt = expf(lv[j] - m);
        if (wgt != 0.f) {  // an empty partial's o is never used (it may hold anything)
          acc += wgt * ov[j];
          wsum += wgt;
        }
      }
    }
    const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
    acc *= inv;
    const int64_t off = (int64_t)b * a.o.sb + (int64_t)s * a.o.ss + (int64_t)h * a.o.sh + d;
    store4(a.o, off, acc[0], acc[1], acc[2], acc[3]);
    if (a.lse && d == 0) a.lse[lse0] = wsum > 0.f ? m + logf(wsum) : kNegInf;
    return;
  }
  // more partials: batches of 8, all loads of a batch issued before any is used
  constexpr int BATCH = 8;
  for (int p0 = 0; p0 < a.P; p0 += BATCH) {
    float lv[BATCH];
#pragma unroll
    for (int j = 0; j < BATCH; ++j) lv[j] = p0 + j < a.P ? a.lse_part[lse0 + (p0 + j) * lse_stride] : kNegInf;
#pragma unroll
    for (int j = 0; j < BATCH; ++j) m = fmaxf(m, lv[j]);
  }
  if (m != kNegInf) {
    for (int p0 = 0; p0 < a.P; p0 += BATCH) {
      float lv[BATCH];
      f32x4 ov[BATCH];
#pragma unroll
      for (int j = 0; j < BATCH; ++j) {
        const bool ok = p0 + j < a.P;
        lv[j] = ok ? a.lse_part[lse0 + (p0 + j) * lse_stride] : kNegInf;
        ov[j] = ok ? ldg128f_nt(a.o_part + o0 + (p0 + j) * o_stride) : f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int j = 0; j < BATCH; ++j) {
        const float wgt = expf(lv[j] - m);
        // a partial with no keys contributes nothing (its weight is exactly 0), and its o is
        // never used (it may hold anything)
        if (wgt != 0.f) {
          acc += wgt * ov[j];
          wsum += wgt;
        }
      }
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  acc *= inv;
  const int64_t off = (int64_t)b * a.o.sb + (int64_t)s * a.o.ss + (int64_t)h * a.o.sh + d;
  store4(a.o, off, acc[0], acc[1], acc[2], acc[3]);
  if (a.lse && d == 0) a.lse[lse0] = wsum > 0.f ? m + logf(wsum) : kNegInf;
}

}  // namespace bsa
