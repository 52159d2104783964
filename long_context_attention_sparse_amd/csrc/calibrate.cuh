// BSFA threshold calibration, selection step ("Block Sparse Flash Attention",
// Abstract and Figure 2: thresholds T^(k) per query row, -inf where fewer than k
// off-diagonal candidates exist).  The page gives no procedure; the one taken:
// for each calibration sample b, head h and query block i, the k-th largest of
// the off-diagonal tile maxima t(i, j), j < i; -inf when i < k; T[h, i] is their
// mean over the B samples (summed in sample order, float32).
//
// One workgroup per (query block, head).  A row has at most kThreshMaxCand candidates,
// staged in LDS; each thread ranks its candidates against the whole row (counts
// of larger and of larger-or-equal values), and the lowest index whose rank
// brackets k gives the k-th largest value — O(i^2 / 256) comparisons per thread,
// a few thousand at 64K tokens, so the pass costs far less than the tile maxima.
#pragma once
#include "common.cuh"

namespace bsa {

__global__ __launch_bounds__(256) void threshold_kernel(ThresholdArgs a) {
  __shared__ float cand[kThreshMaxCand];
  __shared__ int pick;
  const int i = blockIdx.x, h = blockIdx.y;
  const int t = threadIdx.x;
  if (i < a.k) {  // fewer than k off-diagonal candidates: keep every tile
    if (t == 0) a.T[(int64_t)h * a.nqb + i] = kNegInf;
    return;
  }
  float sum = 0.f;
  for (int b = 0; b < a.B; ++b) {
    const float* row = a.tmax + (((int64_t)b * a.Hq + h) * a.nqb + i) * a.nqb;
    for (int j = t; j < i; j += 256) cand[j] = row[j];
    if (t == 0) pick = i;
    __syncthreads();
    for (int j = t; j < i; j += 256) {
      const float v = cand[j];
      int greater = 0, geq = 0;
      for (int x = 0; x < i; ++x) {
        const float c = cand[x];
        greater += c > v;
        geq += c >= v;
      }
      if (greater < a.k && geq >= a.k) atomicMin(&pick, j);
    }
    __syncthreads();
    // some index always brackets k when i >= k (NaN maxima aside, which then propagate)
    if (t == 0) sum += pick < i ? cand[pick] : __builtin_nanf("");
    __syncthreads();  // cand and pick are rewritten for the next sample
  }
  if (t == 0) a.T[(int64_t)h * a.nqb + i] = sum / (float)a.B;
}

}  // namespace bsa
