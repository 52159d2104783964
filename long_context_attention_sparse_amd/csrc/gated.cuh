// BSFA gated causal attention ("Block Sparse Flash Attention", Abstract and
// Figure 2).  For query block i the kernel visits key blocks j <= i (the
// diagonal first, so the running maximum starts high), computes the 128x128
// score tile S_ij with MFMA, takes its exact maximum t(i,j) (lane max, wave
// shuffle reduce, one LDS exchange between the four waves) and keeps the tile
// iff j == i or scale * t(i,j) >= T[b, h, i].  Only kept tiles load V_j and
// run the softmax update and P V product; a skipped tile's scores never enter
// the softmax.  The next key tile is fetched into registers while the current
// one is finished.
//
// Workgroup: 4 waves x 32 query rows (BM = 128); K and V^T tiles of 128 keys
// in LDS (70 KB, two workgroups per CU); same MFMA layouts as the prefill
// kernel (tile.cuh).  Grid remapped XCD-aware, heaviest query blocks first.
#pragma once
#include "tile.cuh"

namespace bsa {


__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void gated_kernel(GatedArgs a) {
  constexpr int D = TD;
  constexpr int BN = 128;
  constexpr int PIECES = D / 8;
  constexpr int L = BN * PIECES / 256;  // 8 consecutive keys per thread per tile
  constexpr int VSTR = BN + 8;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[BN * TKS];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[D * VSTR];
  __shared__ float red[4];

  const int item = xcd_item(wg_x(), a.n_items);
  const int mrev = item % a.nqb;
  int rest = item / a.nqb;
  const int g = rest % a.G;
  rest /= a.G;
  const int hkv = rest % a.Hkv;
  const int b = rest / a.Hkv;
  const int h = hkv * a.G + g;
  const int i = a.nqb - 1 - mrev;

  const int t = tid_x();
  const int w = t >> 6, l = t & 63;
  const int lq = l & 31, hh = l >> 5;

  const uint16_t* qb = reinterpret_cast<const uint16_t*>(a.q.ptr) + (int64_t)b * a.q.sb + (int64_t)h * a.q.sh;
  const uint16_t* kbp = reinterpret_cast<const uint16_t*>(a.k.ptr) + (int64_t)b * a.k.sb + (int64_t)hkv * a.k.sh;
  const uint16_t* vbp = reinterpret_cast<const uint16_t*>(a.v.ptr) + (int64_t)b * a.v.sb + (int64_t)hkv * a.v.sh;

  const int row = i * 128 + w * 32 + lq;
  bf16x8 qreg[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) qreg[ks] = as_bf16x8(ldg128(qb + (int64_t)row * a.q.ss + ks * 16 + hh * 8));

  const int64_t th = ((int64_t)b * a.Hq + h) * a.nqb + i;
  const float T = a.T[th];
  const int64_t mask_row = th * a.nqb;

  // K: 16 lanes per 256-byte row; V: lanes run over the 32 4-key groups of the tile so
  // the transposed LDS stores are conflict-free (two head-dim pieces per thread)
  const int c = t % PIECES, kk = t / PIECES;
  const int kv = t % 32, cv0 = t / 32;
  u32x4 kr[L], vr[2][4];
  auto load_k = [&](int key0) {
#pragma unroll
    for (int jj = 0; jj < L; ++jj) kr[jj] = ldg128(kbp + (int64_t)(key0 + kk * L + jj) * a.k.ss + c * 8);
  };
  auto load_v = [&](int key0) {
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
#pragma unroll
      for (int pp = 0; pp < 2; ++pp)
        vr[pp][jj] = ldg128(vbp + (int64_t)(key0 + kv * 4 + jj) * a.v.ss + (cv0 + pp * 8) * 8);
  };
  auto tile_of = [&](int n) { return n == 0 ? i : n - 1; };  // diagonal first

  float m_run = kNegInf, l_run = 0.f, le_run = 0.f;
  f32x16 oacc[D / 32];
#pragma unroll
  for (int x = 0; x < D / 32; ++x) oacc[x] = f32x16{};

  load_k(tile_of(0) * BN);
  for (int n = 0; n <= i; ++n) {
    const int j = tile_of(n);
    __syncthreads();
#pragma unroll
    for (int jj = 0; jj < L; ++jj) *reinterpret_cast<u32x4*>(Ks + (kk * L + jj) * TKS + c * 8) = kr[jj];
    __syncthreads();

    f32x16 s[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) s[kb] = st_block(Ks, kb * 32, qreg, lq, hh);
    const bool diag = j == i;
    if (diag) {
      const int rl = w * 32 + lq;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kl = kb * 32 + (r >> 2) * 8 + hh * 4 + (r & 3);
          if (kl > rl) s[kb][r] = kNegInf;
        }
    }
    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, shfl_xor_f(mx, off));
    if (l == 0) red[w] = mx;
    __syncthreads();
    const float tile_max = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3])) * a.scale;
    const bool keep = diag || tile_max >= T;
    if (t == 0) {
      if (a.keep) a.keep[mask_row + j] = keep ? 1 : 0;
      if (a.tmax) a.tmax[mask_row + j] = tile_max;
    }
    if (keep) {
      load_v(j * BN);
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) store_vt_group<VSTR>(Vt, vr[pp], kv * 4, cv0 + pp * 8);
      if (n < i) load_k(tile_of(n + 1) * BN);
      __syncthreads();
      softmax_pv64<VSTR>(s[0], s[1], Vt, 0, a.scale_log2, m_run, l_run, le_run, oacc, lq, hh);
      softmax_pv64<VSTR>(s[2], s[3], Vt, 64, a.scale_log2, m_run, l_run, le_run, oacc, lq, hh);
    } else {
      if (n < i) load_k(tile_of(n + 1) * BN);
    }
  }
  const int64_t ob = (int64_t)b * a.o.sb + (int64_t)row * a.o.ss + (int64_t)h * a.o.sh;
  write_row(a.o, ob, a.lse ? a.lse + ((int64_t)b * a.Hq + h) * a.S + row : nullptr, oacc, m_run, l_run, le_run, hh);
}

}  // namespace bsa
