// BSFA gated causal attention ("Block Sparse Flash Attention", Abstract and
// Figure 2).  For query block i the kernel visits key blocks j <= i (the
// diagonal first, so the running maximum starts high), computes the 128x128
// score tile S_ij with MFMA, takes its exact maximum t(i,j) (lane max, wave
// shuffle reduce, one LDS exchange between the four waves) and keeps the tile
// iff j == i or scale * t(i,j) >= T[b, h, i].  Only kept tiles load V_j and
// run the softmax update and P V product; a skipped tile's scores never enter
// the softmax and its V is never requested.
//
// Workgroup: 4 waves x 32 query rows (BM = 128), 128-key tiles.  K and V go
// straight from global memory into LDS (global_load_lds_dwordx4, the swizzled
// row layouts of tile.cuh; 32 KB each, two workgroups per CU); the V^T MFMA
// operand is read with ds_read_b64_tr_b16.  Per tile:
//   [K_j resident] S_ij (8 MFMAs per 32-key block), diagonal mask, tile max
//   -> LDS exchange + barrier (every wave is done with K_j) -> keep decision
//   -> kept tiles: issue V_j, softmax update and P, wait, barrier, issue K_next, PV;
//      skipped tiles: issue K_next -> wait for K_next -> barrier,
// so V_j streams in during the softmax and the next K tile during the PV product (kept
// tiles) or right after the decision (skipped tiles).  (A workgroup-scope barrier waits for
// every outstanding load, so K_next is issued after the V barrier, not
// before it.)  Grid remapped XCD-aware, heaviest query blocks first.
#pragma once
#include "tile.cuh"

namespace bsa {

// CALIB: the threshold-calibration pass — the same S tiles and tile maxima, written to
// a.tmax, with no tile kept: no V load, no P V product and no output.
template <bool CALIB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void gated_kernel(GatedArgs a) {
  constexpr int D = TD;
  constexpr int BN = 128;
  constexpr int RS = D;  // packed 256-byte LDS rows, swizzled
  constexpr int NB = BN / 32;
  __shared__ __attribute__((aligned(16))) uint16_t Kt[BN * RS];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[BN * RS];
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
  const int w = __builtin_amdgcn_readfirstlane(t >> 6), l = t & 63;
  const int lq = l & 31, hh = l >> 5;

  const uint16_t* qb = reinterpret_cast<const uint16_t*>(a.q.ptr) + (int64_t)b * a.q.sb + (int64_t)h * a.q.sh;
  const uint16_t* kbp = reinterpret_cast<const uint16_t*>(a.k.ptr) + (int64_t)b * a.k.sb + (int64_t)hkv * a.k.sh;
  const uint16_t* vbp = reinterpret_cast<const uint16_t*>(a.v.ptr) + (int64_t)b * a.v.sb + (int64_t)hkv * a.v.sh;

  const int row = i * 128 + w * 32 + lq;
  bf16x8 qreg[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) qreg[ks] = as_bf16x8(ldg128(qb + (int64_t)row * a.q.ss + ks * 16 + hh * 8));

  const int64_t th = ((int64_t)b * a.Hq + h) * a.nqb + i;
  const float T = CALIB ? 0.f : a.T[th];
  const int64_t mask_row = th * a.nqb;

  // Direct loads: wave w fills rows 32w..32w+31 of a tile with eight 1 KB instructions
  // (rows 32w + 4x + l/16, lane l into slot l%16; R & 15 = 4(x & 3) + l/16).  Key tiles of a
  // causal self-attention are always complete, so every row address is wave-uniform.
  const int lrow = l >> 4, lslot = l & 15;
  const uint32_t kx = (uint32_t)(lslot ^ lrow) << 4;
  const uint32_t vx = (uint32_t)(lslot ^ (lrow << 2)) << 4;
  const uint32_t k_lane = (uint32_t)(lrow * a.k.ss) * 2u, v_lane = (uint32_t)(lrow * a.v.ss) * 2u + vx;
  auto issue_k = [&](int key0) __attribute__((always_inline)) {
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      const char* p = reinterpret_cast<const char*>(kbp + (int64_t)(key0 + w * 32 + x * 4) * a.k.ss);
      __builtin_amdgcn_global_load_lds(p + (k_lane + (kx ^ ((x & 3) << 6))), BSA_LDS(Kt + (w * 8 + x) * 4 * RS), 16,
                                       0, 0);
    }
  };
  auto issue_v = [&](int key0) __attribute__((always_inline)) {
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      const char* p = reinterpret_cast<const char*>(vbp + (int64_t)(key0 + w * 32 + x * 4) * a.v.ss);
      __builtin_amdgcn_global_load_lds(p + v_lane, BSA_LDS(Vt + (w * 8 + x) * 4 * RS), 16, 0, 0);
    }
  };

  // per-lane LDS offsets of the MFMA operands
  int koff[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) koff[ks] = lq * RS + (((ks * 2 + hh) ^ k_swz(lq)) << 3);
  const int tg = l >> 4, tr = l & 15;
  const int vrow = (tg >> 1) * 4 + (tr >> 2);
  int voff[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    const int col = db * 32 + (tg & 1) * 16 + (tr & 3) * 4;
    voff[db] = vrow * RS + (((col >> 3) ^ v_swz(vrow)) << 3) + (col & 7);
  }

  float m_run = kNegInf, l_run = 0.f, le_run = 0.f;
  f32x16 oacc[D / 32];
#pragma unroll
  for (int x = 0; x < D / 32; ++x) oacc[x] = f32x16{};

  auto tile_of = [&](int n) { return n == 0 ? i : n - 1; };  // diagonal first

  issue_k(tile_of(0) * BN);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int n = 0; n <= i; ++n) {
    const int j = tile_of(n);
    f32x16 s[NB];
#pragma unroll
    for (int kb = 0; kb < NB; ++kb) {
      f32x16 acc = {};
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const u32x4 av = *reinterpret_cast<const u32x4*>(Kt + kb * 32 * RS + koff[ks]);
        acc = mfma32x32x16(as_bf16x8(av), qreg[ks], acc);
      }
      s[kb] = acc;
    }
    const bool diag = j == i;
    if (diag) {
      const int rl = w * 32 + lq;
#pragma unroll
      for (int kb = 0; kb < NB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kl = kb * 32 + (r >> 2) * 8 + hh * 4 + (r & 3);
          if (kl > rl) s[kb][r] = kNegInf;
        }
    }
    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < NB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, shfl_xor_f(mx, off));
    if (l == 0) red[w] = mx;
    // every wave's maximum is in LDS and every wave is done reading K_j
    __syncthreads();
    const float tile_max = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3])) * a.scale;
    const bool keep = !CALIB && (diag || tile_max >= T);
    if (t == 0) {
      if (a.keep) a.keep[mask_row + j] = keep ? 1 : 0;
      if (a.tmax) a.tmax[mask_row + j] = tile_max;
    }
    const bool more = n < i;
    if (keep) {
      issue_v(j * BN);
      // the softmax update and P run while V_j streams in
      softmax_max_n<NB>(s, a.scale_log2, m_run, l_run, le_run, oacc);
      const float m_use = m_run == kNegInf ? 0.f : m_run;
      float psum = 0.f, pesum = 0.f;
      uint32_t pk[NB][8];
#pragma unroll
      for (int kb = 0; kb < NB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; r += 4) {
          const float p0 = exp2_fast(fmaf(s[kb][r], a.scale_log2, -m_use));
          const float p1 = exp2_fast(fmaf(s[kb][r + 1], a.scale_log2, -m_use));
          const float p2 = exp2_fast(fmaf(s[kb][r + 2], a.scale_log2, -m_use));
          const float p3 = exp2_fast(fmaf(s[kb][r + 3], a.scale_log2, -m_use));
          pk[kb][r / 2] = pack_bf16x2(p0, p1);
          pk[kb][r / 2 + 1] = pack_bf16x2(p2, p3);
          psum = bf16x2_sum_acc(pk[kb][r / 2], psum);
          psum = bf16x2_sum_acc(pk[kb][r / 2 + 1], psum);
          pesum += (p0 + p1) + (p2 + p3);
        }
      __builtin_amdgcn_s_waitcnt(0);
      // V_j from every wave is in LDS; K_next streams in during the P V product
      __syncthreads();
      if (more) issue_k(tile_of(n + 1) * BN);
#pragma unroll
      for (int kb = 0; kb < NB; ++kb)
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
          const int ks = kb * 2 + hb;
          const u32x4 pb = {pk[kb][hb * 4], pk[kb][hb * 4 + 1], pk[kb][hb * 4 + 2], pk[kb][hb * 4 + 3]};
#pragma unroll
          for (int db = 0; db < D / 32; ++db) {
            const u32x2 lo = ds_read_tr16(Vt + ks * 16 * RS + voff[db]);
            const u32x2 hi = ds_read_tr16(Vt + (ks * 16 + 8) * RS + voff[db]);
            oacc[db] = mfma32x32x16(as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]}), as_bf16x8(pb), oacc[db]);
          }
        }
      l_run += psum;
      le_run += pesum;
    } else if (more) {
      issue_k(tile_of(n + 1) * BN);
    }
    if (more) {
      // K_next is in LDS and every wave is done reading V_j
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
  }
  if constexpr (!CALIB) {
    const int64_t ob = (int64_t)b * a.o.sb + (int64_t)row * a.o.ss + (int64_t)h * a.o.sh;
    write_row(a.o, ob, a.lse ? a.lse + ((int64_t)b * a.Hq + h) * a.S + row : nullptr, oacc, m_run, l_run, le_run,
              hh);
  }
}

}  // namespace bsa
