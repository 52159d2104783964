// BSFA gated causal attention ("Block Sparse Flash Attention", Abstract and
// Figure 2).  For query block i the kernel visits key blocks j <= i (the
// diagonal first, so the running maximum starts high), computes the 128x128
// score tile S_ij with MFMA, takes its exact maximum t(i,j) (lane max, wave
// shuffle reduce, one LDS exchange between the four waves) and keeps the tile
// iff j == i or scale * t(i,j) >= T[b, h, i].  Only kept tiles load V_j and
// run the P V product; V of a skipped tile is never requested.  The figure
// leaves open what a skipped tile's scores do to the softmax, so both readings
// run: by default they never enter it (the result is attention over the kept
// tiles); with count_skipped they still update the running maximum and the
// normalisers (only the V_j load and the product are skipped).
//
// Workgroup: 4 waves x 32 query rows (BM = 128), 128-key tiles.  K and V go
// straight from global memory into LDS (global_load_lds_dwordx4, the swizzled
// row layouts of tile.cuh); two 32 KB tile buffers, two workgroups per CU; the
// V^T MFMA operand is read with ds_read_b64_tr_b16.  Per tile, with K_j in
// buffer X and the other buffer Y free:
//   issue K_next into Y -> S_ij (8 MFMAs per 32-key block), diagonal mask, tile max
//   -> LDS exchange + bare barrier (every wave is done with K_j; K_next stays in flight)
//   -> keep decision -> kept tiles: issue V_j into X, softmax update and P, wait,
//      barrier, PV; skipped tiles: (count_skipped: softmax update)
//   -> wait for K_next, barrier; X and Y trade roles,
// so the next K tile streams in during the whole of tile j, kept or skipped, and V_j
// during the softmax.  The calibration pass loads no V: it keeps one buffer and requests
// K_next after the barrier.  Grid remapped XCD-aware, heaviest query blocks first.
#pragma once
#include <type_traits>

#include "tile.cuh"

namespace bsa {

// CALIB: the threshold-calibration pass — the same S tiles and tile maxima, written to
// a.tmax, with no tile kept: no V load, no P V product and no output.
// COUNT: a skipped tile's scores still update the running maximum and the normalisers
// (a separate instantiation, so the default one keeps its register allocation).
template <bool CALIB, bool COUNT>
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
  auto issue_k = [&](int key0, uint16_t* buf) __attribute__((always_inline)) {
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      const char* p = reinterpret_cast<const char*>(kbp + (int64_t)(key0 + w * 32 + x * 4) * a.k.ss);
      __builtin_amdgcn_global_load_lds(p + (k_lane + (kx ^ ((x & 3) << 6))), BSA_LDS(buf + (w * 8 + x) * 4 * RS), 16,
                                       0, 0);
    }
  };
  auto issue_v = [&](int key0, uint16_t* buf) __attribute__((always_inline)) {
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      const char* p = reinterpret_cast<const char*>(vbp + (int64_t)(key0 + w * 32 + x * 4) * a.v.ss);
      __builtin_amdgcn_global_load_lds(p + v_lane, BSA_LDS(buf + (w * 8 + x) * 4 * RS), 16, 0, 0);
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

  float m_run = kNegInf, l_run = 0.f;
  f32x16 oacc[D / 32];
#pragma unroll
  for (int x = 0; x < D / 32; ++x) oacc[x] = f32x16{};

  auto tile_of = [&](int n) { return n == 0 ? i : n - 1; };  // diagonal first

  // Online softmax over one tile: the running maximum (lazy rescale), the weights packed to
  // bf16 as the P^T operand, and the sum of the float32 weights (the normaliser).
  auto weights = [&](const f32x16* sc, float row_max, uint32_t (*pk)[8], float& psum) __attribute__((always_inline)) {
    softmax_rescale(row_max * a.scale_log2, m_run, l_run, oacc);
    const float m_use = m_run == kNegInf ? 0.f : m_run;
    psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < NB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; r += 4) {
        const float p0 = exp2_fast(fmaf(sc[kb][r], a.scale_log2, -m_use));
        const float p1 = exp2_fast(fmaf(sc[kb][r + 1], a.scale_log2, -m_use));
        const float p2 = exp2_fast(fmaf(sc[kb][r + 2], a.scale_log2, -m_use));
        const float p3 = exp2_fast(fmaf(sc[kb][r + 3], a.scale_log2, -m_use));
        pk[kb][r / 2] = pack_bf16x2(p0, p1);
        pk[kb][r / 2 + 1] = pack_bf16x2(p2, p3);
        psum += (p0 + p1) + (p2 + p3);
      }
  };
  // O^T += V_j^T P^T, the V^T operands read with the transposing LDS read one 16-key step
  // ahead of their products (read just before, every product waited for its own reads).  The
  // counting reading keeps the reads next to their products: it has no registers to spare.
  auto pv = [&](const uint32_t (*pk)[8], const uint16_t* Vb) __attribute__((always_inline)) {
    constexpr int NKS = NB * 2;
    if constexpr (COUNT) {
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const int kb = ks >> 1, hb = ks & 1;
        const u32x4 pb = {pk[kb][hb * 4], pk[kb][hb * 4 + 1], pk[kb][hb * 4 + 2], pk[kb][hb * 4 + 3]};
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const u32x2 lo = ds_read_tr16(Vb + ks * 16 * RS + voff[db]);
          const u32x2 hi = ds_read_tr16(Vb + (ks * 16 + 8) * RS + voff[db]);
          oacc[db] = mfma32x32x16(as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]}), as_bf16x8(pb), oacc[db]);
        }
      }
      return;
    }
    u32x4 vb[2][D / 32];
    auto read_v = [&](int ks, u32x4* dst) __attribute__((always_inline)) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const u32x2 lo = ds_read_tr16(Vb + ks * 16 * RS + voff[db]);
        const u32x2 hi = ds_read_tr16(Vb + (ks * 16 + 8) * RS + voff[db]);
        dst[db] = u32x4{lo[0], lo[1], hi[0], hi[1]};
      }
    };
    read_v(0, vb[0]);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      if (ks + 1 < NKS) read_v(ks + 1, vb[(ks + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
      const int kb = ks >> 1, hb = ks & 1;
      const u32x4 pb = {pk[kb][hb * 4], pk[kb][hb * 4 + 1], pk[kb][hb * 4 + 2], pk[kb][hb * 4 + 3]};
#pragma unroll
      for (int db = 0; db < D / 32; ++db) oacc[db] = mfma32x32x16(as_bf16x8(vb[ks & 1][db]), as_bf16x8(pb), oacc[db]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  issue_k(tile_of(0) * BN, Kt);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  // One tile; the two tile buffers trade roles from tile to tile (P, the parity, is a
  // compile-time constant so that every LDS access names its array).  K_n sits in X; K_next
  // goes into Y at once and streams in during S_n, the exchange, the softmax and P V_n.
  auto step = [&](int n, auto par) __attribute__((always_inline)) {
    constexpr bool P = decltype(par)::value;
    uint16_t* const X = P ? Vt : Kt;
    uint16_t* const Y = CALIB ? Kt : P ? Kt : Vt;
    const int j = tile_of(n);
    const bool more = n < i;
    // (the calibration pass loads no V: it keeps one buffer and requests K_next after the
    // barrier below, once every wave is done with K_j.  Under 128 registers it runs four waves
    // per SIMD, which hide the load; the two-buffer loop would cost it that)
    if (!CALIB && more) issue_k(tile_of(n + 1) * BN, Y);
    // S_j: the NB key blocks advance together through the head dimension, the K operands of
    // step ks + 1 read before the products of step ks, so each read has a step of products
    // to land behind (one block at a time, every product waited for its own read).  The
    // calibration pass keeps one block at a time: its registers leave room for a fourth wave
    // per SIMD, which hides the reads instead.
    f32x16 s[NB];
#pragma unroll
    for (int kb = 0; kb < NB; ++kb) s[kb] = f32x16{};
    if constexpr (CALIB) {
#pragma unroll
      for (int kb = 0; kb < NB; ++kb)
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks)
          s[kb] = mfma32x32x16(as_bf16x8(*reinterpret_cast<const u32x4*>(X + kb * 32 * RS + koff[ks])), qreg[ks],
                               s[kb]);
    } else {
      u32x4 av[2][NB];
#pragma unroll
      for (int kb = 0; kb < NB; ++kb) av[0][kb] = *reinterpret_cast<const u32x4*>(X + kb * 32 * RS + koff[0]);
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        if (ks + 1 < D / 16) {
#pragma unroll
          for (int kb = 0; kb < NB; ++kb)
            av[(ks + 1) & 1][kb] = *reinterpret_cast<const u32x4*>(X + kb * 32 * RS + koff[ks + 1]);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kb = 0; kb < NB; ++kb) s[kb] = mfma32x32x16(as_bf16x8(av[ks & 1][kb]), qreg[ks], s[kb]);
        __builtin_amdgcn_sched_barrier(0);
      }
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
    // the row maximum (the softmax's) on the way to the wave's maximum (the tile's)
    const float row_max = row_max_n<NB>(s);
    float mx = row_max;
#pragma unroll
    for (int off = 16; off >= 1; off >>= 1) mx = fmaxf(mx, shfl_xor_f(mx, off));
    if (l == 0) red[w] = mx;
    // every wave's maximum is in LDS and every wave is done reading K_j.  A bare barrier
    // after the wait for LDS: the fence of __syncthreads would also wait for K_next.  The
    // empty asm statements with memory clobbers keep LDS accesses on their side of it.
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (CALIB && more) issue_k(tile_of(n + 1) * BN, Y);
    const float tile_max = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3])) * a.scale;
    const bool keep = !CALIB && (diag || tile_max >= T);
    if (t == 0) {
      if (a.keep) a.keep[mask_row + j] = keep ? 1 : 0;
      if (a.tmax) a.tmax[mask_row + j] = tile_max;
    }
    if constexpr (!CALIB) {
      // V_j goes where K_j was; it streams in during the softmax update
      if (keep) issue_v(j * BN, X);
      if (keep || COUNT) {
        uint32_t pk[NB][8];
        float psum;
        weights(s, row_max, pk, psum);
        l_run += psum;
        if (keep) {
          // V_j from every wave is in LDS
          __builtin_amdgcn_s_waitcnt(0);
          __syncthreads();
          pv(pk, X);
        }
      }
    }
    if (more) {
      // K_next is in LDS and every wave is done reading X, which takes K after next
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
  };
  if constexpr (CALIB) {
    for (int n = 0; n <= i; ++n) step(n, std::integral_constant<bool, false>{});
  } else {
    for (int n = 0;; n += 2) {
      step(n, std::integral_constant<bool, false>{});
      if (n + 1 > i) break;
      step(n + 1, std::integral_constant<bool, true>{});
      if (n + 2 > i) break;
    }
  }
  if constexpr (!CALIB) {
    const int64_t ob = (int64_t)b * a.o.sb + (int64_t)row * a.o.ss + (int64_t)h * a.o.sh;
    write_row(a.o, ob, a.lse ? a.lse + ((int64_t)b * a.Hq + h) * a.S + row : nullptr, oacc, m_run, l_run, hh);
  }
}

}  // namespace bsa
