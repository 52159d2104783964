// Prefill kernel with large key chunks: NW waves of 32 query rows (BM = 32 NW),
// chunks of CK = 32 NW keys (128 keys for 128-row tiles, 64 for 64-row tiles)
// made of 64-key segments of the key list, one K and one V tile in LDS.
//
// Same operation as prefill_pipe_kernel for final outputs ("Sparse
// FlashAttention with Incremental Repair", Usage 1; "Implementation: Sgl
// project Sglang Sparse Flash Attention", I/O Contract, for vertical-slash
// windows and columns; dense when no pattern is given).  A segment is 64
// consecutive keys (a dense range, half of a 128-key block or window, a
// 64-key block or window) or up to 64 gathered vertical columns; chunk c holds
// segments NS c .. NS c + NS - 1 (NS = NW/2), wave w loading the 32 rows
// 32w..32w+31 of the chunk, which lie in segment w/2.
//
// Per chunk (as the gated kernel, whose 128-key tiles use the MFMA units
// better than 64-key chunks: the per-iteration latencies are paid once per
// twice the work):
//   [K_c in LDS, V tile free] issue V_c -> S_c (8 MFMAs per 32-key block, V_c
//   streaming in) -> masks, row max -> wait, barrier (V_c visible, K_c free)
//   -> issue K_{c+1} -> softmax + PV_c (K_{c+1} streaming in) -> wait, barrier.
// LDS: 2 x CK x 256 bytes (64 KB for 128-row tiles, two workgroups per CU;
// 32 KB for 64-row tiles, four per CU), rows swizzled as in tile.cuh.
#pragma once
#include "tile.cuh"

namespace bsa {

template <int KIND, int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2))) void prefill_tile_kernel(PrefillArgs a) {
  static_assert(NW == 2 || NW == 4, "64- or 128-row tiles");
  constexpr int D = TD;
  constexpr int NT = NW * 64;
  constexpr int BM = 32 * NW;
  constexpr int CK = 32 * NW;  // keys per chunk
  constexpr int NS = CK / 64;  // 64-key segments per chunk
  constexpr int NB = CK / 32;  // 32-key S blocks per chunk
  constexpr int RS = D;
  __shared__ __attribute__((aligned(16))) uint16_t Kt[CK * RS];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[CK * RS];
  constexpr int kKid = KIND == 2 ? CK : 4;
  __shared__ __attribute__((aligned(16))) int kid_s[kKid];
  constexpr int kEnts = 256;
  constexpr int kCols = KIND == 2 ? 768 : 1;
  __shared__ int ents_s[kEnts];
  __shared__ int cols_s[kCols];

  const int item = KIND == 2 ? head_sync_item(wg_x(), a.nqb, a.n_items) : xcd_item(wg_x(), a.n_items);
  // (b, kv head, query block, group member): the G query heads that share a kv head run
  // the same query block side by side, so the key blocks they visit meet in L2
  const int g = item % a.G;
  int rest = item / a.G;
  const int mrev = rest % a.nqb;
  rest /= a.nqb;
  const int hkv = rest % a.Hkv;
  const int b = rest / a.Hkv;
  const int h = hkv * a.G + g;
  const int m = a.nqb - 1 - mrev;

  int q_start = 0, q_len = a.Sq, k_start = 0, kv_len = a.Sk;
  if (a.cu_q) {
    q_start = a.cu_q[b];
    q_len = a.cu_q[b + 1] - q_start;
    k_start = a.cu_k[b];
    kv_len = a.cu_k[b + 1] - k_start;
  }
  const int r0 = m * BM;
  if (r0 >= q_len) return;  // uniform: no barrier has run yet
  const int delta = kv_len - q_len;
  const int r_last = min(r0 + BM, q_len) - 1;

  const int t = tid_x();
  const int w = __builtin_amdgcn_readfirstlane(t >> 6), l = t & 63;
  const int lq = l & 31, hh = l >> 5;

  const uint16_t* qb = reinterpret_cast<const uint16_t*>(a.q.ptr) +
                       (a.cu_q ? (int64_t)q_start * a.q.ss : (int64_t)b * a.q.sb) + (int64_t)h * a.q.sh;
  const uint16_t* kbp = reinterpret_cast<const uint16_t*>(a.k.ptr) +
                        (a.cu_q ? (int64_t)k_start * a.k.ss : (int64_t)b * a.k.sb) + (int64_t)hkv * a.k.sh;
  const uint16_t* vbp = reinterpret_cast<const uint16_t*>(a.v.ptr) +
                        (a.cu_q ? (int64_t)k_start * a.v.ss : (int64_t)b * a.v.sb) + (int64_t)hkv * a.v.sh;

  const int row = r0 + w * 32 + lq;
  const bool row_ok = row < q_len;
  bf16x8 qreg[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    const u32x4 v = row_ok ? ldg128(qb + (int64_t)row * a.q.ss + ks * 16 + hh * 8) : u32x4{0, 0, 0, 0};
    qreg[ks] = as_bf16x8(v);
  }

  // ---- segment list (64-key segments) ----
  // spe: segments per list entry; nws: window segments (vertical-slash)
  int n_seg = 0, spe = 1, nws = 0, ncol = 0, n_ent = 0;
  const int32_t* list = nullptr;
  const int32_t* cols = nullptr;
  if constexpr (KIND == 0) {
    int kend = kv_len;
    if (a.causal) kend = min(kv_len, r_last + delta + 1);
    n_seg = kend > 0 ? (kend + 63) / 64 : 0;
  } else {
    const int ht = a.list_by_kv ? hkv : h;
    const int64_t lb = (int64_t)b * a.pat.s_b + (int64_t)ht * a.pat.s_h + (int64_t)m * a.pat.s_q;
    n_ent = a.pat.count[lb];
    list = a.pat.index + lb * a.pat.cap;
    spe = a.pat.block_N / 64;
    if constexpr (KIND == 1) {
      n_seg = n_ent * spe;
    } else {
      nws = n_ent * spe;
      ncol = a.pat.col_count[lb];
      cols = a.pat.col_index + lb * a.pat.col_cap;
      n_seg = nws + (ncol + 63) / 64;
    }
  }
  if (kv_len <= 0) n_seg = 0;
  const int n_chunks = (n_seg + NS - 1) / NS;
  if constexpr (KIND != 0) {
    const int nl = min(n_ent, kEnts);
    for (int x = t; x < nl; x += NT) ents_s[x] = list[x];
    if constexpr (KIND == 2) {
      const int nc = min(ncol, kCols);
      for (int x = t; x < nc; x += NT) cols_s[x] = cols[x];
    }
  }

  // A segment: 64 consecutive keys from key0, or up to 64 gathered columns from gbase;
  // absent past the end of the list.  Fields are wave-uniform (scalar registers).
  struct Seg {
    int key0 = 0, gbase = 0;
    bool valid = false, gathered = false, full = false;  // full: all 64 keys inside [0, kv_len)
  };
  auto seg_at = [&](int si, bool staged) -> Seg {
    Seg r;
    if (si >= n_seg) return r;
    r.valid = true;
    if constexpr (KIND == 0) {
      r.key0 = si * 64;
    } else {
      if (KIND == 1 || si < nws) {
        const int e = si / spe;
        const int id = __builtin_amdgcn_readfirstlane(staged && e < kEnts ? lds_int(ents_s, e) : global_int(list, e));
        r.key0 = (KIND == 1 ? id * a.pat.block_N : id) + (si - e * spe) * 64;
      } else {
        r.gathered = true;
        r.gbase = (si - nws) * 64;
      }
    }
    r.full = !r.gathered && r.key0 >= 0 && r.key0 <= kv_len - 64;
    return r;
  };
  // segment-local key i -> key index within the sequence, or -1 when absent
  auto key_of = [&](int i, const Seg& r, bool staged) -> int {
    if (!r.valid) return -1;
    int key;
    if (r.gathered) {
      const int x = r.gbase + i;
      if (x >= ncol) return -1;
      key = (staged && x < kCols) ? lds_int(cols_s, x) : global_int(cols, x);
    } else {
      key = r.key0 + i;
    }
    return (unsigned)key < (unsigned)kv_len ? key : -1;
  };

  // Direct loads: wave w fills chunk rows 32w..32w+31 (segment w/2, segment rows
  // 32(w%2)..+31) with eight 1 KB instructions, rows 32w + 4x + l/16, lane l into slot l%16
  // (R & 15 = 4(x & 3) + l/16).  Contiguous segments go through a buffer resource based at
  // the wave's first row, sized to the rows inside [0, kv_len): rows past the sequence, or a
  // whole absent segment, read zeros (finite, masked out later), with no per-lane test.
  // Gathered columns keep per-lane global addresses (their keys can lie anywhere).
  const int lrow = l >> 4, lslot = l & 15;
  const int srow0 = (w & 1) * 32;  // first row of this wave within its segment
  const uint32_t kx = (uint32_t)(lslot ^ lrow) << 4;
  const uint32_t vx = (uint32_t)(lslot ^ (lrow << 2)) << 4;
  const uint32_t k_lane = (uint32_t)(lrow * a.k.ss) * 2u, v_lane = (uint32_t)(lrow * a.v.ss) * 2u + vx;
  auto issue = [&](uint16_t* tile, const uint16_t* src, int64_t ss, bool is_k, const Seg& r, bool staged)
                   __attribute__((always_inline)) {
    if (!r.gathered) {
      const int row0 = r.key0 + srow0;
      const int nrows = (r.valid && row0 >= 0) ? min(kv_len - row0, 32) : 0;
      const uint32_t row_bytes = (uint32_t)ss * 2u;
      const __amdgpu_buffer_rsrc_t rs =
          rows_rsrc(src + (int64_t)max(row0, 0) * ss, nrows > 0 ? (uint32_t)(nrows - 1) * row_bytes + 256u : 0u);
#pragma unroll
      for (int x = 0; x < 8; ++x)
        buffer_load_lds16(rs, tile + (w * 8 + x) * 4 * RS,
                          (uint32_t)(x * 4) * row_bytes + (is_k ? k_lane + (kx ^ ((x & 3) << 6)) : v_lane));
    } else if constexpr (KIND == 2) {
      // all eight keys first, then the loads: a key read from memory is waited for once, not
      // once per load (each wait would also wait for the loads already in flight)
      int keys[8];
      if (staged && r.gbase + 64 <= kCols) {  // gathered, indices staged in LDS
#pragma unroll
        for (int x = 0; x < 8; ++x) {
          const int xi = r.gbase + srow0 + x * 4 + lrow;
          const int key = xi < ncol ? cols_s[xi] : -1;
          keys[x] = r.valid && (unsigned)key < (unsigned)kv_len ? key : 0;
        }
      } else {
#pragma unroll
        for (int x = 0; x < 8; ++x) keys[x] = max(0, key_of(srow0 + x * 4 + lrow, r, staged));
      }
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        const char* p = reinterpret_cast<const char*>(src + (int64_t)keys[x] * ss);
        __builtin_amdgcn_global_load_lds(p + (is_k ? (kx ^ ((x & 3) << 6)) : vx), BSA_LDS(tile + (w * 8 + x) * 4 * RS),
                                         16, 0, 0);
      }
    }
  };
  // gathered segments record their key indices for the mask (lanes of waves 2s, 2s+1)
  auto record_kid = [&](const Seg& r, bool staged) __attribute__((always_inline)) {
    if constexpr (KIND == 2) {
      if (r.gathered && l < 32) {
        const int key = key_of(srow0 + l, r, staged);
        kid_s[w * 32 + l] = key >= 0 ? key : 0x7fffffff;
      }
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

  // -inf for absent keys and, when causal, keys after the row's diagonal: per 32-key block,
  // the block's segment decides (contiguous: arithmetic on key0; gathered: recorded indices)
  const int wrow_min = r0 + w * 32;
  auto mask_block = [&](f32x16& s, int kb, const Seg& r) __attribute__((always_inline)) {
    const int lim = a.causal ? row + delta : 0x7ffffffe;
    const int half = (kb & 1) * 32;  // key offset of the block within its segment
    if (r.gathered) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int4 k4 = *reinterpret_cast<const int4*>(kid_s + kb * 32 + q4 * 8 + hh * 4);
        if (k4.x > lim) s[q4 * 4 + 0] = kNegInf;
        if (k4.y > lim) s[q4 * 4 + 1] = kNegInf;
        if (k4.z > lim) s[q4 * 4 + 2] = kNegInf;
        if (k4.w > lim) s[q4 * 4 + 3] = kNegInf;
      }
      return;
    }
    const bool need = !r.full || (a.causal && r.key0 + half + 31 > wrow_min + delta);
    if (!need) return;
    // key0 + half + kl is present and visible iff lo <= kl <= hi
    const int hi = r.valid ? min(lim, kv_len - 1) - r.key0 - half : -1;
    const int lo = -r.key0 - half;
#pragma unroll
    for (int rg = 0; rg < 16; ++rg) {
      const int kl = (rg >> 2) * 8 + hh * 4 + (rg & 3);
      if (kl > hi || kl < lo) s[rg] = kNegInf;
    }
  };

  // ---- chunk loop ----
  Seg cur[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) cur[s] = seg_at(s, false);
  // this wave's segment of the current chunk
  auto my_seg = [&](const Seg* c) -> Seg { return (NS == 1 || w < 2) ? c[0] : c[NS - 1]; };
  if (n_chunks > 0) {
    record_kid(my_seg(cur), false);
    issue(Kt, kbp, a.k.ss, true, my_seg(cur), false);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int c = 0; c < n_chunks; ++c) {
    const bool more = c + 1 < n_chunks;
    // V_c streams in while S_c is computed
    issue(Vt, vbp, a.v.ss, false, my_seg(cur), c > 0);
    // S_c: the NB key blocks advance together through the head dimension, so each K
    // operand read has the other blocks' MFMAs to hide behind
    f32x16 s[NB];
#pragma unroll
    for (int kb = 0; kb < NB; ++kb) s[kb] = f32x16{};
    // K operands double-buffered: the reads of step ks + 1 are issued before the products of
    // step ks, so each read has a whole step of products to land behind
    u32x4 av[2][NB];
#pragma unroll
    for (int kb = 0; kb < NB; ++kb) av[0][kb] = *reinterpret_cast<const u32x4*>(Kt + kb * 32 * RS + koff[0]);
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      if (ks + 1 < D / 16) {
#pragma unroll
        for (int kb = 0; kb < NB; ++kb)
          av[(ks + 1) & 1][kb] = *reinterpret_cast<const u32x4*>(Kt + kb * 32 * RS + koff[ks + 1]);
      }
      __builtin_amdgcn_sched_barrier(0);  // keep the order: reads of step ks + 1, then products of step ks
#pragma unroll
      for (int kb = 0; kb < NB; ++kb) s[kb] = mfma32x32x16(as_bf16x8(av[ks & 1][kb]), qreg[ks], s[kb]);
      __builtin_amdgcn_sched_barrier(0);
    }
    softcap_n<NB>(s, a.cap_in, a.cap_out);
#pragma unroll
    for (int kb = 0; kb < NB; ++kb) mask_block(s[kb], kb, cur[kb >> 1]);
    softmax_max_n<NB>(s, a.scale_log2, m_run, l_run, oacc);
    // V_c is in LDS from every wave, and every wave is done reading K_c (and the indices)
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    Seg nxt[NS];
    if (more) {
#pragma unroll
      for (int x = 0; x < NS; ++x) nxt[x] = seg_at((c + 1) * NS + x, true);
      // the key indices first: one read past the staged ones is waited for, and that wait
      // would also wait for loads issued before it
      record_kid(my_seg(nxt), true);
      issue(Kt, kbp, a.k.ss, true, my_seg(nxt), true);
    }
    // softmax weights and PV; the V^T operands of the first two 16-key steps are read
    // before the exponentials
    u32x4 vpre[2][D / 32];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const u32x2 lo = ds_read_tr16(Vt + ks * 16 * RS + voff[db]);
        const u32x2 hi = ds_read_tr16(Vt + (ks * 16 + 8) * RS + voff[db]);
        vpre[ks][db] = u32x4{lo[0], lo[1], hi[0], hi[1]};
      }
    const float m_use = m_run == kNegInf ? 0.f : m_run;
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < NB; ++kb) {
      uint32_t pk[8];
#pragma unroll
      for (int r = 0; r < 16; r += 4) {
        const float p0 = exp2_fast(fmaf(s[kb][r], a.scale_log2, -m_use));
        const float p1 = exp2_fast(fmaf(s[kb][r + 1], a.scale_log2, -m_use));
        const float p2 = exp2_fast(fmaf(s[kb][r + 2], a.scale_log2, -m_use));
        const float p3 = exp2_fast(fmaf(s[kb][r + 3], a.scale_log2, -m_use));
        pk[r / 2] = pack_bf16x2(p0, p1);
        pk[r / 2 + 1] = pack_bf16x2(p2, p3);
        psum += (p0 + p1) + (p2 + p3);
      }
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        const int ks = kb * 2 + hb;
        const u32x4 pb = {pk[hb * 4], pk[hb * 4 + 1], pk[hb * 4 + 2], pk[hb * 4 + 3]};
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          u32x4 av;
          if (ks < 2) {
            av = vpre[ks < 2 ? ks : 0][db];
          } else {
            const u32x2 lo = ds_read_tr16(Vt + ks * 16 * RS + voff[db]);
            const u32x2 hi = ds_read_tr16(Vt + (ks * 16 + 8) * RS + voff[db]);
            av = u32x4{lo[0], lo[1], hi[0], hi[1]};
          }
          oacc[db] = mfma32x32x16(as_bf16x8(av), as_bf16x8(pb), oacc[db]);
        }
      }
    }
    l_run += psum;
    if (more) {
      // K_{c+1} is in LDS and every wave is done reading V_c
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
#pragma unroll
      for (int x = 0; x < NS; ++x) cur[x] = nxt[x];
    }
  }

  if (row_ok) {
    const int64_t ob = (a.cu_q ? (int64_t)(q_start + row) * a.o.ss : (int64_t)b * a.o.sb + (int64_t)row * a.o.ss) +
                       (int64_t)h * a.o.sh;
    float* lp = nullptr;
    if (a.lse) lp = a.lse + (a.cu_q ? (int64_t)h * a.cu_q[a.B] + q_start + row : ((int64_t)b * a.Hq + h) * a.Sq + row);
    write_row(a.o, ob, lp, oacc, m_run, l_run, hh);
  }
}

}  // namespace bsa
