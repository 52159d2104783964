// Selected attention, key-block-outer ("FSA: An Alternative Efficient Implementation of
// Native Sparse Attention Kernel", Abstract, and the Flash-Sparse-Attention README page,
// main features: a batched query-to-KV kernel, a reduction and an online-softmax pass, no
// atomics in the attention arithmetic).  Every query token selects up to topk key blocks
// of 64 keys per kv head (shared by the head's G query heads) and attends to their union.
//
// Instead of one workgroup per query (whose G rows would fill a 32-row MFMA tile poorly
// for small G), the selections are inverted into per-key-block token lists and one
// workgroup takes a key block and up to 128 / G of the tokens that selected it:
//   sel_zero   counts = 0
//   sel_count  count the valid (token, slot) pairs of every (b, kv head, key block),
//              through a per-tile LDS histogram; invalid slots (-1, past the sequence,
//              no causally visible key) get an empty partial (LSE -inf) right away
//   sel_scan   exclusive prefix sums of the counts (list offsets) and of the chunks
//              per list (ceil(count / (128 / G))), one workgroup
//   sel_fill   scatter t * topk + slot into the lists, one reservation per (tile, block)
//              (the order inside a list is not fixed; a row's result does not depend on
//              its place in the MFMA tile)
//   selected   one 64-key block per workgroup: K and V straight into swizzled LDS, the
//              gathered Q rows as the MFMA B operand, S^T = K Q^T, mask, softmax of the
//              64 scores, O^T = V^T P^T, one (o, lse) partial per (token, slot, head)
// and combine_kernel merges each token's topk partials (log-sum-exp).
#pragma once
#include "tile.cuh"

namespace bsa {

__device__ __forceinline__ void sel_lengths(const SelArgs& a, int b, int& q_len, int& kv_len, int& k_start) {
  if (a.cu_q) {
    q_len = a.cu_q[b + 1] - a.cu_q[b];
    k_start = a.cu_k[b];
    kv_len = a.cu_k[b + 1] - k_start;
  } else {
    q_len = a.Sq;
    kv_len = a.Sk;
    k_start = 0;
  }
}

// Partial row offsets: o in floats (row start), lse in floats.
__device__ __forceinline__ int64_t sel_part_o(const SelArgs& a, int slot, int b, int pos, int t, int h) {
  const int bc = a.cu_q ? 0 : b, pc = a.cu_q ? t : pos;
  return ((((int64_t)slot * a.Bc + bc) * a.Sc + pc) * a.Hq + h) * TD;
}
__device__ __forceinline__ int64_t sel_part_lse(const SelArgs& a, int slot, int b, int pos, int t, int h) {
  const int bc = a.cu_q ? 0 : b, pc = a.cu_q ? t : pos;
  return (((int64_t)slot * a.Bc + bc) * a.Hq + h) * a.Sc + pc;
}

__global__ __launch_bounds__(256) void sel_zero_kernel(SelArgs a) {
  const int x = wg_x() * 256 + tid_x();
  if (x < a.B * a.Hkv * a.nkb) a.counts[x] = 0;
}

// Count and fill work on tiles of kSelTile positions of one (sequence, kv head): the tile's
// selections are histogrammed over the key blocks in LDS first, so a block every token
// selects (the first one, the local ones) costs one global atomic per tile, not one per
// token.  Grid: (tiles per sequence, Hkv, B); tiles past a sequence's end exit.
__device__ __forceinline__ bool sel_tile(const SelArgs& a, int& b, int& hkv, int& p0, int& p1, int& q_len,
                                         int& kv_len, int& t0) {
  const int tile = __builtin_amdgcn_workgroup_id_x();
  hkv = __builtin_amdgcn_workgroup_id_y();
  b = __builtin_amdgcn_workgroup_id_z();
  int k_start;
  sel_lengths(a, b, q_len, kv_len, k_start);
  p0 = tile * kSelTile;
  p1 = min(q_len, p0 + kSelTile);
  t0 = a.cu_q ? a.cu_q[b] : b * a.Sq;
  return p0 < q_len;
}

// Key block of slot `slot` of the token at position pos, or -1 when it selects nothing the
// token can see.
__device__ __forceinline__ int sel_valid(const SelArgs& a, int j, int pos, int q_len, int kv_len) {
  if (j < 0 || (int64_t)j * 64 >= kv_len) return -1;
  if (a.causal && (int64_t)j * 64 > (int64_t)pos + (kv_len - q_len)) return -1;
  return j;
}

__global__ __launch_bounds__(256) void sel_count_kernel(SelArgs a) {
  __shared__ int hist[kSelMaxBlocks];
  int b, hkv, p0, p1, q_len, kv_len, t0;
  if (!sel_tile(a, b, hkv, p0, p1, q_len, kv_len, t0)) return;  // uniform
  const int tid = tid_x();
  const int nkb = (kv_len + 63) / 64;
  for (int x = tid; x < nkb; x += 256) hist[x] = 0;
  __syncthreads();
  const int n = (p1 - p0) * a.topk;
  for (int e = tid; e < n; e += 256) {
    const int pos = p0 + e / a.topk, slot = e % a.topk, t = t0 + pos;
    const int j = sel_valid(a, a.sel[((int64_t)t * a.Hkv + hkv) * a.topk + slot], pos, q_len, kv_len);
    if (j >= 0) {
      atomicAdd(&hist[j], 1);
    } else {
      // an empty partial: LSE -inf (the combine gives it weight 0 and never uses its o)
      for (int g = 0; g < a.G; ++g) a.part_lse[sel_part_lse(a, slot, b, pos, t, hkv * a.G + g)] = kNegInf;
    }
  }
  __syncthreads();
  int* counts = a.counts + ((int64_t)b * a.Hkv + hkv) * a.nkb;
  for (int x = tid; x < nkb; x += 256)
    if (hist[x]) atomicAdd(&counts[x], hist[x]);
}

// One workgroup of 1024 threads, four entries per thread per pass.
__global__ __launch_bounds__(1024) void sel_scan_kernel(SelArgs a) {
  __shared__ int s_cnt[1024], s_chk[1024];
  const int n = a.B * a.Hkv * a.nkb;
  const int t = tid_x();
  int carry_c = 0, carry_k = 0;
  for (int base = 0; base < n; base += 4096) {
    int c[4], k[4], sc = 0, sk = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int idx = base + t * 4 + u;
      c[u] = idx < n ? a.counts[idx] : 0;
      k[u] = (c[u] + a.tpc - 1) / a.tpc;
      sc += c[u];
      sk += k[u];
    }
    s_cnt[t] = sc;
    s_chk[t] = sk;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
      const int vc = t >= off ? s_cnt[t - off] : 0;
      const int vk = t >= off ? s_chk[t - off] : 0;
      __syncthreads();
      s_cnt[t] += vc;
      s_chk[t] += vk;
      __syncthreads();
    }
    int ec = carry_c + s_cnt[t] - sc, ek = carry_k + s_chk[t] - sk;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int idx = base + t * 4 + u;
      if (idx < n) {
        a.offsets[idx] = ec;
        a.cursor[idx] = ec;
        a.chunkp[idx] = ek;
      }
      ec += c[u];
      ek += k[u];
    }
    carry_c += s_cnt[1023];
    carry_k += s_chk[1023];
    __syncthreads();  // s_cnt / s_chk are rewritten by the next pass
  }
  if (t == 0) {
    a.offsets[n] = carry_c;
    a.chunkp[n] = carry_k;
  }
}

// The tile's histogram again, then one global reservation per block and the entries
// placed by their LDS rank inside it.
__global__ __launch_bounds__(256) void sel_fill_kernel(SelArgs a) {
  __shared__ int hist[kSelMaxBlocks];
  int b, hkv, p0, p1, q_len, kv_len, t0;
  if (!sel_tile(a, b, hkv, p0, p1, q_len, kv_len, t0)) return;  // uniform
  const int tid = tid_x();
  const int nkb = (kv_len + 63) / 64;
  for (int x = tid; x < nkb; x += 256) hist[x] = 0;
  __syncthreads();
  const int n = (p1 - p0) * a.topk;
  for (int e = tid; e < n; e += 256) {
    const int pos = p0 + e / a.topk, slot = e % a.topk, t = t0 + pos;
    const int j = sel_valid(a, a.sel[((int64_t)t * a.Hkv + hkv) * a.topk + slot], pos, q_len, kv_len);
    if (j >= 0) atomicAdd(&hist[j], 1);
  }
  __syncthreads();
  int* cursor = a.cursor + ((int64_t)b * a.Hkv + hkv) * a.nkb;
  for (int x = tid; x < nkb; x += 256)
    if (hist[x]) hist[x] = atomicAdd(&cursor[x], hist[x]);  // first list position of this tile's run
  __syncthreads();
  for (int e = tid; e < n; e += 256) {
    const int pos = p0 + e / a.topk, slot = e % a.topk, t = t0 + pos;
    const int j = sel_valid(a, a.sel[((int64_t)t * a.Hkv + hkv) * a.topk + slot], pos, q_len, kv_len);
    if (j >= 0) a.entries[atomicAdd(&hist[j], 1)] = t * a.topk + slot;
  }
}

// Workgroup: 4 waves x 32 rows; row r is (token r / G of the chunk, group member r % G).
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void selected_kernel(SelArgs a) {
  constexpr int D = TD;
  constexpr int RS = D;
  constexpr int NB = 2;  // 32-key blocks of the 64-key tile
  __shared__ __attribute__((aligned(16))) uint16_t Kt[64 * RS];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[64 * RS];

  const int n_lists = a.B * a.Hkv * a.nkb;
  const int wg = wg_x();
  if (wg >= a.chunkp[n_lists]) return;  // uniform: the grid is an upper bound
  int lo = 0, hi = n_lists;  // list with chunkp[lo] <= wg < chunkp[lo + 1]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (a.chunkp[mid] <= wg) lo = mid;
    else hi = mid;
  }
  const int list = lo;
  const int j = list % a.nkb;
  const int bh = list / a.nkb;
  const int hkv = bh % a.Hkv, b = bh / a.Hkv;
  const int e0 = a.offsets[list] + (wg - a.chunkp[list]) * a.tpc;
  const int n_tok = min(a.offsets[list + 1] - e0, a.tpc);
  int q_len, kv_len, k_start;
  sel_lengths(a, b, q_len, kv_len, k_start);
  const int q_start = a.cu_q ? a.cu_q[b] : 0;
  const int delta = kv_len - q_len;

  const int t = tid_x();
  const int w = __builtin_amdgcn_readfirstlane(t >> 6), l = t & 63;
  const int lq = l & 31, hh = l >> 5;

  // this lane's query row
  const int r = w * 32 + lq;
  const int it = r / a.G, g = r - it * a.G;
  const bool row_ok = it < n_tok;
  int tok = 0, slot = 0, pos = 0;
  if (row_ok) {
    const int e = a.entries[e0 + it];
    tok = e / a.topk;
    slot = e - tok * a.topk;
    pos = a.cu_q ? tok - q_start : tok - b * a.Sq;
  }
  const int h = hkv * a.G + g;
  const uint16_t* qrow = reinterpret_cast<const uint16_t*>(a.q.ptr) +
                         (a.cu_q ? (int64_t)tok * a.q.ss : (int64_t)b * a.q.sb + (int64_t)pos * a.q.ss) +
                         (int64_t)h * a.q.sh;

  // K and V rows j*64 .. j*64+63 of the sequence: wave w fills rows 16w..16w+15 with four
  // 1 KB instructions (rows 16w + 4x + l/16, lane l into slot l%16); keys past the end
  // load row 0 and are masked
  const uint16_t* kbp = reinterpret_cast<const uint16_t*>(a.k.ptr) +
                        (a.cu_q ? (int64_t)k_start * a.k.ss : (int64_t)b * a.k.sb) + (int64_t)hkv * a.k.sh;
  const uint16_t* vbp = reinterpret_cast<const uint16_t*>(a.v.ptr) +
                        (a.cu_q ? (int64_t)k_start * a.v.ss : (int64_t)b * a.v.sb) + (int64_t)hkv * a.v.sh;
  const int lrow = l >> 4, lslot = l & 15;
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    const int row = w * 16 + x * 4 + lrow;  // row & 15 = 4x + lrow
    int key = j * 64 + row;
    key = key < kv_len ? key : 0;
    const char* kp = reinterpret_cast<const char*>(kbp + (int64_t)key * a.k.ss);
    const char* vp = reinterpret_cast<const char*>(vbp + (int64_t)key * a.v.ss);
    __builtin_amdgcn_global_load_lds(kp + ((lslot ^ k_swz(row)) << 4), BSA_LDS(Kt + (w * 4 + x) * 4 * RS), 16, 0, 0);
    __builtin_amdgcn_global_load_lds(vp + ((lslot ^ v_swz(row)) << 4), BSA_LDS(Vt + (w * 4 + x) * 4 * RS), 16, 0, 0);
  }

  // Every lane loads: a lane without a row reads row 0 of its sequence (a valid address,
  // finite values), and its row is never written (each query row's scores, weights and output
  // stay in its own lane column).  With a branch around each load, or a select on the loaded
  // values, the compiler waited for the loads in flight, the K and V tile included, halfway
  // through issuing them.
  bf16x8 qreg[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) qreg[ks] = as_bf16x8(ldg128(qrow + ks * 16 + hh * 8));
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
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  f32x16 s[NB];
#pragma unroll
  for (int kb = 0; kb < NB; ++kb) s[kb] = f32x16{};
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    u32x4 av[NB];
#pragma unroll
    for (int kb = 0; kb < NB; ++kb) av[kb] = *reinterpret_cast<const u32x4*>(Kt + kb * 32 * RS + koff[ks]);
#pragma unroll
    for (int kb = 0; kb < NB; ++kb) s[kb] = mfma32x32x16(as_bf16x8(av[kb]), qreg[ks], s[kb]);
  }
  softcap_n<NB>(s, a.cap_in, a.cap_out);
  // keys past the sequence, after the row's diagonal (causal), and every key of an empty row
  const int lim = !row_ok ? -1 : (a.causal ? min(pos + delta, kv_len - 1) : kv_len - 1);
#pragma unroll
  for (int kb = 0; kb < NB; ++kb)
#pragma unroll
    for (int rg = 0; rg < 16; ++rg) {
      const int key = j * 64 + kb * 32 + (rg >> 2) * 8 + hh * 4 + (rg & 3);
      if (key > lim) s[kb][rg] = kNegInf;
    }
  float m_run = kNegInf, l_run = 0.f;
  f32x16 oacc[D / 32];
#pragma unroll
  for (int x = 0; x < D / 32; ++x) oacc[x] = f32x16{};
  softmax_max_n<NB>(s, a.scale_log2, m_run, l_run, oacc);
  const float m_use = m_run == kNegInf ? 0.f : m_run;
  float psum = 0.f;
#pragma unroll
  for (int kb = 0; kb < NB; ++kb) {
    uint32_t pk[8];
#pragma unroll
    for (int rg = 0; rg < 16; rg += 4) {
      const float p0 = exp2_fast(fmaf(s[kb][rg], a.scale_log2, -m_use));
      const float p1 = exp2_fast(fmaf(s[kb][rg + 1], a.scale_log2, -m_use));
      const float p2 = exp2_fast(fmaf(s[kb][rg + 2], a.scale_log2, -m_use));
      const float p3 = exp2_fast(fmaf(s[kb][rg + 3], a.scale_log2, -m_use));
      pk[rg / 2] = pack_bf16x2(p0, p1);
      pk[rg / 2 + 1] = pack_bf16x2(p2, p3);
      psum += (p0 + p1) + (p2 + p3);
    }
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const int ks = kb * 2 + hb;
      const u32x4 pb = {pk[hb * 4], pk[hb * 4 + 1], pk[hb * 4 + 2], pk[hb * 4 + 3]};
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const u32x2 vlo = ds_read_tr16(Vt + ks * 16 * RS + voff[db]);
        const u32x2 vhi = ds_read_tr16(Vt + (ks * 16 + 8) * RS + voff[db]);
        oacc[db] = mfma32x32x16(as_bf16x8(u32x4{vlo[0], vlo[1], vhi[0], vhi[1]}), as_bf16x8(pb), oacc[db]);
      }
    }
  }
  l_run += psum;
  if (row_ok) {
    const OutArg po{a.part_o, 0, 0, 0, 1};
    write_row(po, sel_part_o(a, slot, b, pos, tok, h), a.part_lse + sel_part_lse(a, slot, b, pos, tok, h), oacc,
              m_run, l_run, hh);
  }
}

}  // namespace bsa
