// Backward of block-sparse attention: dQ, dK, dV of softmax attention restricted to the
// listed key blocks (the plain derivative of the forward; the "Sparse FlashAttention with
// Incremental Repair" README keeps FA's backward, the FSA and FlagAttention pages list
// forward + backward for their sparse kernels).  With S = scale Q K^T on the key set,
// P = softmax(S), O = P V and the upstream dO:
//   dV = P^T dO,  dP = dO V^T,  D = rowsum(dO * O),  dS = P * (dP - D),
//   dQ = scale dS K,  dK = scale dS^T Q.
// P is rebuilt from the forward's LSE: P = exp(S - LSE).
//
//   bwd_dot     D for every (b, h, row)
//   bwd_bits_* / bwd_list_count / bwd_scan / bwd_list_fill (block patterns): for every
//               sub-block of SB = 64 keys, the list of (query head, query block) pairs whose
//               key lists name it, in a fixed order
//   bwd_dkdv    one workgroup (four waves, two per 32-key group) per chunk of up to
//               kBwdChunk 32-row query slabs of a sub-block's list (a list every query block
//               names, like the first block of a causal pattern, is spread over many
//               workgroups; their float32 partials are summed in chunk order by bwd_reduce,
//               so the result does not depend on scheduling): K or V stays in registers,
//               32-row slabs of Q and dO stream into LDS (double-buffered direct loads) and are
//               shared by the waves; S = Q K^T and dP = dO V^T come out with a key per lane,
//               which makes P and dS directly the B operands of dV^T += dO^T P and
//               dK^T += Q^T dS (dO^T, Q^T read with the transposing LDS read)
//   bwd_dq      one workgroup per (b, head, query block): the forward's tile loop over the
//               listed keys (64-key K and V tiles, double-buffered direct loads), rebuilding
//               P^T and dP^T = V dO^T with a query per lane, then dQ^T += K^T dS^T
// No kernel accumulates with atomics: dK/dV belong to one workgroup, dQ to another.
#pragma once
#include <type_traits>
#include "tile.cuh"

namespace bsa {

__device__ __forceinline__ float bf16_lo(uint32_t x) { return bf16_bits_to_f32(x & 0xffffu); }
__device__ __forceinline__ float bf16_hi(uint32_t x) { return bf16_bits_to_f32(x >> 16); }

// LDS slot of the 16-byte pieces of a tile row that is read both ways: as MFMA row operands
// (16 consecutive rows, one piece each) and with the transposing read (4 consecutive rows,
// 4 pieces each).  Piece p of row R sits in slot p ^ bwd_swz(R): the swizzle is a bijection on
// R & 15 (row reads hit 16 different slots) whose top two bits are R & 3 (the four rows of a
// transposed read land in four different groups of four slots), so neither read conflicts.
__device__ __forceinline__ int bwd_swz(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }

// One sequence of the batch: its lengths and its first token (variable length: from the prefix
// sums; fixed length: b * Sq, b * Sk, the token index in the [B, S, ...] gradients).
struct BwdSeq {
  int q_len, k_len, q_tok, k_tok;
};
__device__ __forceinline__ BwdSeq bwd_seq(const BwdArgs& a, int b) {
  BwdSeq s;
  if (a.cu_q) {
    s.q_tok = a.cu_q[b];
    s.q_len = a.cu_q[b + 1] - s.q_tok;
    s.k_tok = a.cu_k[b];
    s.k_len = a.cu_k[b + 1] - s.k_tok;
  } else {
    s.q_len = a.Sq;
    s.k_len = a.Sk;
    s.q_tok = b * a.Sq;
    s.k_tok = b * a.Sk;
  }
  return s;
}
// Element offset of token `row` of sequence b in an input view: [B, S, H, D] strides, or the
// packed [total, H, D] layout (tok0 = the sequence's first token).
__device__ __forceinline__ int64_t bwd_row(const TensorArg& t, bool packed, int b, int tok0, int row) {
  return packed ? (int64_t)(tok0 + row) * t.ss : (int64_t)b * t.sb + (int64_t)row * t.ss;
}
// Index of (query head h, row) of sequence b in LSE-shaped arrays: [B, Hq, Sq] or [Hq, total_q].
__device__ __forceinline__ int64_t bwd_lse_idx(const BwdArgs& a, int b, const BwdSeq& s, int h, int row) {
  return a.cu_q ? (int64_t)h * a.cu_q[a.B] + s.q_tok + row : ((int64_t)b * a.Hq + h) * a.Sq + row;
}

// D = sum_d dO * O, and the LSE in log2 units with +inf for a row that has no keys (so that
// exp2(s - lse2) is 0 there without a test): 16 threads per row, 16 rows per workgroup.
__global__ __launch_bounds__(256) void bwd_dot_kernel(BwdArgs a) {
  const int64_t row = (int64_t)wg_x() * 16 + (tid_x() >> 4);  // (token, head), head fastest
  const int part = tid_x() & 15;
  const int64_t tokens = a.cu_q ? (int64_t)a.cu_q[a.B] : (int64_t)a.B * a.Sq;
  if (row >= tokens * a.Hq) return;  // whole 16-lane groups
  const int h = (int)(row % a.Hq);
  const int64_t tok = row / a.Hq;
  const int b = a.cu_q ? 0 : (int)(tok / a.Sq);
  const int s = a.cu_q ? 0 : (int)(tok % a.Sq);
  const int64_t dro = a.cu_q ? tok * a.dout.ss : (int64_t)b * a.dout.sb + (int64_t)s * a.dout.ss;
  const uint16_t* dp = reinterpret_cast<const uint16_t*>(a.dout.ptr) + dro + (int64_t)h * a.dout.sh + part * 8;
  const int64_t oo = (a.cu_q ? tok * a.o.ss : (int64_t)b * a.o.sb + (int64_t)s * a.o.ss) + (int64_t)h * a.o.sh +
                     part * 8;
  const u32x4 dv = ldg128(dp);
  float ov[8];
  if (a.o_f32) {
    const f32x4 o0 = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(a.o.ptr) + oo);
    const f32x4 o1 = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(a.o.ptr) + oo + 4);
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      ov[x] = o0[x];
      ov[4 + x] = o1[x];
    }
  } else {
    const u32x4 o = ldg128(reinterpret_cast<const uint16_t*>(a.o.ptr) + oo);
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      ov[2 * x] = bf16_lo(o[x]);
      ov[2 * x + 1] = bf16_hi(o[x]);
    }
  }
  float acc = 0.f;
#pragma unroll
  for (int x = 0; x < 4; ++x) acc += bf16_lo(dv[x]) * ov[2 * x] + bf16_hi(dv[x]) * ov[2 * x + 1];
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) acc += shfl_xor_f(acc, off);
  if (part == 0) {
    const int64_t at = a.cu_q ? (int64_t)h * tokens + tok : ((int64_t)b * a.Hq + h) * a.Sq + s;
    a.dsum[at] = acc;
    const float lv = a.lse[at];
    a.lse2[at] = lv == kNegInf ? kPosInf : lv * kLog2e;
  }
}

// ---- key-sub-block lists ----
// A list belongs to a sub-block of SB keys (SB never exceeds the pattern's key block, so
// every key of a sub-block has the same readers) and holds the (query head, query
// block) pairs whose key lists name its block.  Block patterns build the lists from a bitmap
// (bits[((b * Ht + ht) * nkb + j) * W + i / 32], bit i % 32: list (b, ht, i) names key block
// j) so that a list's order is fixed (by head, then query block) whatever order the bits were
// set in: dK and dV then sum their slabs in the same order on every run.

__global__ __launch_bounds__(256) void bwd_bits_zero_kernel(BwdArgs a) {
  const int64_t x = (int64_t)wg_x() * 256 + tid_x();
  const int Ht = a.list_by_kv ? a.Hkv : a.Hq;
  if (x < (int64_t)a.B * Ht * a.nkb * a.W) a.bits[x] = 0u;
}

// One thread per list entry slot (b, ht, i, c).
__global__ __launch_bounds__(256) void bwd_bits_set_kernel(BwdArgs a) {
  const int64_t x = (int64_t)wg_x() * 256 + tid_x();
  const int Ht = a.list_by_kv ? a.Hkv : a.Hq;
  const int cap = a.pat.cap;
  if (cap <= 0 || x >= (int64_t)a.B * Ht * a.nqb * cap) return;
  const int c = (int)(x % cap);
  const int64_t bi = x / cap;
  const int i = (int)(bi % a.nqb);
  const int64_t bh = bi / a.nqb;
  const int ht = (int)(bh % Ht), b = (int)(bh / Ht);
  const BwdSeq sq = bwd_seq(a, b);
  if ((int64_t)i * a.BM >= sq.q_len) return;  // lists past the sequence are never read
  const int64_t lb = (int64_t)b * a.pat.s_b + (int64_t)ht * a.pat.s_h + (int64_t)i * a.pat.s_q;
  if (c >= min(a.pat.count[lb], cap)) return;
  const int j = a.pat.index[lb * cap + c];
  if (j < 0 || j >= a.nkb || (int64_t)j * a.pat.block_N >= sq.k_len) return;
  atomicOr(&a.bits[(((int64_t)b * Ht + ht) * a.nkb + j) * a.W + (i >> 5)], 1u << (i & 31));
}

// One thread per list: its pair count.
__global__ __launch_bounds__(256) void bwd_list_count_kernel(BwdArgs a) {
  const int x = wg_x() * 256 + tid_x();
  if (x >= a.B * a.Hkv * a.nks) return;
  const int sub = x % a.nks, bh = x / a.nks;
  const int Ht = a.list_by_kv ? a.Hkv : a.Hq;
  const int hkv = bh % a.Hkv, b = bh / a.Hkv;
  const int j = sub * a.SB / a.pat.block_N;
  const int heads = a.list_by_kv ? 1 : a.G;
  int n = 0;
  for (int g = 0; g < heads; ++g) {
    const int ht = a.list_by_kv ? hkv : hkv * a.G + g;
    const uint32_t* col = a.bits + (((int64_t)b * Ht + ht) * a.nkb + j) * a.W;
    for (int wd = 0; wd < a.W; ++wd) n += __builtin_popcount(col[wd]);
  }
  a.counts[x] = a.list_by_kv ? n * a.G : n;
}

// A list entry: query head h and query block i as (h << kBwdEntryShift) | i, so that reading one
// back takes a shift and a mask (the host bounds the query blocks and heads to fit).
constexpr int kBwdEntryShift = 20;

// One wave per list: its pairs (h, i), from offsets[list] on, ordered by query head of
// the group, then query block (lists per kv head: each query block's G heads in turn).  Lane w
// takes bitmap word w (64 words at a time); a prefix sum over the wave of the words' entry
// counts gives each lane where its entries go.
__global__ __launch_bounds__(256) void bwd_list_fill_kernel(BwdArgs a) {
  const int x = wg_x() * 4 + (tid_x() >> 6);
  const int l = tid_x() & 63;
  if (x >= a.B * a.Hkv * a.nks) return;  // wave-uniform
  const int sub = x % a.nks, bh = x / a.nks;
  const int hkv = bh % a.Hkv, b = bh / a.Hkv;
  const int Ht = a.list_by_kv ? a.Hkv : a.Hq;
  const int j = sub * a.SB / a.pat.block_N;
  const int heads = a.list_by_kv ? 1 : a.G;
  const int per = a.list_by_kv ? a.G : 1;  // entries per set bit
  int32_t* out = a.entries + a.offsets[x];
  int base = 0;
  for (int g = 0; g < heads; ++g) {
    const int ht = a.list_by_kv ? hkv : hkv * a.G + g;
    const uint32_t* col = a.bits + (((int64_t)b * Ht + ht) * a.nkb + j) * a.W;
    for (int w0 = 0; w0 < a.W; w0 += 64) {
      const int wd = w0 + l;
      uint32_t m = wd < a.W ? col[wd] : 0u;
      const int c = __builtin_popcount(m) * per;
      int incl = c;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(incl, d, 64);
        if (l >= d) incl += y;
      }
      int k = base + incl - c;
      while (m) {
        const int i = wd * 32 + __builtin_ctz(m);
        m &= m - 1;
        if (a.list_by_kv) {
          for (int gg = 0; gg < a.G; ++gg) out[k++] = ((hkv * a.G + gg) << kBwdEntryShift) | i;
        } else {
          out[k++] = (ht << kBwdEntryShift) | i;
        }
      }
      base += __shfl(incl, 63, 64);
    }
  }
}

// First 32-row query slab that sees key0 (causal: some row r with r + delta >= key0, delta =
// the sequence's key length minus its query length).
__device__ __forceinline__ int bwd_first_slab(const BwdArgs& a, int key0, int delta) {
  return a.causal ? max(0, (key0 - delta) / 32) : 0;
}

// Dense patterns: the units of every list are (query head of the group, slab) pairs.
__global__ __launch_bounds__(256) void bwd_dense_count_kernel(BwdArgs a) {
  const int x = wg_x() * 256 + tid_x();
  if (x >= a.B * a.Hkv * a.nks) return;
  const BwdSeq sq = bwd_seq(a, x / (a.Hkv * a.nks));
  const int key0 = (x % a.nks) * a.SB;
  const int total_slabs = (sq.q_len + 31) / 32;
  a.counts[x] = key0 < sq.k_len ? a.G * max(0, total_slabs - bwd_first_slab(a, key0, sq.k_len - sq.q_len)) : 0;
}

__global__ __launch_bounds__(1024) void bwd_scan_kernel(BwdArgs a) {
  __shared__ int s_cnt[1024], s_chk[1024];
  const int n = a.B * a.Hkv * a.nks;
  const int t = tid_x();
  const bool block = a.pat.kind != 0;
  const int mult = block ? a.BM / 32 : 1;
  int carry = 0, carry_k = 0;
  for (int base = 0; base < n; base += 4096) {
    int c[4], k[4], sc = 0, sk = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int idx = base + t * 4 + u;
      c[u] = idx < n ? a.counts[idx] : 0;
      k[u] = (c[u] * mult + kBwdChunk - 1) / kBwdChunk;
      sc += c[u];
      sk += k[u];
    }
    s_cnt[t] = sc;
    s_chk[t] = sk;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
      const int v = t >= off ? s_cnt[t - off] : 0;
      const int vk = t >= off ? s_chk[t - off] : 0;
      __syncthreads();
      s_cnt[t] += v;
      s_chk[t] += vk;
      __syncthreads();
    }
    int ec = carry + s_cnt[t] - sc, ek = carry_k + s_chk[t] - sk;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int idx = base + t * 4 + u;
      if (idx < n) {
        if (block) a.offsets[idx] = ec;
        a.chunkp[idx] = ek;
      }
      ec += c[u];
      ek += k[u];
    }
    carry += s_cnt[1023];
    carry_k += s_chk[1023];
    __syncthreads();
  }
  if (t == 0) {
    if (block) a.offsets[n] = carry;
    a.chunkp[n] = carry_k;
  }
}

// dK/dV: one workgroup of four waves per chunk of up to kBwdChunk 32-row query slabs of a
// 64-key sub-block's list.  The work of each 32-key group is split over a pair of waves, so
// that a wave holds one operand tile and one accumulator set (168 registers: three waves per
// SIMD): wave 2g (the "P wave") keeps K of its group's keys, builds S^T = K Q^T and
// P = exp(S - LSE), hands P to its partner through LDS and accumulates dV^T += dO^T P; wave
// 2g + 1 (the "dS wave") keeps V, builds dP^T = V dO^T, takes P, forms dS = P * (dP - D) and
// accumulates dK^T += Q^T dS.
template <bool CAP>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void bwd_dkdv_kernel(BwdArgs a) {
  constexpr int D = TD;
  constexpr int SB = 64;
  constexpr int RS = D;  // 256-byte rows; 16-byte pieces swizzled by row (bwd_swz), as written by the DMA
  __shared__ __attribute__((aligned(16))) uint16_t Qs[2][32 * RS];
  __shared__ __attribute__((aligned(16))) uint16_t Ds[2][32 * RS];
  __shared__ __attribute__((aligned(16))) float ls[2][32];
  __shared__ __attribute__((aligned(16))) float dsm[2][32];
  __shared__ __attribute__((aligned(16))) float Ps[2][64 * 16];  // float32 P of each key group, lane layout
  __shared__ int ents_s[kBwdChunk / 2 + 2];                        // this chunk's list entries

  const int n_lists = a.B * a.Hkv * a.nks;
  const int wid = wg_x();
  if (wid >= a.chunkp[n_lists]) return;  // uniform: the grid is an upper bound
  // Neighbouring sub-blocks (lists 2p and 2p + 1) read mostly the same query slabs, in the same
  // order: their chunks are dealt in blocks of eight, list 2p's then list 2p + 1's, so that
  // chunk c of both lands on one XCD (workgroup ids 8 apart) at about the same time and the
  // second reads the slabs from that XCD's L2.
  int lo = 0, hi = (n_lists + 1) >> 1;  // pair with chunkp[2 lo] <= wid < chunkp[2 lo + 2]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (a.chunkp[2 * mid] <= wid) lo = mid;
    else hi = mid;
  }
  const int la = 2 * lo;
  const int n0 = a.chunkp[la + 1] - a.chunkp[la];
  const int n1 = la + 1 < n_lists ? a.chunkp[la + 2] - a.chunkp[la + 1] : 0;
  const int full = min(n0, n1) >> 3;
  int r = wid - a.chunkp[la], list, chunk;
  if (r < 16 * full) {
    list = la + ((r >> 3) & 1);
    chunk = (r >> 4) * 8 + (r & 7);
  } else {
    r -= 16 * full;
    const int ra = n0 - 8 * full;
    list = r < ra ? la : la + 1;
    chunk = 8 * full + (r < ra ? r : r - ra);
  }
  const int sub = list % a.nks;
  const int bh = list / a.nks;
  const int hkv = bh % a.Hkv, b = bh / a.Hkv;
  const int key0 = sub * SB;
  const int slot = a.chunkp[list] + chunk;  // this chunk's partial (bwd_reduce sums them in order)
  const bool split = a.chunkp[list + 1] - a.chunkp[list] > 1;
  const bool packed = a.cu_q != nullptr;
  const BwdSeq sq = bwd_seq(a, b);
  const int delta = sq.k_len - sq.q_len;
  const int t = tid_x();
  const int w = __builtin_amdgcn_readfirstlane(t >> 6), l = t & 63;
  const int kg = w >> 1;         // key group
  const bool ds_wave = w & 1;    // role (wave-uniform)
  const int lq = l & 31, hh = l >> 5;
  const int key = key0 + kg * 32 + lq;  // this lane's key
  // the rows that see it: [rlo, q_len) (causal: from the row of its diagonal on; none past the keys)
  const int rlo = key < sq.k_len ? (a.causal ? key - delta : 0) : INT_MAX;

  // K (P wave) or V (dS wave) rows of the group's keys: the B operand of S^T / dP^T
  const TensorArg& kv = ds_wave ? a.v : a.k;
  const uint16_t* kvbase =
      reinterpret_cast<const uint16_t*>(kv.ptr) + bwd_row(kv, packed, b, sq.k_tok, 0) + (int64_t)hkv * kv.sh;
  bf16x8 kvreg[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks)
    kvreg[ks] =
        as_bf16x8(key < sq.k_len ? ldg128(kvbase + (int64_t)key * kv.ss + ks * 16 + hh * 8) : u32x4{0, 0, 0, 0});
  int aoff[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) aoff[ks] = lq * RS + (((ks * 2 + hh) ^ bwd_swz(lq)) << 3);
  int trlo[D / 32], trhi[D / 32];
  {
    const int tg = l >> 4, tr = l & 15;
    const int rr = (tg >> 1) * 4 + (tr >> 2);
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int col = db * 32 + (tg & 1) * 16 + (tr & 3) * 4;
      trlo[db] = rr * RS + (((col >> 3) ^ bwd_swz(rr)) << 3) + (col & 7);
      trhi[db] = (rr + 8) * RS + (((col >> 3) ^ bwd_swz(rr + 8)) << 3) + (col & 7);
    }
  }
  f32x16 acc[D / 32];  // dV^T (P wave) or dK^T (dS wave)
#pragma unroll
  for (int x = 0; x < D / 32; ++x) acc[x] = f32x16{};

  const int slabs = a.BM / 32;       // 2 or 4
  const int slabs_log2 = a.BM == 128 ? 2 : 1;
  const int total_slabs = (sq.q_len + 31) / 32;
  const bool dense = a.pat.kind == 0;
  const int first_slab = dense ? bwd_first_slab(a, key0, delta) : 0;
  const int list0 = dense ? 0 : a.offsets[list];
  const int n_units = dense ? a.counts[list] : a.counts[list] * slabs;
  const int u0 = chunk * kBwdChunk, u1 = min(n_units, u0 + kBwdChunk);
  // The chunk's list entries (at most kBwdChunk / 2 + 1: an entry covers two or four slabs) are
  // staged in LDS, so that finding the next slab reads no global memory: the wait before each
  // slab's barrier would otherwise include that read.
  const int e0 = u0 >> slabs_log2;
  if (!dense) {
    const int ne = u1 > u0 ? ((u1 - 1) >> slabs_log2) - e0 + 1 : 0;
    for (int x = t; x < ne; x += 256) ents_s[x] = a.entries[list0 + e0 + x];
  }
  __syncthreads();
  auto next_unit = [&](int u, int& h, int& q0) __attribute__((always_inline)) -> int {
    for (; u < u1; ++u) {
      if (dense) {
        const int per = total_slabs - first_slab;
        h = hkv * a.G + u / per;
        q0 = (first_slab + u % per) * 32;
      } else {
        const int e = lds_int(ents_s, (u >> slabs_log2) - e0);
        h = e >> kBwdEntryShift;
        q0 = (e & ((1 << kBwdEntryShift) - 1)) * a.BM + (u & (slabs - 1)) * 32;
      }
      if (q0 < sq.q_len && !(a.causal && q0 + 31 + delta < key0)) return u;
    }
    return u1;
  };
  // this sequence's first Q / dO row, and its LSE-shaped rows: [B, Hq, Sq] or [Hq, total_q]
  const uint16_t* qseq = reinterpret_cast<const uint16_t*>(a.q.ptr) + bwd_row(a.q, packed, b, sq.q_tok, 0);
  const uint16_t* dseq = reinterpret_cast<const uint16_t*>(a.dout.ptr) + bwd_row(a.dout, packed, b, sq.q_tok, 0);
  const int64_t lse_hs = packed ? (int64_t)a.cu_q[a.B] : a.Sq;
  const int64_t lse_seq = packed ? (int64_t)sq.q_tok : (int64_t)b * a.Hq * a.Sq;
  // Q and dO rows q0 + 8w + 4x + l/16 of the slab (clamped to the last row: finite data the
  // mask then ignores), lane l into slot l%16; LSE (wave 0) and D (wave 1) one row per lane
  const int lrow = l >> 4, lslot = l & 15;
  // Q and dO rows go through buffer resources based at the slab's first row and covering its
  // rows inside the sequence: a row past the sequence reads zeros (finite, masked), and the
  // per-lane offsets are the same for every slab
  const uint32_t qrow = (uint32_t)a.q.ss * 2u, drow = (uint32_t)a.dout.ss * 2u;
  auto issue = [&](int h, int q0, uint16_t* __restrict__ nq, uint16_t* __restrict__ nd, float* __restrict__ nl,
                   float* __restrict__ nm) __attribute__((always_inline)) {
    const uint32_t last = (uint32_t)min(sq.q_len - 1 - q0, 31);
    const __amdgpu_buffer_rsrc_t rq = rows_rsrc(qseq + (int64_t)q0 * a.q.ss + (int64_t)h * a.q.sh, last * qrow + 256u);
    const __amdgpu_buffer_rsrc_t rd =
        rows_rsrc(dseq + (int64_t)q0 * a.dout.ss + (int64_t)h * a.dout.sh, last * drow + 256u);
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const uint32_t rl = (uint32_t)(w * 8 + x * 4 + lrow);
      const uint32_t piece = (uint32_t)((lslot ^ bwd_swz(rl)) << 4);
      buffer_load_lds16(rq, nq + (w * 8 + x * 4) * RS, rl * qrow + piece);
      buffer_load_lds16(rd, nd + (w * 8 + x * 4) * RS, rl * drow + piece);
    }
    if (w < 2 && l < 32) {  // LSE (log2 units, wave 0) and D (wave 1) of the 32 rows, one per lane (clamped)
      const int r = min(q0 + l, sq.q_len - 1);
      const float* src = (w == 0 ? a.lse2 : a.dsum) + lse_seq + (int64_t)h * lse_hs + r;
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const char*>(src), BSA_LDS(w == 0 ? nl : nm), 4, 0, 0);
    }
  };

  float* pslot = Ps[kg] + l * 4;  // four 16-byte quarters per lane, 1 KB apart (no bank conflicts)
  int h, q0;
  int u = next_unit(u0, h, q0);
  if (u < u1) issue(h, q0, Qs[0], Ds[0], ls[0], dsm[0]);
  // One slab from the current buffers while the next slab streams into the other ones.  The
  // restrict-qualified buffer parameters tell the compiler that those loads cannot alias the
  // reads of this slab, so it does not make the reads wait for them.
  auto step = [&](const uint16_t* __restrict__ Qb, const uint16_t* __restrict__ Db, const float* __restrict__ lb,
                  const float* __restrict__ mb, uint16_t* __restrict__ nq, uint16_t* __restrict__ nd,
                  float* __restrict__ nl, float* __restrict__ nm) __attribute__((always_inline)) {
    int hn = 0, q0n = 0;
    const int un = next_unit(u + 1, hn, q0n);
    // this slab's tiles are in LDS from every wave, every wave is done with the other buffer
    // and the dS waves have read the previous P
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (un < u1) issue(hn, q0n, nq, nd, nl, nm);  // the next slab streams in during this one
    const uint16_t* rows = ds_wave ? Db : Qb;   // A operand of S^T / dP^T
    const uint16_t* trans = ds_wave ? Qb : Db;  // transposed operand of dK^T / dV^T
    f32x16 x = {};
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
      x = mfma32x32x16(as_bf16x8(*reinterpret_cast<const u32x4*>(rows + aoff[ks])), kvreg[ks], x);
    // lane: key; register r: slab row 8(r/4) + 4hh + r%4
    uint32_t op[8];
    if (!ds_wave) {
      // P (and, with a softcap, what the dS wave multiplies by dP - D) for the slab; FULL: every
      // key of the group sees every row of the slab, so no element needs a test.  Two copies of
      // the code, picked once per slab (wave-uniform), keep the tests out of the common one.
      auto weights = [&](auto full_c) __attribute__((always_inline)) {
        constexpr bool FULL = decltype(full_c)::value;
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const f32x4 lv = *reinterpret_cast<const f32x4*>(lb + g4 * 8 + hh * 4);  // log2 units, +inf: no keys
          float p[4];
          float pf[4];  // what the dS wave multiplies by (dP - D): P, times the cap's derivative
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float xs = x[g4 * 4 + e];
            if constexpr (CAP) xs = softcap_score(xs, a.cap_in, a.cap_out);
            p[e] = exp2_fast(fmaf(xs, a.scale_log2, -lv[e]));
            if constexpr (!FULL) {
              const int row = q0 + g4 * 8 + hh * 4 + e;
              p[e] = row >= rlo && row < sq.q_len ? p[e] : 0.f;
            }
            if constexpr (CAP) {
              const float tc = xs / a.cap_out;  // tanh of the capped argument
              pf[e] = p[e] * (1.f - tc * tc);
            } else {
              pf[e] = p[e];
            }
          }
          op[g4 * 2] = pack_bf16x2(p[0], p[1]);
          op[g4 * 2 + 1] = pack_bf16x2(p[2], p[3]);
          // the dS wave's factor, unrounded
          *reinterpret_cast<f32x4*>(pslot + g4 * 256) = f32x4{pf[0], pf[1], pf[2], pf[3]};
        }
      };
      const int klast = key0 + kg * 32 + 31;
      // (with a softcap one copy, the tested one: two would not fit the registers)
      if (!CAP && klast < sq.k_len && q0 + 31 < sq.q_len && (!a.causal || klast <= q0 + delta))
        weights(std::true_type{});
      else
        weights(std::false_type{});
    }
    // P is in LDS for the dS waves.  The barrier waits for LDS operations only (a release
    // fence would also wait for the next slab's loads, which write LDS); the empty asm
    // statements with memory clobbers keep the compiler from moving LDS accesses across it.
    // (the dS wave takes dP - D first, while the P wave is still on P)
    if (ds_wave) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const f32x4 dm = *reinterpret_cast<const f32x4*>(mb + g4 * 8 + hh * 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) x[g4 * 4 + e] -= dm[e];
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (ds_wave) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const f32x4 pq = *reinterpret_cast<const f32x4*>(pslot + g4 * 256);
        op[g4 * 2] = pack_bf16x2(pq[0] * x[g4 * 4], pq[1] * x[g4 * 4 + 1]);
        op[g4 * 2 + 1] = pack_bf16x2(pq[2] * x[g4 * 4 + 2], pq[3] * x[g4 * 4 + 3]);
      }
    }
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const u32x4 ob = {op[hb * 4], op[hb * 4 + 1], op[hb * 4 + 2], op[hb * 4 + 3]};
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const u32x2 lo2 = ds_read_tr16(trans + hb * 16 * RS + trlo[db]);
        const u32x2 hi2 = ds_read_tr16(trans + hb * 16 * RS + trhi[db]);
        acc[db] = mfma32x32x16(as_bf16x8(u32x4{lo2[0], lo2[1], hi2[0], hi2[1]}), as_bf16x8(ob), acc[db]);
      }
    }
    u = un;
    h = hn;
    q0 = q0n;
  };
  int buf = 0;
  while (u < u1) {
    step(Qs[buf], Ds[buf], ls[buf], dsm[buf], Qs[buf ^ 1], Ds[buf ^ 1], ls[buf ^ 1], dsm[buf ^ 1]);
    buf ^= 1;
  }

    // one chunk: the gradient itself; several: a partial per chunk, summed by bwd_reduce
  const int which = ds_wave ? 0 : 1;  // 0 dK, 1 dV
  float* dst;
  float mul = 1.f;
  if (split) {
    dst = a.part + (((int64_t)slot * 2 + which) * SB + kg * 32 + lq) * D;
  } else {
    dst = (ds_wave ? a.dk : a.dv) + ((int64_t)(sq.k_tok + key) * a.Hkv + hkv) * D;
    if (ds_wave) mul = a.scale;
  }
  if (split || key < sq.k_len) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = db * 32 + g4 * 8 + hh * 4;
        *reinterpret_cast<f32x4*>(dst + d) = f32x4{acc[db][g4 * 4] * mul, acc[db][g4 * 4 + 1] * mul,
                                                   acc[db][g4 * 4 + 2] * mul, acc[db][g4 * 4 + 3] * mul};
      }
  }
}

constexpr int kBwdReduceKeys = 16;  // keys per reduction workgroup

// Lists not written by a single dK/dV workgroup: none (zeros) or several chunks (their
// partials summed in chunk order).  One workgroup per kBwdReduceKeys keys of a list (the first
// block's list has tens of chunks: a workgroup per list would leave its reduction alone at the
// end); each thread sums four independent outputs, so four partial reads are in flight.
__global__ __launch_bounds__(256) void bwd_reduce_kernel(BwdArgs a) {
  constexpr int D = TD;
  constexpr int KR = kBwdReduceKeys;
  static_assert(2 * KR * (D / 4) == 4 * 256, "four outputs per thread");
  const int groups = a.SB / KR;
  const int list = wg_x() / groups;
  const int kg0 = (wg_x() - list * groups) * KR;  // first key of this group within the sub-block
  const int c0 = a.chunkp[list], n = a.chunkp[list + 1] - c0;
  if (n == 1) return;  // written by its workgroup
  const int sub = list % a.nks;
  const int bh = list / a.nks;
  const int hkv = bh % a.Hkv, b = bh / a.Hkv;
  const BwdSeq sq = bwd_seq(a, b);
  const int SB = a.SB;
  const int64_t cstride = (int64_t)2 * SB * D;  // floats per chunk partial
  const float* src[4];
  float* dst[4];
  bool ok[4];
  float mul[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int x = tid_x() + j * 256;
    const int which = x / (KR * D / 4);  // 0 dK, 1 dV
    const int rem = x - which * (KR * D / 4);
    const int kr = kg0 + rem / (D / 4), d4 = rem % (D / 4);
    const int key = sub * SB + kr;
    ok[j] = key < sq.k_len;
    mul[j] = which == 0 ? a.scale : 1.f;
    src[j] = a.part + (((int64_t)c0 * 2 + which) * SB + kr) * D + d4 * 4;
    dst[j] = (which == 0 ? a.dk : a.dv) + ((int64_t)(sq.k_tok + (ok[j] ? key : 0)) * a.Hkv + hkv) * D + d4 * 4;
  }
  f32x4 acc[4] = {};
  for (int c = 0; c < n; ++c) {
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] += *reinterpret_cast<const f32x4*>(src[j] + c * cstride);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (ok[j]) *reinterpret_cast<f32x4*>(dst[j]) = acc[j] * mul[j];
}

template <int NW, bool CAP>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(NW == 4 ? 2 : 1))) void bwd_dq_kernel(BwdArgs a) {
  constexpr int D = TD;
  constexpr int RS = D;  // 256-byte rows, 16-byte pieces swizzled by row (bwd_swz)
  constexpr int RPW = 64 / NW;  // tile rows each wave loads
  __shared__ __attribute__((aligned(16))) uint16_t K0[64 * RS], K1[64 * RS];
  __shared__ __attribute__((aligned(16))) uint16_t V0[64 * RS], V1[64 * RS];
  __shared__ int sub_s[kBwdListLds];  // the first entries of this query block's list

  // (b, kv head, query block, group member), query blocks heaviest (last) first, contiguous
  // ranges per XCD: the G query heads of a kv head take the same query block side by side, so
  // the key blocks they share meet in one L2
  const int item = xcd_item(wg_x(), a.B * a.Hq * a.nqb);
  const int g = item % a.G;
  int rest = item / a.G;
  const int i = a.nqb - 1 - rest % a.nqb;
  rest /= a.nqb;
  const int hkv = rest % a.Hkv, b = rest / a.Hkv;
  const int h = hkv * a.G + g;
  const bool packed = a.cu_q != nullptr;
  const BwdSeq sq = bwd_seq(a, b);
  if ((int64_t)i * a.BM >= sq.q_len) return;  // uniform: query blocks past the sequence
  const int delta = sq.k_len - sq.q_len;
  const int t = tid_x();
  const int w = __builtin_amdgcn_readfirstlane(t >> 6), l = t & 63;
  const int lq = l & 31, hh = l >> 5;
  const int r0 = i * a.BM;
  const int row = r0 + w * 32 + lq;  // this lane's query
  const bool row_ok = row < sq.q_len;

  const int64_t qo = bwd_row(a.q, packed, b, sq.q_tok, row) + (int64_t)h * a.q.sh;
  const int64_t doo = bwd_row(a.dout, packed, b, sq.q_tok, row) + (int64_t)h * a.dout.sh;
  bf16x8 qreg[D / 16], doreg[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    qreg[ks] = as_bf16x8(row_ok ? ldg128(reinterpret_cast<const uint16_t*>(a.q.ptr) + qo + ks * 16 + hh * 8)
                                : u32x4{0, 0, 0, 0});
    doreg[ks] = as_bf16x8(row_ok ? ldg128(reinterpret_cast<const uint16_t*>(a.dout.ptr) + doo + ks * 16 + hh * 8)
                                 : u32x4{0, 0, 0, 0});
  }
  const int64_t rr = bwd_lse_idx(a, b, sq, h, row);
  const float lse2 = row_ok ? a.lse2[rr] : kPosInf;  // +inf: no keys, every weight 0
  const float dsv = row_ok ? a.dsum[rr] : 0.f;
  const int lim = !row_ok ? -1 : (a.causal ? min(row + delta, sq.k_len - 1) : sq.k_len - 1);
  // the last key every row of this wave sees (wave-uniform; -1 when a row is past the sequence)
  const int wrow = r0 + w * 32;
  const int lim_w = wrow + 31 < sq.q_len ? (a.causal ? min(wrow + delta, sq.k_len - 1) : sq.k_len - 1) : -1;
  int koff[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) koff[ks] = lq * RS + (((ks * 2 + hh) ^ bwd_swz(lq)) << 3);
  int trlo[D / 32], trhi[D / 32];
  {
    const int tg = l >> 4, tr = l & 15;
    const int r4 = (tg >> 1) * 4 + (tr >> 2);
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int col = db * 32 + (tg & 1) * 16 + (tr & 3) * 4;
      trlo[db] = r4 * RS + (((col >> 3) ^ bwd_swz(r4)) << 3) + (col & 7);
      trhi[db] = (r4 + 8) * RS + (((col >> 3) ^ bwd_swz(r4 + 8)) << 3) + (col & 7);
    }
  }
  f32x16 dq[D / 32];
#pragma unroll
  for (int x = 0; x < D / 32; ++x) dq[x] = f32x16{};

  // the 64-key sub-blocks to visit
  int n_sub, spe = 1;
  const int32_t* list = nullptr;
  const int last_row = min(r0 + a.BM, sq.q_len) - 1;
  if (a.pat.kind == 0) {
    const int kend = a.causal ? min(sq.k_len, last_row + delta + 1) : sq.k_len;
    n_sub = kend > 0 ? (kend + 63) / 64 : 0;
  } else {
    const int ht = a.list_by_kv ? hkv : h;
    const int64_t lb = (int64_t)b * a.pat.s_b + (int64_t)ht * a.pat.s_h + (int64_t)i * a.pat.s_q;
    list = a.pat.index + lb * a.pat.cap;
    spe = a.pat.block_N / 64;
    n_sub = a.pat.count[lb] * spe;
    // staged in LDS (entries past kBwdListLds are read from global memory), so that finding the
    // next key block reads no global memory before the barrier that waits for every load
    const int ne = min(a.pat.count[lb], kBwdListLds);
    for (int e = tid_x(); e < ne; e += NW * 64) sub_s[e] = list[e];
  }
  __syncthreads();
  auto next_sub = [&](int x, int& key0) __attribute__((always_inline)) -> int {
    for (; x < n_sub; ++x) {
      const int e = x / spe;
      key0 = (a.pat.kind == 0 ? x : (e < kBwdListLds ? lds_int(sub_s, e) : list[e]) * spe + x % spe) * 64;
      if (key0 >= 0 && key0 < sq.k_len && !(a.causal && key0 > last_row + delta)) return x;
    }
    return n_sub;
  };
  // K and V rows key0 + RPW w + 4x + l/16 (clamped to the last key: finite, masked), lane l
  // into slot l%16
  const int lrow = l >> 4, lslot = l & 15;
  const uint16_t* kbase =
      reinterpret_cast<const uint16_t*>(a.k.ptr) + bwd_row(a.k, packed, b, sq.k_tok, 0) + (int64_t)hkv * a.k.sh;
  const uint16_t* vbase =
      reinterpret_cast<const uint16_t*>(a.v.ptr) + bwd_row(a.v, packed, b, sq.k_tok, 0) + (int64_t)hkv * a.v.sh;
  // through buffer resources based at the block's first key and covering its keys inside the
  // sequence: a key past the sequence reads zeros (finite, masked), and the per-lane offsets
  // are the same for every block
  const uint32_t krow = (uint32_t)a.k.ss * 2u, vrow = (uint32_t)a.v.ss * 2u;
  auto issue = [&](int key0, uint16_t* __restrict__ nk, uint16_t* __restrict__ nv) __attribute__((always_inline)) {
    const uint32_t last = (uint32_t)min(sq.k_len - 1 - key0, 63);
    const __amdgpu_buffer_rsrc_t rk = rows_rsrc(kbase + (int64_t)key0 * a.k.ss, last * krow + 256u);
    const __amdgpu_buffer_rsrc_t rv = rows_rsrc(vbase + (int64_t)key0 * a.v.ss, last * vrow + 256u);
#pragma unroll
    for (int x = 0; x < RPW / 4; ++x) {
      const uint32_t rl = (uint32_t)(w * RPW + x * 4 + lrow);
      const uint32_t piece = (uint32_t)((lslot ^ bwd_swz(rl)) << 4);
      buffer_load_lds16(rk, nk + (w * RPW + x * 4) * RS, rl * krow + piece);
      buffer_load_lds16(rv, nv + (w * RPW + x * 4) * RS, rl * vrow + piece);
    }
  };

  int key0 = 0;
  int x = next_sub(0, key0);
  if (x < n_sub) issue(key0, K0, V0);
  // One key block from the current buffers while the next streams into the other ones (the
  // buffers are separate arrays, so the compiler sees that the two cannot alias and the reads
  // of this block do not wait for those loads).
  auto step = [&](const uint16_t* __restrict__ Kb, const uint16_t* __restrict__ Vb, uint16_t* __restrict__ nk,
                  uint16_t* __restrict__ nv) __attribute__((always_inline)) {
    int key0n = 0;
    const int xn = next_sub(x + 1, key0n);
    // this block's K and V are in LDS from every wave; every wave is done with the other buffer
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (xn < n_sub) issue(key0n, nk, nv);
    // every row of this wave sees all 64 keys: no per-element test (wave-uniform)
    const bool full = key0 + 63 <= lim_w;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 st = {}, dpt = {};
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const u32x4 ka = *reinterpret_cast<const u32x4*>(Kb + kb * 32 * RS + koff[ks]);
        const u32x4 va = *reinterpret_cast<const u32x4*>(Vb + kb * 32 * RS + koff[ks]);
        st = mfma32x32x16(as_bf16x8(ka), qreg[ks], st);
        dpt = mfma32x32x16(as_bf16x8(va), doreg[ks], dpt);
      }
      // lane: query; register r: key key0 + 32kb + 8(r/4) + 4hh + r%4.  FULL: every row of the
      // wave sees all 64 keys (wave-uniform), so no element needs a test
      uint32_t dd[8];
      auto weights = [&](auto full_c) __attribute__((always_inline)) {
        constexpr bool FULL = decltype(full_c)::value;
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          float d2[2];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            float xs = st[r + e];
            if constexpr (CAP) xs = softcap_score(xs, a.cap_in, a.cap_out);
            float p = exp2_fast(fmaf(xs, a.scale_log2, -lse2));
            if constexpr (!FULL) {
              const int kk = key0 + kb * 32 + ((r + e) >> 2) * 8 + hh * 4 + ((r + e) & 3);
              p = kk <= lim ? p : 0.f;
            }
            if constexpr (CAP) {
              const float tc = xs / a.cap_out;  // the cap's derivative: 1 - tanh^2
              p *= 1.f - tc * tc;
            }
            d2[e] = p * (dpt[r + e] - dsv);
          }
          dd[r / 2] = pack_bf16x2(d2[0], d2[1]);
        }
      };
      if (full) weights(std::true_type{});
      else weights(std::false_type{});
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        const u32x4 bop = {dd[hb * 4], dd[hb * 4 + 1], dd[hb * 4 + 2], dd[hb * 4 + 3]};
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const u32x2 lo = ds_read_tr16(Kb + (kb * 32 + hb * 16) * RS + trlo[db]);
          const u32x2 hi = ds_read_tr16(Kb + (kb * 32 + hb * 16) * RS + trhi[db]);
          dq[db] = mfma32x32x16(as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]}), as_bf16x8(bop), dq[db]);
        }
      }
    }
    x = xn;
    key0 = key0n;
  };
  int buf = 0;
  while (x < n_sub) {
    step(buf ? K1 : K0, buf ? V1 : V0, buf ? K0 : K1, buf ? V0 : V1);
    buf ^= 1;
  }
  if (row_ok) {
    float* dqp = a.dq + ((int64_t)(sq.q_tok + row) * a.Hq + h) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = db * 32 + g4 * 8 + hh * 4;
        *reinterpret_cast<f32x4*>(dqp + d) =
            f32x4{dq[db][g4 * 4] * a.scale, dq[db][g4 * 4 + 1] * a.scale, dq[db][g4 * 4 + 2] * a.scale,
                  dq[db][g4 * 4 + 3] * a.scale};
      }
  }
}

}  // namespace bsa
