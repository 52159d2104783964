// Prefill kernel: a tile of query rows per workgroup, keys gathered in 64-key
// chunks from a pattern.
//
// Attention restricted to listed keys ("Sparse FlashAttention with
// Incremental Repair", Usage 1 for block lists and Usage 3 for partials;
// "Implementation: Sgl project Sglang Sparse Flash Attention", I/O Contract,
// for vertical-slash block offsets and column indices; dense when no pattern
// is given).  One workgroup owns BM = 32*NW query rows of one (sequence,
// query head); wave w owns rows 32w..32w+31.  Each 64-key chunk is either 64
// consecutive keys (a dense range, half or all of a listed block, or a
// vertical-slash window at any offset) or up to 64 gathered vertical columns.
//
// Per chunk:
//   load   every thread fetches 16-byte pieces of K and V rows (coalesced:
//          16 lanes per 256-byte row); the next chunk's loads are issued
//          before this chunk's MFMAs (register double buffer)
//   LDS    K row-major, V transposed in registers (layouts in tile.cuh)
//   S^T    = K Q^T with v_mfma_f32_32x32x16_bf16, Q^T held in registers
//   softmax online in base 2, scale*log2(e) folded into one FMA; the running
//          max only moves (rescaling O) when it grows by more than 2^8
//   O^T   += V^T P^T, P rounded to bf16
//
// Grid: one workgroup per (b, h_q, query block), remapped so that each XCD
// takes a contiguous range ordered (b, h_kv, h_q, query block descending):
// workgroups sharing a key/value head share an L2, and the longest causal
// rows start first.
#pragma once
#include "tile.cuh"

namespace bsa {


template <int NW, int KIND>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2))) void prefill_kernel(PrefillArgs a) {
  constexpr int D = TD;
  constexpr int NT = NW * 64;
  constexpr int BM = NW * 32;
  constexpr int PIECES = D / 8;
  constexpr int L = 64 * PIECES / NT;  // consecutive keys per thread: 4 (NW=4) or 8 (NW=2)
  static_assert(L % 4 == 0, "each thread must own whole 4-key groups");
  constexpr int VSTR = 64 + 8;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[64 * TKS];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[D * VSTR];
  __shared__ __attribute__((aligned(16))) int kidx_s[64];
  // list entries (block ids or window offsets) and gathered column indices staged in LDS,
  // so a chunk's addresses never wait on a dependent global load
  constexpr int kEnts = 256;
  constexpr int kCols = KIND == 2 ? 768 : 1;
  __shared__ int ents_s[kEnts];
  __shared__ int cols_s[kCols];

  const int item = xcd_item(wg_x(), a.n_items);
  const int mrev = item % a.nqb;
  int rest = item / a.nqb;
  const int g = rest % a.G;
  rest /= a.G;
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

  const int w = tid_x() >> 6, l = tid_x() & 63;
  const int lq = l & 31, hh = l >> 5;

  const int64_t qoff = a.cu_q ? (int64_t)q_start * a.q.ss : (int64_t)b * a.q.sb;
  const uint16_t* qb = reinterpret_cast<const uint16_t*>(a.q.ptr) + qoff + (int64_t)h * a.q.sh;
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

  // ---- chunk list ----
  int n_chunks = 0, cpe = 1, nwin = 0, ncol = 0;
  const int32_t* list = nullptr;
  const int32_t* cols = nullptr;
  if constexpr (KIND == 0) {
    int kend = kv_len;
    if (a.causal) kend = min(kv_len, r_last + delta + 1);
    n_chunks = kend > 0 ? (kend + 63) / 64 : 0;
  } else {
    const int ht = a.list_by_kv ? hkv : h;
    const int64_t lb = (int64_t)b * a.pat.s_b + (int64_t)ht * a.pat.s_h + (int64_t)m * a.pat.s_q;
    const int cnt = a.pat.count[lb];
    list = a.pat.index + lb * a.pat.cap;
    if constexpr (KIND == 1) {
      cpe = a.pat.block_N / 64;
      n_chunks = cnt * cpe;
    } else {
      nwin = cnt;
      ncol = a.pat.col_count[lb];
      cols = a.pat.col_index + lb * a.pat.col_cap;
      n_chunks = nwin + (ncol + 63) / 64;
    }
  }

  const int t = tid_x();
  if constexpr (KIND != 0) {
    const int nl = min(KIND == 1 ? n_chunks / cpe : nwin, kEnts);
    for (int x = t; x < nl; x += NT) ents_s[x] = list[x];
    if constexpr (KIND == 2) {
      const int nc = min(ncol, kCols);
      for (int x = t; x < nc; x += NT) cols_s[x] = cols[x];
    }
  }
  auto entry = [&](int e) -> int { return e < kEnts ? ents_s[e] : list[e]; };
  auto column = [&](int x) -> int {
    if constexpr (KIND == 2) return x < kCols ? cols_s[x] : cols[x];
    return 0;
  };

  // chunk ci -> first key (contiguous) or gather base (columns); staged=false reads global
  auto chunk_key0 = [&](int ci, bool& gathered, int& gbase, bool staged) -> int {
    gathered = false;
    gbase = 0;
    if constexpr (KIND == 0) {
      return ci * 64;
    } else if constexpr (KIND == 1) {
      const int e = ci / cpe;
      return (staged ? entry(e) : list[e]) * a.pat.block_N + (ci - e * cpe) * 64;
    } else {
      if (ci < nwin) return staged ? entry(ci) : list[ci];
      gathered = true;
      gbase = (ci - nwin) * 64;
      return 0;
    }
  };

  // K: 16 lanes per 256-byte row (c = 16-byte piece); V: lanes run over 4-key groups
  // (kv) so the transposed LDS stores are conflict-free; NP (kv, cv) pairs per thread
  const int c = t % PIECES, kk = t / PIECES;
  constexpr int NP = 16 * PIECES / NT;
  const int kv = t % 16, cv0 = t / 16;
  u32x4 kr[L], vr[NP][4];
  // chunk-local key i -> global key index, or -1 when absent
  auto key_of = [&](int i, int key0, bool gathered, int gbase, bool staged) -> int {
    int key;
    if (gathered) {
      if (gbase + i >= ncol) return -1;
      key = staged ? column(gbase + i) : cols[gbase + i];
    } else {
      key = key0 + i;
    }
    return (unsigned)key < (unsigned)kv_len ? key : -1;
  };
  auto load_chunk = [&](int key0, bool gathered, int gbase, bool staged) {
#pragma unroll
    for (int jj = 0; jj < L; ++jj) {
      const int key = key_of(kk * L + jj, key0, gathered, gbase, staged);
      kr[jj] = key >= 0 ? ldg128(kbp + (int64_t)key * a.k.ss + c * 8) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int key = key_of(kv * 4 + jj, key0, gathered, gbase, staged);
#pragma unroll
      for (int pp = 0; pp < NP; ++pp) {
        const int cv = cv0 + pp * (NT / 16);
        vr[pp][jj] = key >= 0 ? ldg128(vbp + (int64_t)key * a.v.ss + cv * 8) : u32x4{0, 0, 0, 0};
      }
    }
  };

  float m_run = kNegInf, l_run = 0.f, le_run = 0.f;
  f32x16 oacc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) oacc[i] = f32x16{};

  auto finish = [&](int slot) {
    if (row_ok) {
      if (!a.partial) {
        const int64_t ob = (a.cu_q ? (int64_t)(q_start + row) * a.o.ss : (int64_t)b * a.o.sb + (int64_t)row * a.o.ss) +
                           (int64_t)h * a.o.sh;
        float* lp = nullptr;
        if (a.lse) lp = a.lse + (a.cu_q ? (int64_t)h * a.cu_q[a.B] + q_start + row : ((int64_t)b * a.Hq + h) * a.Sq + row);
        write_row(a.o, ob, lp, oacc, m_run, l_run, le_run, hh);
      } else {
        const OutArg po{a.part_o, 0, (int64_t)a.Hq * D, D, 1};
        const int64_t ob = (((int64_t)slot * a.B + b) * a.Sq + row) * a.Hq * D + (int64_t)h * D;
        write_row(po, ob, a.part_lse + (((int64_t)slot * a.B + b) * a.Hq + h) * a.Sq + row, oacc, m_run, l_run, le_run, hh);
      }
    }
    m_run = kNegInf;
    l_run = 0.f;
    le_run = 0.f;
#pragma unroll
    for (int i = 0; i < D / 32; ++i) oacc[i] = f32x16{};
  };

  bool g_next = false;
  int gb_next = 0;
  // the first chunk reads its addresses from global memory, so its loads overlap the staging
  int key0_next = n_chunks > 0 ? chunk_key0(0, g_next, gb_next, false) : 0;
  if (n_chunks > 0) load_chunk(key0_next, g_next, gb_next, false);
  __syncthreads();

  const int wrow_min = r0 + w * 32;
  for (int ci = 0; ci < n_chunks; ++ci) {
    const int key0 = key0_next;
    const bool gathered = g_next;
    const int gbase = gb_next;
    __syncthreads();
#pragma unroll
    for (int jj = 0; jj < L; ++jj) *reinterpret_cast<u32x4*>(Ks + (kk * L + jj) * TKS + c * 8) = kr[jj];
#pragma unroll
    for (int pp = 0; pp < NP; ++pp) store_vt_group<VSTR>(Vt, vr[pp], kv * 4, cv0 + pp * (NT / 16));
    if (t < 64) {
      int key = gathered ? (gbase + t < ncol ? column(gbase + t) : -1) : key0 + t;
      if ((unsigned)key >= (unsigned)kv_len) key = 0x7fffffff;
      kidx_s[t] = key;
    }
    __syncthreads();
    if (ci + 1 < n_chunks) {
      key0_next = chunk_key0(ci + 1, g_next, gb_next, true);
      load_chunk(key0_next, g_next, gb_next, true);
    }

    f32x16 s0 = st_block(Ks, 0, qreg, lq, hh);
    f32x16 s1 = st_block(Ks, 32, qreg, lq, hh);

    bool need_mask;
    if (gathered) {
      need_mask = true;
    } else {
      const int kmax = key0 + 63;
      need_mask = kmax >= kv_len || key0 < 0 || (a.causal && kmax > wrow_min + delta);
    }
    if (need_mask) {
      const int lim = a.causal ? row + delta : 0x7ffffffe;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int4 k0 = *reinterpret_cast<const int4*>(kidx_s + q4 * 8 + hh * 4);
        const int4 k1 = *reinterpret_cast<const int4*>(kidx_s + 32 + q4 * 8 + hh * 4);
        if (k0.x > lim) s0[q4 * 4 + 0] = kNegInf;
        if (k0.y > lim) s0[q4 * 4 + 1] = kNegInf;
        if (k0.z > lim) s0[q4 * 4 + 2] = kNegInf;
        if (k0.w > lim) s0[q4 * 4 + 3] = kNegInf;
        if (k1.x > lim) s1[q4 * 4 + 0] = kNegInf;
        if (k1.y > lim) s1[q4 * 4 + 1] = kNegInf;
        if (k1.z > lim) s1[q4 * 4 + 2] = kNegInf;
        if (k1.w > lim) s1[q4 * 4 + 3] = kNegInf;
      }
    }
    softmax_pv64<VSTR>(s0, s1, Vt, 0, a.scale_log2, m_run, l_run, le_run, oacc, lq, hh);

    if constexpr (KIND != 2) {
      if (a.partial && (ci % cpe) == cpe - 1) {
        const int e = ci / cpe;
        if ((e + 1) % a.epp == 0 || ci == n_chunks - 1) finish(e / a.epp);
      }
    }
  }

  if (!a.partial) {
    finish(0);
  } else {
    const int first_empty = n_chunks > 0 ? ((n_chunks - 1) / cpe) / a.epp + 1 : 0;
    for (int s = first_empty; s < a.n_part; ++s) finish(s);
  }
}

}  // namespace bsa
