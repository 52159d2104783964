// Pipelined prefill kernel: NW waves of 32 query rows (BM = 32 NW rows per
// workgroup), keys in chunks of CK = 16 NW (64 keys for 128-row tiles, 32 keys
// for 64-row tiles).
//
// Attention restricted to listed keys ("Sparse FlashAttention with Incremental
// Repair", Usage 1 for block lists and Usage 3 for partials; "Implementation:
// Sgl project Sglang Sparse Flash Attention", I/O Contract, for vertical-slash
// block offsets and column indices; dense when no pattern is given).  A chunk
// is CK consecutive keys (a dense range, part of a listed block or of a
// vertical-slash window at any offset) or up to CK gathered vertical columns.
//
// Built around two gfx950 features:
//   global_load_lds_dwordx4  K and V rows go straight from global memory into
//                            LDS (lane L of a wave instruction fills LDS bytes
//                            16L..16L+15 of a 1 KB slab), no register staging;
//                            each lane picks the global 16-byte piece that its
//                            slot holds under an XOR swizzle, which keeps the
//                            MFMA operand reads free of bank conflicts.
//   ds_read_b64_tr_b16       V^T operands are read transposed out of the
//                            row-major V tile: lane r of a 16-lane group points
//                            at V[k0 + r/4][d0 + 4(r%4)] and receives keys
//                            k0..k0+3 of column d0 + r.
//
// K and V each have two CK-key LDS buffers (64 KB per 128-row workgroup, two per
// CU; 32 KB per 64-row workgroup, four per CU).  Iteration ci holds S(ci) in
// registers and K(ci+1), V(ci) in LDS; it issues the loads of K(ci+2) and
// V(ci+1), runs chunk ci's softmax and PV product, then computes S(ci+1) and its
// row max.  One barrier per iteration: each wave waits for its own loads of the
// previous iteration, the barrier makes every wave's data visible and every wave
// done with the buffers that the next loads overwrite.  The two waves on each
// SIMD come from different workgroups and cover each other's LDS and MFMA waits.
//
// Per wave and chunk: S^T = K Q^T (v_mfma_f32_32x32x16_bf16, Q^T in registers),
// online softmax in base 2 with scale*log2(e) folded into one FMA and a lazy
// rescale (tile.cuh), O^T += V^T P^T with P rounded to bf16.
//
// LDS layout of a buffer: CK rows of 256 bytes (16 pieces of 8 bf16).  K row R
// keeps global piece p in slot p ^ (R & 15); V row R in slot p ^ 4(R & 3).
// Full chunks address K/V from a wave-uniform row pointer plus a fixed per-lane
// offset; only chunks that run past the sequence end or gather columns resolve
// keys per lane.
//
// Grid: one workgroup per (b, h_q, query block), remapped so that each XCD takes
// a contiguous range ordered (b, h_kv, h_q, query block descending): workgroups
// sharing a key/value head share an L2, and the longest causal rows start first.
#pragma once
#include "tile.cuh"

namespace bsa {

template <int KIND, int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2))) void prefill_pipe_kernel(PrefillArgs a) {
  static_assert(NW == 2 || NW == 4, "64- or 128-row tiles");
  constexpr int D = TD;
  constexpr int NT = NW * 64;
  constexpr int BM = 32 * NW;
  constexpr int CK = 16 * NW;   // keys per chunk: every wave loads 16 rows of each tile
  constexpr int NB = CK / 32;   // 32-key S blocks per chunk
  constexpr int NKS = CK / 16;  // 16-key PV steps per chunk
  constexpr int RS = D;         // LDS row stride (bf16): rows are packed, the swizzle spreads banks
  __shared__ __attribute__((aligned(16))) uint16_t K0[CK * RS];
  __shared__ __attribute__((aligned(16))) uint16_t K1[CK * RS];
  __shared__ __attribute__((aligned(16))) uint16_t V0[CK * RS];
  __shared__ __attribute__((aligned(16))) uint16_t V1[CK * RS];
  constexpr int kKid = KIND == 2 ? CK : 4;
  __shared__ __attribute__((aligned(16))) int kid0[kKid];
  __shared__ __attribute__((aligned(16))) int kid1[kKid];
  // list entries (block ids or window offsets) and gathered column indices staged in LDS,
  // so a chunk's addresses never wait on a dependent global load
  constexpr int kEnts = 256;
  constexpr int kCols = KIND == 2 ? 768 : 1;
  __shared__ int ents_s[kEnts];
  __shared__ int cols_s[kCols];

  const int item = xcd_item(wg_x(), a.n_items);
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

  // ---- chunk list ----
  // cpe: chunks per list entry (a block, or a window of block_N keys); nwc: window chunks
  int n_chunks = 0, cpe = 1, nwc = 0, ncol = 0, n_ent = 0;
  const int32_t* list = nullptr;
  const int32_t* cols = nullptr;
  if constexpr (KIND == 0) {
    int kend = kv_len;
    if (a.causal) kend = min(kv_len, r_last + delta + 1);
    n_chunks = kend > 0 ? (kend + CK - 1) / CK : 0;
    cpe = 64 / CK;  // partial outputs group 64-key entries
  } else {
    const int ht = a.list_by_kv ? hkv : h;
    const int64_t lb = (int64_t)b * a.pat.s_b + (int64_t)ht * a.pat.s_h + (int64_t)m * a.pat.s_q;
    n_ent = a.pat.count[lb];
    list = a.pat.index + lb * a.pat.cap;
    cpe = a.pat.block_N / CK;
    if constexpr (KIND == 1) {
      n_chunks = n_ent * cpe;
    } else {
      nwc = n_ent * cpe;
      ncol = a.pat.col_count[lb];
      cols = a.pat.col_index + lb * a.pat.col_cap;
      n_chunks = nwc + (ncol + CK - 1) / CK;
    }
  }
  if (kv_len <= 0) n_chunks = 0;
  if constexpr (KIND != 0) {
    const int nl = min(n_ent, kEnts);
    for (int x = t; x < nl; x += NT) ents_s[x] = list[x];
    if constexpr (KIND == 2) {
      const int nc = min(ncol, kCols);
      for (int x = t; x < nc; x += NT) cols_s[x] = cols[x];
    }
  }

  // A chunk is CK consecutive keys from key0 (possibly running past the sequence end or
  // starting before 0 for a window) or up to CK gathered columns from gbase.  key0 and the
  // flags are wave-uniform and live in scalar registers.
  struct Chunk {
    int key0 = 0, gbase = 0;
    bool gathered = false, full = false;  // full: all CK keys inside [0, kv_len)
  };
  auto chunk_at = [&](int ci, bool staged) -> Chunk {
    Chunk r;
    if constexpr (KIND == 0) {
      r.key0 = ci * CK;
    } else {
      if (KIND == 1 || ci < nwc) {
        const int e = ci / cpe;
        const int id = __builtin_amdgcn_readfirstlane(staged && e < kEnts ? lds_int(ents_s, e) : global_int(list, e));
        r.key0 = (KIND == 1 ? id * a.pat.block_N : id) + (ci - e * cpe) * CK;
      } else {
        r.gathered = true;
        r.gbase = (ci - nwc) * CK;
      }
    }
    r.full = !r.gathered && r.key0 >= 0 && r.key0 <= kv_len - CK;
    return r;
  };
  // chunk-local key i -> key index within the sequence, or -1 when absent
  auto key_of = [&](int i, const Chunk& r, bool staged) -> int {
    int key;
    if (r.gathered) {
      const int x = r.gbase + i;
      if (x >= ncol) return -1;
      key = (staged && x < kCols) ? cols_s[x] : cols[x];
    } else {
      key = r.key0 + i;
    }
    return (unsigned)key < (unsigned)kv_len ? key : -1;
  };

  // Wave w fills LDS rows 16w..16w+15 of a tile with four 1 KB instructions: instruction i
  // covers rows 16w + 4i + l/16, lane l landing in slot l%16.  Row R's slot s holds piece
  // s ^ (R & 15) (K) or s ^ 4(R & 3) (V); with R & 15 = 4i + l/16 the per-lane byte offset
  // within the row is kx ^ 64i (K) or a constant (V).  A full chunk adds these to a
  // wave-uniform row address; otherwise each lane resolves its key, and absent keys load row
  // 0 (finite data, masked out later) so no slot keeps stale bits.
  const int lrow = l >> 4, lslot = l & 15;
  const uint32_t kx = (uint32_t)(lslot ^ lrow) << 4;
  const uint32_t vx = (uint32_t)(lslot ^ (lrow << 2)) << 4;
  const uint32_t k_lane = (uint32_t)(lrow * a.k.ss) * 2u, v_lane = (uint32_t)(lrow * a.v.ss) * 2u + vx;
  auto issue_k = [&](uint16_t* kt, int* kid, const Chunk& r, bool staged) __attribute__((always_inline)) {
    if (r.full) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const char* rowp = reinterpret_cast<const char*>(kbp + (int64_t)(r.key0 + w * 16 + i * 4) * a.k.ss);
        __builtin_amdgcn_global_load_lds(rowp + (k_lane + (kx ^ (i << 6))), BSA_LDS(kt + (w * 4 + i) * 4 * RS), 16,
                                         0, 0);
      }
    } else {
      // the key indices first (a gathered chunk also records them for the mask), then the
      // loads: an index read from memory is waited for, and that wait would also wait for the
      // loads already in flight
      if constexpr (KIND == 2) {
        if (r.gathered && t < CK) {
          const int key = key_of(t, r, staged);
          kid[t] = key >= 0 ? key : 0x7fffffff;
        }
      }
      int keys[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) keys[i] = max(0, key_of(w * 16 + i * 4 + lrow, r, staged));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const char* rowp = reinterpret_cast<const char*>(kbp + (int64_t)keys[i] * a.k.ss);
        __builtin_amdgcn_global_load_lds(rowp + (kx ^ (i << 6)), BSA_LDS(kt + (w * 4 + i) * 4 * RS), 16, 0, 0);
      }
    }
  };
  auto issue_v = [&](uint16_t* vt, const Chunk& r, bool staged) __attribute__((always_inline)) {
    if (r.full) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const char* rowp = reinterpret_cast<const char*>(vbp + (int64_t)(r.key0 + w * 16 + i * 4) * a.v.ss);
        __builtin_amdgcn_global_load_lds(rowp + v_lane, BSA_LDS(vt + (w * 4 + i) * 4 * RS), 16, 0, 0);
      }
    } else {
      // all four indices before any load (as for K)
      int keys[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) keys[i] = max(0, key_of(w * 16 + i * 4 + lrow, r, staged));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const char* rowp = reinterpret_cast<const char*>(vbp + (int64_t)keys[i] * a.v.ss);
        __builtin_amdgcn_global_load_lds(rowp + vx, BSA_LDS(vt + (w * 4 + i) * 4 * RS), 16, 0, 0);
      }
    }
  };

  // per-lane LDS offsets of the MFMA operands (loop invariant)
  int koff[D / 16];  // K: row lq (+32 kb), piece 2ks + hh, swizzled
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) koff[ks] = lq * RS + (((ks * 2 + hh) ^ k_swz(lq)) << 3);
  const int tg = l >> 4, tr = l & 15;  // transpose read: 16-lane group and lane in group
  // V^T: row (tg/2)*4 + tr/4 (+16ks + 8j), column 32db + 16(tg%2) + 4(tr%4)
  const int vrow = (tg >> 1) * 4 + (tr >> 2);
  int voff[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    const int col = db * 32 + (tg & 1) * 16 + (tr & 3) * 4;
    voff[db] = vrow * RS + ((((col >> 3) ^ v_swz(vrow))) << 3) + (col & 7);
  }

  // S^T for the chunk in LDS: block kb holds keys 32kb..32kb+31
  auto s_chunk = [&](const uint16_t* kt, f32x16* s) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < NB; ++kb) {
      f32x16 acc = {};
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const u32x4 av = *reinterpret_cast<const u32x4*>(kt + kb * 32 * RS + koff[ks]);
        acc = mfma32x32x16(as_bf16x8(av), qreg[ks], acc);
      }
      s[kb] = acc;
    }
  };

  float m_run = kNegInf, l_run = 0.f;
  f32x16 oacc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) oacc[i] = f32x16{};

  // exponentials of the chunk's scores, the normaliser and O^T += V^T P^T
  auto exp_pv = [&](const f32x16* s, const uint16_t* vt) __attribute__((always_inline)) {
    // V^T operands of the first two 16-key steps are read before the exponentials, so their
    // LDS latency hides behind the vector work; the rest are read between the MFMAs
    constexpr int NPRE = NKS < 2 ? NKS : 2;
    u32x4 vpre[NPRE][D / 32];
#pragma unroll
    for (int ks = 0; ks < NPRE; ++ks)
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const u32x2 lo = ds_read_tr16(vt + ks * 16 * RS + voff[db]);
        const u32x2 hi = ds_read_tr16(vt + (ks * 16 + 8) * RS + voff[db]);
        vpre[ks][db] = u32x4{lo[0], lo[1], hi[0], hi[1]};
      }
    const float m_use = m_run == kNegInf ? 0.f : m_run;
    uint32_t pk[NB][8];
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < NB; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; r += 4) {
        const float p0 = exp2_fast(fmaf(s[kb][r], a.scale_log2, -m_use));
        const float p1 = exp2_fast(fmaf(s[kb][r + 1], a.scale_log2, -m_use));
        const float p2 = exp2_fast(fmaf(s[kb][r + 2], a.scale_log2, -m_use));
        const float p3 = exp2_fast(fmaf(s[kb][r + 3], a.scale_log2, -m_use));
        pk[kb][r / 2] = pack_bf16x2(p0, p1);
        pk[kb][r / 2 + 1] = pack_bf16x2(p2, p3);
        psum += (p0 + p1) + (p2 + p3);
      }
    }
    l_run += psum;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const int kb = ks >> 1, hb = ks & 1;
      const u32x4 pb = {pk[kb][hb * 4], pk[kb][hb * 4 + 1], pk[kb][hb * 4 + 2], pk[kb][hb * 4 + 3]};
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        u32x4 av;
        if (ks < NPRE) {
          av = vpre[ks < NPRE ? ks : 0][db];
        } else {
          const u32x2 lo = ds_read_tr16(vt + ks * 16 * RS + voff[db]);
          const u32x2 hi = ds_read_tr16(vt + (ks * 16 + 8) * RS + voff[db]);
          av = u32x4{lo[0], lo[1], hi[0], hi[1]};
        }
        oacc[db] = mfma32x32x16(as_bf16x8(av), as_bf16x8(pb), oacc[db]);
      }
    }
  };

  auto finish = [&](int slot) __attribute__((always_inline)) {
    if (row_ok) {
      if (!a.partial) {
        const int64_t ob = (a.cu_q ? (int64_t)(q_start + row) * a.o.ss : (int64_t)b * a.o.sb + (int64_t)row * a.o.ss) +
                           (int64_t)h * a.o.sh;
        float* lp = nullptr;
        if (a.lse) lp = a.lse + (a.cu_q ? (int64_t)h * a.cu_q[a.B] + q_start + row : ((int64_t)b * a.Hq + h) * a.Sq + row);
        write_row(a.o, ob, lp, oacc, m_run, l_run, hh);
      } else {
        const OutArg po{a.part_o, 0, (int64_t)a.Hq * D, D, 1};
        const int64_t ob = (((int64_t)slot * a.B + b) * a.Sq + row) * a.Hq * D + (int64_t)h * D;
        write_row(po, ob, a.part_lse + (((int64_t)slot * a.B + b) * a.Hq + h) * a.Sq + row, oacc, m_run, l_run,
                  hh);
      }
    }
    m_run = kNegInf;
    l_run = 0.f;
#pragma unroll
    for (int i = 0; i < D / 32; ++i) oacc[i] = f32x16{};
  };

  // -inf for absent keys and, when causal, keys after the row's diagonal.  Contiguous
  // chunks compare key0 + (register's key offset) against a per-row limit; gathered
  // chunks read the key indices that issue_k stored.
  const int wrow_min = r0 + w * 32;
  auto mask_chunk = [&](const int* kid, const Chunk& r, f32x16* s) __attribute__((always_inline)) {
    const int lim = a.causal ? row + delta : 0x7ffffffe;
    if (r.gathered) {
#pragma unroll
      for (int kb = 0; kb < NB; ++kb)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int4 k4 = *reinterpret_cast<const int4*>(kid + kb * 32 + q4 * 8 + hh * 4);
          if (k4.x > lim) s[kb][q4 * 4 + 0] = kNegInf;
          if (k4.y > lim) s[kb][q4 * 4 + 1] = kNegInf;
          if (k4.z > lim) s[kb][q4 * 4 + 2] = kNegInf;
          if (k4.w > lim) s[kb][q4 * 4 + 3] = kNegInf;
        }
      return;
    }
    const bool need = !r.full || (a.causal && r.key0 + CK - 1 > wrow_min + delta);
    if (!need) return;
    // key0 + kl is present and visible iff lo <= kl <= hi
    const int hi = min(lim, kv_len - 1) - r.key0;
    const int lo = -r.key0;
#pragma unroll
    for (int kb = 0; kb < NB; ++kb)
#pragma unroll
      for (int rg = 0; rg < 16; ++rg) {
        const int kl = kb * 32 + (rg >> 2) * 8 + hh * 4 + (rg & 3);
        if (kl > hi || kl < lo) s[kb][rg] = kNegInf;
      }
  };

  // ---- pipeline ----
  f32x16 sc[NB];
#pragma unroll
  for (int kb = 0; kb < NB; ++kb) sc[kb] = f32x16{};
  Chunk nxt;
  if (n_chunks > 0) {
    // the first chunks read their addresses from global memory, overlapping the staging
    const Chunk c0 = chunk_at(0, false);
    issue_k(K0, kid0, c0, false);
    issue_v(V0, c0, false);
    if (n_chunks > 1) {
      nxt = chunk_at(1, false);
      issue_k(K1, kid1, nxt, false);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    s_chunk(K0, sc);
    softcap_n<NB>(sc, a.cap_in, a.cap_out);
    mask_chunk(kid0, c0, sc);
    softmax_max_n<NB>(sc, a.scale_log2, m_run, l_run, oacc);
  }

  // Chunk ci: S(ci) in sc; K stages kc / kn (this chunk / the next), V stages vc / vn.
  auto step = [&](int ci, uint16_t* kc, int* kidc, uint16_t* kn, const int* kidn, const uint16_t* vc, uint16_t* vn)
                  __attribute__((always_inline)) {
    // this wave's loads of the previous step (K(ci+1), V(ci)) are done; after the barrier
    // every wave's are, and no wave still reads kc or vn
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    const bool has1 = ci + 1 < n_chunks, has2 = ci + 2 < n_chunks;
    Chunk nn;
    if (has2) {
      nn = chunk_at(ci + 2, true);
      issue_k(kc, kidc, nn, true);
    }
    if (has1) issue_v(vn, nxt, true);
    exp_pv(sc, vc);
    if constexpr (KIND != 2) {
      if (a.partial && (ci % cpe) == cpe - 1) {
        const int e = ci / cpe;
        if ((e + 1) % a.epp == 0 || ci == n_chunks - 1) finish(e / a.epp);
      }
    }
    if (has1) {
      s_chunk(kn, sc);
      softcap_n<NB>(sc, a.cap_in, a.cap_out);
      mask_chunk(kidn, nxt, sc);
      softmax_max_n<NB>(sc, a.scale_log2, m_run, l_run, oacc);
    }
    nxt = nn;
  };
  for (int ci = 0; ci < n_chunks; ci += 2) {
    step(ci, K0, kid0, K1, kid1, V0, V1);
    if (ci + 1 < n_chunks) step(ci + 1, K1, kid1, K0, kid0, V1, V0);
  }

  if (!a.partial) {
    finish(0);
  } else {
    const int first_empty = n_chunks > 0 ? ((n_chunks - 1) / cpe) / a.epp + 1 : 0;
    for (int s = first_empty; s < a.n_part; ++s) finish(s);
  }
}

}  // namespace bsa
