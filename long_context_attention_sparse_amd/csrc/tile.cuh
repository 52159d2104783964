// MFMA tile steps shared by the prefill and gated kernels (head dim 128,
// 32 query rows per wave, v_mfma_f32_32x32x16_bf16).
//
// Layout conventions (lane l of a wave, lq = l % 32, hh = l / 32):
//   Q^T operand  qreg[ks] = Q[row lq][16ks + 8hh .. +8]      (8 registers x 4 dwords)
//   K in LDS     Ks[key][d], row stride KS (D + 8) bf16
//   S^T block    lane holds query lq, keys 8(r/4) + 4hh + r%4 of the 32-key block (r = 0..15)
//   V^T in LDS   Vt[d][pos], row stride VSTR; within each 16-key group the
//                positions hold keys (0-3, 8-11, 4-7, 12-15) so that S^T
//                registers 8hb..8hb+7 of a block are the P^T operand of the
//                16-key MFMA step (block, hb) without any data movement
//   O^T          oacc[db]: lane holds query lq, dims 32db + 8(r/4) + 4hh + r%4
#pragma once
#include "common.cuh"

namespace bsa {

constexpr int TD = 128;           // head dim of the tile kernels
constexpr int TKS = TD + 8;       // K row stride in LDS (bf16)
constexpr float kSlack = 8.0f;    // lazy rescale threshold (log2 units)

// Position of the first key of a 4-key group inside the V^T row.
__device__ __forceinline__ int vt_pos(int key4) {
  const int grp = (key4 >> 2) & 3;
  return (key4 & ~15) | ((((grp & 1) << 1) | (grp >> 1)) << 2);
}

// Store 4 V rows (keys key4..key4+3, head dims 8cv..8cv+7) transposed into V^T.  V is
// loaded with the 4-key group index running fastest across lanes, so the 16 (or 32)
// lanes of one store instruction write consecutive 8-byte slots of the same V^T row:
// no LDS bank conflicts.
template <int VSTR>
__device__ __forceinline__ void store_vt_group(uint16_t* Vt, const u32x4* v4, int key4, int cv) {
  const int pos = vt_pos(key4);
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    uint16_t* dst = Vt + (cv * 8 + 2 * p) * VSTR + pos;
    *reinterpret_cast<u32x2*>(dst) = u32x2{lo_halves(v4[0][p], v4[1][p]), lo_halves(v4[2][p], v4[3][p])};
    *reinterpret_cast<u32x2*>(dst + VSTR) = u32x2{hi_halves(v4[0][p], v4[1][p]), hi_halves(v4[2][p], v4[3][p])};
  }
}

// S^T for the 32 keys in LDS rows krow0 .. krow0+31.
__device__ __forceinline__ f32x16 st_block(const uint16_t* Ks, int krow0, const bf16x8* qreg, int lq, int hh) {
  f32x16 s = {};
#pragma unroll
  for (int ks = 0; ks < TD / 16; ++ks) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(Ks + (krow0 + lq) * TKS + ks * 16 + hh * 8);
    s = mfma32x32x16(as_bf16x8(a), qreg[ks], s);
  }
  return s;
}

// Online softmax over 64 keys, in two steps so a pipelined loop can place them apart.
// s0 holds keys 0-31 and s1 keys 32-63 of the chunk (V^T columns vcol0..vcol0+63);
// masked scores are -inf; m_run is in scaled log2 units.  Two normalisers are kept:
// l_run sums the bf16-rounded weights the PV product uses (O is then an exact convex
// combination of V rows, so a dominant key's rounding cancels) and le_run sums the exact
// weights (for LSE).
//
// Step 1: the chunk's row maximum, and the lazy rescale: the reference maximum only
// moves (rescaling O and the sums) when the new maximum exceeds it by more than 2^8.
// s holds NB blocks of 32 keys.
// Soft-caps NB blocks of 32 raw scores in place (softcap_score); a no-op when cap_in == 0.
template <int NB>
__device__ __forceinline__ void softcap_n(f32x16* s, float cap_in, float cap_out) {
  if (cap_in == 0.f) return;
#pragma unroll
  for (int kb = 0; kb < NB; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) s[kb][r] = softcap_score(s[kb][r], cap_in, cap_out);
}

template <int NB>
__device__ __forceinline__ void softmax_max_n(const f32x16* s, float scale_log2, float& m_run, float& l_run,
                                              float& le_run, f32x16* oacc) {
  float mx = kNegInf;
#pragma unroll
  for (int kb = 0; kb < NB; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
  mx = fmaxf(mx, shfl_xor_f(mx, 32)) * scale_log2;
  const float m_new = fmaxf(m_run, mx);
  const bool need = m_new > m_run + kSlack;
  if (__any(need)) {
    const float alpha = need ? exp2_fast(m_run - m_new) : 1.f;
    if (need) m_run = m_new;
    l_run *= alpha;
    le_run *= alpha;
#pragma unroll
    for (int db = 0; db < TD / 32; ++db) oacc[db] *= alpha;
  }
}

__device__ __forceinline__ void softmax_max(const f32x16& s0, const f32x16& s1, float scale_log2, float& m_run,
                                            float& l_run, float& le_run, f32x16* oacc) {
  const f32x16 s[2] = {s0, s1};
  softmax_max_n<2>(s, scale_log2, m_run, l_run, le_run, oacc);
}

// Step 2: weights, both normalisers, and O^T += V^T P^T.
template <int VSTR>
__device__ __forceinline__ void softmax_pv(const f32x16& s0, const f32x16& s1, const uint16_t* Vt, int vcol0,
                                           float scale_log2, float m_run, float& l_run, float& le_run,
                                           f32x16* oacc, int lq, int hh) {
  const float m_use = m_run == kNegInf ? 0.f : m_run;
  uint32_t pk[2][8];
  float psum = 0.f, pesum = 0.f;
#pragma unroll
  for (int r = 0; r < 16; r += 2) {
    const float p0 = exp2_fast(fmaf(s0[r], scale_log2, -m_use));
    const float p1 = exp2_fast(fmaf(s0[r + 1], scale_log2, -m_use));
    const float p2 = exp2_fast(fmaf(s1[r], scale_log2, -m_use));
    const float p3 = exp2_fast(fmaf(s1[r + 1], scale_log2, -m_use));
    pk[0][r / 2] = pack_bf16x2(p0, p1);
    pk[1][r / 2] = pack_bf16x2(p2, p3);
    psum = bf16x2_sum_acc(pk[0][r / 2], psum);
    psum = bf16x2_sum_acc(pk[1][r / 2], psum);
    pesum += (p0 + p1) + (p2 + p3);
  }
  l_run += psum;
  le_run += pesum;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const u32x4 pb = {pk[kb][hb * 4], pk[kb][hb * 4 + 1], pk[kb][hb * 4 + 2], pk[kb][hb * 4 + 3]};
      const int ks = kb * 2 + hb;
#pragma unroll
      for (int db = 0; db < TD / 32; ++db) {
        const u32x4 av = *reinterpret_cast<const u32x4*>(Vt + (db * 32 + lq) * VSTR + vcol0 + ks * 16 + hh * 8);
        oacc[db] = mfma32x32x16(as_bf16x8(av), as_bf16x8(pb), oacc[db]);
      }
    }
}

// Both steps back to back.
template <int VSTR>
__device__ __forceinline__ void softmax_pv64(const f32x16& s0, const f32x16& s1, const uint16_t* Vt, int vcol0,
                                             float scale_log2, float& m_run, float& l_run, float& le_run,
                                             f32x16* oacc, int lq, int hh) {
  softmax_max(s0, s1, scale_log2, m_run, l_run, le_run, oacc);
  softmax_pv<VSTR>(s0, s1, Vt, vcol0, scale_log2, m_run, l_run, le_run, oacc, lq, hh);
}

// Normalise and store one query row's O (32 rows per wave, 64 dims per lane) and its LSE.
// o_off: element offset of the row start (head dim 0) in the output.
__device__ __forceinline__ void write_row(const OutArg& o, int64_t o_off, float* lse_ptr, const f32x16* oacc,
                                          float m_run, float l_run, float le_run, int hh) {
  const float lt = l_run + shfl_xor_f(l_run, 32);
  const float le = le_run + shfl_xor_f(le_run, 32);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
#pragma unroll
  for (int db = 0; db < TD / 32; ++db)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int d = db * 32 + g4 * 8 + hh * 4;
      store4(o, o_off + d, oacc[db][g4 * 4] * inv, oacc[db][g4 * 4 + 1] * inv, oacc[db][g4 * 4 + 2] * inv,
             oacc[db][g4 * 4 + 3] * inv);
    }
  if (hh == 0 && lse_ptr) *lse_ptr = le > 0.f ? (m_run + log2f(le)) * kLn2 : kNegInf;
}

// ---- direct global->LDS tiles (global_load_lds_dwordx4) and transposed LDS reads ----
// A 64-key tile is 64 rows of 256 bytes (16 pieces of 8 bf16).  K row R keeps global piece
// p in slot p ^ (R & 15), V row R in slot p ^ 4(R & 3): both keep the MFMA operand reads
// (b128 rows of K, b64 transposed reads of V) free of bank conflicts.
__device__ __forceinline__ int k_swz(int row) { return row & 15; }
__device__ __forceinline__ int v_swz(int row) { return (row & 3) << 2; }

typedef short s16x4 __attribute__((ext_vector_type(4)));
#define BSA_LDS(p) ((__attribute__((address_space(3))) void*)(p))

// Loads through explicitly typed LDS / global pointers.
__device__ __forceinline__ int lds_int(const int* p, int i) {
  return ((const __attribute__((address_space(3))) int*)p)[i];
}
__device__ __forceinline__ int global_int(const int* p, int i) {
  return ((const __attribute__((address_space(1))) int*)p)[i];
}

__device__ __forceinline__ u32x2 ds_read_tr16(const uint16_t* p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
  return __builtin_bit_cast(u32x2, v);
}


// Work item for an XCD-aware, heavy-first launch: workgroup lid of n_items ->
// item index such that XCD x (= lid % 8) runs the contiguous item range x.
__device__ __forceinline__ int xcd_item(int lid, int n_items) {
  const int xcd = lid & 7, j8 = lid >> 3;
  const int per = n_items >> 3, rem = n_items & 7;
  return xcd * per + min(xcd, rem) + j8;
}

// Work order for patterns whose key sets stream through a head's whole K/V (vertical-slash):
// every XCD works on the same (b, head) at the same time, so that head's K/V stays in the
// memory-side cache, and each XCD takes runs of kRun consecutive query blocks, so the
// near-diagonal windows and the columns the blocks of a run share hit in its L2.  Runs are
// dealt to the XCDs in turn, heaviest (last) query block first.  Returns the item index in
// the (b, kv head, reversed query block, group member) order of the prefill kernels (with G
// query heads per kv head a run holds kRun / G query blocks of each of them).
__device__ __forceinline__ int head_sync_item(int lid, int nqb, int n_items) {
  constexpr int kRun = 16;
  if (nqb % (8 * kRun) || n_items % nqb) return xcd_item(lid, n_items);
  const int xcd = lid & 7, j = lid >> 3;
  const int share = nqb >> 3;  // query blocks of one head per XCD
  const int head = j / share, jj = j - head * share;
  const int c = jj / kRun, r = jj - c * kRun;
  return head * nqb + (c * 8 + xcd) * kRun + r;
}

}  // namespace bsa
