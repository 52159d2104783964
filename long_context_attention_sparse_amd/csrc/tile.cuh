// MFMA tile steps shared by the prefill, gated, selected-attention and backward kernels
// (head dim 128, 32 query rows per wave, v_mfma_f32_32x32x16_bf16).
//
// Layout conventions (lane l of a wave, lq = l % 32, hh = l / 32):
//   Q^T operand  qreg[ks] = Q[row lq][16ks + 8hh .. +8]      (8 registers x 4 dwords)
//   K/V tiles    64- or 128-key tiles in LDS, 256-byte rows written straight from global
//                memory (global_load_lds_dwordx4); the 16-byte pieces of row R are swizzled
//                (K: piece p in slot p ^ (R & 15), V: p ^ 4(R & 3)) so the MFMA operand
//                reads are free of bank conflicts
//   S^T block    lane holds query lq, keys 8(r/4) + 4hh + r%4 of the 32-key block (r = 0..15);
//                registers 8hb..8hb+7, rounded to bf16, are the P^T operand of the 16-key
//                step hb, matched by V^T operands read with the transposing LDS read
//   O^T          oacc[db]: lane holds query lq, dims 32db + 8(r/4) + 4hh + r%4
#pragma once
#include "common.cuh"

namespace bsa {

constexpr int TD = 128;           // head dim of the tile kernels
constexpr float kSlack = 8.0f;    // lazy rescale threshold (log2 units)

// Soft-caps NB blocks of 32 raw scores in place (softcap_score); a no-op when cap_in == 0.
template <int NB>
__device__ __forceinline__ void softcap_n(f32x16* s, float cap_in, float cap_out) {
  if (cap_in == 0.f) return;
#pragma unroll
  for (int kb = 0; kb < NB; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) s[kb][r] = softcap_score(s[kb][r], cap_in, cap_out);
}

// Online softmax, first step of a chunk (the weights and the P V product follow in the
// kernel): the chunk's row maximum over NB blocks of 32 keys (masked scores -inf; m_run in
// scaled log2 units) and the lazy rescale — the reference maximum only moves, rescaling O
// and the normaliser, when the new maximum exceeds it by more than 2^8.  One normaliser is
// kept: l_run sums the float32 weights before their rounding to bf16 for the P V product.
// It divides O and gives LSE, so O's error is the weights' bf16 rounding alone: at most
// 2^-9 times the weighted mean of |v| over the attended keys.
// The lazy rescale for a chunk whose row maximum (scaled log2 units) is mx.
__device__ __forceinline__ void softmax_rescale(float mx, float& m_run, float& l_run, f32x16* oacc) {
  const float m_new = fmaxf(m_run, mx);
  const bool need = m_new > m_run + kSlack;
  if (__any(need)) {
    const float alpha = need ? exp2_fast(m_run - m_new) : 1.f;
    if (need) m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int db = 0; db < TD / 32; ++db) oacc[db] *= alpha;
  }
}

// Row maximum of NB blocks of 32 raw scores (the two lanes 32 apart hold one row).
template <int NB>
__device__ __forceinline__ float row_max_n(const f32x16* s) {
  float mx = kNegInf;
#pragma unroll
  for (int kb = 0; kb < NB; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
  return fmaxf(mx, shfl_xor_f(mx, 32));
}

template <int NB>
__device__ __forceinline__ void softmax_max_n(const f32x16* s, float scale_log2, float& m_run, float& l_run,
                                              f32x16* oacc) {
  softmax_rescale(row_max_n<NB>(s) * scale_log2, m_run, l_run, oacc);
}

// Normalise and store one query row's O (32 rows per wave, 64 dims per lane) and its LSE.
// o_off: element offset of the row start (head dim 0) in the output.
__device__ __forceinline__ void write_row(const OutArg& o, int64_t o_off, float* lse_ptr, const f32x16* oacc,
                                          float m_run, float l_run, int hh) {
  const float lt = l_run + shfl_xor_f(l_run, 32);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
#pragma unroll
  for (int db = 0; db < TD / 32; ++db)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int d = db * 32 + g4 * 8 + hh * 4;
      store4(o, o_off + d, oacc[db][g4 * 4] * inv, oacc[db][g4 * 4 + 1] * inv, oacc[db][g4 * 4 + 2] * inv,
             oacc[db][g4 * 4 + 3] * inv);
    }
  if (hh == 0 && lse_ptr) *lse_ptr = lt > 0.f ? (m_run + log2f(lt)) * kLn2 : kNegInf;
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

// Raw buffer resource over `bytes` bytes from `base`: untyped loads at offsets past `bytes`
// return zeros (the range check takes the per-lane offset, so every row-dependent part of an
// address goes into it).  Dword 3 selects 32-bit data, the setting untyped loads need.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
// 16 bytes per lane from a buffer straight into LDS (lane i -> lds + 16 i)
__device__ __forceinline__ void buffer_load_lds16(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, BSA_LDS(lds), 16, voff, 0, 0, 0);
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
// memory-side cache, and each XCD takes runs of kRun consecutive query blocks (or pairs of
// them), so the near-diagonal windows and the columns the blocks of a run share hit in its
// L2.  Runs are dealt to the XCDs in turn, heaviest (last) query block first; with kMirror
// every second round is dealt in reverse XCD order (x, 15 - x, 16 + x, ...), so that each XCD's
// runs of a head carry about the same work when the work per block grows along the sequence
// (otherwise the XCDs drift onto different heads).  Returns the item index in the (b, kv
// head, reversed query block, group member) order of the prefill kernels (with G query heads
// per kv head a run holds kRun / G query blocks of each of them).
template <int kRun, bool kMirror = false>
__device__ __forceinline__ int head_sync_item_n(int lid, int nqb, int n_items) {
  if (nqb % (8 * kRun) || n_items % nqb) return xcd_item(lid, n_items);
  const int xcd = lid & 7, j = lid >> 3;
  const int share = nqb >> 3;  // query blocks of one head per XCD
  const int head = j / share, jj = j - head * share;
  const int c = jj / kRun, r = jj - c * kRun;
  return head * nqb + (c * 8 + (kMirror && (c & 1) ? 7 - xcd : xcd)) * kRun + r;
}
// runs of 16 single query blocks (runs of 8, 32 and 64 measured slower)
__device__ __forceinline__ int head_sync_item(int lid, int nqb, int n_items) {
  return head_sync_item_n<16>(lid, nqb, n_items);
}

}  // namespace bsa
