// C ABI of the block-sparse attention library (declared in include/bsa.h).
//
// Each entry point validates its arguments on the host, picks a kernel, fills
// a plain argument block and enqueues the launch on the caller's stream.  No
// memory is allocated, no stream is synchronised, no exception escapes.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdint>
#include <cstring>

#include "bsa.h"
#include "combine.cuh"
#include "decode.cuh"
#include "gated.cuh"
#include "prefill.cuh"
#include "vs_convert.cuh"

using namespace bsa;

namespace {

constexpr int kTargetWorkgroups = 2048;  // decode split heuristic: ~8 resident workgroups per CU

bool valid_dtype(int32_t d) { return d == BSA_BF16 || d == BSA_F32; }

float scale_of(const bsa_problem& p) {
  return p.softmax_scale > 0.f ? p.softmax_scale : 1.0f / std::sqrt((float)p.D);
}

TensorArg targ(const bsa_tensor& t) { return TensorArg{t.ptr, t.stride_b, t.stride_s, t.stride_h}; }
OutArg oarg(const bsa_tensor& t) { return OutArg{t.ptr, t.stride_b, t.stride_s, t.stride_h, t.dtype == BSA_F32}; }

PatternArg parg(const bsa_pattern* p) {
  PatternArg a{};
  if (!p) return a;
  a.kind = p->kind;
  a.block_M = p->block_M;
  a.block_N = p->block_N;
  a.cap = p->cap;
  a.col_cap = p->col_cap;
  a.count = p->count;
  a.index = p->index;
  a.col_count = p->col_count;
  a.col_index = p->col_index;
  a.s_b = p->s_b;
  a.s_h = p->s_h;
  a.s_q = p->s_q;
  return a;
}

bsa_status launch_status() {
  return hipGetLastError() == hipSuccess ? BSA_OK : BSA_ERR_HIP;
}

// 16-byte alignment of every row start: base pointer and all strides must keep
// head-dim rows 16-byte aligned for the vector loads.
bool aligned_rows(const bsa_tensor& t, int elem_bytes) {
  const uintptr_t p = reinterpret_cast<uintptr_t>(t.ptr);
  auto ok = [&](int64_t s) { return ((s * elem_bytes) & 15) == 0; };
  return (p & 15) == 0 && ok(t.stride_b) && ok(t.stride_s) && ok(t.stride_h);
}

bsa_status check_problem(const bsa_problem* prob, const bsa_tensor& q, const bsa_tensor& k, const bsa_tensor& v,
                         const bsa_tensor& o) {
  if (!prob) return BSA_ERR_INVALID_ARG;
  const bsa_problem& p = *prob;
  if (p.B <= 0 || p.Hq <= 0 || p.Hkv <= 0 || p.Sq <= 0 || p.Sk <= 0 || p.D <= 0) return BSA_ERR_INVALID_ARG;
  if (p.Hq % p.Hkv) return BSA_ERR_INVALID_ARG;
  if ((p.cu_seqlens_q == nullptr) != (p.cu_seqlens_k == nullptr)) return BSA_ERR_INVALID_ARG;
  if (p.cu_seqlens_q && (p.max_seqlen_q <= 0 || p.max_seqlen_k <= 0)) return BSA_ERR_INVALID_ARG;
  if (!q.ptr || !k.ptr || !v.ptr || !o.ptr) return BSA_ERR_INVALID_ARG;
  if (q.dtype != BSA_BF16 || k.dtype != BSA_BF16 || v.dtype != BSA_BF16) return BSA_ERR_UNSUPPORTED;
  if (!valid_dtype(o.dtype)) return BSA_ERR_INVALID_ARG;
  if (p.D != 64 && p.D != 128) return BSA_ERR_UNSUPPORTED;
  if (!aligned_rows(q, 2) || !aligned_rows(k, 2) || !aligned_rows(v, 2)) return BSA_ERR_INVALID_ARG;
  if (!aligned_rows(o, o.dtype == BSA_F32 ? 4 : 2)) return BSA_ERR_INVALID_ARG;
  return BSA_OK;
}

bsa_status check_pattern(const bsa_problem& p, const bsa_pattern* pat) {
  if (!pat || pat->kind == BSA_PAT_DENSE) return BSA_OK;
  if (pat->kind != BSA_PAT_BLOCK && pat->kind != BSA_PAT_VS) return BSA_ERR_INVALID_ARG;
  if (pat->Ht != p.Hq && pat->Ht != p.Hkv) return BSA_ERR_INVALID_ARG;
  if (!pat->count || !pat->index || pat->cap < 0) return BSA_ERR_INVALID_ARG;
  if (pat->s_b < 0 || pat->s_h < 0 || pat->s_q < 0) return BSA_ERR_INVALID_ARG;
  if (pat->block_M != 64 && pat->block_M != 128) return BSA_ERR_UNSUPPORTED;
  if (pat->block_N != 64 && pat->block_N != 128) return BSA_ERR_UNSUPPORTED;
  if (pat->kind == BSA_PAT_BLOCK) {
    if (!p.cu_seqlens_q && p.Sk % pat->block_N) return BSA_ERR_INVALID_ARG;
  } else {
    if (!pat->col_count || !pat->col_index || pat->col_cap < 0) return BSA_ERR_INVALID_ARG;
    if (!p.causal) return BSA_ERR_UNSUPPORTED;
    if (pat->block_M > pat->block_N) return BSA_ERR_UNSUPPORTED;
  }
  return BSA_OK;
}

// ---------------------------------------------------------------------------
// Decode path selection and split heuristic
// ---------------------------------------------------------------------------

struct DecodePlan {
  bool use = false;
  int Gp = 1, R = 0;
  int n_entries = 0, entries_per_split = 0, splits = 0;
  int cpe = 1;
};

DecodePlan plan_decode(const bsa_problem& p, const bsa_pattern* pat) {
  DecodePlan d;
  const int kind = pat ? pat->kind : BSA_PAT_DENSE;
  if (p.cu_seqlens_q || kind == BSA_PAT_VS) return d;
  const int G = p.Hq / p.Hkv;
  const bool shared = kind == BSA_PAT_DENSE || pat->Ht == p.Hkv;
  d.Gp = shared ? G : 1;
  d.R = d.Gp * p.Sq;
  if (d.R > 16) return d;
  if (kind == BSA_PAT_BLOCK && p.Sq > pat->block_M) return d;
  if (kind == BSA_PAT_DENSE) {
    d.n_entries = (p.Sk + 63) / 64;
    d.cpe = 1;
  } else {
    d.n_entries = pat->cap;
    d.cpe = pat->block_N / 64;
  }
  const int groups = p.B * (p.Hq / d.Gp);
  int splits = (kTargetWorkgroups + groups - 1) / groups;
  splits = std::max(1, std::min(splits, std::max(1, d.n_entries)));
  d.entries_per_split = std::max(1, (d.n_entries + splits - 1) / splits);
  d.splits = std::max(1, (d.n_entries + d.entries_per_split - 1) / d.entries_per_split);
  d.use = true;
  return d;
}

size_t decode_ws_bytes(const bsa_problem& p, const DecodePlan& d) {
  if (d.splits <= 1) return 0;
  const size_t rows = (size_t)p.B * p.Sq * p.Hq;
  return (size_t)d.splits * rows * (p.D + 1) * sizeof(float) + 256;
}

template <int D, int CPE>
void launch_decode_t(const DecodeArgs& a, int splits, int groups, int B, hipStream_t st) {
  hipLaunchKernelGGL((decode_kernel<D, CPE>), dim3(splits, groups, B), dim3(256), 0, st, a);
}

void launch_decode(const DecodeArgs& a, int D, int cpe, int splits, int groups, int B, hipStream_t st) {
  if (D == 128) {
    if (cpe == 2) launch_decode_t<128, 2>(a, splits, groups, B, st);
    else launch_decode_t<128, 1>(a, splits, groups, B, st);
  } else {
    if (cpe == 2) launch_decode_t<64, 2>(a, splits, groups, B, st);
    else launch_decode_t<64, 1>(a, splits, groups, B, st);
  }
}

void launch_combine(const CombineArgs& c, hipStream_t st) {
  const int64_t rows = (int64_t)c.B * c.Sq * c.Hq;
  const int rows_per_block = 256 / (c.D / 4);
  const int64_t blocks = (rows + rows_per_block - 1) / rows_per_block;
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)blocks), dim3(256), 0, st, c);
}

bsa_status run_decode(const bsa_problem& p, const DecodePlan& d, const bsa_tensor& q, const bsa_tensor& k,
                      const bsa_tensor& v, const bsa_pattern* pat, float* part_o, float* part_lse,
                      const bsa_tensor* o, float* lse, hipStream_t st) {
  DecodeArgs a{};
  a.q = targ(q);
  a.k = targ(k);
  a.v = targ(v);
  a.pat = parg(pat);
  a.B = p.B;
  a.Hq = p.Hq;
  a.Hkv = p.Hkv;
  a.Sq = p.Sq;
  a.Sk = p.Sk;
  a.G = p.Hq / p.Hkv;
  a.Gp = d.Gp;
  a.R = d.R;
  a.n_entries = d.n_entries;
  a.entries_per_split = d.entries_per_split;
  a.causal = p.causal != 0;
  a.scale_log2 = scale_of(p) * kLog2e;
  if (o) {
    a.direct = 1;
    a.o = oarg(*o);
    a.lse = lse;
  } else {
    a.direct = 0;
    a.part_o = part_o;
    a.part_lse = part_lse;
  }
  launch_decode(a, p.D, d.cpe, d.splits, p.Hq / d.Gp, p.B, st);
  return launch_status();
}


// ---------------------------------------------------------------------------
// Prefill path
// ---------------------------------------------------------------------------

template <int NW, int KIND>
void launch_prefill_t(const PrefillArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((prefill_kernel<NW, KIND>), dim3(a.n_items), dim3(NW * 64), 0, st, a);
}

bsa_status run_prefill(const bsa_problem& p, const bsa_tensor& q, const bsa_tensor& k, const bsa_tensor& v,
                       const bsa_pattern* pat, const bsa_tensor* o, float* lse, int epp, int n_part, float* part_o,
                       float* part_lse, hipStream_t st) {
  if (p.D != 128) return BSA_ERR_UNSUPPORTED;
  const int kind = pat ? pat->kind : BSA_PAT_DENSE;
  const int BM = kind == BSA_PAT_DENSE ? 128 : pat->block_M;
  const int Sq = p.cu_seqlens_q ? p.max_seqlen_q : p.Sq;
  PrefillArgs a{};
  a.q = targ(q);
  a.k = targ(k);
  a.v = targ(v);
  a.pat = parg(pat);
  a.cu_q = p.cu_seqlens_q;
  a.cu_k = p.cu_seqlens_k;
  a.B = p.B;
  a.Hq = p.Hq;
  a.Hkv = p.Hkv;
  a.G = p.Hq / p.Hkv;
  a.Sq = Sq;
  a.Sk = p.cu_seqlens_q ? p.max_seqlen_k : p.Sk;
  a.nqb = (Sq + BM - 1) / BM;
  a.list_by_kv = pat && kind != BSA_PAT_DENSE && pat->Ht == p.Hkv && p.Hkv != p.Hq;
  a.causal = p.causal != 0;
  a.scale_log2 = scale_of(p) * kLog2e;
  const int64_t items = (int64_t)p.B * p.Hq * a.nqb;
  if (items > INT_MAX) return BSA_ERR_UNSUPPORTED;
  a.n_items = (int)items;
  if (o) {
    a.o = oarg(*o);
    a.lse = lse;
  } else {
    a.partial = 1;
    a.epp = epp;
    a.n_part = n_part;
    a.part_o = part_o;
    a.part_lse = part_lse;
  }
  if (BM == 128) {
    if (kind == BSA_PAT_DENSE) launch_prefill_t<4, 0>(a, st);
    else if (kind == BSA_PAT_BLOCK) launch_prefill_t<4, 1>(a, st);
    else launch_prefill_t<4, 2>(a, st);
  } else {
    if (kind == BSA_PAT_DENSE) launch_prefill_t<2, 0>(a, st);
    else if (kind == BSA_PAT_BLOCK) launch_prefill_t<2, 1>(a, st);
    else launch_prefill_t<2, 2>(a, st);
  }
  return launch_status();
}

// Entries (list entries, or 64-key chunks for a dense pattern) and the number of
// partials bsa_fwd_partials writes for a given grouping.
int partial_entries(const bsa_problem& p, const bsa_pattern* pat) {
  if (!pat || pat->kind == BSA_PAT_DENSE) return (p.Sk + 63) / 64;
  return pat->cap;
}

}  // namespace

extern "C" {

const char* bsa_status_string(bsa_status s) {
  switch (s) {
    case BSA_OK: return "ok";
    case BSA_ERR_INVALID_ARG: return "invalid argument";
    case BSA_ERR_UNSUPPORTED: return "unsupported configuration";
    case BSA_ERR_WORKSPACE: return "workspace too small";
    case BSA_ERR_HIP: return "HIP launch failure";
  }
  return "unknown status";
}

size_t bsa_workspace_size(const bsa_problem* prob, const bsa_pattern* pat) {
  if (!prob || prob->B <= 0 || prob->Hkv <= 0 || prob->Hq % prob->Hkv) return 0;
  if (check_pattern(*prob, pat) != BSA_OK) return 0;
  const DecodePlan d = plan_decode(*prob, pat);
  if (d.use) return decode_ws_bytes(*prob, d);
  return 0;
}

bsa_status bsa_fwd(const bsa_problem* prob, bsa_tensor q, bsa_tensor k, bsa_tensor v, const bsa_pattern* pat,
                   bsa_tensor o, float* lse, void* ws, size_t ws_bytes, bsa_stream stream) {
  bsa_status st = check_problem(prob, q, k, v, o);
  if (st != BSA_OK) return st;
  const bsa_problem& p = *prob;
  st = check_pattern(p, pat);
  if (st != BSA_OK) return st;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  const DecodePlan d = plan_decode(p, pat);
  if (!d.use) return run_prefill(p, q, k, v, pat, &o, lse, 0, 0, nullptr, nullptr, hs);
  if (d.splits == 1) return run_decode(p, d, q, k, v, pat, nullptr, nullptr, &o, lse, hs);
  const size_t need = decode_ws_bytes(p, d);
  if (!ws || ws_bytes < need || (reinterpret_cast<uintptr_t>(ws) & 15)) return BSA_ERR_WORKSPACE;
  const size_t rows = (size_t)p.B * p.Sq * p.Hq;
  float* part_o = reinterpret_cast<float*>(ws);
  float* part_lse = part_o + (size_t)d.splits * rows * p.D;
  st = run_decode(p, d, q, k, v, pat, part_o, part_lse, nullptr, nullptr, hs);
  if (st != BSA_OK) return st;
  CombineArgs c{d.splits, p.B, p.Hq, p.Sq, p.D, part_o, part_lse, oarg(o), lse};
  launch_combine(c, hs);
  return launch_status();
}

int32_t bsa_num_partials(const bsa_problem* prob, const bsa_pattern* pat, int32_t entries_per_partial) {
  if (!prob || prob->B <= 0 || prob->Hkv <= 0 || prob->Sk <= 0 || prob->Hq % prob->Hkv) return -1;
  if (check_pattern(*prob, pat) != BSA_OK || (pat && pat->kind == BSA_PAT_VS)) return -1;
  const int n = partial_entries(*prob, pat);
  int e = entries_per_partial;
  if (e <= 0) {
    const DecodePlan d = plan_decode(*prob, pat);
    e = d.use ? d.entries_per_split : 1;
  }
  return n > 0 ? (n + e - 1) / e : 0;
}

bsa_status bsa_fwd_partials(const bsa_problem* prob, bsa_tensor q, bsa_tensor k, bsa_tensor v,
                            const bsa_pattern* pat, int32_t entries_per_partial, float* o_part, float* lse_part,
                            bsa_stream stream) {
  if (!o_part || !lse_part) return BSA_ERR_INVALID_ARG;
  bsa_tensor o_dummy{o_part, BSA_F32, 0, 0, 0};
  bsa_status st = check_problem(prob, q, k, v, o_dummy);
  if (st != BSA_OK) return st;
  const bsa_problem& p = *prob;
  if (p.cu_seqlens_q || (pat && pat->kind == BSA_PAT_VS)) return BSA_ERR_UNSUPPORTED;
  st = check_pattern(p, pat);
  if (st != BSA_OK) return st;
  if (reinterpret_cast<uintptr_t>(o_part) & 15) return BSA_ERR_INVALID_ARG;
  const int n = partial_entries(p, pat);
  DecodePlan d = plan_decode(p, pat);
  const int epp = entries_per_partial > 0 ? entries_per_partial : (d.use ? d.entries_per_split : 1);
  const int n_part = n > 0 ? (n + epp - 1) / epp : 0;
  if (n_part == 0) return BSA_OK;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  if (d.use) {
    d.entries_per_split = epp;
    d.splits = n_part;
    return run_decode(p, d, q, k, v, pat, o_part, lse_part, nullptr, nullptr, hs);
  }
  return run_prefill(p, q, k, v, pat, nullptr, nullptr, epp, n_part, o_part, lse_part, hs);
}

bsa_status bsa_combine(int32_t P, int32_t B, int32_t Hq, int32_t Sq, int32_t D, const float* o_part,
                       const float* lse_part, bsa_tensor o, float* lse, bsa_stream stream) {
  if (P < 1 || B <= 0 || Hq <= 0 || Sq <= 0 || !o_part || !lse_part || !o.ptr) return BSA_ERR_INVALID_ARG;
  if (D != 64 && D != 128) return BSA_ERR_UNSUPPORTED;
  if (!valid_dtype(o.dtype) || !aligned_rows(o, o.dtype == BSA_F32 ? 4 : 2)) return BSA_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(o_part) & 15) return BSA_ERR_INVALID_ARG;
  CombineArgs c{P, B, Hq, Sq, D, o_part, lse_part, oarg(o), lse};
  launch_combine(c, reinterpret_cast<hipStream_t>(stream));
  return launch_status();
}

bsa_status bsa_fwd_gated(const bsa_problem* prob, bsa_tensor q, bsa_tensor k, bsa_tensor v, const float* T,
                         int32_t block_M, int32_t block_N, bsa_tensor o, float* lse, uint8_t* keep_mask,
                         float* tile_max, bsa_stream stream) {
  bsa_status st = check_problem(prob, q, k, v, o);
  if (st != BSA_OK) return st;
  const bsa_problem& p = *prob;
  if (!T) return BSA_ERR_INVALID_ARG;
  if (block_M != 128 || block_N != 128 || p.D != 128) return BSA_ERR_UNSUPPORTED;
  if (!p.causal || p.cu_seqlens_q || p.Sq != p.Sk || p.Sq % 128) return BSA_ERR_UNSUPPORTED;
  GatedArgs a{};
  a.q = targ(q);
  a.k = targ(k);
  a.v = targ(v);
  a.o = oarg(o);
  a.lse = lse;
  a.T = T;
  a.keep = keep_mask;
  a.tmax = tile_max;
  a.B = p.B;
  a.Hq = p.Hq;
  a.Hkv = p.Hkv;
  a.G = p.Hq / p.Hkv;
  a.S = p.Sq;
  a.nqb = p.Sq / 128;
  a.scale = scale_of(p);
  a.scale_log2 = a.scale * kLog2e;
  const int64_t items = (int64_t)p.B * p.Hq * a.nqb;
  if (items > INT_MAX) return BSA_ERR_UNSUPPORTED;
  a.n_items = (int)items;
  hipLaunchKernelGGL(gated_kernel, dim3(a.n_items), dim3(256), 0, reinterpret_cast<hipStream_t>(stream), a);
  return launch_status();
}

bsa_status vs_convert_indexes(const int32_t* q_seqlens, const int32_t* kv_seqlens, const int32_t* vertical,
                              const int32_t* slash, int32_t B, int32_t H, int32_t nnz_v, int32_t nnz_s,
                              int32_t context_size, int32_t block_M, int32_t block_N, int32_t causal,
                              int32_t* block_count, int32_t* block_offset, int32_t* column_count,
                              int32_t* column_index, bsa_stream stream) {
  if (!q_seqlens || !kv_seqlens || !block_count || !column_count) return BSA_ERR_INVALID_ARG;
  if (B <= 0 || H <= 0 || nnz_v < 0 || nnz_s < 0 || context_size <= 0 || block_M <= 0 || block_N <= 0)
    return BSA_ERR_INVALID_ARG;
  if ((nnz_v > 0 && (!vertical || !column_index)) || (nnz_s > 0 && (!slash || !block_offset)))
    return BSA_ERR_INVALID_ARG;
  if (!causal || block_M > block_N) return BSA_ERR_UNSUPPORTED;
  VSConvArgs a{q_seqlens, kv_seqlens, vertical, slash, B, H, nnz_v, nnz_s, 0, block_M, block_N,
               block_count, block_offset, column_count, column_index};
  a.rows = (context_size + block_M - 1) / block_M;
  const int lds_ints = nnz_s + nnz_v <= kVSConvLdsInts ? nnz_s + nnz_v : 0;
  dim3 grid((a.rows + kVSConvThreads - 1) / kVSConvThreads, B * H);
  hipLaunchKernelGGL(vs_convert_kernel, grid, dim3(kVSConvThreads), lds_ints * sizeof(int32_t),
                     reinterpret_cast<hipStream_t>(stream), a);
  return launch_status();
}

}  // extern "C"
