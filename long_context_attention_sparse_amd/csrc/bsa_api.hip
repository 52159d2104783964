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
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "args.cuh"
#include "bsa.h"
#include "decode_plan.h"
#include "host_args.h"
#include "launch.h"

using namespace bsa;

namespace {

bsa_status check_problem(const bsa_problem* prob, const bsa_tensor& q, const bsa_tensor& k, const bsa_tensor& v,
                         const bsa_tensor& o) {
  if (!prob) return BSA_ERR_INVALID_ARG;
  const bsa_problem& p = *prob;
  if (p.B <= 0 || p.Hq <= 0 || p.Hkv <= 0 || p.Sq <= 0 || p.Sk <= 0 || p.D <= 0) return BSA_ERR_INVALID_ARG;
  if (p.Hq % p.Hkv) return BSA_ERR_INVALID_ARG;
  if ((p.cu_seqlens_q == nullptr) != (p.cu_seqlens_k == nullptr)) return BSA_ERR_INVALID_ARG;
  if (p.cu_seqlens_q && (p.max_seqlen_q <= 0 || p.max_seqlen_k <= 0)) return BSA_ERR_INVALID_ARG;
  if (!(p.softcap >= 0.f) || std::isinf(p.softcap)) return BSA_ERR_INVALID_ARG;
  if (!q.ptr || !k.ptr || !v.ptr || !o.ptr) return BSA_ERR_INVALID_ARG;
  if (q.dtype != BSA_BF16 || k.dtype != BSA_BF16 || v.dtype != BSA_BF16) return BSA_ERR_UNSUPPORTED;
  if (!valid_dtype(o.dtype)) return BSA_ERR_INVALID_ARG;
  if (p.D != 64 && p.D != 128) return BSA_ERR_UNSUPPORTED;
  if (!aligned_rows(q, 2) || !aligned_rows(k, 2) || !aligned_rows(v, 2)) return BSA_ERR_INVALID_ARG;
  if (!aligned_rows(o, o.dtype == BSA_F32 ? 4 : 2)) return BSA_ERR_INVALID_ARG;
  if (!row_stride_ok(q, 2) || !row_stride_ok(k, 2) || !row_stride_ok(v, 2)) return BSA_ERR_UNSUPPORTED;
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
    if (pat->block_M > pat->block_N) return BSA_ERR_UNSUPPORTED;
  }
  return BSA_OK;
}

// Pattern validation on the device (bsa_check_pattern; BSA_DEBUG_CHECKS).
CheckArgs check_args(const bsa_problem& p, const bsa_pattern* pat, int32_t* result) {
  CheckArgs a{};
  a.pat = parg(pat);
  a.cu_q = p.cu_seqlens_q;
  a.cu_k = p.cu_seqlens_k;
  a.B = p.B;
  a.Ht = pat->Ht;
  const int sq = p.cu_seqlens_q ? p.max_seqlen_q : p.Sq;
  a.nqb = (sq + pat->block_M - 1) / pat->block_M;
  a.Sk = p.cu_seqlens_q ? p.max_seqlen_k : p.Sk;
  a.result = result;
  return a;
}

bool debug_checks_on() {
  const char* e = std::getenv("BSA_DEBUG_CHECKS");
  return e && *e && std::strcmp(e, "0") != 0;
}

// With BSA_DEBUG_CHECKS set: check the pattern on the device, wait for the answer and refuse
// a violating one before anything is launched.
bsa_status debug_validate(const bsa_problem& p, const bsa_pattern* pat, bsa_stream stream) {
  if (!pat || pat->kind == BSA_PAT_DENSE || !debug_checks_on()) return BSA_OK;
  const int r = debug_check(check_args(p, pat, nullptr), reinterpret_cast<hipStream_t>(stream));
  return r == 0 ? BSA_OK : (r < 0 ? BSA_ERR_HIP : BSA_ERR_INVALID_ARG);
}

// ---------------------------------------------------------------------------
// Prefill path
// ---------------------------------------------------------------------------

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
  cap_consts(p, a.cap_in, a.cap_out);
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
  if (o && kind == BSA_PAT_VS && BM == 64) {
    // final outputs of 64-row vertical-slash blocks: pairs of neighbouring query blocks
    a.n_items = (int)((int64_t)p.B * p.Hq * ((a.nqb + 1) / 2));
    launch_vs_pair(a, st);
  } else {
    launch_prefill(a, BM / 32, kind, st);
  }
  return launch_status();
}

// ---------------------------------------------------------------------------
// Library-resident scratch of bsa_speculative_sparse_noalloc
// ---------------------------------------------------------------------------

// One copy per device.  In host code this name is only a handle for the symbol lookup: its
// device address comes from hipGetSymbolAddress, made once per device with that device
// current, and only that address is ever handed to a kernel.
static __device__ __align__(256) unsigned char scratch[BSA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

// Device address of the current device's scratch area (looked up on first use).
bsa_status scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return BSA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return BSA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return BSA_ERR_HIP;
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return BSA_OK;
}

// Entries (list entries, or 64-key chunks for a dense pattern) and the number of
// partials bsa_fwd_partials writes for a given grouping.
int partial_entries(const bsa_problem& p, const bsa_pattern* pat) {
  if (!pat || pat->kind == BSA_PAT_DENSE) return (p.Sk + 63) / 64;
  return pat->cap;
}

}  // namespace

extern "C" {

const char* bsa_status_string(int32_t status) {
  // an int, not the enum: a value outside bsa_status must not be loaded as one
  switch (status) {
    case BSA_OK: return "ok";
    case BSA_ERR_INVALID_ARG: return "invalid argument";
    case BSA_ERR_UNSUPPORTED: return "unsupported configuration";
    case BSA_ERR_WORKSPACE: return "workspace too small";
    case BSA_ERR_HIP: return "HIP launch failure";
  }
  return "unknown status";
}

size_t bsa_workspace_size(const bsa_problem* prob, const bsa_pattern* pat) {
  if (!prob || prob->B <= 0 || prob->Hkv <= 0 || prob->Hq <= 0 || prob->Hq % prob->Hkv) return 0;
  if (check_pattern(*prob, pat) != BSA_OK) return 0;
  const DecodePlan d = plan_decode(*prob, pat);
  if (!d.use) return 0;
  const SegPlan sp = fwd_decode_plan(*prob, pat, d);
  return sp.splits > 1 ? partial_bytes(*prob, sp.splits) : 0;
}

bsa_status bsa_fwd(const bsa_problem* prob, bsa_tensor q, bsa_tensor k, bsa_tensor v, const bsa_pattern* pat,
                   bsa_tensor o, float* lse, void* ws, size_t ws_bytes, bsa_stream stream) {
  bsa_status st = check_problem(prob, q, k, v, o);
  if (st != BSA_OK) return st;
  const bsa_problem& p = *prob;
  st = check_pattern(p, pat);
  if (st != BSA_OK) return st;
  st = debug_validate(p, pat, stream);
  if (st != BSA_OK) return st;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  const DecodePlan d = plan_decode(p, pat);
  if (!d.use) return run_prefill(p, q, k, v, pat, &o, lse, 0, 0, nullptr, nullptr, hs);
  const SegPlan sp = fwd_decode_plan(p, pat, d);
  const DecodeSeg seg = make_seg(k, v, pat, p.Sk, p.causal, sp, 0);
  if (sp.splits == 1) return run_decode(p, d, q, &seg, 1, nullptr, nullptr, &o, lse, hs);
  const size_t need = partial_bytes(p, sp.splits);
  if (!ws || ws_bytes < need || (reinterpret_cast<uintptr_t>(ws) & 15)) return BSA_ERR_WORKSPACE;
  const size_t rows = (size_t)p.B * p.Sq * p.Hq;
  float* part_o = reinterpret_cast<float*>(ws);
  float* part_lse = part_o + (size_t)sp.splits * rows * p.D;
  st = run_decode(p, d, q, &seg, 1, part_o, part_lse, nullptr, nullptr, hs);
  if (st != BSA_OK) return st;
  CombineArgs c{sp.splits, p.B, p.Hq, p.Sq, p.D, part_o, part_lse, oarg(o), lse};
  launch_combine(c, hs);
  return launch_status();
}

// Entries per partial and partial count of bsa_fwd_partials (E <= 0: the split plan).
static SegPlan partials_plan(const bsa_problem& p, const bsa_pattern* pat, int E) {
  const DecodePlan d = plan_decode(p, pat);
  SegPlan sp = seg_entries(p.Sk, pat);
  if (E > 0) {
    sp.eps = E;
    sp.splits = sp.n_entries > 0 ? (sp.n_entries + E - 1) / E : 0;
  } else if (d.use) {
    split_segments(&sp, 1, p.B * (p.Hq / d.Gp));
  } else {
    sp.eps = 1;
    sp.splits = sp.n_entries;
  }
  if (sp.n_entries <= 0) sp.splits = 0;
  return sp;
}

int32_t bsa_num_partials(const bsa_problem* prob, const bsa_pattern* pat, int32_t entries_per_partial) {
  if (!prob || prob->B <= 0 || prob->Hkv <= 0 || prob->Hq <= 0 || prob->Sk <= 0 || prob->Hq % prob->Hkv) return -1;
  if (check_pattern(*prob, pat) != BSA_OK || (pat && pat->kind == BSA_PAT_VS)) return -1;
  return partials_plan(*prob, pat, entries_per_partial).splits;
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
  st = debug_validate(p, pat, stream);
  if (st != BSA_OK) return st;
  if (reinterpret_cast<uintptr_t>(o_part) & 15) return BSA_ERR_INVALID_ARG;
  const SegPlan sp = partials_plan(p, pat, entries_per_partial);
  if (sp.splits == 0) return BSA_OK;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  const DecodePlan d = plan_decode(p, pat);
  if (d.use) {
    const DecodeSeg seg = make_seg(k, v, pat, p.Sk, p.causal, sp, 0);
    return run_decode(p, d, q, &seg, 1, o_part, lse_part, nullptr, nullptr, hs);
  }
  return run_prefill(p, q, k, v, pat, nullptr, nullptr, sp.eps, sp.splits, o_part, lse_part, hs);
}

int32_t bsa_speculative_num_partials(const bsa_problem* prob, int32_t Sk_spec, const bsa_pattern* missed) {
  if (!prob || prob->B <= 0 || prob->Hkv <= 0 || prob->Hq <= 0 || prob->Hq % prob->Hkv || Sk_spec <= 0) return -1;
  if (!missed || missed->kind != BSA_PAT_BLOCK || check_pattern(*prob, missed) != BSA_OK) return -1;
  SegPlan segs[2];
  DecodePlan d;
  speculative_plan(*prob, Sk_spec, missed, segs, &d);
  return segs[0].splits + segs[1].splits;
}

size_t bsa_speculative_workspace_size(const bsa_problem* prob, int32_t Sk_spec, const bsa_pattern* missed) {
  const int32_t n = bsa_speculative_num_partials(prob, Sk_spec, missed);
  return n > 0 ? partial_bytes(*prob, n) : 0;
}

bsa_status bsa_speculative_partials(const bsa_problem* prob, bsa_tensor q, bsa_tensor k_spec, bsa_tensor v_spec,
                                    int32_t Sk_spec, int32_t causal_spec, bsa_tensor k, bsa_tensor v,
                                    const bsa_pattern* missed, float* o_part, float* lse_part, bsa_stream stream) {
  if (!o_part || !lse_part || (reinterpret_cast<uintptr_t>(o_part) & 15)) return BSA_ERR_INVALID_ARG;
  bsa_tensor o_dummy{o_part, BSA_F32, 0, 0, 0};
  bsa_status st = check_problem(prob, q, k, v, o_dummy);
  if (st != BSA_OK) return st;
  const bsa_problem& p = *prob;
  if (p.cu_seqlens_q) return BSA_ERR_UNSUPPORTED;
  if (Sk_spec <= 0 || !k_spec.ptr || !v_spec.ptr) return BSA_ERR_INVALID_ARG;
  if (k_spec.dtype != BSA_BF16 || v_spec.dtype != BSA_BF16) return BSA_ERR_UNSUPPORTED;
  if (!aligned_rows(k_spec, 2) || !aligned_rows(v_spec, 2)) return BSA_ERR_INVALID_ARG;
  if (!missed || missed->kind != BSA_PAT_BLOCK) return BSA_ERR_INVALID_ARG;
  st = check_pattern(p, missed);
  if (st != BSA_OK) return st;
  st = debug_validate(p, missed, stream);
  if (st != BSA_OK) return st;
  SegPlan segs[2];
  DecodePlan d;
  speculative_plan(p, Sk_spec, missed, segs, &d);
  const size_t rows = (size_t)p.B * p.Sq * p.Hq;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  if (d.use) {
    // both passes in one launch: the speculative keys (dense, causal_spec) and the
    // missed blocks of the full cache (never masked)
    const DecodeSeg sg[2] = {make_seg(k_spec, v_spec, nullptr, Sk_spec, causal_spec, segs[0], 0),
                             make_seg(k, v, missed, p.Sk, 0, segs[1], segs[0].splits)};
    return run_decode(p, d, q, sg, 2, o_part, lse_part, nullptr, nullptr, hs);
  }
  bsa_problem ps = p;
  ps.Sk = Sk_spec;
  ps.causal = causal_spec;
  st = run_prefill(ps, q, k_spec, v_spec, nullptr, nullptr, nullptr, segs[0].eps, 1, o_part, lse_part, hs);
  if (st != BSA_OK) return st;
  bsa_problem pr = p;
  pr.causal = 0;
  return run_prefill(pr, q, k, v, missed, nullptr, nullptr, segs[1].eps, 1, o_part + rows * p.D, lse_part + rows, hs);
}

bsa_status bsa_speculative_sparse(const bsa_problem* prob, bsa_tensor q, bsa_tensor k_spec, bsa_tensor v_spec,
                                  int32_t Sk_spec, int32_t causal_spec, bsa_tensor k, bsa_tensor v,
                                  const bsa_pattern* missed, bsa_tensor o, float* lse, void* ws, size_t ws_bytes,
                                  bsa_stream stream) {
  bsa_status st = check_problem(prob, q, k, v, o);
  if (st != BSA_OK) return st;
  const int32_t slots = bsa_speculative_num_partials(prob, Sk_spec, missed);
  if (slots <= 0) return BSA_ERR_INVALID_ARG;
  const bsa_problem& p = *prob;
  const size_t need = partial_bytes(p, slots);
  if (!ws || ws_bytes < need || (reinterpret_cast<uintptr_t>(ws) & 15)) return BSA_ERR_WORKSPACE;
  const size_t rows = (size_t)p.B * p.Sq * p.Hq;
  float* part_o = reinterpret_cast<float*>(ws);
  float* part_lse = part_o + (size_t)slots * rows * p.D;
  st = bsa_speculative_partials(prob, q, k_spec, v_spec, Sk_spec, causal_spec, k, v, missed, part_o, part_lse,
                                stream);
  if (st != BSA_OK) return st;
  CombineArgs c{slots, p.B, p.Hq, p.Sq, p.D, part_o, part_lse, oarg(o), lse};
  launch_combine(c, reinterpret_cast<hipStream_t>(stream));
  return launch_status();
}

bsa_status bsa_speculative_sparse_noalloc(const bsa_problem* prob, bsa_tensor q, bsa_tensor k_spec,
                                          bsa_tensor v_spec, int32_t Sk_spec, int32_t causal_spec, bsa_tensor k,
                                          bsa_tensor v, const bsa_pattern* missed, bsa_tensor o, float* lse,
                                          bsa_stream stream) {
  bsa_status st = check_problem(prob, q, k, v, o);
  if (st != BSA_OK) return st;
  const int32_t slots = bsa_speculative_num_partials(prob, Sk_spec, missed);
  if (slots <= 0) return BSA_ERR_INVALID_ARG;
  if (partial_bytes(*prob, slots) > BSA_NOALLOC_SCRATCH_BYTES) return BSA_ERR_WORKSPACE;
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != BSA_OK) return st;
  return bsa_speculative_sparse(prob, q, k_spec, v_spec, Sk_spec, causal_spec, k, v, missed, o, lse, ws,
                                BSA_NOALLOC_SCRATCH_BYTES, stream);
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
                         int32_t block_M, int32_t block_N, int32_t skipped, bsa_tensor o, float* lse,
                         uint8_t* keep_mask, float* tile_max, bsa_stream stream) {
  bsa_status st = check_problem(prob, q, k, v, o);
  if (st != BSA_OK) return st;
  const bsa_problem& p = *prob;
  if (!T) return BSA_ERR_INVALID_ARG;
  if (skipped != BSA_GATE_DROP_SKIPPED && skipped != BSA_GATE_COUNT_SKIPPED) return BSA_ERR_INVALID_ARG;
  if (block_M != 128 || block_N != 128 || p.D != 128) return BSA_ERR_UNSUPPORTED;
  if (!p.causal || p.cu_seqlens_q || p.Sq != p.Sk || p.Sq % 128) return BSA_ERR_UNSUPPORTED;
  if (p.softcap > 0.f) return BSA_ERR_UNSUPPORTED;
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
  a.count_skipped = skipped == BSA_GATE_COUNT_SKIPPED;
  const int64_t items = (int64_t)p.B * p.Hq * a.nqb;
  if (items > INT_MAX) return BSA_ERR_UNSUPPORTED;
  a.n_items = (int)items;
  launch_gated(a, false, reinterpret_cast<hipStream_t>(stream));
  return launch_status();
}

// ---------------------------------------------------------------------------
// Backward of block-sparse attention
// ---------------------------------------------------------------------------

}  // extern "C"

namespace {

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct BwdLayout {
  int BM = 0, SB = 0, nqb = 0, nks = 0, nkb = 0, W = 0, n_lists = 0, chunk_bound = 0;
  size_t dsum = 0, lse2 = 0, counts = 0, offsets = 0, entries = 0, chunkp = 0, bits = 0, part = 0, total = 0;
};

// Shapes the backward kernels take; total == 0 otherwise.
BwdLayout bwd_layout(const bsa_problem& p, const bsa_pattern* pat) {
  BwdLayout L;
  if (p.B <= 0 || p.Hq <= 0 || p.Hkv <= 0 || p.Hq % p.Hkv || p.Sq <= 0 || p.Sk <= 0) return L;
  if (p.D != 128) return L;
  const bool block = pat && pat->kind == BSA_PAT_BLOCK;
  if (pat && pat->kind != BSA_PAT_DENSE && !block) return L;
  const int Sq = p.cu_seqlens_q ? p.max_seqlen_q : p.Sq;  // variable length: the longest sequence
  const int Sk = p.cu_seqlens_q ? p.max_seqlen_k : p.Sk;
  L.BM = block ? pat->block_M : 128;
  L.SB = 64;  // a sub-block never spans two pattern key blocks (block_N is 64 or 128)
  L.nqb = (Sq + L.BM - 1) / L.BM;
  L.nks = (Sk + L.SB - 1) / L.SB;
  L.n_lists = p.B * p.Hkv * L.nks;
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t at = off; off = align256(off + bytes); return at; };
  L.dsum = take(sizeof(float) * (size_t)p.B * p.Hq * Sq);  // at least Hq * total_q
  L.lse2 = take(sizeof(float) * (size_t)p.B * p.Hq * Sq);
  L.counts = take(sizeof(int32_t) * L.n_lists);
  L.chunkp = take(sizeof(int32_t) * (L.n_lists + 1));
  size_t units;  // upper bound on the 32-row slabs over all lists
  if (block) {
    const int Ht = pat->Ht;
    const int mult = Ht == p.Hkv ? p.Hq / p.Hkv : 1;
    // each (list head, query block) names a key block at most once in the bitmap
    const size_t per = (size_t)std::min(pat->cap, (Sk + pat->block_N - 1) / pat->block_N);
    const size_t pairs = (size_t)p.B * Ht * L.nqb * per * (pat->block_N / L.SB) * mult;
    if (pairs >= (size_t)INT_MAX) return BwdLayout{};
    if (L.nqb > (1 << 20) || p.Hq > (1 << 11)) return BwdLayout{};  // list entries: (head << 20) | block
    L.nkb = (Sk + pat->block_N - 1) / pat->block_N;
    L.W = (L.nqb + 31) / 32;
    L.offsets = take(sizeof(int32_t) * (L.n_lists + 1));
    L.entries = take(sizeof(int32_t) * std::max<size_t>(pairs, 1));
    L.bits = take(sizeof(uint32_t) * (size_t)p.B * Ht * L.nkb * L.W);
    units = pairs * (L.BM / 32);
  } else {
    units = (size_t)L.n_lists * (p.Hq / p.Hkv) * ((Sq + 31) / 32);
  }
  const size_t chunks = units / kBwdChunk + L.n_lists;  // ceil per list: at most one extra each
  if (chunks >= (size_t)INT_MAX / 2) return BwdLayout{};
  L.chunk_bound = (int)chunks;
  L.part = take(sizeof(float) * chunks * 2 * L.SB * 128);
  L.total = off;
  return L;
}

}  // namespace

extern "C" {

size_t bsa_bwd_workspace_size(const bsa_problem* prob, const bsa_pattern* pat) {
  if (!prob || check_pattern(*prob, pat) != BSA_OK) return 0;
  return bwd_layout(*prob, pat).total;
}

bsa_status bsa_bwd(const bsa_problem* prob, bsa_tensor q, bsa_tensor k, bsa_tensor v, const bsa_pattern* pat,
                   bsa_tensor o, const float* lse, bsa_tensor dout, float* dq, float* dk, float* dv, void* ws,
                   size_t ws_bytes, bsa_stream stream) {
  bsa_status st = check_problem(prob, q, k, v, o);
  if (st != BSA_OK) return st;
  const bsa_problem& p = *prob;
  st = check_pattern(p, pat);
  if (st != BSA_OK) return st;
  st = debug_validate(p, pat, stream);
  if (st != BSA_OK) return st;
  if (!lse || !dout.ptr || !dq || !dk || !dv) return BSA_ERR_INVALID_ARG;
  if (dout.dtype != BSA_BF16) return BSA_ERR_UNSUPPORTED;
  if (!aligned_rows(dout, 2)) return BSA_ERR_INVALID_ARG;
  if (!row_stride_ok(dout, 2)) return BSA_ERR_UNSUPPORTED;
  if ((reinterpret_cast<uintptr_t>(dq) | reinterpret_cast<uintptr_t>(dk) | reinterpret_cast<uintptr_t>(dv)) & 15)
    return BSA_ERR_INVALID_ARG;
  const BwdLayout L = bwd_layout(p, pat);
  if (L.total == 0) return BSA_ERR_UNSUPPORTED;
  if (!ws || ws_bytes < L.total || (reinterpret_cast<uintptr_t>(ws) & 255)) return BSA_ERR_WORKSPACE;
  char* base = reinterpret_cast<char*>(ws);
  BwdArgs a{};
  a.q = targ(q);
  a.k = targ(k);
  a.v = targ(v);
  a.o = targ(o);
  a.o_f32 = o.dtype == BSA_F32;
  a.dout = targ(dout);
  a.lse = lse;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.dsum = reinterpret_cast<float*>(base + L.dsum);
  a.lse2 = reinterpret_cast<float*>(base + L.lse2);
  a.pat = parg(pat);
  a.cu_q = p.cu_seqlens_q;
  a.cu_k = p.cu_seqlens_k;
  a.B = p.B;
  a.Hq = p.Hq;
  a.Hkv = p.Hkv;
  a.G = p.Hq / p.Hkv;
  a.Sq = p.cu_seqlens_q ? p.max_seqlen_q : p.Sq;
  a.Sk = p.cu_seqlens_q ? p.max_seqlen_k : p.Sk;
  a.list_by_kv = pat && pat->kind == BSA_PAT_BLOCK && pat->Ht == p.Hkv && p.Hkv != p.Hq;
  a.causal = p.causal;
  a.scale = scale_of(p);
  a.scale_log2 = a.scale * kLog2e;
  cap_consts(p, a.cap_in, a.cap_out);
  a.BM = L.BM;
  a.SB = L.SB;
  a.nqb = L.nqb;
  a.nks = L.nks;
  a.nkb = L.nkb;
  a.W = L.W;
  a.counts = reinterpret_cast<int32_t*>(base + L.counts);
  a.chunkp = reinterpret_cast<int32_t*>(base + L.chunkp);
  a.part = reinterpret_cast<float*>(base + L.part);
  if (pat && pat->kind == BSA_PAT_BLOCK) {
    a.offsets = reinterpret_cast<int32_t*>(base + L.offsets);
    a.entries = reinterpret_cast<int32_t*>(base + L.entries);
    a.bits = reinterpret_cast<uint32_t*>(base + L.bits);
  }
  launch_bwd(a, L.chunk_bound, reinterpret_cast<hipStream_t>(stream));
  return launch_status();
}

// ---------------------------------------------------------------------------
// Selected attention (top-k key blocks per query token)
// ---------------------------------------------------------------------------

}  // extern "C"

namespace {

struct SelLayout {
  int T = 0, nkb = 0, n_lists = 0, Bc = 0, Sc = 0;
  size_t counts = 0, offsets = 0, cursor = 0, chunkp = 0, entries = 0, part_o = 0, part_lse = 0, total = 0;
};

constexpr int kSelD = 128;  // head dim of the selected-attention kernel

// Workspace carve-up; total == 0 for shapes outside the supported set.
SelLayout sel_layout(const bsa_problem& p, int32_t total_q, int32_t topk) {
  SelLayout L;
  if (p.B <= 0 || p.Hq <= 0 || p.Hkv <= 0 || p.Hq % p.Hkv || topk < 1) return L;
  const bool varlen = p.cu_seqlens_q != nullptr;
  const int64_t T = varlen ? (int64_t)total_q : (int64_t)p.B * p.Sq;
  const int kmax = varlen ? p.max_seqlen_k : p.Sk;
  if (T <= 0 || kmax <= 0) return L;
  const int64_t nkb = (kmax + 63) / 64;
  if (nkb > kSelMaxBlocks) return L;
  const int64_t n_lists = (int64_t)p.B * p.Hkv * nkb;
  const int64_t pairs = T * p.Hkv * topk;
  if (T * topk >= INT_MAX || pairs >= INT_MAX || n_lists >= INT_MAX / 2) return L;
  L.T = (int)T;
  L.nkb = (int)nkb;
  L.n_lists = (int)n_lists;
  L.Bc = varlen ? 1 : p.B;
  L.Sc = varlen ? (int)T : p.Sq;
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t at = off; off = align256(off + bytes); return at; };
  L.counts = take(sizeof(int32_t) * n_lists);
  L.offsets = take(sizeof(int32_t) * (n_lists + 1));
  L.cursor = take(sizeof(int32_t) * n_lists);
  L.chunkp = take(sizeof(int32_t) * (n_lists + 1));
  L.entries = take(sizeof(int32_t) * pairs);
  L.part_o = take(sizeof(float) * (size_t)topk * T * p.Hq * kSelD);
  L.part_lse = take(sizeof(float) * (size_t)topk * T * p.Hq);
  L.total = off;
  return L;
}

}  // namespace

extern "C" {

size_t bsa_selected_workspace_size(const bsa_problem* prob, int32_t total_q, int32_t topk, int32_t block_size) {
  if (!prob || block_size != 64) return 0;
  return sel_layout(*prob, total_q, topk).total;
}

bsa_status bsa_fwd_selected(const bsa_problem* prob, bsa_tensor q, bsa_tensor k, bsa_tensor v, const int32_t* sel,
                            int32_t total_q, int32_t topk, int32_t block_size, bsa_tensor o, float* lse, void* ws,
                            size_t ws_bytes, bsa_stream stream) {
  bsa_status st = check_problem(prob, q, k, v, o);
  if (st != BSA_OK) return st;
  const bsa_problem& p = *prob;
  if (!sel || topk < 1) return BSA_ERR_INVALID_ARG;
  if (p.cu_seqlens_q && total_q <= 0) return BSA_ERR_INVALID_ARG;
  const int G = p.Hq / p.Hkv;
  if (p.D != 128 || block_size != 64 || G > 16 || 128 % G) return BSA_ERR_UNSUPPORTED;
  const SelLayout L = sel_layout(p, total_q, topk);
  if (L.total == 0) return BSA_ERR_UNSUPPORTED;
  if (!ws || ws_bytes < L.total || (reinterpret_cast<uintptr_t>(ws) & 255)) return BSA_ERR_WORKSPACE;
  char* base = reinterpret_cast<char*>(ws);
  SelArgs a{};
  a.q = targ(q);
  a.k = targ(k);
  a.v = targ(v);
  a.sel = sel;
  a.cu_q = p.cu_seqlens_q;
  a.cu_k = p.cu_seqlens_k;
  a.B = p.B;
  a.Hq = p.Hq;
  a.Hkv = p.Hkv;
  a.G = G;
  a.Sq = p.cu_seqlens_q ? p.max_seqlen_q : p.Sq;
  a.Sk = p.cu_seqlens_q ? p.max_seqlen_k : p.Sk;
  a.T = L.T;
  a.topk = topk;
  a.nkb = L.nkb;
  a.tpc = 128 / G;
  a.causal = p.causal;
  a.scale_log2 = scale_of(p) * kLog2e;
  cap_consts(p, a.cap_in, a.cap_out);
  a.counts = reinterpret_cast<int32_t*>(base + L.counts);
  a.offsets = reinterpret_cast<int32_t*>(base + L.offsets);
  a.cursor = reinterpret_cast<int32_t*>(base + L.cursor);
  a.chunkp = reinterpret_cast<int32_t*>(base + L.chunkp);
  a.entries = reinterpret_cast<int32_t*>(base + L.entries);
  a.part_o = reinterpret_cast<float*>(base + L.part_o);
  a.part_lse = reinterpret_cast<float*>(base + L.part_lse);
  a.Bc = L.Bc;
  a.Sc = L.Sc;
  // chunks <= sum over lists of (count / tpc + 1) <= pairs / tpc + lists
  const int64_t grid = ((int64_t)L.T * p.Hkv * topk + a.tpc - 1) / a.tpc + L.n_lists;
  if (grid > INT_MAX) return BSA_ERR_UNSUPPORTED;
  const hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  launch_selected(a, (int)grid, hs);
  if (hipPeekAtLastError() != hipSuccess) return launch_status();
  CombineArgs c{topk, L.Bc, p.Hq, L.Sc, kSelD, a.part_o, a.part_lse, oarg(o), lse};
  launch_combine(c, hs);
  return launch_status();
}

bsa_status bsfa_calibrate(const bsa_problem* prob, bsa_tensor q, bsa_tensor k, int32_t k_keep, float* tile_max,
                          float* T, bsa_stream stream) {
  if (!prob || !q.ptr || !k.ptr || !tile_max || !T || k_keep < 1) return BSA_ERR_INVALID_ARG;
  const bsa_problem& p = *prob;
  if (p.B <= 0 || p.Hq <= 0 || p.Hkv <= 0 || p.Sq <= 0 || p.Sk <= 0 || p.D <= 0 || p.Hq % p.Hkv)
    return BSA_ERR_INVALID_ARG;
  if (!(p.softcap >= 0.f) || std::isinf(p.softcap)) return BSA_ERR_INVALID_ARG;
  if (q.dtype != BSA_BF16 || k.dtype != BSA_BF16) return BSA_ERR_UNSUPPORTED;
  if (!aligned_rows(q, 2) || !aligned_rows(k, 2)) return BSA_ERR_INVALID_ARG;
  if (p.D != 128 || !p.causal || p.cu_seqlens_q || p.Sq != p.Sk || p.Sq % 128 || p.softcap > 0.f)
    return BSA_ERR_UNSUPPORTED;
  const int nqb = p.Sq / 128;
  if (nqb > kThreshMaxCand) return BSA_ERR_UNSUPPORTED;
  GatedArgs a{};
  a.q = targ(q);
  a.k = targ(k);
  a.v = targ(k);  // not read by the calibration pass
  a.tmax = tile_max;
  a.B = p.B;
  a.Hq = p.Hq;
  a.Hkv = p.Hkv;
  a.G = p.Hq / p.Hkv;
  a.S = p.Sq;
  a.nqb = nqb;
  a.scale = scale_of(p);
  a.scale_log2 = a.scale * kLog2e;
  const int64_t items = (int64_t)p.B * p.Hq * nqb;
  if (items > INT_MAX) return BSA_ERR_UNSUPPORTED;
  a.n_items = (int)items;
  const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  launch_gated(a, true, st);
  if (hipPeekAtLastError() != hipSuccess) return launch_status();
  launch_threshold(ThresholdArgs{tile_max, T, p.B, p.Hq, nqb, k_keep}, st);
  return launch_status();
}

static bsa_status vs_convert_impl(const int32_t* q_seqlens, const int32_t* kv_seqlens, const int32_t* vertical,
                                  const int32_t* slash, const int32_t* v_count, const int32_t* s_count, int32_t B,
                                  int32_t H, int32_t nnz_v, int32_t nnz_s, int32_t context_size, int32_t block_M,
                                  int32_t block_N, int32_t causal, int32_t* block_count, int32_t* block_offset,
                                  int32_t* column_count, int32_t* column_index, bsa_stream stream) {
  if (!q_seqlens || !kv_seqlens || !block_count || !column_count) return BSA_ERR_INVALID_ARG;
  if (B <= 0 || H <= 0 || nnz_v < 0 || nnz_s < 0 || context_size <= 0 || block_M <= 0 || block_N <= 0)
    return BSA_ERR_INVALID_ARG;
  if ((nnz_v > 0 && (!vertical || !column_index)) || (nnz_s > 0 && (!slash || !block_offset)))
    return BSA_ERR_INVALID_ARG;
  if (!causal || block_M > block_N) return BSA_ERR_UNSUPPORTED;
  VSConvArgs a{q_seqlens, kv_seqlens, vertical, slash, v_count, s_count, B, H, nnz_v, nnz_s, 0, block_M, block_N,
               block_count, block_offset, column_count, column_index};
  a.rows = (context_size + block_M - 1) / block_M;
  launch_vs_convert(a, reinterpret_cast<hipStream_t>(stream));
  return launch_status();
}

bsa_status bsa_check_pattern(const bsa_problem* prob, const bsa_pattern* pat, int32_t* result, bsa_stream stream) {
  if (!prob || !pat || !result || (reinterpret_cast<uintptr_t>(result) & 3)) return BSA_ERR_INVALID_ARG;
  const bsa_problem& p = *prob;
  if (p.B <= 0 || p.Hq <= 0 || p.Hkv <= 0 || p.Sq <= 0 || p.Sk <= 0 || p.Hq % p.Hkv) return BSA_ERR_INVALID_ARG;
  if ((p.cu_seqlens_q == nullptr) != (p.cu_seqlens_k == nullptr)) return BSA_ERR_INVALID_ARG;
  if (p.cu_seqlens_q && (p.max_seqlen_q <= 0 || p.max_seqlen_k <= 0)) return BSA_ERR_INVALID_ARG;
  const bsa_status st = check_pattern(p, pat);
  if (st != BSA_OK) return st;
  if (pat->kind == BSA_PAT_DENSE) return BSA_ERR_INVALID_ARG;
  launch_check(check_args(p, pat, result), reinterpret_cast<hipStream_t>(stream));
  return launch_status();
}

bsa_status vs_convert_indexes(const int32_t* q_seqlens, const int32_t* kv_seqlens, const int32_t* vertical,
                              const int32_t* slash, int32_t B, int32_t H, int32_t nnz_v, int32_t nnz_s,
                              int32_t context_size, int32_t block_M, int32_t block_N, int32_t causal,
                              int32_t* block_count, int32_t* block_offset, int32_t* column_count,
                              int32_t* column_index, bsa_stream stream) {
  return vs_convert_impl(q_seqlens, kv_seqlens, vertical, slash, nullptr, nullptr, B, H, nnz_v, nnz_s, context_size,
                         block_M, block_N, causal, block_count, block_offset, column_count, column_index, stream);
}

bsa_status vs_convert_indexes_mergehead(const int32_t* q_seqlens, const int32_t* kv_seqlens,
                                        const int32_t* vertical, const int32_t* slash,
                                        const int32_t* vertical_count, const int32_t* slash_count, int32_t B,
                                        int32_t H, int32_t nnz_v, int32_t nnz_s, int32_t context_size,
                                        int32_t block_M, int32_t block_N, int32_t causal, int32_t* block_count,
                                        int32_t* block_offset, int32_t* column_count, int32_t* column_index,
                                        bsa_stream stream) {
  if (!vertical_count || !slash_count) return BSA_ERR_INVALID_ARG;
  return vs_convert_impl(q_seqlens, kv_seqlens, vertical, slash, vertical_count, slash_count, B, H, nnz_v, nnz_s,
                         context_size, block_M, block_N, causal, block_count, block_offset, column_count,
                         column_index, stream);
}

}  // extern "C"
