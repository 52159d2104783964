// Shared device helpers for the gfx950 attention kernels: vector types, the
// bf16 MFMA builtins, bf16 packing, shuffles and the argument structs the
// host passes to every kernel.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "args.cuh"

namespace bsa {

// Workgroup and thread indices straight from the hardware registers (the builtins stay
// inline whatever floating-point mode a kernel is compiled in; the library calls behind
// blockIdx / threadIdx are not inlined into kernels built without IEEE mode, which turns
// every value derived from them into a per-lane one).
__device__ __forceinline__ int wg_x() { return (int)__builtin_amdgcn_workgroup_id_x(); }
__device__ __forceinline__ int tid_x() { return (int)__builtin_amdgcn_workitem_id_x(); }

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;
constexpr float kNegInf = -__builtin_inff();
constexpr float kPosInf = __builtin_inff();

// ---------------------------------------------------------------------------
// Small helpers
// ---------------------------------------------------------------------------

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Logit soft-capping ("Implementation: Sgl project Sglang Sparse Flash Attention",
// Signature: softcap, 0 = off), applied to the raw score s = <q, k> so that the
// softmax scale still multiplies it afterwards: with cap c and scale t,
//   s <- (c / t) tanh(t s / c) = cap_out (1 - 2 / (2^(cap_in s) + 1)),
// cap_in = 2 t log2(e) / c, cap_out = c / t.  2^x overflowing to +inf gives
// cap_out, underflowing to 0 gives -cap_out; near 0 the absolute error is a few
// float32 ulps of cap_out.
__device__ __forceinline__ float softcap_score(float s, float cap_in, float cap_out) {
  const float e = exp2_fast(s * cap_in);
  return fmaf(-2.f * cap_out, __builtin_amdgcn_rcpf(e + 1.f), cap_out);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Round two floats to bf16 (nearest-even) and pack, lo in bits 0..15: one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// acc + (both bf16 values packed in u), as one v_dot2_f32_bf16 against (1, 1).
__device__ __forceinline__ float bf16x2_sum_acc(uint32_t u, float acc) {
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, u), ones, acc, false);
}

// 16-bit halves of two dwords, one v_perm_b32 each: (a.lo, b.lo) and (a.hi, b.hi).
__device__ __forceinline__ uint32_t lo_halves(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x05040100u); }
__device__ __forceinline__ uint32_t hi_halves(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x07060302u); }

__device__ __forceinline__ float shfl_xor_f(float v, int mask) { return __shfl_xor(v, mask, 64); }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ bf16x4 as_bf16x4(u32x2 v) { return __builtin_bit_cast(bf16x4, v); }

__device__ __forceinline__ u32x4 ldg128(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16x16x16(bf16x4 a, bf16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// Store 4 consecutive head-dim values of one output row.
__device__ __forceinline__ void store4(const OutArg& o, int64_t off, float a, float b, float c, float d) {
  if (o.f32) {
    f32x4 v = {a, b, c, d};
    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(o.ptr) + off) = v;
  } else {
    u32x2 v = {pack_bf16x2(a, b), pack_bf16x2(c, d)};
    *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(o.ptr) + off) = v;
  }
}

}  // namespace bsa
