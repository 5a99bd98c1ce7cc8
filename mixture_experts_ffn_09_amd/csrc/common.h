// Shared device helpers of the gfx950 MoE FFN kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float floatx4_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float floatx16_t;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2_t;

#define MOE_WAVE 64
#define MOE_MAX_EXPERTS 1024
#define MOE_FP8_BLOCK 128

// bfloat16 <-> float32.  bf16 is the top half of a binary32 word.
__device__ __forceinline__ float bf16_to_f32(uint32_t b16) {
  return __uint_as_float(b16 << 16);
}

// Round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
}

// Logistic function in float32 (no overflow: exp of a non-positive value).
__device__ __forceinline__ float sigmoid_f32(float z) {
  float e = __expf(-fabsf(z));
  float p = 1.0f / (1.0f + e);
  return z >= 0.0f ? p : e * p;
}

// silu(z) = z / (1 + e^-z) with the hardware exponential and reciprocal
// (about 1 ulp each; the result is rounded to bfloat16 or used in float32
// with a tolerance far above that).  z -> -inf: e^-z overflows to inf and
// the product is -0; z -> +inf: z.
__device__ __forceinline__ float silu_f32(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

// Two floats -> two bfloat16 in one dword (lo in the low half), rounded to
// nearest even by the hardware conversion.
__device__ __forceinline__ uint32_t pack_bf16x2_rne(float lo, float hi) {
  typedef float f2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 b2_t __attribute__((ext_vector_type(2)));
  const f2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, b2_t));
}

// Two OCP E4M3 codes (the low or high 16 bits of `w`) -> two bf16 in one
// dword.  E4M3 values are exact in bf16, so the conversion is exact.
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w) {
  typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
  bf16x2_t v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI);
  return __builtin_bit_cast(uint32_t, v);
}

// 8 E2M1 codes (one 32-bit word, element 2i in the low nibble of byte i) ->
// 8 bf16 = one MFMA operand, each times 2^(e - 127) (exact: an E2M1 value
// times a power of two is a bf16 value; e = 0 scales by 2^-127, e = 255 is
// the E8M0 NaN).  The conversion takes the exponent field of its float scale
// operand as an E8M0 exponent, so the byte shifted into that field is the
// scale as it stands: for every one of the 256 codes and all 16 E2M1 values
// this decodes bit for bit like the float 2^(e - 127) (the subnormal 2^-127
// for e = 0, a NaN for e = 255) on gfx950, without the selects those two
// codes would otherwise need.
__device__ __forceinline__ u32x4_t fp4_word_to_bf16(uint32_t q, uint32_t e) {
  const float sc = __uint_as_float(e << 23);
  u32x4_t r;
  r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, sc, 0));
  r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, sc, 1));
  r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, sc, 2));
  r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, sc, 3));
  return r;
}

__device__ __forceinline__ floatx4_t mfma16x16x32(const u32x4_t& a, const u32x4_t& b,
                                                  floatx4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Fourth dword of a raw buffer resource on gfx950 (32-bit data format, no
// swizzle), as used for bounds-checked byte-addressed loads.
constexpr int BUF_DWORD3 = 0x00020000;

// s_waitcnt vmcnt(N) leaving the other counters untouched (gfx9 encoding:
// vmcnt low bits 3:0 and high bits 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier without the release/acquire fences of __syncthreads():
// those would wait for every outstanding global-to-LDS copy (vmcnt(0)) and
// drain the ring.  The copies are ordered by explicit wait_vmcnt() instead;
// the empty asm statements keep the compiler from moving memory accesses
// across the barrier.
__device__ __forceinline__ void barrier_no_fence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__host__ __device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Instruction-scheduling patterns for software-pipelined MFMA loops (masks:
// 0x008 MFMA, 0x100 LDS read, 0x010 vector memory).
// MFMA slices and LDS reads of one copy group: D reads, each preceded by a
// share of M MFMAs, then the rest of the MFMAs.
template <int I, int D, int M>
__device__ __forceinline__ void group_pattern() {
  if constexpr (I < D) {
    constexpr int m = (I + 1) * M / (D + 1) - I * M / (D + 1);
    if constexpr (m > 0) __builtin_amdgcn_sched_group_barrier(0x008, m, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    group_pattern<I + 1, D, M>();
  } else {
    constexpr int m = M - D * M / (D + 1);
    if constexpr (m > 0) __builtin_amdgcn_sched_group_barrier(0x008, m, 0);
  }
}

// NB groups of V VALU instructions (an operand decode), each followed by its
// share of M MFMAs.
template <int Q, int NB, int V, int M>
__device__ __forceinline__ void decode_pattern() {
  if constexpr (Q < NB) {
    constexpr int m = (Q + 1) * M / NB - Q * M / NB;
    __builtin_amdgcn_sched_group_barrier(0x002, V, 0);
    if constexpr (m > 0) __builtin_amdgcn_sched_group_barrier(0x008, m, 0);
    decode_pattern<Q + 1, NB, V, M>();
  }
}

// Scheduling pattern of one step: group q of LPS issues one copy, then its
// share of the NRD fragment reads interleaved with its share of the NMF MFMAs.
template <int Q, int LPS, int NRD, int NMF>
__device__ __forceinline__ void stage_pattern() {
  if constexpr (Q < LPS) {
    constexpr int d = (Q + 1) * NRD / LPS - Q * NRD / LPS;   // reads in this group
    constexpr int m = (Q + 1) * NMF / LPS - Q * NMF / LPS;   // MFMAs in this group
    __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);       // one copy
    group_pattern<0, d, m>();
    stage_pattern<Q + 1, LPS, NRD, NMF>();
  }
}
