// gfx950 device primitives: FP4 dequantisation into MFMA operands, bf16 packing, MFMA wrapper.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// D += A * B for a 16x16x32 bf16 step. Lane l holds A[l%16][8*(l/16) + j] and
// B[8*(l/16) + j][l%16] (j = 0..7); D row 4*(l/16) + i, column l%16 in element i.
__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// E4M3FN byte -> float (OCP FP8): bias 7, exponent field 0 subnormal, S.1111.111 NaN.
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
  uint32_t mag = b & 0x7Fu;
  float f = __uint_as_float((mag << 20) + (120u << 23));           // normal numbers
  if ((mag & 0x78u) == 0) f = float(mag & 7u) * 0x1p-9f;            // subnormals (and zero)
  if (mag == 0x7Fu) f = __uint_as_float(0x7FC00000u);
  return (b & 0x80u) ? -f : f;
}

// E8M0 byte -> the float whose exponent field is that byte. The gfx950 scaled FP4
// converts apply only the exponent of their f32 scale operand, so this is exactly
// 2^(b-127) as far as they are concerned (b = 0 gives 2^-127, b = 255 NaN/inf).
__device__ __forceinline__ float e8m0_as_scale(uint32_t b) { return __uint_as_float(b << 23); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 r;
  r[0] = (__bf16)lo;
  r[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, r);
}

// 8 E2M1 codes (one dword, code j in bits 4j..4j+3) times a power-of-two scale -> 8 bf16.
// Exact: every E2M1 value times 2^e has at most two significant bits.
__device__ __forceinline__ bf16x8 dq8_pow2(uint32_t q, float pow2_scale) {
  u32x4 r;
  r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, pow2_scale, 0));
  r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, pow2_scale, 1));
  r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, pow2_scale, 2));
  r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, pow2_scale, 3));
  return __builtin_bit_cast(bf16x8, r);
}

// 8 E2M1 codes times an arbitrary float scale (an E4M3 value) -> 8 bf16. The product of
// an E2M1 value (2 significant bits) and an E4M3 value (4 significant bits) has at most
// 6 significant bits and lies in [2^-10, 2688], so the bf16 result is exact.
__device__ __forceinline__ bf16x8 dq8_scaled(uint32_t q, float scale) {
  u32x4 r;
  f32x2 v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, 1.0f, 0);
  f32x2 v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, 1.0f, 1);
  f32x2 v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, 1.0f, 2);
  f32x2 v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, 1.0f, 3);
  r[0] = pack_bf16x2(v0[0] * scale, v0[1] * scale);
  r[1] = pack_bf16x2(v1[0] * scale, v1[1] * scale);
  r[2] = pack_bf16x2(v2[0] * scale, v2[1] * scale);
  r[3] = pack_bf16x2(v3[0] * scale, v3[1] * scale);
  return __builtin_bit_cast(bf16x8, r);
}

// Dequantise one lane's share of a K-step: `q` holds 8 codes, `sbyte` the scale byte.
template <int FMT>
__device__ __forceinline__ bf16x8 dq8(uint32_t q, uint32_t sbyte);
template <>
__device__ __forceinline__ bf16x8 dq8<1>(uint32_t q, uint32_t sbyte) { return dq8_scaled(q, e4m3_to_f32(sbyte)); }
template <>
__device__ __forceinline__ bf16x8 dq8<2>(uint32_t q, uint32_t sbyte) { return dq8_pow2(q, e8m0_as_scale(sbyte)); }

__device__ __forceinline__ bf16x8 zero_bf16x8() {
  u32x4 z = {0u, 0u, 0u, 0u};
  return __builtin_bit_cast(bf16x8, z);
}

__device__ __forceinline__ bf16x8 load_bf16x8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

// Workgroup barrier that orders LDS only. __syncthreads() also waits for every outstanding
// global load of the wave (gfx9 counts loads and stores in one vmcnt), which would drain
// the weight prefetch; LDS hand-offs between waves need only lgkmcnt.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ float silu_f32(float z) {
  // z * sigmoid(z) with the hardware exp2 and reciprocal; the oracle uses exact exp and the
  // bf16 tolerance absorbs the few-ulp difference.
  return z * __frcp_rn(1.0f + __expf(-z));
}

}  // namespace moe
