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
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));

// D += A * B for a 16x16x32 bf16 step. Lane l holds A[l%16][8*(l/16) + j] and
// B[8*(l/16) + j][l%16] (j = 0..7); D row 4*(l/16) + i, column l%16 in element i.
__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Same for the f16 MFMA (identical lane layout).
__device__ __forceinline__ f32x4 mfma16h(const f16x8& a, const f16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Four scale bytes of one K block (byte s = the scale of MFMA step s) -> four floats.
// NVFP4: OCP E4M3FN values, decoded by the hardware FP8 convert (exact, subnormals included).
// MXFP4: the float whose exponent field is the E8M0 byte. The gfx950 scaled FP4 converts
// apply only the exponent of their f32 scale operand, so this is exactly 2^(b-127) as far
// as they are concerned (b = 0 gives 2^-127).
template <int FMT>
__device__ __forceinline__ void decode_scales(uint32_t w, float s[4]);
template <>
__device__ __forceinline__ void decode_scales<1>(uint32_t w, float s[4]) {
  const f32x2 lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, false);
  const f32x2 hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, true);
  s[0] = lo[0];
  s[1] = lo[1];
  s[2] = hi[0];
  s[3] = hi[1];
}
template <>
__device__ __forceinline__ void decode_scales<2>(uint32_t w, float s[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) s[i] = __uint_as_float(((w >> (8 * i)) & 0xFFu) << 23);
}

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

// Dequantise one lane's share of a K-step to bf16: `q` holds 8 codes, `scale` comes from
// decode_scales.
template <int FMT>
__device__ __forceinline__ bf16x8 dq8(uint32_t q, float scale);
template <>
__device__ __forceinline__ bf16x8 dq8<1>(uint32_t q, float scale) { return dq8_scaled(q, scale); }
template <>
__device__ __forceinline__ bf16x8 dq8<2>(uint32_t q, float scale) { return dq8_pow2(q, scale); }

// NVFP4 to f16. The four E4M3 scale bytes of a K block (byte s = the scale of MFMA step s)
// decode exactly to f16 (every E4M3 value, subnormals, sign and NaN included, is an f16
// value), two per hardware FP8 convert: pair 0 holds steps 0 and 1, pair 1 steps 2 and 3.
struct NvScalesF16 {
  f16x2 p[2];
  __device__ __forceinline__ _Float16 step(int s) const { return p[s >> 1][s & 1]; }
};
__device__ __forceinline__ NvScalesF16 nv_scales_f16(uint32_t w) {
  NvScalesF16 r;
  r.p[0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);
  r.p[1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true);
  return r;
}
// 8 E2M1 codes times one E4M3 scale (as f16) -> 8 f16: the FP4 convert gives the E2M1 values,
// one packed multiply (the scale taken from one half of its register) applies the scale. Every
// E2M1 x E4M3 product lies in [2^-10, 2688] with at most 6 significant bits, so the f16
// result is exact -- at half the VALU work of the f32 route.
__device__ __forceinline__ f16x8 dq8_nv_f16(uint32_t q, _Float16 scale) {
  const f16x2 m = {scale, scale};
  f16x2 v[4];
  v[0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q, 1.0f, 0) * m;
  v[1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q, 1.0f, 1) * m;
  v[2] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q, 1.0f, 2) * m;
  v[3] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q, 1.0f, 3) * m;
  return __builtin_bit_cast(f16x8, v);
}

__device__ __forceinline__ f16x8 zero_f16x8() {
  u32x4 z = {0u, 0u, 0u, 0u};
  return __builtin_bit_cast(f16x8, z);
}

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
constexpr uint32_t kOutOfRange = 0x80000000u;           // set in a buffer offset: past every num_records, loads 0

// s_waitcnt with only the vector-memory counter bounded (gfx9 encoding: vmcnt in bits 3:0
// and 15:14; expcnt and lgkmcnt at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit counter");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// A pointer the compiler cannot prove wave-uniform, moved to scalar registers (it is uniform).
__device__ __forceinline__ void* uniform_ptr(const void* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(v >> 32));
  return reinterpret_cast<void*>((uint64_t(hi) << 32) | lo);
}

// 16 bytes per lane from a buffer into LDS at lds_dst + 16 * lane.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, const uint8_t* lds_dst, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_dst, 16, int(voff), 0, 0, 0);
}

// The same with a wave-uniform part of the offset in the scalar offset (no VALU add per load).
__device__ __forceinline__ void dma16s(__amdgpu_buffer_rsrc_t r, const uint8_t* lds_dst, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_dst, 16, int(voff), int(soff), 0, 0);
}

// 4 bytes per lane from a buffer into LDS at lds_dst + 4 * lane.
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, const void* lds_dst, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_dst, 4, int(voff), 0, 0, 0);
}

// Buffer resource over `bytes` bytes at p (raw, no stride; loads past the end return 0).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(p), 0, int(bytes), 0x00020000);
}

// Load through the scalar cache: `i` must be wave-uniform and the data must not change
// during the launch (it was written by an earlier launch).
__device__ __forceinline__ int32_t scalar_load(const int32_t* p, int i) {
  return ((const __attribute__((address_space(4))) int32_t*)p)[i];
}
__device__ __forceinline__ float scalar_load(const float* p, int i) {
  return ((const __attribute__((address_space(4))) float*)p)[i];
}

// FC1's activation output: four consecutive intermediate columns of one slot row, in bf16
// (W4A16), or in fp32 for the W4A8 variant's MXFP8 rounding pass (rounding to bf16 first
// would round twice: a bf16 value lies on an E4M3 midpoint once in 16). P: the fused-layer
// parameter block.
template <typename P>
__device__ __forceinline__ void store_inter4(const P& p, int64_t slot, int64_t col, const float* v) {
  if (p.w4a8)
    *reinterpret_cast<f32x4*>(p.inter32 + slot * p.g.ip + col) = f32x4{v[0], v[1], v[2], v[3]};
  else
    *reinterpret_cast<uint2*>(p.inter + slot * p.g.ip + col) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
}

__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ float silu_f32(float z) {
  // z * sigmoid(z) with the hardware exp2 and reciprocal; the oracle uses exact exp and the
  // bf16 tolerance absorbs the few-ulp difference.
  return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

// MXFP8 (OCP MX v1.0 with OCP FP8 E4M3FN elements, one E8M0 scale per 32 along K), the W4A8
// variant's FC2 operand. Scale 2^e with e = ceil(log2(amax / 448)) clamped to [-127, 127], so
// the largest element lands in (224, 448] and nothing saturates; codes round to nearest, ties
// to even; an all-zero group stores scale byte 0 and zero codes.

// e for a group maximum amax > 0, exactly: amax = fr 2^ex with fr in [0.5, 1), so amax / 448 =
// (fr / 0.875) 2^(ex - 9) with fr / 0.875 in [0.57, 1.15), above 1 only for fr > 0.875.
__device__ __forceinline__ int mx8_exponent(float amax) {
  const int ex = __builtin_amdgcn_frexp_expf(amax);
  const float fr = __builtin_amdgcn_frexp_mantf(amax);
  const int e = ex - 9 + (fr > 0.875f ? 1 : 0);
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// Round |s| <= 448 to the nearest E4M3FN value, ties to even: 3 fraction bits from 2^-6 up
// (the normal range), multiples of 2^-9 below it (the subnormal range).
__device__ __forceinline__ float e4m3_rne(float s) {
  const float a = fabsf(s);
  float q;
  if (a >= 0.015625f) {
    const uint32_t b = __float_as_uint(a);
    q = __uint_as_float((b + 0x7FFFFu + ((b >> 20) & 1u)) & 0xFFF00000u);
  } else {
    q = __builtin_rintf(a * 512.f) * (1.f / 512.f);
  }
  return copysignf(q, s);
}

// The E4M3FN code of a value q that is already on the grid (|q| <= 448).
__device__ __forceinline__ uint32_t e4m3_code(float q) {
  const uint32_t b = __float_as_uint(q), sign = (b >> 24) & 0x80u;
  const float a = fabsf(q);
  if (a >= 0.015625f) return sign | ((((b >> 23) & 0xFFu) - 120u) << 3) | ((b >> 20) & 7u);   // biased 127 -> 7
  return sign | uint32_t(a * 512.f);                                                          // subnormal: multiples of 2^-9
}

// Four values of one group (scale exponent e, group maximum amax) -> four E4M3 codes, value i
// in byte i.
__device__ __forceinline__ uint32_t mx8_codes4(const float* v, int e, float amax) {
  uint32_t w = 0u;
  if (amax > 0.f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) w |= e4m3_code(e4m3_rne(ldexpf(v[i], -e))) << (8 * i);
  }
  return w;
}

// 4 x 4 transpose of one dword per lane quarter (lanes 16 q .. 16 q + 15): afterwards lane
// (c, q) holds in dword t what lane (c, t) held in dword q. Two rounds of gfx950 lane swaps:
// quarters {0,1} <-> {2,3} between dwords (0, 2) and (1, 3), then quarters 1 <-> 0 and 3 <-> 2
// between dwords (0, 1) and (2, 3).
__device__ __forceinline__ u32x4 transpose_quarters(const u32x4& d) {
  const auto a = __builtin_amdgcn_permlane32_swap(d[0], d[2], false, false);
  const auto b = __builtin_amdgcn_permlane32_swap(d[1], d[3], false, false);
  const auto c = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);
  const auto e = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
  return u32x4{c[0], c[1], e[0], e[1]};
}

}  // namespace moe
