// W4A8 variant of the fused MoE layer: the FC2 operand rounded to MXFP8 between FC1 and FC2.
//
// FlashInfer PR 4255, review: a grouped MXFP8 quantisation of the SiLU-mul output (checked
// there against a Torch reference with the exact silu). MXFP8 per the OCP MX v1.0 and OCP FP8
// specifications: E4M3FN elements with one E8M0 scale per 32 along the intermediate axis, the
// scale being the power-of-two ceiling 2^ceil(log2(amax / 448)) (so nothing saturates), codes
// rounded to nearest, ties to even. Each valid intermediate row (fp32, slot order, written by
// FC1 without the router weight) is rounded and stored as the exact values of its codes into
// the bf16 rows FC2 reads: an E4M3 value times a power of two has at most 4 significant bits,
// so bf16 holds it exactly and FC2 multiplies exactly the MXFP8 operand on the bf16 MFMA. Only
// the decode path's fallback FC2 (routes whose K slices do not fit in its LDS) uses this pass:
// elsewhere the rounding happens inside FC1's epilogue or FC2's staging, to E4M3 codes for the
// block-scaled MFMA.
#include <hip/hip_runtime.h>

#include "device.hpp"
#include "kernels.hpp"
#include "layout.hpp"

namespace moe {

namespace {

constexpr int kRequantThreads = 256;

// Lane l of a wave holds columns 8 l .. 8 l + 7 of a 512-column slice (fp32 in, bf16 out);
// lanes 4 g .. 4 g + 3 hold MX group g of the slice, so the group maximum is two xor shuffles.
__global__ __launch_bounds__(kRequantThreads) void mxfp8_requant_kernel(const float* __restrict__ inter32,
                                                                        uint16_t* __restrict__ inter, int64_t ip,
                                                                        const int32_t* __restrict__ sorted_route_ids,
                                                                        const int32_t* __restrict__ live) {
  const int rows = live[1];                                  // padded slots of this call
  const int lane = threadIdx.x & 63;
  const int64_t waves = int64_t(gridDim.x) * (kRequantThreads / 64);
  const int chunks = int(ip / 8);                            // ip is a multiple of 128: whole groups
  for (int64_t r = int64_t(blockIdx.x) * (kRequantThreads / 64) + (threadIdx.x >> 6); r < rows; r += waves) {
    if (sorted_route_ids[r] < 0) continue;                   // padding slot: never a valid FC2 column
    const float* src = inter32 + r * ip;
    uint16_t* row = inter + r * ip;
    for (int c0 = 0; c0 < chunks; c0 += 64) {
      const int c = c0 + lane;
      const bool in = c < chunks;
      f32x4 v0 = {0.f, 0.f, 0.f, 0.f}, v1 = {0.f, 0.f, 0.f, 0.f};
      if (in) {
        v0 = *reinterpret_cast<const f32x4*>(src + 8 * c);
        v1 = *reinterpret_cast<const f32x4*>(src + 8 * c + 4);
      }
      const float f[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
      float amax = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
      amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
      amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
      const int e = amax > 0.f ? mx8_exponent(amax) : 0;
      u32x4 o;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t h[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const float q = amax > 0.f ? ldexpf(e4m3_rne(ldexpf(f[2 * i + j], -e)), e) : 0.f;
          h[j] = __float_as_uint(q) >> 16;                   // exact: at most 4 significant bits
        }
        o[i] = h[0] | (h[1] << 16);
      }
      if (in) *reinterpret_cast<u32x4*>(row + 8 * c) = o;
    }
  }
}

}  // namespace

hipError_t launch_mxfp8_requant(const FusedParams& p, hipStream_t stream) {
  // one wave per row, grid-stride over the padded slots (their count is read on the device)
  int64_t grid = (p.cap_blocks * kBlockM + 3) / 4;
  if (grid > 2048) grid = 2048;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(mxfp8_requant_kernel, dim3(grid), dim3(kRequantThreads), 0, stream, p.inter32, p.inter,
                     int64_t(p.g.ip), p.sorted_route_ids, p.live);
  return hipGetLastError();
}

}  // namespace moe
