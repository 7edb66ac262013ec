// Weight preparation: canonical packed FP4 codes and scale bytes -> the gfx950 fragment
// layout (FlashInfer PR 4255, Tests: preparation is lossless and bit-identical across
// source formats and activations; Walkthrough: layout normalisation, scale packing and
// the W13 rotation, read here as interleaving gate and up row groups). Runs once per
// weight load; apart from the NVFP4 FC1 row-norm bounds it is a byte shuffle.
#include <hip/hip_runtime.h>

#include "device.hpp"
#include "kernels.hpp"
#include "layout.hpp"

namespace moe {

namespace {

// Canonical row of prepared row (group rg, row r in group) of FC1; -1 for padding rows.
__device__ __forceinline__ int64_t fc1_row(const PreparedGeom& g, int64_t rg, int r) {
  if (g.act == ACT_SWIGLU) {
    int64_t i = (rg >> 1) * kRowGroup + r;
    return i < g.I ? (rg & 1) * g.I + i : -1;
  }
  int64_t i = rg * kRowGroup + r;
  return i < g.I ? i : -1;
}

// Source row of canonical FC1 row `row`: up-half-first checkpoints swap the halves,
// row-interleaved ones store row i of the first half at 2i and of the second at 2i + 1.
__device__ __forceinline__ int64_t fc1_src_row(const PrepareParams& p, int64_t row) {
  if (row < 0 || p.g.act != ACT_SWIGLU) return row;
  int64_t half = row < p.g.I ? 0 : 1;
  const int64_t i = row - half * p.g.I;
  half ^= p.w13_up_first;
  return p.w13_interleaved ? 2 * i + half : half * p.g.I + i;
}

__device__ __forceinline__ int64_t fc2_row(const PreparedGeom& g, int64_t rg, int r) {
  int64_t i = rg * kRowGroup + r;
  return i < g.H ? i : -1;
}

// One prepared nibble dword: codes of row `row` at K = k0 .. k0+7 (k0 a multiple of 8).
__device__ __forceinline__ uint32_t gather_codes(const uint8_t* src_row, int64_t K, int64_t k0) {
  uint32_t v = 0;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    int64_t byte = k0 / 2 + b;
    if (byte < K / 2) v |= uint32_t(src_row[byte]) << (8 * b);
  }
  return v;
}

template <bool FC1>
__global__ void prepare_nibbles_kernel(PrepareParams p) {
  const PreparedGeom& g = p.g;
  const int64_t groups = FC1 ? g.n1_groups : g.n2_groups;
  const int64_t kbs = FC1 ? g.kb1 : g.kb2;
  const int64_t K = FC1 ? g.H : g.I;
  const int64_t rows_src = FC1 ? (g.act == ACT_SWIGLU ? 2 * g.I : g.I) : g.H;
  const uint8_t* src = FC1 ? p.w13 : p.w2;
  uint32_t* dst = reinterpret_cast<uint32_t*>(p.out + (FC1 ? g.off_nib1 : g.off_nib2));
  const int64_t total = int64_t(g.E) * groups * kbs * 256;   // dwords (64 lanes x 4)
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < total;
       i += int64_t(gridDim.x) * blockDim.x) {
    const int s = int(i & 3);
    const int lane = int((i >> 2) & 63);
    int64_t rest = i >> 8;
    const int64_t kb = rest % kbs; rest /= kbs;
    const int64_t rg = rest % groups;
    const int64_t e = rest / groups;
    const int r = lane & 15;
    const int64_t row = FC1 ? fc1_src_row(p, fc1_row(g, rg, r)) : fc2_row(g, rg, r);
    const int64_t k0 = kb * kKBlock + 32 * s + 8 * (lane >> 4);
    uint32_t v = 0;
    if (row >= 0) v = gather_codes(src + (e * rows_src + row) * (K / 2), K, k0);
    dst[i] = v;
  }
}

template <bool FC1>
__global__ void prepare_scales_kernel(PrepareParams p) {
  const PreparedGeom& g = p.g;
  const int64_t groups = FC1 ? g.n1_groups : g.n2_groups;
  const int64_t kbs = FC1 ? g.kb1 : g.kb2;
  const int64_t per_group = FC1 ? g.sc1_per_group : g.sc2_per_group;
  const int64_t K = FC1 ? g.H : g.I;
  const int64_t rows_src = FC1 ? (g.act == ACT_SWIGLU ? 2 * g.I : g.I) : g.H;
  const bool nv = g.fmt == FMT_NVFP4;
  const int64_t G = nv ? 16 : 32;
  const int64_t ngroups = (K + G - 1) / G;                 // scale groups along K
  const int64_t ngroups_src = p.scale_per_row ? 1 : ngroups;   // stored per row
  const uint8_t* src = FC1 ? p.s13 : p.s2;
  uint8_t* dst = p.out + (FC1 ? g.off_sc1 : g.off_sc2);
  const uint8_t pad = nv ? 0 : 127;   // E4M3 0 or E8M0 2^0: finite, and the padded codes are 0
  const int64_t total = int64_t(g.E) * groups * per_group;
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < total;
       i += int64_t(gridDim.x) * blockDim.x) {
    const int64_t eg = i / per_group;          // e * groups + rg
    const int64_t within = i % per_group;
    const int64_t chunk = within / g.sc_chunk_bytes;
    const int b = int(within % g.sc_chunk_bytes);
    const int s = b & 3, kbm = (b >> 2) & 3;
    int r, h = 0;
    if (nv) { r = (b >> 4) & 15; h = b >> 8; } else { r = b >> 4; }
    const int64_t kb = chunk * kScaleChunkKB + kbm;
    const int64_t grp = nv ? 8 * kb + 2 * s + h : 4 * kb + s;
    const int64_t rg = eg % groups, e = eg / groups;
    const int64_t row = FC1 ? fc1_src_row(p, fc1_row(g, rg, r)) : fc2_row(g, rg, r);
    uint8_t v = pad;
    if (row >= 0 && kb < kbs && grp < ngroups) v = src[(e * rows_src + row) * ngroups_src + (p.scale_per_row ? 0 : grp)];
    dst[i] = v;
  }
}

__global__ void prepare_globals_kernel(PrepareParams p) {
  const PreparedGeom& g = p.g;
  float* d13 = reinterpret_cast<float*>(p.out + g.off_g13);
  float* d2 = reinterpret_cast<float*>(p.out + g.off_g2);
  for (int e = blockIdx.x * blockDim.x + threadIdx.x; e < g.E; e += gridDim.x * blockDim.x) {
    const bool nv = g.fmt == FMT_NVFP4;
    // encode-sense globals: the correctly rounded fp32 quotient 1 / stored
    d13[e] = nv ? (p.global_reciprocal ? __fdiv_rn(1.0f, p.g13[e]) : p.g13[e]) : 1.0f;
    d2[e] = nv ? (p.global_reciprocal ? __fdiv_rn(1.0f, p.g2[e]) : p.g2[e]) : 1.0f;
  }
}

// NVFP4 FC1 row-norm bounds: for each expert the largest Euclidean norm of a dequantised
// (E2M1 x E4M3, global scale excluded) gate row and of an up row; relu2 stores its largest
// row norm in both entries. By Cauchy-Schwarz they bound every FC1 output of a token by the
// norm of its activation row, from which the grouped GEMM picks the power of two that keeps
// each f16 intermediate row in range. One wave per canonical row, a fixed-order sum, and the
// maximum over rows by an integer atomic max on the non-negative fp32 bits (order-free), so
// the bytes do not depend on scheduling.
__global__ void prepare_norms_zero_kernel(PrepareParams p) {
  float* n = reinterpret_cast<float*>(p.out + p.g.off_n13);
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < 2 * p.g.E; i += gridDim.x * blockDim.x) n[i] = 0.f;
}

__global__ void prepare_norms_kernel(PrepareParams p) {
  const PreparedGeom& g = p.g;
  const int lane = threadIdx.x & 63;
  const int64_t rows = g.act == ACT_SWIGLU ? 2 * int64_t(g.I) : g.I;
  const int64_t kbytes = g.H / 2;
  const int64_t ngroups_src = p.scale_per_row ? 1 : (g.H + 15) / 16;
  uint32_t* n13 = reinterpret_cast<uint32_t*>(p.out + g.off_n13);
  const int64_t waves = int64_t(gridDim.x) * (blockDim.x / 64);
  for (int64_t w = int64_t(blockIdx.x) * (blockDim.x / 64) + (threadIdx.x >> 6); w < int64_t(g.E) * rows; w += waves) {
    const int64_t e = w / rows, row = w % rows;
    const int64_t src = e * rows + fc1_src_row(p, row);
    const uint8_t* codes = p.w13 + src * kbytes;
    const uint8_t* scales = p.s13 + src * ngroups_src;
    float ss = 0.f;
    for (int64_t b = lane; b < kbytes; b += 64) {
      const uint32_t c = codes[b];
      const float sc = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(uint32_t(scales[p.scale_per_row ? 0 : b / 8]), 1.0f, false)[0];
      const f32x2 v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 0);   // low code, high code
      ss = fmaf(v[0] * sc, v[0] * sc, ss);
      ss = fmaf(v[1] * sc, v[1] * sc, ss);
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) ss += __shfl_xor(ss, d, 64);
    if (lane == 0) {
      const uint32_t bits = __float_as_uint(sqrtf(ss));
      if (g.act == ACT_SWIGLU) {
        atomicMax(n13 + 2 * e + (row < g.I ? 0 : 1), bits);
      } else {
        atomicMax(n13 + 2 * e, bits);
        atomicMax(n13 + 2 * e + 1, bits);
      }
    }
  }
}

int grid_for(int64_t n, int threads) {
  int64_t b = (n + threads - 1) / threads;
  return int(b < 65536 ? (b > 0 ? b : 1) : 65536);
}

}  // namespace

hipError_t launch_prepare(const PrepareParams& p, hipStream_t stream) {
  const PreparedGeom& g = p.g;
  const int T = 256;
  hipLaunchKernelGGL(prepare_nibbles_kernel<true>, dim3(grid_for(int64_t(g.E) * g.n1_groups * g.kb1 * 256, T)),
                     dim3(T), 0, stream, p);
  hipLaunchKernelGGL(prepare_nibbles_kernel<false>, dim3(grid_for(int64_t(g.E) * g.n2_groups * g.kb2 * 256, T)),
                     dim3(T), 0, stream, p);
  hipLaunchKernelGGL(prepare_scales_kernel<true>, dim3(grid_for(int64_t(g.E) * g.n1_groups * g.sc1_per_group, T)),
                     dim3(T), 0, stream, p);
  hipLaunchKernelGGL(prepare_scales_kernel<false>, dim3(grid_for(int64_t(g.E) * g.n2_groups * g.sc2_per_group, T)),
                     dim3(T), 0, stream, p);
  hipLaunchKernelGGL(prepare_globals_kernel, dim3(grid_for(g.E, T)), dim3(T), 0, stream, p);
  hipLaunchKernelGGL(prepare_norms_zero_kernel, dim3(grid_for(2 * int64_t(g.E), T)), dim3(T), 0, stream, p);
  if (g.fmt == FMT_NVFP4) {
    const int64_t rows = int64_t(g.E) * (g.act == ACT_SWIGLU ? 2 * int64_t(g.I) : g.I);
    hipLaunchKernelGGL(prepare_norms_kernel, dim3(grid_for(rows * 64, T)), dim3(T), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace moe
