// Small-batch (decode) path of the fused W4A16 MoE layer on gfx950.
//
// FlashInfer PR 4255, Description: a tensor-core decode path for small batches that folds
// the top-k sum into the FC2 store epilogue and removes a separate launch; Reviewer
// Notes: the decode path is chosen up to a small m. At m <= 16 the layer is bound by the
// weight bytes streamed from HBM, so both kernels are organised around streaming:
//  * FC1: one workgroup (8 waves) per (route block, 16 or 32 FC1 columns); the waves
//    split K, each issues every 128-bit weight load of its K range up front, dequantises
//    in registers straight into MFMA operands (no LDS for weights), and the partial sums
//    meet in LDS. The activation, the expert's FC1 global scale, the router weight and the
//    FC2 global scale are applied once, and the bf16 row goes to the workspace.
//  * FC2: one workgroup per 16 hidden rows, looping over every live route block; route
//    results are summed per token in LDS (the top-k sum) and the bf16 output row slice is
//    stored once -- deterministic, no atomics in global memory.
#include <hip/hip_runtime.h>

#include "device.hpp"
#include "kernels.hpp"
#include "layout.hpp"

namespace moe {

namespace {

constexpr int kDecThreads = 512;
constexpr int kDecWaves = kDecThreads / 64;
constexpr int kKPW = 4;              // K blocks whose loads a wave keeps in flight at once
constexpr int kMaxDecodeTokens = 16;

__device__ __forceinline__ uint32_t scale_dword(const uint8_t* sc_group, int64_t kb, int lane, bool nv) {
  // Scales of K block kb for this lane: NVFP4 chunk [h][row][kb%4][s], MXFP4 [row][kb%4][s].
  const int r = lane & 15;
  const int64_t chunk = kb >> 2;
  const int sub = int(kb & 3);
  const int64_t off = nv ? chunk * 512 + ((lane >> 5) * 16 + r) * 16 + sub * 4 : chunk * 256 + r * 16 + sub * 4;
  return *reinterpret_cast<const uint32_t*>(sc_group + off);
}

__device__ __forceinline__ bf16x8 load_x8(const uint16_t* x, int64_t H, int64_t t, int64_t k) {
  if (t < 0 || k >= H) return zero_bf16x8();
  return load_bf16x8(x + t * H + k);
}

template <int FMT>
__global__ __launch_bounds__(kDecThreads) void decode_fc1_kernel(FusedParams p) {
  __shared__ f32x4 red[kDecWaves][2][64];
  const PreparedGeom& g = p.g;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const bool nv = FMT == FMT_NVFP4;
  const int64_t live_blocks = p.live[2];
  const int64_t n_it = g.n1_groups / 2;                 // items per block: two row groups each
  const int64_t n_items = live_blocks * n_it;
  const int64_t kpw = (g.kb1 + kDecWaves - 1) / kDecWaves;
  const int64_t kb_begin = wave * kpw;
  const int64_t kb_end = min(g.kb1, kb_begin + kpw);
  const int col = lane & 15;

  for (int64_t item = blockIdx.x; item < n_items; item += gridDim.x) {
    const int64_t blk = item / n_it, it = item % n_it;
    const int e = p.block_expert[blk];
    const int64_t slot = blk * kBlockM + col;
    const int2 info = p.slot_info[slot];
    const int64_t tok = info.x;
    const int64_t rg0 = 2 * it, rg1 = 2 * it + 1;
    const uint8_t* nb0 = p.nib1 + ((int64_t(e) * g.n1_groups + rg0) * g.kb1) * kFragBytes + lane * 16;
    const uint8_t* nb1 = p.nib1 + ((int64_t(e) * g.n1_groups + rg1) * g.kb1) * kFragBytes + lane * 16;
    const uint8_t* sg0 = p.sc1 + (int64_t(e) * g.n1_groups + rg0) * g.sc1_per_group;
    const uint8_t* sg1 = p.sc1 + (int64_t(e) * g.n1_groups + rg1) * g.sc1_per_group;
    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};

    for (int64_t kb0 = kb_begin; kb0 < kb_end; kb0 += kKPW) {
      u32x4 q0[kKPW], q1[kKPW];
      uint32_t s0[kKPW], s1[kKPW];
      bf16x8 xb[kKPW][4];
#pragma unroll
      for (int j = 0; j < kKPW; ++j) {
        const int64_t kb = kb0 + j;
        if (kb < kb_end) {
          q0[j] = *reinterpret_cast<const u32x4*>(nb0 + kb * kFragBytes);
          q1[j] = *reinterpret_cast<const u32x4*>(nb1 + kb * kFragBytes);
          s0[j] = scale_dword(sg0, kb, lane, nv);
          s1[j] = scale_dword(sg1, kb, lane, nv);
#pragma unroll
          for (int s = 0; s < 4; ++s) xb[j][s] = load_x8(p.x, g.H, tok, kb * kKBlock + 32 * s + 8 * (lane >> 4));
        }
      }
#pragma unroll
      for (int j = 0; j < kKPW; ++j) {
        if (kb0 + j < kb_end) {
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            const bf16x8 a0 = dq8<FMT>(q0[j][s], (s0[j] >> (8 * s)) & 0xFF);
            const bf16x8 a1 = dq8<FMT>(q1[j][s], (s1[j] >> (8 * s)) & 0xFF);
            acc0 = mfma16(a0, xb[j][s], acc0);
            acc1 = mfma16(a1, xb[j][s], acc1);
          }
        }
      }
    }
    red[wave][0][lane] = acc0;
    red[wave][1][lane] = acc1;
    __syncthreads();
    if (wave == 0) {
      f32x4 h0 = red[0][0][lane], h1 = red[0][1][lane];
      for (int w = 1; w < kDecWaves; ++w) {
        h0 += red[w][0][lane];
        h1 += red[w][1][lane];
      }
      const float g13 = p.g13[e], g2 = p.g2[e];
      const float rw = (tok >= 0) ? __int_as_float(info.y) * g2 : 0.f;
      uint16_t* dst = p.inter + slot * g.ip;
      const int r0 = 4 * (lane >> 4);
      if (g.act == ACT_SWIGLU) {
        float a[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = silu_f32(h0[i] * g13) * (h1[i] * g13) * rw;
        uint2 v = make_uint2(pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]));
        *reinterpret_cast<uint2*>(dst + it * 16 + r0) = v;
      } else {
        float a[4], b[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float u = fmaxf(h0[i] * g13, 0.f), v = fmaxf(h1[i] * g13, 0.f);
          a[i] = u * u * rw;
          b[i] = v * v * rw;
        }
        *reinterpret_cast<uint2*>(dst + rg0 * 16 + r0) = make_uint2(pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]));
        *reinterpret_cast<uint2*>(dst + rg1 * 16 + r0) = make_uint2(pack_bf16x2(b[0], b[1]), pack_bf16x2(b[2], b[3]));
      }
    }
    __syncthreads();
  }
}

template <int FMT>
__global__ __launch_bounds__(kDecThreads) void decode_fc2_kernel(FusedParams p) {
  __shared__ float tacc[kDecWaves][kMaxDecodeTokens][16];
  const PreparedGeom& g = p.g;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const bool nv = FMT == FMT_NVFP4;
  const int64_t ht = blockIdx.x;                          // 16 hidden rows per workgroup
  const int64_t live_blocks = p.live[2];
  const int col = lane & 15;
  for (int i = threadIdx.x; i < kDecWaves * kMaxDecodeTokens * 16; i += kDecThreads) (&tacc[0][0][0])[i] = 0.f;
  __syncthreads();

  for (int64_t blk = wave; blk < live_blocks; blk += kDecWaves) {
    const int e = p.block_expert[blk];
    const int64_t slot = blk * kBlockM + col;
    const int tok = p.slot_info[slot].x;
    const uint16_t* irow = p.inter + slot * g.ip + 8 * (lane >> 4);
    const uint8_t* nb = p.nib2 + ((int64_t(e) * g.n2_groups + ht) * g.kb2) * kFragBytes + lane * 16;
    const uint8_t* sg = p.sc2 + (int64_t(e) * g.n2_groups + ht) * g.sc2_per_group;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int64_t kb0 = 0; kb0 < g.kb2; kb0 += kKPW) {
      u32x4 q[kKPW];
      uint32_t sc[kKPW];
      bf16x8 ib[kKPW][4];
#pragma unroll
      for (int j = 0; j < kKPW; ++j) {
        const int64_t kb = kb0 + j;
        if (kb < g.kb2) {
          q[j] = *reinterpret_cast<const u32x4*>(nb + kb * kFragBytes);
          sc[j] = scale_dword(sg, kb, lane, nv);
#pragma unroll
          for (int s = 0; s < 4; ++s) ib[j][s] = tok >= 0 ? load_bf16x8(irow + kb * kKBlock + 32 * s) : zero_bf16x8();
        }
      }
#pragma unroll
      for (int j = 0; j < kKPW; ++j) {
        if (kb0 + j < g.kb2) {
#pragma unroll
          for (int s = 0; s < 4; ++s) acc = mfma16(dq8<FMT>(q[j][s], (sc[j] >> (8 * s)) & 0xFF), ib[j][s], acc);
        }
      }
    }
    if (tok >= 0) {
      const int r0 = 4 * (lane >> 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) atomicAdd(&tacc[wave][tok][r0 + i], acc[i]);
    }
  }
  __syncthreads();
  // Sum the waves in a fixed order and store the bf16 slice out[t, 16*ht .. 16*ht + 15].
  for (int i = threadIdx.x; i < kMaxDecodeTokens * 16; i += kDecThreads) {
    const int t = i >> 4, j = i & 15;
    const int64_t h = ht * 16 + j;
    if (t < p.m && h < g.H) {
      float s = 0.f;
      for (int w = 0; w < kDecWaves; ++w) s += tacc[w][t][j];
      bf16x2 v;
      v[0] = (__bf16)s;
      p.out[t * g.H + h] = __builtin_bit_cast(uint16_t, v[0]);
    }
  }
}

}  // namespace

hipError_t launch_decode(const FusedParams& p, int num_cus, hipStream_t stream) {
  const int64_t n_it = p.g.n1_groups / 2;
  int64_t items = p.cap_blocks * n_it;
  int64_t grid1 = items < int64_t(num_cus) * 8 ? items : int64_t(num_cus) * 8;
  if (grid1 < 1) grid1 = 1;
  const int64_t grid2 = p.g.n2_groups;
  if (p.g.fmt == FMT_NVFP4) {
    hipLaunchKernelGGL(decode_fc1_kernel<FMT_NVFP4>, dim3(grid1), dim3(kDecThreads), 0, stream, p);
    hipLaunchKernelGGL(decode_fc2_kernel<FMT_NVFP4>, dim3(grid2), dim3(kDecThreads), 0, stream, p);
  } else {
    hipLaunchKernelGGL(decode_fc1_kernel<FMT_MXFP4>, dim3(grid1), dim3(kDecThreads), 0, stream, p);
    hipLaunchKernelGGL(decode_fc2_kernel<FMT_MXFP4>, dim3(grid2), dim3(kDecThreads), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace moe
