// Router front end on gfx950: top-k experts of each token's router logits and their
// weights (FlashInfer PR 4255, Summary: configurable routing; Walkthrough: routing modes).
//
// One wave per token. Lane l holds the logits of experts l + 64 i as 64-bit keys
// (order-preserving bits of the fp32 value, then the complement of the expert id), so the
// largest key is the largest logit and, among equal logits, the lowest id. k rounds of a
// wave-wide key maximum pick the experts in order; the winner's lane clears its key. Lane j
// keeps the j-th pick, and the weights are the softmax (or sigmoid) scores of the picks,
// renormalised over the k of them or not. Loads of one token's logits are coalesced; the
// kernel is bound by reading m x E x 4 bytes.
#include <hip/hip_runtime.h>

#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kRouterThreads = 256;
constexpr int kRouterWaves = kRouterThreads / 64;

__device__ __forceinline__ uint64_t router_key(float v, int e) {
  if (v == 0.f) v = 0.f;                                      // -0 and +0 are equal logits
  const uint32_t b = __float_as_uint(v);
  const uint32_t ord = (b & 0x80000000u) ? ~b : (b | 0x80000000u);   // increasing in v
  return (uint64_t(ord) << 32) | uint32_t(0xFFFFFFFFu - uint32_t(e));
}

__device__ __forceinline__ float key_value(uint64_t key) {
  const uint32_t ord = uint32_t(key >> 32);
  return __uint_as_float((ord & 0x80000000u) ? (ord & 0x7FFFFFFFu) : ~ord);
}

__device__ __forceinline__ uint64_t wave_max(uint64_t k) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    const uint64_t o = __shfl_xor(k, d, 64);
    k = o > k ? o : k;
  }
  return k;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
  return v;
}

template <int PER>
__global__ __launch_bounds__(kRouterThreads) void router_kernel(RouterParams p) {
  const int lane = threadIdx.x & 63;
  const int64_t t = int64_t(blockIdx.x) * kRouterWaves + (threadIdx.x >> 6);
  if (t >= p.m) return;                                       // whole waves only
  const float* row = p.logits + t * p.num_experts;
  uint64_t key[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = lane + 64 * i;
    key[i] = e < p.num_experts ? router_key(row[e], e) : 0ull;   // 0: absent (below every real key)
  }
  int my_id = -1;
  float my_val = 0.f;
  for (int j = 0; j < p.topk; ++j) {
    uint64_t best = 0ull;
#pragma unroll
    for (int i = 0; i < PER; ++i) best = key[i] > best ? key[i] : best;
    best = wave_max(best);
    const int e = int(0xFFFFFFFFu - uint32_t(best));
#pragma unroll
    for (int i = 0; i < PER; ++i)
      if (lane == (e & 63) && i == (e >> 6)) key[i] = 0ull;   // taken
    if (lane == j) {
      my_id = e;
      my_val = key_value(best);
    }
  }
  // Scores of the picks (lanes j < k), in float32.
  const bool mine = lane < p.topk;
  const float top = __shfl(my_val, 0, 64);                    // the largest logit
  float s = 0.f;
  if (p.scoring == 0) {
    s = mine ? expf(my_val - top) : 0.f;
    if (!p.renormalize) {
      float z = 0.f;                                          // full softmax denominator over every expert
      for (int e = lane; e < p.num_experts; e += 64) z += expf(row[e] - top);
      const float zs = wave_sum(z);
      if (mine) {
        p.topk_ids[t * p.topk + lane] = my_id;
        p.topk_weights[t * p.topk + lane] = s / zs;
      }
      return;
    }
  } else {
    s = mine ? 1.f / (1.f + expf(-my_val)) : 0.f;
  }
  const float denom = p.renormalize ? wave_sum(s) : 1.f;
  if (mine) {
    p.topk_ids[t * p.topk + lane] = my_id;
    p.topk_weights[t * p.topk + lane] = s / denom;
  }
}

}  // namespace

hipError_t launch_router(const RouterParams& p, hipStream_t stream) {
  if (p.m == 0) return hipSuccess;
  const int64_t blocks = (p.m + kRouterWaves - 1) / kRouterWaves;
  const int per = (p.num_experts + 63) / 64;
  if (per <= 2) hipLaunchKernelGGL(router_kernel<2>, dim3(blocks), dim3(kRouterThreads), 0, stream, p);
  else if (per <= 4) hipLaunchKernelGGL(router_kernel<4>, dim3(blocks), dim3(kRouterThreads), 0, stream, p);
  else if (per <= 8) hipLaunchKernelGGL(router_kernel<8>, dim3(blocks), dim3(kRouterThreads), 0, stream, p);
  else hipLaunchKernelGGL(router_kernel<16>, dim3(blocks), dim3(kRouterThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace moe
