// Route packing on gfx950: group token x expert routes by local expert into a padded,
// power-of-two-capacity workspace (FlashInfer PR 4255, Description: shape-stable route
// packing; Tests: expert_map and invalid expert ids). One 1024-thread workgroup does the
// whole pack; for the grouped-GEMM path with NVFP4 weights every other workgroup of the
// same launch converts the activation rows to f16 (exact up to f16 subnormals, below
// 2^-38 of the row maximum) times a per-token power of two, so that no separate launch is
// needed.
#include <hip/hip_runtime.h>

#include "kernels.hpp"
#include "layout.hpp"

namespace moe {

namespace {

constexpr int kPackThreads = 1024;
constexpr int kPackWaves = kPackThreads / 64;

__device__ __forceinline__ int local_expert(const RoutePackParams& p, int64_t r) {
  if (r >= p.num_routes) return -1;
  int g = p.topk_ids[r];
  if (g < 0 || g >= p.num_global_experts) return -1;
  int l = p.expert_map ? p.expert_map[g] : g;
  return (l >= 0 && l < p.num_experts) ? l : -1;
}

// Exclusive scan of one int per thread over the 1024-thread workgroup.
__device__ int block_exclusive_scan(int v, int* wave_tot, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane == 63) wave_tot[w] = x;
  __syncthreads();
  if (w == 0) {
    int t = lane < kPackWaves ? wave_tot[lane] : 0;
    int s = t;
#pragma unroll
    for (int d = 1; d < kPackWaves; d <<= 1) {
      int y = __shfl_up(s, d, 64);
      if (lane >= d) s += y;
    }
    if (lane < kPackWaves) wave_tot[lane] = s - t;       // exclusive wave base
    if (lane == kPackWaves - 1) wave_tot[kPackWaves] = s;  // workgroup total
  }
  __syncthreads();
  int r = x - v + wave_tot[w];
  *total = wave_tot[kPackWaves];
  __syncthreads();
  return r;
}

__device__ void pack_routes(const RoutePackParams& p, uint8_t* smem) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = p.num_experts, B = p.block_m;
  int* cnt = reinterpret_cast<int*>(smem);                 // [E] counts, then running slot
  int* wave_tot = cnt + E;                                 // [32] scan scratch; [20] = valid routes
  uint8_t* wcnt = reinterpret_cast<uint8_t*>(wave_tot + 32);  // [kPackWaves][E] per-wave counts

  // The first chunk's local id and router weight stay in registers for the scatter, so
  // small batches read topk_ids / expert_map / topk_weights from memory only once.
  const int l_first = local_expert(p, tid);
  const float w_first = (p.topk_weights && tid < p.num_routes) ? p.topk_weights[tid] : 0.f;
  for (int e = tid; e < E; e += kPackThreads) cnt[e] = 0;
  if (tid == 0) wave_tot[kPackWaves + 4] = 0;
  for (int i = tid; i < kPackWaves * E; i += kPackThreads) wcnt[i] = 0;
  __syncthreads();
  if (l_first >= 0) atomicAdd(&cnt[l_first], 1);
  for (int64_t r = kPackThreads + tid; r < p.num_routes; r += kPackThreads) {
    int l = local_expert(p, r);
    if (l >= 0) atomicAdd(&cnt[l], 1);
  }
  __syncthreads();

  // Padded segment offsets and the M-tile table, kPackThreads experts per pass of the scan.
  // Full tiles (kTileBlocks blocks) come first, then each expert's partial tail tile, so a
  // queue that hands the tiles out in order starts the longest work first.
  int carry = 0, tile_carry = 0;
  for (int base = 0; base < E; base += kPackThreads) {
    int e = base + tid;
    int c = e < E ? cnt[e] : 0;
    int padded = (c + B - 1) / B * B;
    int nfull = padded / B / kTileBlocks;
    int tot, ttot;
    int off = block_exclusive_scan(padded, wave_tot, &tot) + carry;
    int toff = block_exclusive_scan(nfull, wave_tot, &ttot) + tile_carry;
    if (e < E) {
      p.expert_counts[e] = c;
      p.expert_offsets[e] = off;
      for (int b = off / B; b < (off + padded) / B; ++b) p.block_expert[b] = e;
      for (int s = off + c; s < off + padded; ++s) {
        p.sorted_route_ids[s] = -1;
        if (p.slot_info) p.slot_info[s] = make_int2(-1, 0);
      }
      if (p.tiles) {
        for (int t = 0; t < nfull; ++t)
          p.tiles[toff + t] = make_int2(off / B + t * kTileBlocks, kTileBlocks | (e << 8));
      }
      cnt[e] = off;                                        // running slot of expert e
    }
    carry += tot;
    tile_carry += ttot;
  }
  const int total_padded = carry;
  const int full_tiles = tile_carry;
  if (p.tiles) {
    // Partial tiles after all full ones. Thread e reads back the offsets it wrote above.
    for (int base = 0; base < E; base += kPackThreads) {
      int e = base + tid;
      int blocks = 0, off = 0;
      if (e < E) {
        off = p.expert_offsets[e];
        blocks = (p.expert_counts[e] + B - 1) / B;
      }
      int rem = blocks % kTileBlocks;
      int ttot;
      int toff = block_exclusive_scan(rem > 0 ? 1 : 0, wave_tot, &ttot) + tile_carry;
      if (rem > 0) p.tiles[toff] = make_int2(off / B + blocks - rem, rem | (e << 8));
      tile_carry += ttot;
    }
  }
  if (tid == 0) {
    p.expert_offsets[E] = total_padded;
    p.live[1] = total_padded;
    p.live[2] = total_padded / B;
    p.live[3] = int(p.m);
    p.live[4] = tile_carry;
    p.live[5] = full_tiles;
  }
  if (tid < 16) p.live[8 + tid] = 0;                       // grouped-GEMM work queues: 8 per phase
  for (int64_t s = total_padded + tid; s < p.cap_routes; s += kPackThreads) {
    p.sorted_route_ids[s] = -1;
    if (p.slot_info) p.slot_info[s] = make_int2(-1, 0);
  }
  for (int64_t b = total_padded / B + tid; b < p.cap_blocks; b += kPackThreads) p.block_expert[b] = -1;
  for (int64_t r = p.num_routes + tid; r < p.cap_k; r += kPackThreads) p.route_slot[r] = -1;
  __syncthreads();

  // Stable scatter, 1024 routes per chunk: rank inside the wave by matching equal expert
  // ids, then add the counts of lower waves of the chunk and the running slot.
  int valid_total = 0;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int64_t base = 0; base < p.num_routes; base += kPackThreads) {
    const int64_t r = base + tid;
    const int l = base == 0 ? l_first : local_expert(p, r);
    int rank = 0;
    uint64_t todo = __ballot(l >= 0);
    valid_total += __popcll(todo);
    while (todo) {
      const int leader = __ffsll((long long)todo) - 1;
      const int ev = __builtin_amdgcn_readlane(l, leader);
      const uint64_t same = __ballot(l == ev);
      if (l == ev) {
        rank = __popcll(same & lt_mask);
        if (lane == leader) wcnt[wave * E + ev] = (uint8_t)__popcll(same);
      }
      todo &= ~same;
    }
    __syncthreads();
    if (l >= 0) {
      int pos = cnt[l] + rank;
      for (int w2 = 0; w2 < wave; ++w2) pos += wcnt[w2 * E + l];
      p.sorted_route_ids[pos] = int(r);
      p.route_slot[r] = pos;
      if (p.slot_info) {
        const float wt = base == 0 ? w_first : (p.topk_weights ? p.topk_weights[r] : 0.f);
        p.slot_info[pos] = make_int2(int(r / p.topk), __float_as_int(wt));
      }
    } else if (r < p.num_routes) {
      p.route_slot[r] = -1;
    }
    if (base + kPackThreads < p.num_routes) {                // more chunks: advance the running slots
      __syncthreads();
      for (int e = tid; e < E; e += kPackThreads) {
        int add = 0;
        for (int w2 = 0; w2 < kPackWaves; ++w2) {
          add += wcnt[w2 * E + e];
          wcnt[w2 * E + e] = 0;
        }
        cnt[e] += add;
      }
      __syncthreads();
    }
  }
  // valid_total is per wave (ballots are wave-wide); lane 0 of each wave adds its share.
  if (lane == 0) atomicAdd(&wave_tot[kPackWaves + 4], valid_total);
  __syncthreads();
  if (tid == 0) p.live[0] = wave_tot[kPackWaves + 4];
}

}  // namespace

__global__ __launch_bounds__(kPackThreads) void route_pack_kernel(RoutePackParams p) {
  extern __shared__ __align__(16) uint8_t smem[];
  if (blockIdx.x == 0) {
    pack_routes(p, smem);
    return;
  }
  // One wave per activation row: row maximum, exponent p with max * 2^-p in [2^14, 2^15),
  // then the scaled f16 row (hidden % 8 == 0: 16-byte chunks).
  const int lane = threadIdx.x & 63;
  const int64_t waves = int64_t(gridDim.x - 1) * (blockDim.x / 64);
  const int64_t chunks = p.hidden / 8;
  for (int64_t t = int64_t(blockIdx.x - 1) * (blockDim.x / 64) + (threadIdx.x >> 6); t < p.m; t += waves) {
    const uint4* row = reinterpret_cast<const uint4*>(p.x + t * p.hidden);
    float amax = 0.f;
    for (int64_t c = lane; c < chunks; c += 64) {
      const uint4 v = row[c];
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; ++i)
        amax = fmaxf(amax, fmaxf(fabsf(__uint_as_float(w[i] << 16)), fabsf(__uint_as_float(w[i] & 0xFFFF0000u))));
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) amax = fmaxf(amax, __shfl_xor(amax, d, 64));
    int e = 0;
    if (amax > 0.f && amax <= 3.4e38f) (void)frexpf(amax, &e);   // amax = f * 2^e, f in [0.5, 1)
    const int pexp = amax > 0.f && amax <= 3.4e38f ? e - 15 : 0;
    const float inv = ldexpf(1.f, -pexp);
    uint4* dst = reinterpret_cast<uint4*>(p.x16 + t * p.hidden);
    for (int64_t c = lane; c < chunks; c += 64) {
      const uint4 v = row[c];
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
      uint32_t o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const _Float16 lo = (_Float16)(__uint_as_float(w[i] << 16) * inv);
        const _Float16 hi = (_Float16)(__uint_as_float(w[i] & 0xFFFF0000u) * inv);
        o[i] = uint32_t(__builtin_bit_cast(uint16_t, lo)) | (uint32_t(__builtin_bit_cast(uint16_t, hi)) << 16);
      }
      dst[c] = make_uint4(o[0], o[1], o[2], o[3]);
    }
    if (lane == 0) p.xexp[t] = pexp;
  }
}

size_t route_pack_lds_bytes(int num_experts) {
  return size_t(num_experts) * 4 + 32 * 4 + size_t(kPackWaves) * num_experts + 16;
}

hipError_t launch_route_pack(const RoutePackParams& p, int side_blocks, hipStream_t stream) {
  const size_t lds = route_pack_lds_bytes(p.num_experts);
  hipLaunchKernelGGL(route_pack_kernel, dim3(1 + (p.x16 ? side_blocks : 0)), dim3(kPackThreads), lds, stream, p);
  return hipGetLastError();
}

}  // namespace moe
