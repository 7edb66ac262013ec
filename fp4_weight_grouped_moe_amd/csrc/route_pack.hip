// Route packing on gfx950: group token x expert routes by local expert into a padded,
// power-of-two-capacity workspace (FlashInfer PR 4255, Description: shape-stable route
// packing; Tests: expert_map and invalid expert ids). One 1024-thread workgroup does the
// whole pack; for the NVFP4 weights' f16 MFMA route every other workgroup of the same
// launch converts the activation rows to f16 (exact up to f16 subnormals, below
// 2^-38 of the row maximum) times a per-token power of two, so that no separate launch is
// needed.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "device.hpp"
#include "kernels.hpp"
#include "layout.hpp"

namespace moe {

namespace {

constexpr int kPackThreads = 1024;
constexpr int kPackWaves = kPackThreads / 64;
constexpr int kValidSlot = 36;                 // scan scratch entries 0 .. 2 kPackWaves + 1 are the scans'
__host__ __device__ inline size_t route_pack_base_lds(int num_experts) {
  // counts, scan scratch, kept counts, per-wave counts; rounded to 16 bytes
  return (size_t(num_experts) * 8 + 40 * 4 + size_t(kPackWaves) * num_experts + 16 + 15) / 16 * 16;
}
constexpr int kRowRegs = 8;                    // 16-byte chunks per lane per batch of the row conversion

// Local expert of route r, or -1 (r at or past the routes in use `rl`, an invalid or unmapped id).
__device__ __forceinline__ int local_expert(const RoutePackParams& p, int64_t r, int64_t rl) {
  if (r >= rl) return -1;
  int g = p.topk_ids[r];
  if (g < 0 || g >= p.num_global_experts) return -1;
  int l = p.expert_map ? p.expert_map[g] : g;
  return (l >= 0 && l < p.num_experts) ? l : -1;
}

// Batches of more than one chunk and at most kCacheRoutes routes over at most kSegExperts
// experts keep every route's local id (int16) in LDS, read once in batches of kLoadBatch
// loads per thread, and scatter by wave segments: wave w ranks its contiguous segment of
// routes 64 at a time against its own running per-expert counts (no barriers), one scan over
// the waves turns the counts into segment bases, and every route's slot is its segment base
// plus its rank. Two barriers in all, instead of three per 1024 routes.
constexpr int kCacheRoutes = 16384;
constexpr int kSegExperts = 1024;
constexpr int kLoadBatch = 8;

__host__ __device__ inline bool segmented_pack(int64_t num_routes, int num_experts) {
  return num_routes > kPackThreads && num_routes <= kCacheRoutes && num_experts <= kSegExperts;
}
// Up to this many experts the segmented pack ranks each 64-route chunk with per-wave 64-bit
// lane masks per expert in LDS (one atomic OR and one read per lane) instead of one ballot
// pass per distinct expert (30 of the 46 us of a 16 384-route, 256-expert pack).
constexpr int kMaskExperts = 256;
__host__ __device__ inline bool mask_ranks(int num_experts) { return num_experts <= kMaskExperts; }

// Segmented packs whose slot range fits in LDS as 16-bit route ids write the slot-ordered
// tables (sorted route ids, token + weight per slot, padding included) in slot order, from a
// slot -> route map built in LDS: coalesced stores instead of one cache line per route and per
// padding slot (27 of the 56 us of a 16 384-route pack were those scattered stores). The map
// sits after the cached ids and ranks, over the per-wave counts and lane masks, followed by
// the block -> expert table (a block's first slot always holds a route: its expert is the
// block's); the router weights are staged over the ids and ranks once those are in registers.
constexpr size_t kPackLdsMax = 163840;
constexpr int kRoutesPerThread = kCacheRoutes / kPackThreads;
constexpr int kSlotBits = 17;                  // slot | local expert << kSlotBits in one register
__host__ __device__ inline size_t slot_map_offset(int num_experts) {
  return route_pack_base_lds(num_experts) + size_t(kCacheRoutes) * 4;
}
__host__ __device__ inline size_t block_map_offset(int num_experts, int64_t cap_routes) {
  return slot_map_offset(num_experts) + (size_t(cap_routes) * 2 + 15) / 16 * 16;
}
__host__ __device__ inline bool slot_map_pass(int64_t num_routes, int num_experts, int64_t cap_routes, int block_m) {
  return segmented_pack(num_routes, num_experts) && cap_routes < (int64_t(1) << kSlotBits) &&
         block_map_offset(num_experts, cap_routes) + size_t(cap_routes / block_m) * 2 <= kPackLdsMax;
}

__device__ void cache_routes(const RoutePackParams& p, int16_t* lc, int* cnt, int64_t rl) {
  const int tid = threadIdx.x;
  const int64_t R = p.num_routes;
  for (int64_t base = 0; base < R; base += int64_t(kPackThreads) * kLoadBatch) {
    int g[kLoadBatch];
#pragma unroll
    for (int j = 0; j < kLoadBatch; ++j) {
      const int64_t r = base + j * kPackThreads + tid;
      g[j] = r < rl ? p.topk_ids[r] : -1;
    }
#pragma unroll
    for (int j = 0; j < kLoadBatch; ++j) {
      const bool ok = g[j] >= 0 && g[j] < p.num_global_experts;
      g[j] = ok ? (p.expert_map ? p.expert_map[g[j]] : g[j]) : -1;
    }
#pragma unroll
    for (int j = 0; j < kLoadBatch; ++j) {
      const int64_t r = base + j * kPackThreads + tid;
      const int l = (g[j] >= 0 && g[j] < p.num_experts) ? g[j] : -1;
      if (r < R) {
        lc[r] = int16_t(l);
        if (l >= 0) atomicAdd(&cnt[l], 1);
      }
    }
  }
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

// Exclusive scans of two ints per thread at once (one set of barriers); wave_tot needs
// 2 * (kPackWaves + 1) ints.
__device__ int2 block_exclusive_scan2(int v0, int v1, int* wave_tot, int* total0, int* total1) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int x0 = v0, x1 = v1;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y0 = __shfl_up(x0, d, 64), y1 = __shfl_up(x1, d, 64);
    if (lane >= d) { x0 += y0; x1 += y1; }
  }
  if (lane == 63) { wave_tot[w] = x0; wave_tot[kPackWaves + 1 + w] = x1; }
  __syncthreads();
  if (w == 0) {
    const int t0 = lane < kPackWaves ? wave_tot[lane] : 0;
    const int t1 = lane < kPackWaves ? wave_tot[kPackWaves + 1 + lane] : 0;
    int s0 = t0, s1 = t1;
#pragma unroll
    for (int d = 1; d < kPackWaves; d <<= 1) {
      const int y0 = __shfl_up(s0, d, 64), y1 = __shfl_up(s1, d, 64);
      if (lane >= d) { s0 += y0; s1 += y1; }
    }
    if (lane < kPackWaves) { wave_tot[lane] = s0 - t0; wave_tot[kPackWaves + 1 + lane] = s1 - t1; }
    if (lane == kPackWaves - 1) { wave_tot[kPackWaves] = s0; wave_tot[2 * kPackWaves + 1] = s1; }
  }
  __syncthreads();
  const int2 r = make_int2(x0 - v0 + wave_tot[w], x1 - v1 + wave_tot[kPackWaves + 1 + w]);
  *total0 = wave_tot[kPackWaves];
  *total1 = wave_tot[2 * kPackWaves + 1];
  __syncthreads();
  return r;
}

__device__ void pack_routes(const RoutePackParams& p, uint8_t* smem) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = p.num_experts, B = p.block_m;
  int* cnt = reinterpret_cast<int*>(smem);                 // [E] counts, then running slot
  int* wave_tot = cnt + E;                                 // [40] scan scratch; [kValidSlot] = valid routes
  int* ecnt = wave_tot + 40;                               // [E] counts (kept for the tile table)
  uint8_t* wcnt = reinterpret_cast<uint8_t*>(ecnt + E);    // [kPackWaves][E] per-wave counts
  const int64_t rl = routes_in_use(p, p.m, p.topk);         // routes past rl are dropped
  const bool cached = segmented_pack(p.num_routes, E);
  const bool slot_pass = slot_map_pass(p.num_routes, E, p.cap_routes, B);
  int16_t* lc = reinterpret_cast<int16_t*>(smem + route_pack_base_lds(E));                          // [R] local ids
  uint16_t* srank = reinterpret_cast<uint16_t*>(smem + route_pack_base_lds(E) + size_t(kCacheRoutes) * 2);   // [R] rank in segment
  uint16_t* scnt = srank + kCacheRoutes;                                                            // [waves][E] counts, then bases
  uint64_t* wmask = reinterpret_cast<uint64_t*>(smem + route_pack_base_lds(E) + size_t(kCacheRoutes) * 4 +
                                                (size_t(kPackWaves) * E * 2 + 7) / 8 * 8);          // [waves][E] lane masks

  // Small batches (one chunk) keep the first chunk's local id and router weight in
  // registers; larger ones up to kCacheRoutes keep every route's in LDS. Either way
  // topk_ids / expert_map / topk_weights are read from memory once.
  const int l_first = cached ? -1 : local_expert(p, tid, rl);
  const float w_first = (!cached && p.topk_weights && tid < p.num_routes) ? p.topk_weights[tid] : 0.f;
  for (int e = tid; e < E; e += kPackThreads) cnt[e] = 0;
  if (tid == 0) wave_tot[kValidSlot] = 0;
  for (int i = tid; i < kPackWaves * E; i += kPackThreads) wcnt[i] = 0;
  if (cached)
    for (int i = tid; i < kPackWaves * E; i += kPackThreads) scnt[i] = 0;
  if (cached && mask_ranks(E))
    for (int i = tid; i < kPackWaves * E; i += kPackThreads) wmask[i] = 0;
  __syncthreads();
  if (cached) {
    cache_routes(p, lc, cnt, rl);
  } else {
    if (l_first >= 0) atomicAdd(&cnt[l_first], 1);
    for (int64_t r = kPackThreads + tid; r < p.num_routes; r += kPackThreads) {
      int l = local_expert(p, r, rl);
      if (l >= 0) atomicAdd(&cnt[l], 1);
    }
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
    const int2 sc2 = block_exclusive_scan2(padded, nfull, wave_tot, &tot, &ttot);
    const int off = sc2.x + carry, toff = sc2.y + tile_carry;
    if (e < E) {
      p.expert_counts[e] = c;
      p.expert_offsets[e] = off;
      if (!slot_pass) {
        for (int b = off / B; b < (off + padded) / B; ++b) p.block_expert[b] = e;
        for (int s = off + c; s < off + padded; ++s) {
          p.sorted_route_ids[s] = -1;
          if (p.slot_info) p.slot_info[s] = make_int2(-1, 0);
        }
      }
      if (p.tiles) {
        for (int t = 0; t < nfull; ++t)
          p.tiles[toff + t] = make_int2(off / B + t * kTileBlocks, kTileBlocks | (e << 8));
      }
      cnt[e] = off;                                        // running slot of expert e
      ecnt[e] = c;
    }
    carry += tot;
    tile_carry += ttot;
  }
  const int total_padded = carry;
  const int full_tiles = tile_carry;
  if (p.tiles) {
    // Partial tiles after all full ones (counts and offsets kept in LDS by the pass above).
    for (int base = 0; base < E; base += kPackThreads) {
      int e = base + tid;
      int blocks = 0, off = 0;
      if (e < E) {
        off = cnt[e];
        blocks = (ecnt[e] + B - 1) / B;
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
    p.live[3] = int(rl / p.topk);
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

  int valid_total = 0;
  if (cached) {
    // Wave segments (see cache_routes): ranks against the wave's running counts.
    const int R = int(p.num_routes);
    const int S = ((R + kPackWaves - 1) / kPackWaves + 63) / 64 * 64;
    const int s0 = wave * S, s1 = min(R, s0 + S);
    uint16_t* myc = scnt + wave * E;
    const uint64_t lt_mask = lane == 0 ? 0ull : (~0ull >> (64 - lane));
    for (int j0 = s0; j0 < s1; j0 += 64) {
      const int r = j0 + lane;
      const int l = r < s1 ? int(lc[r]) : -1;
      // One pass per distinct expert among the 64 routes: the lanes of expert v are one
      // ballot; a lane's rank is the number of them below it.
      int rank = 0, same = 0;
      uint64_t todo = __ballot(l >= 0);
      valid_total += __popcll(todo);
      if (mask_ranks(E)) {
        // The lanes of expert v set their bits in this wave's mask of v, then read it back; a
        // lane's rank is the number of set bits below it (one wave's LDS operations complete in
        // order, so every read sees all the ORs, and the clear below comes after all reads).
        uint64_t* mym = wmask + wave * E;
        if (l >= 0) atomicOr(reinterpret_cast<unsigned long long*>(mym + l), 1ull << lane);
        const uint64_t mv = l >= 0 ? mym[l] : 0ull;
        rank = __popcll(mv & lt_mask);
        same = __popcll(mv);
        if (l >= 0 && rank == 0) mym[l] = 0ull;
      } else {
        while (todo) {
          const int v = __builtin_amdgcn_readlane(l, __builtin_ctzll(todo));
          const uint64_t mv = __ballot(l == v);
          if (l == v) {
            rank = __popcll(mv & lt_mask);
            same = __popcll(mv);
          }
          todo &= ~mv;
        }
      }
      // Every lane reads the running count before the expert's first lane bumps it (one
      // wave's LDS operations complete in order).
      const int run = l >= 0 ? int(myc[l]) : 0;
      if (r < s1) srank[r] = uint16_t(run + rank);
      if (l >= 0 && rank == 0) myc[l] = uint16_t(run + same);
    }
    __syncthreads();
    // Segment bases: expert e's slots for wave w start after the earlier waves' routes of e.
    // Kept relative to the expert's padded offset cnt[e] (below kCacheRoutes, so 16 bits
    // hold them; the offsets themselves reach cap_routes, beyond 16 bits for large E x B).
    for (int e = tid; e < E; e += kPackThreads) {
      int run = 0;
      for (int w2 = 0; w2 < kPackWaves; ++w2) {
        const int c = scnt[w2 * E + e];
        scnt[w2 * E + e] = uint16_t(run);
        run += c;
      }
    }
    __syncthreads();
    if (slot_pass) {
      // Each thread's routes' router weights (loads in flight meanwhile) and slots into
      // registers (route order: coalesced route_slot), then the slot -> route map in LDS
      // (0xFFFF: padding) with the block -> expert table, then one pass in slot order.
      const bool wts = p.slot_info != nullptr;
      float wreg[kRoutesPerThread];
#pragma unroll
      for (int k = 0; k < kRoutesPerThread; ++k) {
        const int r = tid + k * kPackThreads;
        wreg[k] = (wts && p.topk_weights && r < R) ? p.topk_weights[r] : 0.f;
      }
      int pos[kRoutesPerThread];
#pragma unroll
      for (int k = 0; k < kRoutesPerThread; ++k) {
        const int r = tid + k * kPackThreads;
        int q = -1;
        if (r < R) {
          const int l = lc[r];
          if (l >= 0) q = cnt[l] + int(scnt[(r / S) * E + l]) + int(srank[r]);
          p.route_slot[r] = q;
          if (l >= 0) q |= l << kSlotBits;
        }
        pos[k] = q;
      }
      __syncthreads();                                     // ids, ranks, counts and masks are free now
      uint16_t* smap = reinterpret_cast<uint16_t*>(smem + slot_map_offset(E));                 // [total_padded]
      uint16_t* bmap = reinterpret_cast<uint16_t*>(smem + block_map_offset(E, p.cap_routes));  // [total_padded / B]
      float* wst = reinterpret_cast<float*>(smem + route_pack_base_lds(E));                     // [R] router weights
      for (int s = tid; s < total_padded; s += kPackThreads) smap[s] = 0xFFFF;
      if (wts) {
#pragma unroll
        for (int k = 0; k < kRoutesPerThread; ++k)
          if (tid + k * kPackThreads < R) wst[tid + k * kPackThreads] = wreg[k];
      }
      __syncthreads();
#pragma unroll
      for (int k = 0; k < kRoutesPerThread; ++k) {
        if (pos[k] >= 0) {
          const int q = pos[k] & ((1 << kSlotBits) - 1);
          smap[q] = uint16_t(tid + k * kPackThreads);
          if ((q & (B - 1)) == 0) bmap[q / B] = uint16_t(pos[k] >> kSlotBits);
        }
      }
      __syncthreads();
      for (int s = tid; s < total_padded; s += kPackThreads) {
        const int v = smap[s];
        const bool pad = v == 0xFFFF;
        p.sorted_route_ids[s] = pad ? -1 : v;
        if (wts) p.slot_info[s] = pad ? make_int2(-1, 0) : make_int2(v / p.topk, __float_as_int(wst[v]));
      }
      for (int b = tid; b < total_padded / B; b += kPackThreads) p.block_expert[b] = bmap[b];
    } else {
      for (int r = tid; r < R; r += kPackThreads) {
        const int l = lc[r];
        if (l >= 0) {
          const int pos = cnt[l] + int(scnt[(r / S) * E + l]) + int(srank[r]);
          p.sorted_route_ids[pos] = r;
          p.route_slot[r] = pos;
          if (p.slot_info)
            p.slot_info[pos] = make_int2(r / p.topk, __float_as_int(p.topk_weights ? p.topk_weights[r] : 0.f));
        } else {
          p.route_slot[r] = -1;
        }
      }
    }
  }
  // Stable scatter, 1024 routes per chunk: rank inside the wave by matching equal expert
  // ids, then add the counts of lower waves of the chunk and the running slot.
  for (int64_t base = 0; base < (cached ? 0 : p.num_routes); base += kPackThreads) {
    const int64_t r = base + tid;
    const int l = base == 0 ? l_first : local_expert(p, r, rl);
    // Stable rank among the wave's earlier lanes with the same expert, and the wave's count
    // per expert (written by the expert's first lane): one pass over the 64 lanes' ids.
    int rank = 0, same = 0;
    const uint64_t valid_mask = __ballot(l >= 0);
    valid_total += __popcll(valid_mask);
    if (valid_mask) {
      const int nl = 64 - __builtin_clzll(valid_mask);          // lanes at and above the last valid one hold no route
      for (int j = 0; j < nl; ++j) {
        const int lj = __builtin_amdgcn_readlane(l, j);
        const int eq = lj == l;
        same += eq;
        rank += eq & (j < lane);
      }
      if (l >= 0 && rank == 0) wcnt[wave * E + l] = (uint8_t)same;
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
  if (lane == 0) atomicAdd(&wave_tot[kValidSlot], valid_total);
  __syncthreads();
  if (tid == 0) p.live[0] = wave_tot[kValidSlot];
}

}  // namespace

__global__ __launch_bounds__(kPackThreads) void route_pack_kernel(RoutePackParams p) {
  extern __shared__ __align__(16) uint8_t smem[];
  if (blockIdx.x == 0) {
    pack_routes(p, smem);
    return;
  }
  // One wave per activation row: row maximum, exponent p with max * 2^-p in [2^14, 2^15),
  // then the scaled f16 row (hidden % 8 == 0: 16-byte chunks) and the sum of its squares (the
  // grouped GEMM bounds each intermediate row with it).
  const int lane = threadIdx.x & 63;
  const int64_t waves = int64_t(gridDim.x - 1) * (blockDim.x / 64);
  const int chunks = int(p.hidden / 8);
  auto pexp_of = [](float amax) {
    int e = 0;
    if (amax > 0.f && amax <= 3.4e38f) (void)frexpf(amax, &e);   // amax = f * 2^e, f in [0.5, 1)
    return amax > 0.f && amax <= 3.4e38f ? e - 15 : 0;
  };
  auto row_max = [&](float amax) {
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) amax = fmaxf(amax, __shfl_xor(amax, d, 64));
    return amax;
  };
  auto chunk_max = [](const u32x4 v, float amax) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      amax = fmaxf(amax, fmaxf(fabsf(__uint_as_float(v[i] << 16)), fabsf(__uint_as_float(v[i] & 0xFFFF0000u))));
    return amax;
  };
  // Each value times 2^-pexp by ldexp: a row whose maximum is below 2^-113 has pexp <= -128,
  // where the factor 2^-pexp alone would overflow to +inf.
  auto to_f16 = [](const u32x4 v, int pexp, float& ss) {
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const _Float16 lo = (_Float16)ldexpf(__uint_as_float(v[i] << 16), -pexp);
      const _Float16 hi = (_Float16)ldexpf(__uint_as_float(v[i] & 0xFFFF0000u), -pexp);
      ss = fmaf(float(lo), float(lo), ss);
      ss = fmaf(float(hi), float(hi), ss);
      o[i] = uint32_t(__builtin_bit_cast(uint16_t, lo)) | (uint32_t(__builtin_bit_cast(uint16_t, hi)) << 16);
    }
    return o;
  };
  for (int64_t t = int64_t(blockIdx.x - 1) * (blockDim.x / 64) + (threadIdx.x >> 6); t < p.m; t += waves) {
    // Row buffers: loads past the row return 0 and stores past it are dropped.
    const __amdgpu_buffer_rsrc_t src = buffer_rsrc(p.x + t * p.hidden, uint32_t(p.hidden * 2));
    const __amdgpu_buffer_rsrc_t dst = buffer_rsrc(p.x16 + t * p.hidden, uint32_t(p.hidden * 2));
    // Batches of kRowRegs chunks per lane, all loads of a batch in flight together; a row of
    // one batch stays in registers, longer rows are read a second time for the conversion.
    u32x4 v[kRowRegs];
#pragma unroll
    for (int i = 0; i < kRowRegs; ++i) v[i] = __builtin_amdgcn_raw_buffer_load_b128(src, (lane + 64 * i) * 16, 0, 0);
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < kRowRegs; ++i) amax = chunk_max(v[i], amax);
    for (int base = 64 * kRowRegs; base < chunks; base += 64 * kRowRegs) {
      u32x4 w[kRowRegs];
#pragma unroll
      for (int i = 0; i < kRowRegs; ++i) w[i] = __builtin_amdgcn_raw_buffer_load_b128(src, (base + lane + 64 * i) * 16, 0, 0);
#pragma unroll
      for (int i = 0; i < kRowRegs; ++i) amax = chunk_max(w[i], amax);
    }
    const int pexp = pexp_of(row_max(amax));
    float ss = 0.f;       // (chunks past the row load as zeros)
    if (chunks <= 64 * kRowRegs) {
#pragma unroll
      for (int i = 0; i < kRowRegs; ++i) {
        const u32x4 o = to_f16(v[i], pexp, ss);
        if (lane + 64 * i < chunks) __builtin_amdgcn_raw_buffer_store_b128(o, dst, (lane + 64 * i) * 16, 0, 0);
      }
    } else {
      // (half batches here: the full ones made the kernel spill registers)
      constexpr int kHalf = kRowRegs / 2;
      for (int base = 0; base < chunks; base += 64 * kHalf) {
        u32x4 w[kHalf];
#pragma unroll
        for (int i = 0; i < kHalf; ++i) w[i] = __builtin_amdgcn_raw_buffer_load_b128(src, (base + lane + 64 * i) * 16, 0, 0);
#pragma unroll
        for (int i = 0; i < kHalf; ++i) {
          const u32x4 o = to_f16(w[i], pexp, ss);
          if (base + lane + 64 * i < chunks) __builtin_amdgcn_raw_buffer_store_b128(o, dst, (base + lane + 64 * i) * 16, 0, 0);
        }
      }
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) ss += __shfl_xor(ss, d, 64);
    if (lane == 0) {
      p.xexp[t] = pexp;
      if (p.xss) p.xss[t] = ss;
    }
  }
}

size_t route_pack_lds_bytes(int num_experts, int64_t num_routes, int64_t cap_routes, int block_m) {
  if (!segmented_pack(num_routes, num_experts)) return route_pack_base_lds(num_experts);
  const size_t ranks = route_pack_base_lds(num_experts) + size_t(kCacheRoutes) * 4 +
                       (size_t(kPackWaves) * num_experts * 2 + 7) / 8 * 8 +
                       (mask_ranks(num_experts) ? size_t(kPackWaves) * num_experts * 8 : 0);
  const size_t map = slot_map_pass(num_routes, num_experts, cap_routes, block_m)
                         ? (block_map_offset(num_experts, cap_routes) + size_t(cap_routes / block_m) * 2 + 15) / 16 * 16
                         : 0;
  return std::max(ranks, map);
}

hipError_t launch_route_pack(const RoutePackParams& p, int side_blocks, hipStream_t stream) {
  static const hipError_t lds_ok = hipFuncSetAttribute(reinterpret_cast<const void*>(&route_pack_kernel),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, int(kPackLdsMax));
  if (lds_ok != hipSuccess) return lds_ok;
  const size_t lds = route_pack_lds_bytes(p.num_experts, p.num_routes, p.cap_routes, p.block_m);
  hipLaunchKernelGGL(route_pack_kernel, dim3(1 + (p.x16 ? side_blocks : 0)), dim3(kPackThreads), lds, stream, p);
  return hipGetLastError();
}

}  // namespace moe
