// Kernel parameter blocks and launch entry points shared by the HIP sources and the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "layout.hpp"

namespace moe {

struct RoutePackParams {
  const int32_t* topk_ids;       // [m * topk]
  const float* topk_weights;     // [m * topk] or null (only the fused layer passes it)
  const int32_t* expert_map;     // [num_global_experts] or null
  int64_t m, num_routes, cap_k, cap_routes, cap_blocks;
  int32_t topk, num_global_experts, num_experts, block_m;
  int32_t* expert_counts;
  int32_t* expert_offsets;
  int32_t* sorted_route_ids;
  int32_t* block_expert;
  int32_t* live;                 // [8]: valid, padded, live blocks, m, M tiles, two queue counters
  int32_t* route_slot;
  int2* tiles;                   // [cap_blocks] (first block, blocks | expert << 8) or null
  int2* slot_info;               // [cap_routes] (token, router weight bits) or null
  float* acc;                    // fp32 accumulator cleared by the extra workgroups, or null
  int64_t acc_elems;
  int32_t* zero_ints;            // counters cleared by the packing workgroup, or null
  int64_t n_zero_ints;
};

struct PrepareParams {
  PreparedGeom g;
  const uint8_t* w13;
  const uint8_t* s13;
  const float* g13;
  const uint8_t* w2;
  const uint8_t* s2;
  const float* g2;
  uint8_t* out;
};

// Everything the fused-layer kernels read; pointers into the prepared buffer and workspace.
struct FusedParams {
  PreparedGeom g;
  const uint8_t* nib1;
  const uint8_t* sc1;
  const uint8_t* nib2;
  const uint8_t* sc2;
  const float* g13;
  const float* g2;
  const uint16_t* x;             // bf16 [m, H]
  uint16_t* out;                 // bf16 [m, H]
  int64_t m;
  int32_t topk;
  const int32_t* sorted_route_ids;
  const int32_t* block_expert;
  int32_t* live;                 // route-pack counts; [5], [6] = grouped-GEMM work queues
  const int2* tiles;
  const int2* slot_info;
  const int32_t* route_slot;      // [m * topk] packed slot of each route or -1
  uint16_t* inter;               // bf16 [cap_routes, ip]
  float* acc;                    // fp32 [m, H] (grouped GEMM)
  float* ybuf;                   // fp32 [cap_routes, hp] route partials (decode)
  int32_t* fc2_arrivals;         // [hp / 64] decode FC2 arrival counters, zero on entry
  int64_t cap_blocks;
  int64_t lds_block_table;       // decode FC1: bytes of LDS before the staged activations
};

size_t route_pack_lds_bytes(int num_experts);
hipError_t launch_route_pack(const RoutePackParams& p, int zero_blocks, hipStream_t stream);
hipError_t launch_prepare(const PrepareParams& p, hipStream_t stream);
// `marks` (nullable) receives an event record after each kernel: FC1, FC2, final cast
// (the decode path records its last mark right after FC2).
hipError_t launch_decode(const FusedParams& p, int num_cus, hipStream_t stream, hipEvent_t* marks);
hipError_t launch_gemm(const FusedParams& p, int num_cus, hipStream_t stream, hipEvent_t* marks);

}  // namespace moe
