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
  // Token count read on the device (or null): routes of tokens at or past *m_dev are dropped,
  // and m / num_routes above are then the capacity's bounds.
  const int32_t* m_dev;
  int64_t m, num_routes, cap_k, cap_routes, cap_blocks;
  int32_t topk, num_global_experts, num_experts, block_m;
  int32_t* expert_counts;
  int32_t* expert_offsets;
  int32_t* sorted_route_ids;
  int32_t* block_expert;
  int32_t* live;                 // [64]: valid, padded, live blocks, m, M tiles, full M tiles; [8..23] GEMM queues
  int32_t* route_slot;
  int2* tiles;                   // [cap_blocks] (first block, blocks | expert << 8) or null
  int2* slot_info;               // [cap_routes] (token, router weight bits) or null
  // Side work of the extra workgroups (grouped-GEMM path with NVFP4 weights): activation
  // rows to f16 times a per-token power of two, or null.
  const uint16_t* x;             // bf16 [m, hidden]
  uint16_t* x16;                 // f16 [m, hidden]
  int32_t* xexp;                 // [m] exponent p: x = x16 * 2^p
  float* xss;                    // [m] sum of squares of each f16 row (x16), or null
  int64_t hidden;
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
  // Source layout variants (all 0: canonical).
  int32_t w13_up_first;          // SwiGLU W13 rows [0, I) are up, [I, 2I) gate
  int32_t w13_interleaved;       // SwiGLU W13 rows alternate between the halves
  int32_t global_reciprocal;     // g13 / g2 hold 1 / (dequant multiplier)
  int32_t scale_per_row;         // one scale byte per row for all of K: s [E, N, 1]
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
  const int32_t* m_dev;          // token count read on the device (or null; m is then its bound)
  int32_t topk;
  int32_t* sorted_route_ids;
  int32_t* block_expert;
  int32_t* live;                 // route-pack counts; [8..15] FC1, [16..23] FC2 work queues
  const int2* tiles;
  int2* slot_info;
  int32_t* route_slot;           // [m * topk] packed slot of each route or -1
  // Decode FC1 packing the routes itself (no route-pack launch): its inputs. Workgroup 0
  // writes the tables above that FC2 reads.
  const int32_t* topk_ids;       // [m * topk]
  const float* topk_weights;     // [m * topk]
  const int32_t* expert_map;     // [num_global_experts] or null
  int32_t num_global_experts;
  // W4A8 variant: the activation output (without the router weight) rounded to MXFP8 codes and
  // E8M0 scales -- by the grouped GEMM's FC1 epilogue, on the decode path from FC1's fp32 rows --
  // and FC2 on the block-scaled MFMA, applying router weight x FC2 global scale per route.
  int32_t w4a8;
  // Grouped-GEMM path, opt-in: FC2 adds each route's weighted row into the bf16 output with
  // packed-bf16 atomics (FC1 zeroes the output first); no per-route rows, no combine pass.
  int32_t atomic_bf16;
  float* inter32;                // W4A8, decode path: fp32 [cap_routes, ip] activation output of FC1
  uint8_t* inter8;               // W4A8: MXFP8 codes [cap_routes, ip] (E4M3)
  uint8_t* sc8;                  //   and their E8M0 scales [cap_routes, ip / 32]
  uint16_t* inter;               // [cap_routes, ip] bf16 (NVFP4 grouped GEMM: f16, the row times 2^-sexp)
  const uint16_t* x16;           // f16 [m, H] scaled activations (NVFP4 f16 MFMA route)
  const int32_t* xexp;           // [m] their per-token exponents
  const float* xss;              // [m] sums of squares of the f16 rows
  const float* n13;              // [E][2] FC1 gate / up row-norm bounds (prepared buffer)
  int32_t* sexp;                 // [cap_routes] NVFP4 grouped GEMM: exponent q of each slot's
                                 // f16 intermediate row (the row = inter * 2^q)
  uint16_t* y;                   // bf16 [m * topk, H] weighted FC2 rows per route (grouped GEMM)
  float* part;                   // fp32 [K splits, m, H] FC2 partial sums (decode)
  int32_t* f2_count;             // [n2_groups] FC2 K-split arrival counts (decode)
  int64_t cap_blocks;
  int64_t xs_pitch;              // decode FC1: elements per staged activation row in LDS
};

// Routes in use: m * topk, or with a device token count min(max(*m_dev, 0), m) * topk (the
// value was written before the launch, so every lane reads the same).
template <typename P>
__device__ __forceinline__ int64_t routes_in_use(const P& p, int64_t m, int topk) {
  if (!p.m_dev) return m * topk;
  const int64_t v = *p.m_dev;
  return (v < 0 ? 0 : (v > m ? m : v)) * topk;
}

// Sets the message moe_last_error() returns on this thread; returns `code`.
int report_error(int code, const char* fmt, ...);

// Router front end: top-k of fp32 logits [m, num_experts] per token.
struct RouterParams {
  const float* logits;
  int64_t m;
  int32_t num_experts, topk;
  int32_t scoring;               // 0 softmax, 1 sigmoid
  int32_t renormalize;
  int32_t* topk_ids;
  float* topk_weights;
};
constexpr int kRouterMaxExperts = 1024;
constexpr int kRouterMaxTopk = 64;
hipError_t launch_router(const RouterParams& p, hipStream_t stream);

size_t route_pack_lds_bytes(int num_experts, int64_t num_routes, int64_t cap_routes, int block_m);
// `side_blocks` extra workgroups do the activation conversion when p.x16 is set.
hipError_t launch_route_pack(const RoutePackParams& p, int side_blocks, hipStream_t stream);
hipError_t launch_prepare(const PrepareParams& p, hipStream_t stream);
// Measurement marks: after each kernel a launcher enqueues, one event record on the same
// stream and the kernel's id (MOE_KERNEL_* of the C ABI) -- only for kernels that launched.
struct LaunchMarks {
  hipEvent_t* events;            // events[0] is recorded before the first launch
  int32_t* ids;
  int n;
  void after(hipStream_t stream, int id) {
    (void)hipEventRecord(events[n + 1], stream);
    ids[n++] = id;
  }
};
enum KernelId : int32_t { KID_ROUTE_PACK = 0, KID_FC1 = 1, KID_REQUANT = 2, KID_FC2 = 3, KID_COMBINE = 4 };
constexpr int kMaxMarks = 5;

// `marks` (nullable) receives a mark after each kernel launched.
hipError_t launch_decode(const FusedParams& p, int num_cus, hipStream_t stream, LaunchMarks* marks);
// True when the decode FC1 launch packs the routes itself for these sizes (the fused call then
// launches no route pack); false for the grouped-GEMM path.
bool decode_fc1_packs(const PreparedGeom& g, int64_t m, int topk);
hipError_t launch_gemm(const FusedParams& p, int num_cus, hipStream_t stream, LaunchMarks* marks);
// out = bf16 of the sum of each token's valid route rows y[route] (route order).
void launch_combine(const FusedParams& p, hipStream_t stream);
// W4A8, decode path's bf16 fallback FC2: every valid intermediate row rounded to MXFP8 (between
// FC1 and FC2), stored as the exact values in the bf16 rows.
hipError_t launch_mxfp8_requant(const FusedParams& p, hipStream_t stream);

}  // namespace moe
