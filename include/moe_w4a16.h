/*
 * moe_w4a16.h -- C ABI of the MI355X (gfx950) fused W4A16 mixture-of-experts layer.
 *
 * What the layer computes (FlashInfer PR 4255, "feat(moe): sync SM12x W4A16 fused
 * MoE family to b12x HEAD", Description and Performance sections): for every token t
 * and each of its top-k routes (t, j) to expert e,
 *     h = W13_e x_t,  a = silu(h_gate) * h_up   (SiLU-SwiGLU)  or  a = max(h, 0)^2 (relu2),
 *     out_t += w[t, j] * (W2_e a),
 * with bf16 activations x and 4-bit E2M1 weights dequantised on the fly from
 *   NVFP4 (one E4M3 scale per 16 along K plus one fp32 global scale per expert and
 *          matrix), or
 *   MXFP4 (one E8M0 scale per 32 along K; the last group of a row holds K mod 32
 *          elements when K is not a multiple of 32 -- the page's scale tail).
 *
 * Conventions for every call:
 *   - Return 0 (MOE_OK) or a negative moe_status. No exception crosses the ABI.
 *     moe_last_error() gives a message for the last failure on the calling thread.
 *   - Pointers named device_* or documented as device memory are HIP device
 *     pointers; everything else is host memory. Inputs are never modified.
 *   - All device work is enqueued on the caller's `stream`, in order. No call
 *     allocates device or pinned memory, synchronises the stream, or reads device
 *     data on the host; they are safe to issue during HIP graph capture. (The page's
 *     review found a packing entry point that silently dropped its stream argument.)
 *   - The caller owns every buffer. Sizes come from the *_size queries; a buffer that
 *     is too small is rejected with MOE_ERR_WORKSPACE, never grown (the b12x
 *     PR 136 Root cause: capture failed on an un-provisioned scratch arena).
 *   - Out-of-range expert ids are data, not errors: they are dropped on the device.
 *   - bf16 tensors are passed as uint16_t bit patterns.
 */
#ifndef MOE_W4A16_H
#define MOE_W4A16_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1,   /* a size, pointer or enum value is out of its documented range */
  MOE_ERR_UNSUPPORTED = -2,   /* a valid request this library does not handle (device arch, shape) */
  MOE_ERR_WORKSPACE = -3,     /* a caller buffer is smaller than its size query */
  MOE_ERR_HIP = -4            /* a HIP runtime call or kernel launch failed */
} moe_status;

/* Weight source formats (page: Description, the fp4_e8m0_k32 source format; NVFP4 e4m3_k16). */
typedef enum moe_source_format {
  MOE_FMT_NVFP4_E4M3_K16 = 1,
  MOE_FMT_MXFP4_E8M0_K32 = 2
} moe_source_format;

/* Activations between FC1 and FC2 (page: Performance, relu2 and silu rows). */
typedef enum moe_activation {
  MOE_ACT_SILU_SWIGLU = 1,    /* W13 rows [0, I) are gate, [I, 2I) are up; a = silu(gate) * up */
  MOE_ACT_RELU2 = 2           /* W1 has I rows; a = max(h, 0)^2 */
} moe_activation;

/* Shape of one MoE layer's weights. hidden (H) and inter (I) must be even
 * (two E2M1 codes per byte along K). */
typedef struct moe_w4a16_dims {
  int32_t fmt;          /* moe_source_format */
  int32_t act;          /* moe_activation */
  int32_t num_experts;  /* E, local experts held by this device */
  int32_t hidden;       /* H */
  int32_t inter;        /* I */
} moe_w4a16_dims;

/* ------------------------------------------------------------------ route packing
 * Page: Description (shape-stable route packing on a power-of-two capacity, with
 * workspaces sized to that capacity), Tests (expert_map, invalid ids, preallocated
 * buffers, capacity contract), Review round 1 (capacity helper; minimum-one clamps).
 *
 * Route r = t*k + j of token t. Its local expert is expert_map[g] (or g without a
 * map) for g = topk_ids[t][j]; the route is dropped when g < 0, g >= num_global_experts
 * or the local id is outside [0, E). Each expert's segment lists its routes in
 * ascending r, padded with -1 to a multiple of block_m. With cap = token capacity:
 *   cap_routes = max(round_up(cap*k + min(E, cap*k)*(block_m-1), block_m), block_m),
 *   cap_blocks = cap_routes / block_m.
 */

/* next power of two of max(m, 1); -1 when m < 0. One capacity serves every m <= it. */
int64_t moe_route_pack_token_capacity(int64_t m);

/* Device arrays written by moe_route_pack, all int32, pointing into the workspace. */
typedef struct moe_route_pack_view {
  int32_t* expert_counts;     /* [E]            valid routes per expert */
  int32_t* expert_offsets;    /* [E+1]          padded segment starts, multiples of block_m */
  int32_t* sorted_route_ids;  /* [cap_routes]   route id per packed slot; -1 = padding */
  int32_t* block_expert;      /* [cap_blocks]   expert of each block; -1 after the live blocks */
  int32_t* live;              /* [4]            {valid routes, padded routes, live blocks, m} */
  int32_t* route_slot;        /* [cap*k]        packed slot of each route; -1 if dropped or r >= m*k */
  int64_t token_capacity;
  int64_t cap_routes;
  int64_t cap_blocks;
  int32_t block_m;
  int32_t num_experts;
} moe_route_pack_view;

/* Bytes of device workspace moe_route_pack needs. block_m in {16, 32, 64, 128};
 * num_local_experts in [1, 2048]; topk in [1, 64]; token_capacity a power of two
 * in [1, 2^24]. */
int moe_route_pack_workspace_size(int64_t token_capacity, int topk, int num_local_experts,
                                  int block_m, size_t* bytes);

/* Pack routes. topk_ids: device int32 [m, topk] row-major; expert_map: device int32
 * [num_global_experts] or NULL (identity); m <= token_capacity. workspace: device,
 * >= moe_route_pack_workspace_size bytes, 256-byte aligned. On success *out (host)
 * receives the device sub-pointers. The result depends only on the inputs, never on
 * previous contents of the workspace. */
int moe_route_pack(const int32_t* topk_ids, int64_t m, int topk, const int32_t* expert_map,
                   int num_global_experts, int num_local_experts, int block_m,
                   int64_t token_capacity, void* workspace, size_t workspace_bytes,
                   moe_route_pack_view* out, hipStream_t stream);

/* ------------------------------------------------------------------ weight preparation
 * Page: Tests (weight preparation is bit-identical across source formats and
 * activations), Walkthrough (layout normalisation, scale packing, W13 rotation).
 *
 * Canonical source layout (device memory, row-major, K fastest):
 *   w13 u8 [E, N1, H/2]  E2M1 codes, element 2i in the low nibble; N1 = 2I (SwiGLU:
 *                        rows [0, I) gate, [I, 2I) up) or I (relu2)
 *   s13 u8 [E, N1, ceil(H/G)]  E4M3 (NVFP4, G = 16) or E8M0 (MXFP4, G = 32) scale bytes
 *   g13 f32 [E]          NVFP4 global dequant multiplier (ignored, may be NULL, for MXFP4)
 *   w2  u8 [E, H, I/2], s2 u8 [E, H, ceil(I/G)], g2 f32 [E]   likewise for FC2.
 * The prepared buffer is an opaque, lossless gfx950 layout: 16-row x 128-K fragments
 * whose nibbles each lane reads with one 128-bit load in MFMA operand order, scales
 * packed four K-blocks per 128-bit load, K and rows zero-padded to multiples of 128,
 * SwiGLU gate and up row groups interleaved; with NVFP4 it also holds each expert's largest
 * dequantised FC1 gate and up row norms, which bound the intermediate rows that the grouped
 * GEMM keeps in f16 (see moe_w4a16_fused). */
int moe_w4a16_prepared_size(const moe_w4a16_dims* dims, size_t* bytes);

int moe_w4a16_prepare(const moe_w4a16_dims* dims, const uint8_t* w13, const uint8_t* s13,
                      const float* g13, const uint8_t* w2, const uint8_t* s2, const float* g2,
                      void* prepared, size_t prepared_bytes, hipStream_t stream);

/* Source layouts other than the canonical one (page: Summary, ModelOpt / CompressedTensors
 * formats; Walkthrough, weight format preparation and layout normalisation; review of the
 * preparation module, single-scale branch). Each flag is 0 (canonical) or 1:
 *   w13_up_first             SwiGLU W13 rows [0, I) are up and [I, 2I) gate (s13 likewise);
 *                            ignored for relu2.
 *   global_scale_reciprocal  NVFP4 g13 / g2 hold the encode scale 1/g; the prepared buffer
 *                            keeps the correctly rounded fp32 quotient 1/stored. Ignored for
 *                            MXFP4.
 *   scale_per_row            s13 is [E, N1, 1] and s2 [E, H, 1]: one scale byte per row for
 *                            all of K (group size -1).
 *   w13_interleaved          SwiGLU W13 rows (and s13 rows) alternate between the halves:
 *                            row 2i is row i of the first half, 2i + 1 row i of the second
 *                            (the first half is gate, or up with w13_up_first); ignored for
 *                            relu2.
 * The prepared buffer equals, byte for byte, the one moe_w4a16_prepare makes from the
 * canonical arrays these describe. layout may be NULL (canonical). Errors as for
 * moe_w4a16_prepare, plus MOE_ERR_INVALID_ARG for a flag outside {0, 1}. */
typedef struct moe_w4a16_source_layout {
  int32_t w13_up_first;
  int32_t global_scale_reciprocal;
  int32_t scale_per_row;
  int32_t w13_interleaved;
} moe_w4a16_source_layout;

int moe_w4a16_prepare_layout(const moe_w4a16_dims* dims, const moe_w4a16_source_layout* layout,
                             const uint8_t* w13, const uint8_t* s13, const float* g13, const uint8_t* w2,
                             const uint8_t* s2, const float* g2, void* prepared, size_t prepared_bytes,
                             hipStream_t stream);

/* ------------------------------------------------------------------ the fused layer
 * Page: Description (fused FC1/FC2 kernel with cooperative persistent launches; a
 * small-batch decode path that folds the top-k sum into the FC2 store epilogue),
 * Performance (the m = 2048 stall: grid-wide barriers without co-residency),
 * Reviewer Notes (decode path cap m <= 4 here, m <= 8 upstream).
 *
 * A call whose m is at most the decode threshold and whose token_capacity is at most
 * MOE_DECODE_MAX_M takes the decode path: two weight-streaming MFMA kernels; FC2 gives
 * each workgroup a range of hidden rows and a slice of K for every route, sums each
 * token's routes in LDS, and the last K slice of a row range to finish adds the slices in
 * order before one bf16 store. Other calls take the grouped-GEMM path: FC1 + activation
 * epilogue over (route tile, weight tile) items, FC2 writing each route's weighted row
 * rounded to bf16, and a combine pass that sums every token's top-k rows in fp32 in route
 * order and casts to bf16 -- deterministic, no atomics on data. Persistent workgroups take items from a
 * queue; no workgroup waits on another that may not be resident. The intermediate (activation
 * output) rows are 16-bit: bf16, except on the grouped-GEMM path with NVFP4 weights, where both
 * GEMMs run on f16 operands and each route's row is stored in f16 times a power of two chosen
 * from a bound on the row (the token's activation norm, the expert's largest FC1 row norms, the
 * global scales and the router weight): no value can overflow, and each is stored within
 * 2^-11 of itself plus 2^-32 of the bound (bf16: 2^-9 of itself). */
#define MOE_DECODE_MAX_M 16

/* Workspace bytes for moe_w4a16_fused at a token capacity (route packing included). */
int moe_w4a16_workspace_size(const moe_w4a16_dims* dims, int64_t token_capacity, int topk,
                             size_t* bytes);

/* x: device bf16 [m, H]; topk_ids: device int32 [m, topk]; topk_weights: device f32
 * [m, topk]; expert_map: device int32 [num_global_experts] or NULL; out: device bf16
 * [m, H], fully written (a token without a surviving route gets a zero row).
 * prepared: the buffer filled by moe_w4a16_prepare for the same dims. m may be 0. */
int moe_w4a16_fused(const moe_w4a16_dims* dims, const void* prepared, size_t prepared_bytes,
                    const uint16_t* x, int64_t m, const int32_t* topk_ids,
                    const float* topk_weights, int topk, const int32_t* expert_map,
                    int num_global_experts, int64_t token_capacity, void* workspace,
                    size_t workspace_bytes, uint16_t* out, hipStream_t stream);

/* The same layer with the token count read from device memory when the call executes, so that
 * one captured HIP graph serves every m up to the capacity (page: Description, shape-stable
 * route packing on a power-of-two capacity, so that batch-size changes need no new launch
 * shapes; b12x PR 136: capture-safe small-M dispatch). m = min(max(*m_device, 0),
 * token_capacity), where m_device is a device int32 written before the call runs (e.g. by a
 * copy between graph replays). Every launch is sized for token_capacity tokens: x, topk_ids,
 * topk_weights and out must hold token_capacity rows; rows at or past m of the inputs are
 * never used for the result (x rows may be read), routes of those tokens are dropped, and rows
 * m .. token_capacity - 1 of out are written with zeros. The path follows token_capacity (the
 * decode path when it is at most the decode threshold and MOE_DECODE_MAX_M). On the grouped-GEMM
 * path the result equals moe_w4a16_fused at that m bit for bit; on the decode path it is the
 * same layer, equal within the layer's tolerance (the kernels' launch shapes follow the
 * capacity, which can change the order of the top-k sums). Other arguments, ownership and
 * errors as moe_w4a16_fused, plus MOE_ERR_INVALID_ARG for a NULL or misaligned m_device. */
int moe_w4a16_fused_device_m(const moe_w4a16_dims* dims, const void* prepared, size_t prepared_bytes,
                             const uint16_t* x, const int32_t* m_device, const int32_t* topk_ids,
                             const float* topk_weights, int topk, const int32_t* expert_map,
                             int num_global_experts, int64_t token_capacity, void* workspace,
                             size_t workspace_bytes, uint16_t* out, hipStream_t stream);

/* W4A8 variant of the same layer. Page: PR 4255 review (a grouped MXFP8 quantisation of the
 * SiLU-mul output, checked against a Torch reference with the exact silu). The activation
 * output of every route is rounded to MXFP8 before FC2 -- E4M3FN elements, one E8M0 scale per
 * 32 along the intermediate axis, scale 2^ceil(log2(amax / 448)), ties to even -- and the
 * router weight is applied after FC2, outside the quantisation; FC1 is the W4A16 one.
 * out[t] = sum_j w[t, j] * W2_e @ MXFP8(act(W13_e @ x_t)) over surviving routes.
 * Arguments, layouts, ownership and errors as moe_w4a16_fused (same prepared buffer and
 * workspace); MOE_ERR_UNSUPPORTED unless dims->fmt is MOE_FMT_MXFP4_E8M0_K32 (the gfx950
 * block-scaled MFMA applies E8M0 scales only). The rounding is taken from FC1's fp32 result
 * (one rounding, as defined): in the grouped-GEMM path's FC1 epilogue, on the decode path by
 * each FC2 workgroup for its K slice. FC2 multiplies the E4M3 codes on gfx950's block-scaled
 * FP4 x FP8 MFMA on both paths (the decode path falls back to the exact MXFP8 values on the
 * bf16 MFMA when the routes' slices do not fit in its LDS). */
int moe_w4a8_fused(const moe_w4a16_dims* dims, const void* prepared, size_t prepared_bytes,
                   const uint16_t* x, int64_t m, const int32_t* topk_ids,
                   const float* topk_weights, int topk, const int32_t* expert_map,
                   int num_global_experts, int64_t token_capacity, void* workspace,
                   size_t workspace_bytes, uint16_t* out, hipStream_t stream);

/* Opt-in approximate top-k combine. Page: the FlashInfer fused-MoE kernel source's atomic
 * reduction helpers (a bf16 scatter-add, f32 rounded to bf16 to nearest and then added
 * atomically, offered as an opt-in approximate mode beside the f32 reduction). The same layer
 * as moe_w4a16_fused; on the grouped-GEMM path (m above the decode threshold) FC2 rounds each
 * route's weighted row to bf16 and adds it into its token's output row with gfx950's
 * packed-bf16 global atomic (FC1 zeroes `out` first), instead of writing per-route rows for
 * the fixed-order combine pass. Every partial sum is rounded to bf16 and the order of the adds
 * varies, so results can differ from run to run and from moe_w4a16_fused by a few bf16 ulps
 * of the row's magnitude. On the decode path it is moe_w4a16_fused exactly (that path sums
 * the top-k in registers). Arguments, layouts, ownership and errors as moe_w4a16_fused. */
int moe_w4a16_fused_atomic_bf16(const moe_w4a16_dims* dims, const void* prepared,
                                size_t prepared_bytes, const uint16_t* x, int64_t m,
                                const int32_t* topk_ids, const float* topk_weights, int topk,
                                const int32_t* expert_map, int num_global_experts,
                                int64_t token_capacity, void* workspace, size_t workspace_bytes,
                                uint16_t* out, hipStream_t stream);

/* Allocation-free variant, for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc. moe_w4a16_fused with
 * its workspace in a device array the library itself holds: MOE_STATIC_WORKSPACE_BYTES on each
 * GPU the library runs on, from the load of its code object until the process ends. Arguments,
 * layouts, ownership and results as moe_w4a16_fused, without the workspace arguments; the call
 * allocates and frees nothing. Errors as moe_w4a16_fused, and MOE_ERR_WORKSPACE, before any
 * device work, when the layer at token_capacity needs more workspace than the array holds
 * (moe_w4a16_workspace_size gives the need; 64 MiB covers, e.g., the 128-expert
 * hidden-4096 decode shape up to a capacity of 64 tokens). All calls on one GPU share its
 * array, which keeps the last call's contents: calls that overlap on one GPU (other streams
 * or threads) race and must be serialised by the caller. */
#define MOE_STATIC_WORKSPACE_BYTES (64u << 20)

int moe_w4a16_fused_static_workspace(const moe_w4a16_dims* dims, const void* prepared,
                                     size_t prepared_bytes, const uint16_t* x, int64_t m,
                                     const int32_t* topk_ids, const float* topk_weights, int topk,
                                     const int32_t* expert_map, int num_global_experts,
                                     int64_t token_capacity, uint16_t* out, hipStream_t stream);

/* ------------------------------------------------------------------ diagnostics */

/* Measurement twin of moe_w4a16_fused: the same launches on `stream`, with a HIP event
 * record before the first kernel (events[0]) and one after every kernel that the call
 * launches: events[j + 1] follows the j-th kernel launched, whose id (moe_kernel_id) is
 * written to kernel_ids[j] (host memory); *num_kernels (host) receives the number of kernels
 * launched (0 for m = 0 and on an argument error). Which kernels run depends on the path: the
 * decode path packs the routes inside its FC1 launch for small m and has no combine pass.
 * The caller creates the events (num_events >= 6) and provides room for 5 ids. Not for graph
 * capture. Errors as moe_w4a16_fused, plus MOE_ERR_INVALID_ARG for too few events or NULL
 * kernel_ids / num_kernels. */
typedef enum moe_kernel_id {
  MOE_KERNEL_ROUTE_PACK = 0,
  MOE_KERNEL_FC1 = 1,          /* FC1 + activation epilogue */
  MOE_KERNEL_REQUANT = 2,      /* the W4A8 variant's MXFP8 rounding pass */
  MOE_KERNEL_FC2 = 3,          /* FC2 (+ the top-k sum on the decode path) */
  MOE_KERNEL_COMBINE = 4       /* the grouped-GEMM path's top-k combine pass */
} moe_kernel_id;

int moe_w4a16_fused_profiled(const moe_w4a16_dims* dims, const void* prepared, size_t prepared_bytes,
                             const uint16_t* x, int64_t m, const int32_t* topk_ids,
                             const float* topk_weights, int topk, const int32_t* expert_map,
                             int num_global_experts, int64_t token_capacity, void* workspace,
                             size_t workspace_bytes, uint16_t* out, hipStream_t stream,
                             hipEvent_t* events, int num_events, int32_t* kernel_ids,
                             int* num_kernels);

/* ------------------------------------------------------------------ router front end
 * Page: Summary (New Features: configurable routing) and Walkthrough (kernel compilation and
 * execution: routing modes); the pages print no formula, so the operation follows the
 * workload definitions (softmax top-k over the router logits; sigmoid scores, top-k,
 * renormalised):
 *   topk_ids[t, j]     = the j-th largest of logits[t, :] (equal logits: ascending expert id;
 *                        the comparison is on the fp32 values, -0 equal to +0),
 *   topk_weights[t, j] = score of that expert, score = softmax or sigmoid of the logits,
 *                        divided by the sum of the k selected scores when renormalize != 0
 *                        (for softmax this is the softmax of the k selected logits).
 * logits: device fp32 [m, num_experts], finite values, row-major. topk_ids: device int32
 * [m, topk]; topk_weights: device fp32 [m, topk]; both caller-owned, written in selection
 * order. One wave per token; no allocation, no synchronisation.
 * Errors: MOE_ERR_INVALID_ARG for m < 0, num_experts outside [1, 1024], topk outside
 * [1, min(64, num_experts)], an unknown scoring, or NULL pointers with m > 0;
 * MOE_ERR_UNSUPPORTED off gfx950; MOE_ERR_HIP when the launch fails. */
typedef enum moe_router_scoring {
  MOE_ROUTER_SOFTMAX = 0,
  MOE_ROUTER_SIGMOID = 1
} moe_router_scoring;

int moe_router_topk(const float* logits, int64_t m, int num_experts, int topk, int scoring, int renormalize,
                    int32_t* topk_ids, float* topk_weights, hipStream_t stream);

/* Message for the calling thread's last failing call ("" if none). */
const char* moe_last_error(void);

/* Path selection for tests and tuning: 0 = automatic (decode for m <= the decode
 * threshold), 1 = force decode (token_capacity <= MOE_DECODE_MAX_M, else the call
 * fails with MOE_ERR_UNSUPPORTED), 2 = force grouped GEMM.
 * Process-wide; the environment variable MOE_W4A16_FORCE_PATH=decode|gemm sets the
 * initial value. Returns the previous value, or MOE_ERR_INVALID_ARG. */
int moe_w4a16_set_path(int path);

/* Decode threshold (default MOE_DECODE_MAX_M, measured faster than the grouped GEMM at
 * every m up to it; MOE_W4A16_DECODE_MAX_M overrides it at load).
 * Values outside [0, MOE_DECODE_MAX_M] are rejected. Returns the previous value. */
int moe_w4a16_set_decode_max_m(int max_m);

/* Test setting: later fused calls size their persistent and grid-stride launches (the grouped
 * GEMM's FC1 and FC2, the decode path's FC1, the route pack's conversion workgroups) as if the
 * device had at most max_cus compute units; 0 (the default) uses every CU. With a limit of one,
 * a single workgroup works through every item of the grouped GEMM. Results are identical bit
 * for bit at every limit: no workgroup waits for another, so none relies on co-residency (the
 * page's m = 2048 stall came from grid-wide barriers without a cooperative launch; PR 4255,
 * Performance). Negative values are rejected. Returns the previous value. */
int moe_w4a16_set_grid_limit(int max_cus);

#ifdef __cplusplus
}
#endif

#endif /* MOE_W4A16_H */
