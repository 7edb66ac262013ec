// The C ABI (include/moe_w4a16.h): argument validation, size queries and kernel launches.
// No call allocates memory, synchronises, or reads device data on the host.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <cstdint>
#include <string>

#include "../../include/moe_w4a16.h"
#include "kernels.hpp"
#include "layout.hpp"

using namespace moe;

namespace {

thread_local std::string g_last_error;

int vfail(int code, const char* fmt, va_list ap) {
  char buf[512];
  vsnprintf(buf, sizeof buf, fmt, ap);
  g_last_error = buf;
  return code;
}

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  const int rc = vfail(code, fmt, ap);
  va_end(ap);
  return rc;
}

int ok() {
  g_last_error.clear();
  return MOE_OK;
}

bool is_pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }
bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int initial_path() {
  const char* s = std::getenv("MOE_W4A16_FORCE_PATH");
  if (!s) return 0;
  if (!std::strcmp(s, "decode")) return 1;
  if (!std::strcmp(s, "gemm")) return 2;
  return 0;
}

int initial_decode_max_m() {
  const char* s = std::getenv("MOE_W4A16_DECODE_MAX_M");
  if (!s) return MOE_DECODE_MAX_M;
  int v = std::atoi(s);
  return (v >= 0 && v <= MOE_DECODE_MAX_M) ? v : MOE_DECODE_MAX_M;
}

std::mutex g_cfg_mu;
int g_path = initial_path();
int g_decode_max_m = initial_decode_max_m();
int g_grid_limit = 0;           // 0: launch for every CU of the device

struct DeviceInfo {
  bool probed = false;
  bool gfx950 = false;
  int num_cus = 0;
  std::string arch;
};
constexpr int kMaxDevices = 64;
DeviceInfo g_devices[kMaxDevices];
std::mutex g_dev_mu;

// The current device must be a gfx950 part; returns its CU count through *cus.
int check_device(int* cus) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(MOE_ERR_HIP, "hipGetDevice failed: no usable HIP device");
  if (dev < 0 || dev >= kMaxDevices) return fail(MOE_ERR_UNSUPPORTED, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lk(g_dev_mu);
  DeviceInfo& d = g_devices[dev];
  if (!d.probed) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return fail(MOE_ERR_HIP, "hipGetDeviceProperties failed");
    d.arch = prop.gcnArchName;
    d.gfx950 = d.arch.rfind("gfx950", 0) == 0;
    d.num_cus = prop.multiProcessorCount;
    d.probed = true;
  }
  if (!d.gfx950) return fail(MOE_ERR_UNSUPPORTED, "device %d is %s; this library is built for gfx950 only", dev, d.arch.c_str());
  *cus = d.num_cus;
  return MOE_OK;
}

int check_dims(const moe_w4a16_dims* d) {
  if (!d) return fail(MOE_ERR_INVALID_ARG, "dims is NULL");
  if (d->fmt != MOE_FMT_NVFP4_E4M3_K16 && d->fmt != MOE_FMT_MXFP4_E8M0_K32)
    return fail(MOE_ERR_UNSUPPORTED, "unsupported source format %d", d->fmt);
  if (d->act != MOE_ACT_SILU_SWIGLU && d->act != MOE_ACT_RELU2)
    return fail(MOE_ERR_UNSUPPORTED, "unsupported activation %d", d->act);
  if (d->num_experts < 1 || d->num_experts > kMaxExperts)
    return fail(MOE_ERR_INVALID_ARG, "num_experts %d outside [1, %d]", d->num_experts, kMaxExperts);
  if (d->hidden <= 0 || d->inter <= 0) return fail(MOE_ERR_INVALID_ARG, "hidden and inter must be positive");
  if ((d->hidden & 1) || (d->inter & 1))
    return fail(MOE_ERR_UNSUPPORTED, "hidden (%d) and inter (%d) must be even: two E2M1 codes per byte", d->hidden, d->inter);
  if (d->hidden % 8)
    return fail(MOE_ERR_UNSUPPORTED, "hidden (%d) must be a multiple of 8 (16-byte activation rows)", d->hidden);
  if (d->hidden > (1 << 20) || d->inter > (1 << 20)) return fail(MOE_ERR_INVALID_ARG, "hidden / inter too large");
  return MOE_OK;
}

int check_capacity(int64_t cap) {
  if (!is_pow2(cap) || cap > (int64_t(1) << 24))
    return fail(MOE_ERR_INVALID_ARG, "token_capacity %lld must be a power of two in [1, 2^24]", (long long)cap);
  return MOE_OK;
}

int check_pack_args(int64_t cap, int topk, int num_local_experts, int block_m) {
  if (int rc = check_capacity(cap)) return rc;
  if (topk < 1 || topk > kMaxTopk) return fail(MOE_ERR_INVALID_ARG, "topk %d outside [1, %d]", topk, kMaxTopk);
  if (num_local_experts < 1 || num_local_experts > kMaxExperts)
    return fail(MOE_ERR_INVALID_ARG, "num_local_experts %d outside [1, %d]", num_local_experts, kMaxExperts);
  if (block_m != 16 && block_m != 32 && block_m != 64 && block_m != 128)
    return fail(MOE_ERR_INVALID_ARG, "block_m %d not in {16, 32, 64, 128}", block_m);
  return MOE_OK;
}

int launch_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

}  // namespace

int moe::report_error(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  const int rc = vfail(code, fmt, ap);
  va_end(ap);
  return rc;
}

extern "C" {

int64_t moe_route_pack_token_capacity(int64_t m) {
  if (m < 0) return -1;
  int64_t c = 1;
  while (c < m) c <<= 1;
  return c;
}

int moe_route_pack_workspace_size(int64_t token_capacity, int topk, int num_local_experts, int block_m, size_t* bytes) {
  if (!bytes) return fail(MOE_ERR_INVALID_ARG, "bytes is NULL");
  if (int rc = check_pack_args(token_capacity, topk, num_local_experts, block_m)) return rc;
  *bytes = make_pack_geom(token_capacity, topk, num_local_experts, block_m).total;
  return ok();
}

int moe_route_pack(const int32_t* topk_ids, int64_t m, int topk, const int32_t* expert_map, int num_global_experts,
                   int num_local_experts, int block_m, int64_t token_capacity, void* workspace,
                   size_t workspace_bytes, moe_route_pack_view* out, hipStream_t stream) {
  if (!out) return fail(MOE_ERR_INVALID_ARG, "out view is NULL");
  if (int rc = check_pack_args(token_capacity, topk, num_local_experts, block_m)) return rc;
  if (m < 0 || m > token_capacity)
    return fail(MOE_ERR_INVALID_ARG, "m = %lld outside [0, token_capacity = %lld]", (long long)m, (long long)token_capacity);
  if (num_global_experts < 1) return fail(MOE_ERR_INVALID_ARG, "num_global_experts must be >= 1");
  if (m > 0 && !topk_ids) return fail(MOE_ERR_INVALID_ARG, "topk_ids is NULL");
  if (!workspace || !aligned(workspace, 256)) return fail(MOE_ERR_INVALID_ARG, "workspace must be a 256-byte aligned device pointer");
  const PackGeom pg = make_pack_geom(token_capacity, topk, num_local_experts, block_m);
  if (workspace_bytes < pg.total)
    return fail(MOE_ERR_WORKSPACE, "route-pack workspace %zu bytes < required %zu", workspace_bytes, pg.total);
  int cus = 0;
  if (int rc = check_device(&cus)) return rc;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  RoutePackParams rp{};
  rp.topk_ids = topk_ids;
  rp.topk_weights = nullptr;
  rp.expert_map = expert_map;
  rp.m_dev = nullptr;
  rp.m = m;
  rp.num_routes = m * topk;
  rp.cap_k = token_capacity * topk;
  rp.cap_routes = pg.cap_routes;
  rp.cap_blocks = pg.cap_blocks;
  rp.topk = topk;
  rp.num_global_experts = num_global_experts;
  rp.num_experts = num_local_experts;
  rp.block_m = block_m;
  rp.expert_counts = reinterpret_cast<int32_t*>(ws + pg.off_counts);
  rp.expert_offsets = reinterpret_cast<int32_t*>(ws + pg.off_offsets);
  rp.sorted_route_ids = reinterpret_cast<int32_t*>(ws + pg.off_sorted);
  rp.block_expert = reinterpret_cast<int32_t*>(ws + pg.off_block_expert);
  rp.live = reinterpret_cast<int32_t*>(ws + pg.off_live);
  rp.route_slot = reinterpret_cast<int32_t*>(ws + pg.off_route_slot);
  rp.tiles = nullptr;
  rp.slot_info = nullptr;
  rp.x16 = nullptr;
  out->expert_counts = rp.expert_counts;
  out->expert_offsets = rp.expert_offsets;
  out->sorted_route_ids = rp.sorted_route_ids;
  out->block_expert = rp.block_expert;
  out->live = rp.live;
  out->route_slot = rp.route_slot;
  out->token_capacity = token_capacity;
  out->cap_routes = pg.cap_routes;
  out->cap_blocks = pg.cap_blocks;
  out->block_m = block_m;
  out->num_experts = num_local_experts;
  return launch_status(launch_route_pack(rp, 0, stream), "route pack launch");
}

int moe_w4a16_prepared_size(const moe_w4a16_dims* dims, size_t* bytes) {
  if (!bytes) return fail(MOE_ERR_INVALID_ARG, "bytes is NULL");
  if (int rc = check_dims(dims)) return rc;
  *bytes = make_prepared_geom(dims->fmt, dims->act, dims->num_experts, dims->hidden, dims->inter).total;
  return ok();
}

int moe_w4a16_prepare(const moe_w4a16_dims* dims, const uint8_t* w13, const uint8_t* s13, const float* g13,
                      const uint8_t* w2, const uint8_t* s2, const float* g2, void* prepared, size_t prepared_bytes,
                      hipStream_t stream) {
  return moe_w4a16_prepare_layout(dims, nullptr, w13, s13, g13, w2, s2, g2, prepared, prepared_bytes, stream);
}

int moe_w4a16_prepare_layout(const moe_w4a16_dims* dims, const moe_w4a16_source_layout* layout, const uint8_t* w13,
                             const uint8_t* s13, const float* g13, const uint8_t* w2, const uint8_t* s2, const float* g2,
                             void* prepared, size_t prepared_bytes, hipStream_t stream) {
  if (int rc = check_dims(dims)) return rc;
  moe_w4a16_source_layout lay{};
  if (layout) lay = *layout;
  if ((lay.w13_up_first & ~1) || (lay.global_scale_reciprocal & ~1) || (lay.scale_per_row & ~1) ||
      (lay.w13_interleaved & ~1))
    return fail(MOE_ERR_INVALID_ARG, "source layout flags must be 0 or 1");
  if (!w13 || !s13 || !w2 || !s2) return fail(MOE_ERR_INVALID_ARG, "a weight or scale pointer is NULL");
  if (dims->fmt == MOE_FMT_NVFP4_E4M3_K16 && (!g13 || !g2))
    return fail(MOE_ERR_INVALID_ARG, "NVFP4 needs the global scales g13 and g2");
  if (!prepared || !aligned(prepared, 256)) return fail(MOE_ERR_INVALID_ARG, "prepared must be a 256-byte aligned device pointer");
  const PreparedGeom g = make_prepared_geom(dims->fmt, dims->act, dims->num_experts, dims->hidden, dims->inter);
  if (prepared_bytes < g.total) return fail(MOE_ERR_WORKSPACE, "prepared buffer %zu bytes < required %zu", prepared_bytes, g.total);
  int cus = 0;
  if (int rc = check_device(&cus)) return rc;
  PrepareParams pp{};
  pp.g = g;
  pp.w13 = w13; pp.s13 = s13; pp.g13 = g13;
  pp.w2 = w2; pp.s2 = s2; pp.g2 = g2;
  pp.out = static_cast<uint8_t*>(prepared);
  pp.w13_up_first = lay.w13_up_first;
  pp.w13_interleaved = lay.w13_interleaved;
  pp.global_reciprocal = lay.global_scale_reciprocal;
  pp.scale_per_row = lay.scale_per_row;
  return launch_status(launch_prepare(pp, stream), "prepare launch");
}

int moe_w4a16_workspace_size(const moe_w4a16_dims* dims, int64_t token_capacity, int topk, size_t* bytes) {
  if (!bytes) return fail(MOE_ERR_INVALID_ARG, "bytes is NULL");
  if (int rc = check_dims(dims)) return rc;
  if (int rc = check_pack_args(token_capacity, topk, dims->num_experts, kBlockM)) return rc;
  const PreparedGeom g = make_prepared_geom(dims->fmt, dims->act, dims->num_experts, dims->hidden, dims->inter);
  *bytes = make_fused_geom(g, token_capacity, topk).total;
  return ok();
}

}  // extern "C"

namespace {

int fused_impl(const moe_w4a16_dims* dims, const void* prepared, size_t prepared_bytes, const uint16_t* x, int64_t m,
               const int32_t* topk_ids, const float* topk_weights, int topk, const int32_t* expert_map,
               int num_global_experts, int64_t token_capacity, void* workspace, size_t workspace_bytes, uint16_t* out,
               hipStream_t stream, LaunchMarks* marks, bool w4a8 = false, bool atomic_bf16 = false,
               const int32_t* m_dev = nullptr) {
  if (int rc = check_dims(dims)) return rc;
  if (w4a8 && dims->fmt != MOE_FMT_MXFP4_E8M0_K32)
    return fail(MOE_ERR_UNSUPPORTED, "the W4A8 variant needs MXFP4 weights (E8M0 block scales)");
  if (int rc = check_pack_args(token_capacity, topk, dims->num_experts, kBlockM)) return rc;
  if (m < 0 || m > token_capacity)
    return fail(MOE_ERR_INVALID_ARG, "m = %lld outside [0, token_capacity = %lld]", (long long)m, (long long)token_capacity);
  if (num_global_experts < 1) return fail(MOE_ERR_INVALID_ARG, "num_global_experts must be >= 1");
  const PreparedGeom g = make_prepared_geom(dims->fmt, dims->act, dims->num_experts, dims->hidden, dims->inter);
  const FusedGeom fg = make_fused_geom(g, token_capacity, topk);
  if (!prepared || !aligned(prepared, 256)) return fail(MOE_ERR_INVALID_ARG, "prepared must be a 256-byte aligned device pointer");
  if (prepared_bytes < g.total) return fail(MOE_ERR_WORKSPACE, "prepared buffer %zu bytes < required %zu", prepared_bytes, g.total);
  if (!workspace || !aligned(workspace, 256)) return fail(MOE_ERR_INVALID_ARG, "workspace must be a 256-byte aligned device pointer");
  if (workspace_bytes < fg.total) return fail(MOE_ERR_WORKSPACE, "workspace %zu bytes < required %zu", workspace_bytes, fg.total);
  if (m > 0) {
    if (!x || !topk_ids || !topk_weights || !out) return fail(MOE_ERR_INVALID_ARG, "x, topk_ids, topk_weights and out must be non-NULL");
    if (!aligned(x, 16) || !aligned(out, 16)) return fail(MOE_ERR_INVALID_ARG, "x and out must be 16-byte aligned");
  }
  int path, dmax, grid_limit;
  {
    std::lock_guard<std::mutex> lk(g_cfg_mu);
    path = g_path;
    dmax = g_decode_max_m;
    grid_limit = g_grid_limit;
  }
  const bool decode = path == 1 || (path == 0 && m <= dmax && token_capacity <= kDecodeMaxM);
  if (decode && token_capacity > kDecodeMaxM)
    return fail(MOE_ERR_UNSUPPORTED, "decode path needs token_capacity <= %d (got %lld)", kDecodeMaxM,
                (long long)token_capacity);
  // The grouped GEMM addresses activation and intermediate rows with 32-bit buffer offsets.
  if (!decode && (m * int64_t(dims->hidden) * 2 > INT32_MAX - 4096 ||
                  fg.pack.cap_routes * g.ip * 2 > INT32_MAX - 4096))
    return fail(MOE_ERR_UNSUPPORTED, "grouped GEMM: m x hidden or the intermediate rows exceed 2 GiB");
  int cus = 0;
  if (int rc = check_device(&cus)) return rc;
  if (m == 0) return ok();
  if (grid_limit > 0 && grid_limit < cus) cus = grid_limit;   // launches sized as for that many CUs

  uint8_t* ws = static_cast<uint8_t*>(workspace);
  uint8_t* pk = ws + fg.off_pack;
  const PackGeom& pg = fg.pack;
  RoutePackParams rp{};
  rp.topk_ids = topk_ids;
  rp.topk_weights = topk_weights;
  rp.expert_map = expert_map;
  rp.m_dev = m_dev;
  rp.m = m;
  rp.num_routes = m * topk;
  rp.cap_k = token_capacity * topk;
  rp.cap_routes = pg.cap_routes;
  rp.cap_blocks = pg.cap_blocks;
  rp.topk = topk;
  rp.num_global_experts = num_global_experts;
  rp.num_experts = dims->num_experts;
  rp.block_m = kBlockM;
  rp.expert_counts = reinterpret_cast<int32_t*>(pk + pg.off_counts);
  rp.expert_offsets = reinterpret_cast<int32_t*>(pk + pg.off_offsets);
  rp.sorted_route_ids = reinterpret_cast<int32_t*>(pk + pg.off_sorted);
  rp.block_expert = reinterpret_cast<int32_t*>(pk + pg.off_block_expert);
  rp.live = reinterpret_cast<int32_t*>(pk + pg.off_live);
  rp.route_slot = reinterpret_cast<int32_t*>(pk + pg.off_route_slot);
  rp.tiles = decode ? nullptr : reinterpret_cast<int2*>(pk + pg.off_tiles);   // M tiles: grouped GEMM only
  rp.slot_info = reinterpret_cast<int2*>(pk + pg.off_tok_of_slot);
  // At small m the decode FC1 launch packs the routes itself (no route-pack launch) and
  // converts the activation rows in LDS.
  const bool fc1_packs = decode && decode_fc1_packs(g, m, topk);
  // NVFP4 weights run on the f16 MFMA wherever the activations are staged whole: the grouped
  // GEMM always, the decode path when its rows fit in LDS.
  const bool convert = dims->fmt == MOE_FMT_NVFP4_E4M3_K16 && !fc1_packs && (!decode || decode_stages_x(g, m));
  rp.x = x;
  rp.x16 = convert ? reinterpret_cast<uint16_t*>(ws + fg.off_x16) : nullptr;
  rp.xexp = convert ? reinterpret_cast<int32_t*>(ws + fg.off_xexp) : nullptr;
  rp.xss = convert ? reinterpret_cast<float*>(ws + fg.off_xss) : nullptr;
  rp.hidden = dims->hidden;

  FusedParams fp{};
  const uint8_t* pw = static_cast<const uint8_t*>(prepared);
  fp.g = g;
  fp.nib1 = pw + g.off_nib1;
  fp.sc1 = pw + g.off_sc1;
  fp.nib2 = pw + g.off_nib2;
  fp.sc2 = pw + g.off_sc2;
  fp.g13 = reinterpret_cast<const float*>(pw + g.off_g13);
  fp.g2 = reinterpret_cast<const float*>(pw + g.off_g2);
  fp.x = x;
  fp.out = out;
  fp.m = m;
  fp.m_dev = m_dev;
  fp.topk = topk;
  fp.sorted_route_ids = rp.sorted_route_ids;
  fp.block_expert = rp.block_expert;
  fp.live = rp.live;
  fp.tiles = rp.tiles;
  fp.slot_info = rp.slot_info;
  fp.route_slot = rp.route_slot;
  fp.inter = reinterpret_cast<uint16_t*>(ws + fg.off_inter);
  fp.x16 = rp.x16;
  fp.xexp = rp.xexp;
  fp.xss = rp.xss;
  fp.n13 = reinterpret_cast<const float*>(pw + g.off_n13);
  fp.sexp = reinterpret_cast<int32_t*>(ws + fg.off_sexp);
  fp.y = reinterpret_cast<uint16_t*>(ws + fg.off_y);
  fp.part = reinterpret_cast<float*>(ws + fg.off_part);
  fp.f2_count = decode ? reinterpret_cast<int32_t*>(ws + fg.off_count) : nullptr;
  fp.cap_blocks = pg.cap_blocks;
  fp.w4a8 = w4a8 ? 1 : 0;
  fp.atomic_bf16 = atomic_bf16 && !decode ? 1 : 0;
  fp.inter32 = w4a8 && decode ? reinterpret_cast<float*>(ws + fg.off_inter32) : nullptr;
  fp.inter8 = w4a8 ? ws + fg.off_inter8 : nullptr;
  fp.sc8 = w4a8 ? ws + fg.off_sc8 : nullptr;
  fp.topk_weights = topk_weights;
  if (fc1_packs) {
    fp.topk_ids = topk_ids;
    fp.expert_map = expert_map;
    fp.num_global_experts = num_global_experts;
  }

  if (marks) (void)hipEventRecord(marks->events[0], stream);
  // extra route-pack workgroups for the conversion: one wave per row, 16 waves each
  const int side_blocks = decode ? int((m + 15) / 16) : cus;
  if (!fc1_packs) {
    if (hipError_t e = launch_route_pack(rp, side_blocks, stream); e != hipSuccess)
      return launch_status(e, "route pack launch");
    if (marks) marks->after(stream, KID_ROUTE_PACK);
  }
  hipError_t e = decode ? launch_decode(fp, cus, stream, marks) : launch_gemm(fp, cus, stream, marks);
  return launch_status(e, decode ? "decode launch" : "grouped GEMM launch");
}

}  // namespace

extern "C" {

int moe_w4a16_fused(const moe_w4a16_dims* dims, const void* prepared, size_t prepared_bytes, const uint16_t* x,
                    int64_t m, const int32_t* topk_ids, const float* topk_weights, int topk,
                    const int32_t* expert_map, int num_global_experts, int64_t token_capacity, void* workspace,
                    size_t workspace_bytes, uint16_t* out, hipStream_t stream) {
  return fused_impl(dims, prepared, prepared_bytes, x, m, topk_ids, topk_weights, topk, expert_map,
                    num_global_experts, token_capacity, workspace, workspace_bytes, out, stream, nullptr);
}

int moe_w4a16_fused_device_m(const moe_w4a16_dims* dims, const void* prepared, size_t prepared_bytes,
                             const uint16_t* x, const int32_t* m_device, const int32_t* topk_ids,
                             const float* topk_weights, int topk, const int32_t* expert_map, int num_global_experts,
                             int64_t token_capacity, void* workspace, size_t workspace_bytes, uint16_t* out,
                             hipStream_t stream) {
  if (!m_device || !aligned(m_device, 4)) return fail(MOE_ERR_INVALID_ARG, "m_device must be a 4-byte aligned device pointer");
  if (int rc = check_capacity(token_capacity)) return rc;
  // Every launch is sized for token_capacity tokens; the kernels read the live count.
  return fused_impl(dims, prepared, prepared_bytes, x, token_capacity, topk_ids, topk_weights, topk, expert_map,
                    num_global_experts, token_capacity, workspace, workspace_bytes, out, stream, nullptr, false, false,
                    m_device);
}

int moe_w4a8_fused(const moe_w4a16_dims* dims, const void* prepared, size_t prepared_bytes, const uint16_t* x,
                   int64_t m, const int32_t* topk_ids, const float* topk_weights, int topk,
                   const int32_t* expert_map, int num_global_experts, int64_t token_capacity, void* workspace,
                   size_t workspace_bytes, uint16_t* out, hipStream_t stream) {
  return fused_impl(dims, prepared, prepared_bytes, x, m, topk_ids, topk_weights, topk, expert_map,
                    num_global_experts, token_capacity, workspace, workspace_bytes, out, stream, nullptr, true);
}

int moe_w4a16_fused_atomic_bf16(const moe_w4a16_dims* dims, const void* prepared, size_t prepared_bytes,
                                const uint16_t* x, int64_t m, const int32_t* topk_ids, const float* topk_weights,
                                int topk, const int32_t* expert_map, int num_global_experts, int64_t token_capacity,
                                void* workspace, size_t workspace_bytes, uint16_t* out, hipStream_t stream) {
  return fused_impl(dims, prepared, prepared_bytes, x, m, topk_ids, topk_weights, topk, expert_map,
                    num_global_experts, token_capacity, workspace, workspace_bytes, out, stream, nullptr, false, true);
}

int moe_w4a16_fused_profiled(const moe_w4a16_dims* dims, const void* prepared, size_t prepared_bytes,
                             const uint16_t* x, int64_t m, const int32_t* topk_ids, const float* topk_weights,
                             int topk, const int32_t* expert_map, int num_global_experts, int64_t token_capacity,
                             void* workspace, size_t workspace_bytes, uint16_t* out, hipStream_t stream,
                             hipEvent_t* events, int num_events, int32_t* kernel_ids, int* num_kernels) {
  if (!events || num_events < kMaxMarks + 1)
    return fail(MOE_ERR_INVALID_ARG, "events must hold at least %d HIP events", kMaxMarks + 1);
  if (!kernel_ids || !num_kernels) return fail(MOE_ERR_INVALID_ARG, "kernel_ids and num_kernels must be non-NULL");
  LaunchMarks marks{events, kernel_ids, 0};
  *num_kernels = 0;
  const int rc = fused_impl(dims, prepared, prepared_bytes, x, m, topk_ids, topk_weights, topk, expert_map,
                            num_global_experts, token_capacity, workspace, workspace_bytes, out, stream, &marks);
  *num_kernels = marks.n;
  return rc;
}

const char* moe_last_error(void) { return g_last_error.c_str(); }

int moe_w4a16_set_path(int path) {
  if (path < 0 || path > 2) return fail(MOE_ERR_INVALID_ARG, "path %d not in {0, 1, 2}", path);
  std::lock_guard<std::mutex> lk(g_cfg_mu);
  int prev = g_path;
  g_path = path;
  return prev;
}

int moe_router_topk(const float* logits, int64_t m, int num_experts, int topk, int scoring, int renormalize,
                    int32_t* topk_ids, float* topk_weights, hipStream_t stream) {
  if (m < 0) return fail(MOE_ERR_INVALID_ARG, "m = %lld is negative", (long long)m);
  if (num_experts < 1 || num_experts > kRouterMaxExperts)
    return fail(MOE_ERR_INVALID_ARG, "num_experts %d outside [1, %d]", num_experts, kRouterMaxExperts);
  if (topk < 1 || topk > kRouterMaxTopk || topk > num_experts)
    return fail(MOE_ERR_INVALID_ARG, "topk %d outside [1, min(%d, num_experts = %d)]", topk, kRouterMaxTopk, num_experts);
  if (scoring != MOE_ROUTER_SOFTMAX && scoring != MOE_ROUTER_SIGMOID)
    return fail(MOE_ERR_INVALID_ARG, "unknown scoring %d", scoring);
  if (m > 0 && (!logits || !topk_ids || !topk_weights)) return fail(MOE_ERR_INVALID_ARG, "NULL device pointer");
  int cus = 0;
  if (int rc = check_device(&cus); rc != MOE_OK) return rc;
  RouterParams p{};
  p.logits = logits;
  p.m = m;
  p.num_experts = num_experts;
  p.topk = topk;
  p.scoring = scoring;
  p.renormalize = renormalize ? 1 : 0;
  p.topk_ids = topk_ids;
  p.topk_weights = topk_weights;
  return launch_status(launch_router(p, stream), "router launch");
}

int moe_w4a16_set_grid_limit(int max_cus) {
  if (max_cus < 0) return fail(MOE_ERR_INVALID_ARG, "grid limit %d is negative", max_cus);
  std::lock_guard<std::mutex> lk(g_cfg_mu);
  int prev = g_grid_limit;
  g_grid_limit = max_cus;
  return prev;
}

int moe_w4a16_set_decode_max_m(int max_m) {
  if (max_m < 0 || max_m > MOE_DECODE_MAX_M) return fail(MOE_ERR_INVALID_ARG, "decode max m %d outside [0, %d]", max_m, MOE_DECODE_MAX_M);
  std::lock_guard<std::mutex> lk(g_cfg_mu);
  int prev = g_decode_max_m;
  g_decode_max_m = max_m;
  return prev;
}

}  // extern "C"
