// Grouped-GEMM (prefill) path of the fused W4A16 MoE layer on gfx950.
//
// FlashInfer PR 4255, Description: cooperative persistent launches for the fused FC1/FC2
// kernel with occupancy-aware tiles; Performance: at m = 2048 the old kernel stalled on
// grid-wide barriers because it was not launched cooperatively. Here FC1 -> FC2 -> cast
// are ordered by stream order between persistent launches, so no workgroup ever waits
// for another one that might not be resident.
//
// M tiles are up to 8 route blocks (128 rows) of one expert; N tiles are 16 row groups
// (256 weight rows). Each of the 4 waves owns 4 row groups: it streams their E2M1
// fragments with 128-bit loads one K block ahead, dequantises them in registers into
// MFMA A operands, and reads the activation rows (B operand) from a double-buffered LDS
// tile that the whole workgroup stages. Route blocks past the tile's live rows issue no
// MFMA.
//  * FC1 epilogue: expert FC1 global scale, SiLU-SwiGLU (gate and up fragments sit in
//    the same lanes) or relu2, times router weight and the expert's FC2 global scale,
//    bf16 store into the intermediate workspace row of the route.
//  * FC2 epilogue: the top-k sum -- fp32 atomic adds of the weighted rows into the
//    token's accumulator row; a last pass casts the accumulator to bf16.
#include <hip/hip_runtime.h>

#include "device.hpp"
#include "kernels.hpp"
#include "layout.hpp"

namespace moe {

namespace {

constexpr int kGemmThreads = 256;
constexpr uint32_t kOutOfRange = 0x80000000u;           // set in a buffer offset: past every num_records, loads 0
constexpr int kRowBytes = kKBlock * 2;                  // one activation row of a K block: 256 B
constexpr int kWaveW = 4 * kFragBytes;                  // one wave's four fragment blocks of a K block
constexpr int kLdsBytes = 147456;                       // the pipeline ring (144 KiB of the 160 KiB LDS)

// Ring of K-block stages in LDS, filled by buffer loads that write LDS directly (no register
// staging): an activation tile of 16 NB rows x 256 B, then each wave's 4 fragment blocks.
template <int NB>
struct Ring {
  static constexpr int kStage = NB * kBlockM * kRowBytes + 4 * kWaveW;
  static constexpr int kDepth = kLdsBytes / kStage;                  // 3 (NB 8) .. 7 (NB 1)
  static constexpr int kLoads = NB + 4 + 4;                          // vector loads a wave issues per stage
};

// s_waitcnt with only the vector-memory counter bounded (gfx9 encoding: vmcnt in bits 3:0
// and 15:14; expcnt and lgkmcnt at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit counter");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Workgroup barrier for the stage ring. A release fence would make every wave wait for all of
// its loads into LDS, including the stages still meant to be in flight; instead each wave
// waits explicitly for the stage it needs (wait_vmcnt) and for its own LDS reads (lgkmcnt 0,
// so the slot about to be refilled is no longer being read), then meets the others. The
// acquire fence keeps later LDS reads below the barrier.
__device__ __forceinline__ void stage_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt and expcnt at their maxima
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// A pointer the compiler cannot prove wave-uniform, moved to scalar registers (it is uniform).
__device__ __forceinline__ void* uniform_ptr(const void* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(v >> 32));
  return reinterpret_cast<void*>((uint64_t(hi) << 32) | lo);
}

__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, const uint8_t* lds_dst, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_dst, 16, int(voff), 0, 0, 0);
}

// Per-launch constants shared by every item of a workgroup.
struct GemmCtx {
  int groups, kbs;
  int64_t sc_per_group;
  const uint8_t* nib;
  const uint8_t* scb;
  __amdgpu_buffer_rsrc_t act;        // x (FC1) or the intermediate rows (FC2), bounds-checked
  int act_row_bytes, k_bytes;        // row pitch of that buffer and its K extent, in bytes
};

// One item: NB route blocks (16 NB rows) of one expert x 256 weight rows (16 row groups,
// 4 per wave), full K.
template <int FMT, int PHASE, int NB>
__device__ __forceinline__ void gemm_item(const FusedParams& p, const GemmCtx& c, uint8_t* lds, int mt, int nt) {
  using R = Ring<NB>;
  constexpr int D = R::kDepth;
  const PreparedGeom& g = p.g;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int2 tile = p.tiles[mt];
  const int64_t fb = tile.x;
  const int nb = __builtin_amdgcn_readfirstlane(tile.y & 0xFF);
  const int e = __builtin_amdgcn_readfirstlane(tile.y >> 8);
  const int kbs = c.kbs;

  // Activation rows. Load j of wave w fills tile rows 4q .. 4q+3 (q = w NB + j), lane l the
  // 16-byte chunk position l % 16 of row 4q + l / 16 with the row's chunk (l % 16) ^ (row % 16):
  // the XOR swizzle lets the 16 lanes that read one chunk column of 16 rows hit 16 distinct
  // bank groups. Padding slots and blocks past the tile read 0 through the bounds check.
  uint32_t src[NB], chunk[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int row = 4 * (wave * NB + j) + (lane >> 4);
    const int64_t slot = fb * kBlockM + row;
    const int t = row < nb * kBlockM ? p.slot_info[slot].x : -1;
    const int64_t src_row = PHASE == 1 ? int64_t(t) : slot;   // x row of the token, or the slot's own row
    chunk[j] = uint32_t((lane & 15) ^ (row & 15)) << 4;
    src[j] = t >= 0 ? uint32_t(src_row * c.act_row_bytes) + chunk[j] : kOutOfRange;
  }
  // This wave's four row groups are contiguous in the prepared buffer; groups past the end
  // (last N tile only) fall outside the resource and read 0.
  const int rg_base = nt * 16 + wave * 4;
  const int live_groups = max(0, min(4, c.groups - rg_base));
  const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc(
      uniform_ptr(c.nib + (int64_t(e) * c.groups + min(rg_base, c.groups - 1)) * kbs * kFragBytes), 0,
      __builtin_amdgcn_readfirstlane(live_groups * kbs * kFragBytes), 0x00020000);
  const uint8_t* sgp[4];
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    const int rg = min(rg_base + f, c.groups - 1);
    sgp[f] = c.scb + (int64_t(e) * c.groups + rg) * c.sc_per_group;
  }
  const int sc_lane = FMT == FMT_NVFP4 ? ((lane >> 5) * 16 + (lane & 15)) * 16 : (lane & 15) * 16;

  // One stage: the activation K block and this wave's weight K block into LDS slot `slot`, its
  // scale dwords into registers. Blocks past K are clamped (weights) or read 0 (activations):
  // every stage issues the same R::kLoads loads, so the vmcnt arithmetic below is exact.
  uint32_t sc[D][4];
  auto issue = [&](int kb, int slot, uint32_t* scd) {
    uint8_t* st = lds + slot * R::kStage;
    const uint32_t k = uint32_t(kb) * kRowBytes;
#pragma unroll
    for (int j = 0; j < NB; ++j)
      dma16(c.act, st + (wave * NB + j) * 1024, (src[j] + k) | (k + chunk[j] < uint32_t(c.k_bytes) ? 0u : kOutOfRange));
    const int kc = min(kb, kbs - 1);
    uint8_t* wst = st + NB * kBlockM * kRowBytes + wave * kWaveW;
#pragma unroll
    for (int f = 0; f < 4; ++f) dma16(wres, wst + f * kFragBytes, uint32_t((f * kbs + kc) * kFragBytes + lane * 16));
#pragma unroll
    for (int f = 0; f < 4; ++f)
      scd[f] = *reinterpret_cast<const uint32_t*>(sgp[f] + int64_t(kc >> 2) * g.sc_chunk_bytes + sc_lane + (kc & 3) * 4);
  };

  f32x4 acc[4][NB];
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[f][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  // One K block: four MFMA K-steps. The activation reads and dequantisation of step s+1 are
  // issued ahead of the MFMAs of step s, and the scheduler is asked to interleave them one
  // MFMA at a time so the matrix pipe stays busy while LDS and the VALU work.
  constexpr int kDqValu = FMT == FMT_NVFP4 ? 16 : 4;           // VALU ops of one dq8
  constexpr int kValuPerMfma = (4 * kDqValu + 4 * NB - 1) / (4 * NB);
  auto compute = [&](int slot, const uint32_t* scd) {
    const uint8_t* st = lds + slot * R::kStage;
    const uint8_t* xrow = st + (lane & 15) * kRowBytes;
    const int sw = lane & 15;
    u32x4 wq[4];
#pragma unroll
    for (int f = 0; f < 4; ++f)
      wq[f] = *reinterpret_cast<const u32x4*>(st + NB * kBlockM * kRowBytes + wave * kWaveW + f * kFragBytes + lane * 16);
    float scl[4][4];
#pragma unroll
    for (int f = 0; f < 4; ++f) decode_scales<FMT>(scd[f], scl[f]);
    auto xread = [&](int b, int s) {
      return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
          xrow + b * kBlockM * kRowBytes + (((4 * s + (lane >> 4)) ^ sw) << 4)));
    };
    bf16x8 xb[2][NB], a[2][4];
#pragma unroll
    for (int b = 0; b < NB; ++b) xb[0][b] = xread(b, 0);
#pragma unroll
    for (int f = 0; f < 4; ++f) a[0][f] = dq8<FMT>(wq[f][0], scl[f][0]);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int cur = s & 1, nxt = cur ^ 1;
      if (s < 3) {
#pragma unroll
        for (int b = 0; b < NB; ++b) xb[nxt][b] = xread(b, s + 1);
#pragma unroll
        for (int f = 0; f < 4; ++f) a[nxt][f] = dq8<FMT>(wq[f][s + 1], scl[f][s + 1]);
      }
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int f = 0; f < 4; ++f) acc[f][b] = mfma16(a[cur][f], xb[cur][b], acc[f][b]);
      if (s < 3) {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                 // one LDS read
#pragma unroll
          for (int f = 0; f < 4; ++f) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);               // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, kValuPerMfma, 0);    // dequant VALU
          }
        }
      }
    }
  };

  // Pipeline: stages 0 .. D-2 in flight before the loop; step kb waits until its own stage has
  // landed (at most D-2 later stages still outstanding), meets the other waves at a barrier
  // (their loads have landed too, and all are done with slot (kb-1) % D), refills that slot
  // with stage kb+D-1 and computes stage kb. Barriers order LDS only.
  auto step = [&](int kb, int j) {
    wait_vmcnt<(D - 2) * R::kLoads>();
    stage_barrier();
    __builtin_amdgcn_sched_barrier(0);
    issue(kb + D - 1, (j + D - 1) % D, sc[(j + D - 1) % D]);
    __builtin_amdgcn_sched_barrier(0);
    compute(j, sc[j]);
  };
#pragma unroll
  for (int j = 0; j < D - 1; ++j) issue(j, j, sc[j]);
  __builtin_amdgcn_sched_barrier(0);
  int kb = 0;
  for (; kb + D <= kbs; kb += D) {
#pragma unroll
    for (int j = 0; j < D; ++j) step(kb + j, j);
  }
#pragma unroll
  for (int j = 0; j < D - 1; ++j)
    if (kb + j < kbs) step(kb + j, j);
  // Drain the stages issued past K before the slots are reused by the next item.
  wait_vmcnt<0>();

  // Epilogue. Lane (r0 = 4 (lane / 16), col = lane % 16) holds rows r0..r0+3 of each
  // 16-row group, route column col of each block.
  const int r0 = 4 * (lane >> 4), col = lane & 15;
  if (PHASE == 1) {
    const float g13 = p.g13[e], g2 = p.g2[e];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      if (b < nb) {
        const int64_t slot = (fb + b) * kBlockM + col;
        const int2 info = p.slot_info[slot];
        const float rw = info.x >= 0 ? __int_as_float(info.y) * g2 : 0.f;
        uint16_t* dst = p.inter + slot * g.ip;
        if (g.act == ACT_SWIGLU) {
#pragma unroll
          for (int pr = 0; pr < 2; ++pr) {
            if (rg_base + 2 * pr < c.groups) {
              float a[4];
#pragma unroll
              for (int i = 0; i < 4; ++i)
                a[i] = silu_f32(acc[2 * pr][b][i] * g13) * (acc[2 * pr + 1][b][i] * g13) * rw;
              const int64_t icol = int64_t((rg_base + 2 * pr) >> 1) * 16 + r0;
              *reinterpret_cast<uint2*>(dst + icol) = make_uint2(pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]));
            }
          }
        } else {
#pragma unroll
          for (int f = 0; f < 4; ++f) {
            if (rg_base + f < c.groups) {
              float a[4];
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const float u = fmaxf(acc[f][b][i] * g13, 0.f);
                a[i] = u * u * rw;
              }
              const int64_t icol = int64_t(rg_base + f) * 16 + r0;
              *reinterpret_cast<uint2*>(dst + icol) = make_uint2(pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]));
            }
          }
        }
      }
    }
  } else {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      if (b < nb) {
        const int64_t slot = (fb + b) * kBlockM + col;
        const int t = p.slot_info[slot].x;
        if (t >= 0) {
#pragma unroll
          for (int f = 0; f < 4; ++f) {
            if (rg_base + f < c.groups) {
              const int64_t h = int64_t(rg_base + f) * 16 + r0;
              float* dst = p.acc + int64_t(t) * g.H + h;
#pragma unroll
              for (int i = 0; i < 4; ++i)
                if (h + i < g.H) atomicAdd(dst + i, acc[f][b][i]);
            }
          }
        }
      }
    }
  }
}

template <int FMT, int PHASE>
__global__ __launch_bounds__(kGemmThreads, 1) void gemm_kernel(FusedParams p) {
  extern __shared__ __align__(16) uint8_t lds[];
  const PreparedGeom& g = p.g;
  GemmCtx c;
  c.groups = int(PHASE == 1 ? g.n1_groups : g.n2_groups);
  c.kbs = int(PHASE == 1 ? g.kb1 : g.kb2);
  c.nib = PHASE == 1 ? p.nib1 : p.nib2;
  c.scb = PHASE == 1 ? p.sc1 : p.sc2;
  c.sc_per_group = PHASE == 1 ? g.sc1_per_group : g.sc2_per_group;
  if (PHASE == 1) {
    c.act_row_bytes = g.H * 2;
    c.k_bytes = g.H * 2;
    c.act = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p.x), 0, int(int64_t(p.m) * g.H * 2), 0x00020000);
  } else {
    c.act_row_bytes = int(g.ip * 2);
    c.k_bytes = int(g.ip * 2);
    c.act = __builtin_amdgcn_make_buffer_rsrc(p.inter, 0, int(p.cap_blocks * kBlockM * g.ip * 2), 0x00020000);
  }
  const int n_mt = p.live[4];
  const int n_nt = (c.groups + 15) / 16;
  const int n_items = n_mt * n_nt;
  // Persistent workgroups take items from a queue (reset by the route packer) in M-tile
  // order, N fastest: the workgroups that share an activation tile, and the consecutive M
  // tiles of one expert that share its weight tiles, run at the same time, so the re-reads
  // hit the caches; full tiles are queued first, so the load stays balanced to the end.
  __shared__ int s_item;
  int* queue = p.live + (PHASE == 1 ? 5 : 6);
  for (;;) {
    if (threadIdx.x == 0) s_item = atomicAdd(queue, 1);
    lds_barrier();
    const int item = __builtin_amdgcn_readfirstlane(s_item);
    if (item >= n_items) break;
    // Every item starts with a barrier after this read, so thread 0 cannot overwrite
    // s_item before all threads have taken it.
    const int mt = item / n_nt, nt = item % n_nt;
    const int nb = __builtin_amdgcn_readfirstlane(p.tiles[mt].y & 0xFF);
    // Tiles are compiled for 1, 2, 4 or 8 route blocks so that the MFMA loop is straight-line.
    if (nb <= 1) gemm_item<FMT, PHASE, 1>(p, c, lds, mt, nt);
    else if (nb <= 2) gemm_item<FMT, PHASE, 2>(p, c, lds, mt, nt);
    else if (nb <= 4) gemm_item<FMT, PHASE, 4>(p, c, lds, mt, nt);
    else gemm_item<FMT, PHASE, 8>(p, c, lds, mt, nt);
  }
}

// out[i] = bf16(acc[i]) for the m x H accumulator.
__global__ void finalize_kernel(const float* __restrict__ acc, uint16_t* __restrict__ out, int64_t n) {
  const int64_t n2 = n / 2;
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n2; i += int64_t(gridDim.x) * blockDim.x) {
    const float2 v = reinterpret_cast<const float2*>(acc)[i];
    reinterpret_cast<uint32_t*>(out)[i] = pack_bf16x2(v.x, v.y);
  }
  if (blockIdx.x == 0 && threadIdx.x == 0 && (n & 1)) {
    bf16x2 v;
    v[0] = (__bf16)acc[n - 1];
    out[n - 1] = __builtin_bit_cast(uint16_t, v[0]);
  }
}

}  // namespace

template <int FMT, int PHASE>
hipError_t allow_large_lds(size_t lds) {
  // The stage ring needs more than the 64 KiB default of dynamic LDS.
  static hipError_t once = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_kernel<FMT, PHASE>),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
  return once;
}

hipError_t launch_gemm(const FusedParams& p, int num_cus, hipStream_t stream, hipEvent_t* marks) {
  // One 4-wave workgroup per CU: 128 accumulator AGPRs + ~230 VGPRs per wave leave room for one.
  const int grid = num_cus;
  const size_t lds = kLdsBytes;
  hipError_t e = p.g.fmt == FMT_NVFP4 ? allow_large_lds<FMT_NVFP4, 1>(lds) : allow_large_lds<FMT_MXFP4, 1>(lds);
  if (e == hipSuccess) e = p.g.fmt == FMT_NVFP4 ? allow_large_lds<FMT_NVFP4, 2>(lds) : allow_large_lds<FMT_MXFP4, 2>(lds);
  if (e != hipSuccess) return e;
  const bool nv = p.g.fmt == FMT_NVFP4;
  if (nv) hipLaunchKernelGGL((gemm_kernel<FMT_NVFP4, 1>), dim3(grid), dim3(kGemmThreads), lds, stream, p);
  else hipLaunchKernelGGL((gemm_kernel<FMT_MXFP4, 1>), dim3(grid), dim3(kGemmThreads), lds, stream, p);
  if (marks) (void)hipEventRecord(marks[0], stream);
  if (nv) hipLaunchKernelGGL((gemm_kernel<FMT_NVFP4, 2>), dim3(grid), dim3(kGemmThreads), lds, stream, p);
  else hipLaunchKernelGGL((gemm_kernel<FMT_MXFP4, 2>), dim3(grid), dim3(kGemmThreads), lds, stream, p);
  if (marks) (void)hipEventRecord(marks[1], stream);
  const int64_t n = p.m * p.g.H;
  int64_t fb = (n / 2 + 255) / 256;
  if (fb < 1) fb = 1;
  if (fb > 4096) fb = 4096;
  hipLaunchKernelGGL(finalize_kernel, dim3(fb), dim3(256), 0, stream, p.acc, p.out, n);
  if (marks) (void)hipEventRecord(marks[2], stream);
  return hipGetLastError();
}

}  // namespace moe
