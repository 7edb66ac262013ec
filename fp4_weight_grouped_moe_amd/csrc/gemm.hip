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
constexpr int kTileRows = kTileBlocks * kBlockM;        // 128
constexpr int kLdsStride = kKBlock + 8;                 // bf16 per LDS row (16 B pad vs bank conflicts)
constexpr int kLdsBuf = kTileRows * kLdsStride;         // bf16 per buffer
constexpr int kStageChunks = kTileRows * (kKBlock / 8) / kGemmThreads;   // 16-byte chunks per thread: 8
constexpr int kXcds = 8;


struct WRegs {
  u32x4 q[4];                        // one 1 KiB fragment block per row group
  uint32_t s[4];                     // its scale dword
};

template <int FMT, int PHASE>
__global__ __launch_bounds__(kGemmThreads, 1) void gemm_kernel(FusedParams p) {
  extern __shared__ __align__(16) uint16_t lds[];
  const PreparedGeom& g = p.g;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n_mt = p.live[4];
  const int groups = int(PHASE == 1 ? g.n1_groups : g.n2_groups);
  const int n_nt = (groups + 15) / 16;
  const int kbs = int(PHASE == 1 ? g.kb1 : g.kb2);
  const uint8_t* nib = PHASE == 1 ? p.nib1 : p.nib2;
  const uint8_t* scb = PHASE == 1 ? p.sc1 : p.sc2;
  const int64_t sc_per_group = PHASE == 1 ? g.sc1_per_group : g.sc2_per_group;
  const int n_items = n_mt * n_nt;
  // Items run M tile by M tile (N fastest) in contiguous ranges per XCD (workgroups are dealt
  // to the XCDs round robin): the workgroups of one XCD share an activation tile in their L2,
  // and the M tiles of one expert revisit its weight tiles while they are still in the
  // Infinity Cache.
  const int xcd = blockIdx.x % kXcds, wg_in_xcd = blockIdx.x / kXcds, wgs_per_xcd = gridDim.x / kXcds;
  const int per_xcd = (n_items + kXcds - 1) / kXcds;
  const int item_lo = xcd * per_xcd;
  const int item_hi = min(n_items, item_lo + per_xcd);
  const int seg = tid & 15;              // staging: this thread's 16-byte column segment
  const int srow0 = tid >> 4;            // and its first row (rows srow0 + 16 j)
  const int sc_lane = FMT == FMT_NVFP4 ? ((lane >> 5) * 16 + (lane & 15)) * 16 : (lane & 15) * 16;

  for (int item = item_lo + wg_in_xcd; item < item_hi; item += wgs_per_xcd) {
    const int mt = item / n_nt, nt = item % n_nt;
    const int2 tile = p.tiles[mt];
    const int64_t fb = tile.x;
    const int nb = tile.y & 0xFF;
    const int e = __builtin_amdgcn_readfirstlane(tile.y >> 8);
    const int rows = nb * kBlockM;

    // Source offsets (in bf16 elements, at K block 0) of this thread's staging rows; -1 = zero row.
    int64_t src[kStageChunks];
#pragma unroll
    for (int j = 0; j < kStageChunks; ++j) {
      const int row = srow0 + 16 * j;
      src[j] = -1;
      if (row < rows) {
        const int64_t slot = fb * kBlockM + row;
        if (PHASE == 1) {
          const int t = p.slot_info[slot].x;
          if (t >= 0) src[j] = int64_t(t) * g.H + seg * 8;
        } else {
          src[j] = slot * g.ip + seg * 8;
        }
      }
    }
    const uint16_t* bsrc = PHASE == 1 ? p.x : p.inter;
    const int64_t kmax = PHASE == 1 ? g.H : g.ip;
    auto stage_load = [&](int kb, u32x4* r) {
#pragma unroll
      for (int j = 0; j < kStageChunks; ++j) {
        const int64_t k = int64_t(kb) * kKBlock;
        if (src[j] >= 0 && k + seg * 8 < kmax) r[j] = *reinterpret_cast<const u32x4*>(bsrc + src[j] + k);
        else r[j] = u32x4{0u, 0u, 0u, 0u};
      }
    };
    auto stage_store = [&](int buf, const u32x4* r) {
#pragma unroll
      for (int j = 0; j < kStageChunks; ++j) {
        const int row = srow0 + 16 * j;
        if (row < rows) *reinterpret_cast<u32x4*>(lds + buf * kLdsBuf + row * kLdsStride + seg * 8) = r[j];
      }
    };

    // This wave's four row groups (wave-uniform base addresses; lanes add 32-bit offsets).
    const int rg_base = nt * 16 + wave * 4;
    bool fvalid[4];
    const uint8_t* nbp[4];
    const uint8_t* sgp[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      const int rg = rg_base + f;
      fvalid[f] = rg < groups;
      const int64_t gi = int64_t(e) * groups + (fvalid[f] ? rg : 0);
      nbp[f] = nib + gi * kbs * kFragBytes;
      sgp[f] = scb + gi * sc_per_group;
    }
    // Loads are unconditional (a K block past the end re-reads the last one, never used) so
    // the wait counters stay exact across the three-deep ring below.
    auto load_w = [&](int kb, WRegs& w) {
      kb = min(kb, kbs - 1);
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        w.q[f] = *reinterpret_cast<const u32x4*>(nbp[f] + int64_t(kb) * kFragBytes + lane * 16);
        w.s[f] = *reinterpret_cast<const uint32_t*>(sgp[f] + int64_t(kb >> 2) * g.sc_chunk_bytes + sc_lane + (kb & 3) * 4);
      }
    };

    f32x4 acc[4][kTileBlocks];
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
      for (int b = 0; b < kTileBlocks; ++b) acc[f][b] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](int buf_idx, const WRegs& w) {
      const uint16_t* buf = lds + buf_idx * kLdsBuf;
      float scl[4][4];
#pragma unroll
      for (int f = 0; f < 4; ++f) decode_scales<FMT>(w.s[f], scl[f]);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        bf16x8 a[4];
#pragma unroll
        for (int f = 0; f < 4; ++f) a[f] = dq8<FMT>(w.q[f][s], scl[f][s]);
#pragma unroll
        for (int b = 0; b < kTileBlocks; ++b) {
          if (b < nb) {
            const bf16x8 xb = load_bf16x8(buf + (b * kBlockM + (lane & 15)) * kLdsStride + 32 * s + 8 * (lane >> 4));
#pragma unroll
            for (int f = 0; f < 4; ++f)
              if (fvalid[f]) acc[f][b] = mfma16(a[f], xb, acc[f][b]);
          }
        }
      }
    };

    // One K block per step: weights two blocks ahead in registers, activations one block
    // ahead in the other LDS buffer; barriers order LDS only, so the weight loads in flight
    // are not drained.
    u32x4 xr[kStageChunks];
    auto step = [&](int kb, const WRegs& cur, WRegs& ahead2) {
      if (kb < kbs) {
        load_w(kb + 2, ahead2);
        const bool more = kb + 1 < kbs;
        if (more) stage_load(kb + 1, xr);
        compute(kb & 1, cur);
        if (more) stage_store((kb + 1) & 1, xr);
      }
      lds_barrier();
    };
    WRegs wa, wb, wc;
    stage_load(0, xr);
    load_w(0, wa);
    load_w(1, wb);
    stage_store(0, xr);
    lds_barrier();
    for (int kb = 0; kb < kbs; kb += 3) {
      step(kb, wa, wc);
      step(kb + 1, wb, wa);
      step(kb + 2, wc, wb);
    }

    // Epilogue.
    const int r0 = 4 * (lane >> 4), col = lane & 15;
    if (PHASE == 1) {
      const float g13 = p.g13[e], g2 = p.g2[e];
#pragma unroll
      for (int b = 0; b < kTileBlocks; ++b) {
        if (b < nb) {
          const int64_t slot = (fb + b) * kBlockM + col;
          const int2 info = p.slot_info[slot];
          const float rw = info.x >= 0 ? __int_as_float(info.y) * g2 : 0.f;
          uint16_t* dst = p.inter + slot * g.ip;
          if (g.act == ACT_SWIGLU) {
#pragma unroll
            for (int pr = 0; pr < 2; ++pr) {
              if (fvalid[2 * pr]) {
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
              if (fvalid[f]) {
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
      for (int b = 0; b < kTileBlocks; ++b) {
        if (b < nb) {
          const int64_t slot = (fb + b) * kBlockM + col;
          const int t = p.slot_info[slot].x;
          if (t >= 0) {
#pragma unroll
            for (int f = 0; f < 4; ++f) {
              if (fvalid[f]) {
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
  // The double-buffered tile needs more than the 64 KiB default of dynamic LDS.
  static hipError_t once = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_kernel<FMT, PHASE>),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
  return once;
}

hipError_t launch_gemm(const FusedParams& p, int num_cus, hipStream_t stream, hipEvent_t* marks) {
  // One 4-wave workgroup per CU: 128 accumulator AGPRs + ~230 VGPRs per wave leave room for one.
  const int grid = ((num_cus + kXcds - 1) / kXcds) * kXcds;
  const size_t lds = size_t(2) * kLdsBuf * sizeof(uint16_t);
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
