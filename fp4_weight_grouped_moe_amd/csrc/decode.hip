// Small-batch (decode) path of the fused W4A16 MoE layer on gfx950.
//
// FlashInfer PR 4255, Description: a tensor-core decode path for small batches that folds
// the top-k sum into the FC2 store epilogue and removes a separate launch; Reviewer
// Notes: the decode path is chosen up to a small m. At m <= 16 the layer is bound by the
// weight bytes streamed from HBM, so both kernels are built as weight streams: each wave
// walks a list of units (a few 16 x 128 fragment blocks), always holding the next unit's
// 128-bit loads in flight in a second register set while it dequantises the current one
// in registers straight into MFMA A operands. Loop bounds are wave-uniform and loads are
// unconditional (addresses clamped, contributions masked), so no load waits on a branch.
//  * FC1: a workgroup (4 waves) owns one (route block, 16 or 32 FC1 columns) item at a
//    time; its K blocks are dealt to the waves in slices, partial sums meet in LDS, and
//    wave 0 applies the FC1 global scale, the activation, the router weight and the FC2
//    global scale and stores the bf16 row slice of each route. The activation rows of
//    all m tokens sit in LDS.
//  * FC2: a workgroup (16 waves) owns 16 hidden rows for every route block; each unit's
//    route results are added into per-wave, per-token LDS sums (the top-k sum), which are
//    reduced in a fixed order and stored once as bf16 -- deterministic, no global atomics.
#include <hip/hip_runtime.h>

#include "device.hpp"
#include "kernels.hpp"
#include "layout.hpp"

namespace moe {

namespace {

constexpr int kF1Threads = 256;
constexpr int kF1Waves = kF1Threads / 64;
constexpr int kF1Slice = 4;          // K blocks per FC1 unit
constexpr int kF2Threads = 1024;
constexpr int kF2Waves = kF2Threads / 64;
constexpr int kF2Slice = 2;          // K blocks per FC2 unit

__device__ __forceinline__ uint32_t scale_dword(const uint8_t* sc_group, int64_t kb, int lane, bool nv) {
  // Scales of K block kb for this lane: NVFP4 chunk [h][row][kb%4][s], MXFP4 [row][kb%4][s].
  const int r = lane & 15;
  const int64_t chunk = kb >> 2;
  const int sub = int(kb & 3);
  const int64_t off = nv ? chunk * 512 + ((lane >> 5) * 16 + r) * 16 + sub * 4 : chunk * 256 + r * 16 + sub * 4;
  return *reinterpret_cast<const uint32_t*>(sc_group + off);
}

// 16-byte chunk j of LDS row `row` is stored at chunk j ^ (row & 7) inside every complete
// group of 8 chunks, so lanes reading the same K of different rows hit different banks.
__device__ __forceinline__ int64_t swz(int64_t j, int row, int64_t chunks_per_row) {
  return ((j | 7) < chunks_per_row) ? (j ^ (row & 7)) : j;
}

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// ----------------------------------------------------------------------------- FC1

struct F1Unit {
  u32x4 q0[kF1Slice], q1[kF1Slice];
  uint32_t s0[kF1Slice], s1[kF1Slice];
  int2 info;                         // (token, router weight) of this lane's route column
};

template <int FMT, bool STAGED>
__global__ __launch_bounds__(kF1Threads, 2) void decode_fc1_kernel(FusedParams p) {
  extern __shared__ __align__(16) uint8_t dyn[];
  __shared__ f32x4 red[kF1Waves][2][64];
  const PreparedGeom& g = p.g;
  const int tid = threadIdx.x, lane = tid & 63, wave = uniform(tid >> 6);
  const bool nv = FMT == FMT_NVFP4;
  const int64_t H = g.H, xchunks = H / 8;
  const int64_t live_blocks = p.live[2];
  int4* bt = reinterpret_cast<int4*>(dyn);                   // block -> (expert, g13, g2)
  uint16_t* xs = reinterpret_cast<uint16_t*>(dyn + p.lds_block_table);   // [m][H], chunk-swizzled

  for (int64_t b = tid; b < live_blocks; b += kF1Threads) {
    const int e = p.block_expert[b];
    bt[b] = make_int4(e, __float_as_int(p.g13[e]), __float_as_int(p.g2[e]), 0);
  }
  if (STAGED) {
    for (int64_t c = tid; c < p.m * xchunks; c += kF1Threads) {
      const int64_t t = c / xchunks, j = c % xchunks;
      *reinterpret_cast<u32x4*>(xs + t * H + swz(j, int(t), xchunks) * 8) =
          *reinterpret_cast<const u32x4*>(p.x + t * H + j * 8);
    }
  }
  lds_barrier();

  const int64_t n_it = g.n1_groups / 2;                      // items per block: two row groups
  const int64_t n_items = live_blocks * n_it;
  const int64_t nsl = (g.kb1 + kF1Slice - 1) / kF1Slice;      // K slices per item
  const int64_t spw = (nsl + kF1Waves - 1) / kF1Waves;        // slices per wave per item
  const int64_t my_items = n_items > blockIdx.x ? (n_items - blockIdx.x + gridDim.x - 1) / gridDim.x : 0;
  const int64_t U = my_items * spw;
  const int64_t U2 = (U + 1) & ~int64_t(1);                  // even: the loop below takes units in pairs
  const int col = lane & 15;

  auto unit_item = [&](int64_t u) { return int64_t(blockIdx.x) + (u / spw) * gridDim.x; };
  auto unit_slice = [&](int64_t u) { return wave + kF1Waves * (u % spw); };

  // Loads are unconditional so that the wait counters stay exact: units past the end and
  // slices past K re-read a valid block (an L2 hit) whose contribution is masked.
  auto issue = [&](int64_t u, F1Unit& r) {
    u = min(u, U - 1);
    const int64_t item = unit_item(u), sl = min(unit_slice(u), nsl - 1);
    const int64_t blk = item / n_it, it = item % n_it;
    r.info = p.slot_info[blk * kBlockM + col];
    const int64_t gi = int64_t(bt[blk].x) * g.n1_groups + 2 * it;
    const uint8_t* nb0 = p.nib1 + gi * g.kb1 * kFragBytes + lane * 16;
    const uint8_t* nb1 = nb0 + g.kb1 * kFragBytes;
    const uint8_t* sg0 = p.sc1 + gi * g.sc1_per_group;
    const uint8_t* sg1 = sg0 + g.sc1_per_group;
#pragma unroll
    for (int j = 0; j < kF1Slice; ++j) {
      const int64_t kb = min(sl * kF1Slice + j, g.kb1 - 1);
      r.q0[j] = *reinterpret_cast<const u32x4*>(nb0 + kb * kFragBytes);
      r.q1[j] = *reinterpret_cast<const u32x4*>(nb1 + kb * kFragBytes);
      r.s0[j] = scale_dword(sg0, kb, lane, nv);
      r.s1[j] = scale_dword(sg1, kb, lane, nv);
    }
  };

  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  auto compute = [&](int64_t u, const F1Unit& r) {
    const int64_t sl = unit_slice(u);
    if (u < U && sl < nsl) {
      const int tok = r.info.x;
#pragma unroll
      for (int j = 0; j < kF1Slice; ++j) {
        const int64_t kb = sl * kF1Slice + j;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int64_t k = kb * kKBlock + 32 * s + 8 * (lane >> 4);
          bf16x8 xb = zero_bf16x8();
          if (tok >= 0 && k < H) {
            if (STAGED) xb = load_bf16x8(xs + int64_t(tok) * H + swz(k >> 3, tok, xchunks) * 8);
            else xb = load_bf16x8(p.x + int64_t(tok) * H + k);
          }
          acc0 = mfma16(dq8<FMT>(r.q0[j][s], (r.s0[j] >> (8 * s)) & 0xFF), xb, acc0);
          acc1 = mfma16(dq8<FMT>(r.q1[j][s], (r.s1[j] >> (8 * s)) & 0xFF), xb, acc1);
        }
      }
    }
  };

  auto finish = [&](int64_t u, const F1Unit& r) {
    if (u >= U || u % spw != spw - 1) return;                 // not the item's last slice
    red[wave][0][lane] = acc0;
    red[wave][1][lane] = acc1;
    acc0 = f32x4{0.f, 0.f, 0.f, 0.f};
    acc1 = f32x4{0.f, 0.f, 0.f, 0.f};
    lds_barrier();
    if (wave == 0) {
      f32x4 h0 = red[0][0][lane], h1 = red[0][1][lane];
#pragma unroll
      for (int w = 1; w < kF1Waves; ++w) {
        h0 += red[w][0][lane];
        h1 += red[w][1][lane];
      }
      const int64_t item = unit_item(u);
      const int64_t blk = item / n_it, it = item % n_it;
      const int4 b4 = bt[blk];
      const int tok = r.info.x;
      const float g13 = __int_as_float(b4.y), g2 = __int_as_float(b4.z);
      const float rw = (tok >= 0) ? __int_as_float(r.info.y) * g2 : 0.f;
      uint16_t* dst = p.inter + (blk * kBlockM + col) * g.ip;
      const int r0 = 4 * (lane >> 4);
      if (g.act == ACT_SWIGLU) {
        float a[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = silu_f32(h0[i] * g13) * (h1[i] * g13) * rw;
        *reinterpret_cast<uint2*>(dst + it * 16 + r0) = make_uint2(pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]));
      } else {
        float a[4], b[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float x0 = fmaxf(h0[i] * g13, 0.f), x1 = fmaxf(h1[i] * g13, 0.f);
          a[i] = x0 * x0 * rw;
          b[i] = x1 * x1 * rw;
        }
        *reinterpret_cast<uint2*>(dst + 32 * it + r0) = make_uint2(pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]));
        *reinterpret_cast<uint2*>(dst + 32 * it + 16 + r0) = make_uint2(pack_bf16x2(b[0], b[1]), pack_bf16x2(b[2], b[3]));
      }
    }
    lds_barrier();
  };

  if (U == 0) return;
  F1Unit ra, rb;
  issue(0, ra);
  for (int64_t u = 0; u < U2; u += 2) {
    issue(u + 1, rb);
    compute(u, ra);
    finish(u, ra);
    issue(u + 2, ra);
    compute(u + 1, rb);
    finish(u + 1, rb);
  }
}

// ----------------------------------------------------------------------------- FC2

struct F2Unit {
  u32x4 q[kF2Slice];
  uint32_t s[kF2Slice];
  bf16x8 b[kF2Slice][4];
};

template <int FMT>
__global__ __launch_bounds__(kF2Threads, 1) void decode_fc2_kernel(FusedParams p) {
  extern __shared__ __align__(16) uint8_t dyn[];
  __shared__ float tacc[kF2Waves][kDecodeMaxM][16];
  const PreparedGeom& g = p.g;
  const int tid = threadIdx.x, lane = tid & 63, wave = uniform(tid >> 6);
  const bool nv = FMT == FMT_NVFP4;
  const int64_t ht = blockIdx.x;                             // 16 hidden rows per workgroup
  const int64_t live_blocks = p.live[2];
  int* be = reinterpret_cast<int*>(dyn);                     // block -> expert
  int* stok = be + p.cap_blocks;                             // slot -> token (-1 = padding)
  for (int64_t b = tid; b < live_blocks; b += kF2Threads) be[b] = p.block_expert[b];
  for (int64_t s = tid; s < live_blocks * kBlockM; s += kF2Threads) stok[s] = p.slot_info[s].x;
  for (int i = tid; i < kF2Waves * kDecodeMaxM * 16; i += kF2Threads) (&tacc[0][0][0])[i] = 0.f;
  lds_barrier();

  const int64_t nsl = (g.kb2 + kF2Slice - 1) / kF2Slice;
  const int64_t units = live_blocks * nsl;
  const int64_t U = units > wave ? (units - wave + kF2Waves - 1) / kF2Waves : 0;
  const int64_t U2 = (U + 1) & ~int64_t(1);
  const int col = lane & 15;

  // Unconditional loads (units past the end re-read the last one, masked) keep the wait
  // counters exact across the ping-pong.
  auto issue = [&](int64_t u, F2Unit& r) {
    const int64_t unit = wave + min(u, U - 1) * kF2Waves;
    const int64_t blk = unit / nsl, sl = unit % nsl;
    const int64_t e = be[blk];
    const uint8_t* nb = p.nib2 + ((e * g.n2_groups + ht) * g.kb2) * kFragBytes + lane * 16;
    const uint8_t* sg = p.sc2 + (e * g.n2_groups + ht) * g.sc2_per_group;
    const int64_t slot = blk * kBlockM + col;
    const bool valid = stok[slot] >= 0;
    const uint16_t* irow = p.inter + slot * g.ip + 8 * (lane >> 4);
#pragma unroll
    for (int j = 0; j < kF2Slice; ++j) {
      const int64_t kb = sl * kF2Slice + j;
      const int64_t kbc = min(kb, g.kb2 - 1);                 // clamped; masked through the B operand
      r.q[j] = *reinterpret_cast<const u32x4*>(nb + kbc * kFragBytes);
      r.s[j] = scale_dword(sg, kbc, lane, nv);
#pragma unroll
      for (int s = 0; s < 4; ++s)
        r.b[j][s] = (valid && kb < g.kb2) ? load_bf16x8(irow + kb * kKBlock + 32 * s) : zero_bf16x8();
    }
  };
  auto compute = [&](int64_t u, const F2Unit& r) {
    if (u >= U) return;
    const int64_t unit = wave + u * kF2Waves;
    const int64_t blk = unit / nsl;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < kF2Slice; ++j)
#pragma unroll
      for (int s = 0; s < 4; ++s) acc = mfma16(dq8<FMT>(r.q[j][s], (r.s[j] >> (8 * s)) & 0xFF), r.b[j][s], acc);
    const int tok = stok[blk * kBlockM + col];
    if (tok >= 0) {
      const int r0 = 4 * (lane >> 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) atomicAdd(&tacc[wave][tok][r0 + i], acc[i]);
    }
  };

  if (U > 0) {
    F2Unit ra, rb;
    issue(0, ra);
    for (int64_t u = 0; u < U2; u += 2) {
      issue(u + 1, rb);
      compute(u, ra);
      issue(u + 2, ra);
      compute(u + 1, rb);
    }
  }
  lds_barrier();
  // Sum the waves in a fixed order and store out[t, 16*ht .. 16*ht + 15] (zero for tokens
  // whose every route was dropped).
  for (int i = tid; i < kDecodeMaxM * 16; i += kF2Threads) {
    const int t = i >> 4, j = i & 15;
    const int64_t h = ht * 16 + j;
    if (t < p.m && h < g.H) {
      float s = 0.f;
      for (int w = 0; w < kF2Waves; ++w) s += tacc[w][t][j];
      bf16x2 v;
      v[0] = (__bf16)s;
      p.out[t * g.H + h] = __builtin_bit_cast(uint16_t, v[0]);
    }
  }
}

template <typename K>
hipError_t allow_lds(K kernel, int bytes) {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
}

template <int FMT>
hipError_t launch_decode_fmt(const FusedParams& p0, int num_cus, hipStream_t stream, hipEvent_t* marks) {
  static const hipError_t lds_ok = [] {
    hipError_t e = allow_lds(&decode_fc1_kernel<FMT, true>, kDecodeStageBytes + 16384);
    if (e == hipSuccess) e = allow_lds(&decode_fc1_kernel<FMT, false>, 16384);
    if (e == hipSuccess) e = allow_lds(&decode_fc2_kernel<FMT>, 65536);
    return e;
  }();
  if (lds_ok != hipSuccess) return lds_ok;
  FusedParams p = p0;
  const PreparedGeom& g = p.g;
  const size_t table = align256(size_t(p.cap_blocks) * sizeof(int4));
  p.lds_block_table = int64_t(table);
  const int64_t items = p.cap_blocks * (g.n1_groups / 2);
  const int64_t grid1 = max(int64_t(1), min(items, int64_t(num_cus) * 2));
  const size_t xs_bytes = size_t(p.m) * g.H * 2;
  if (xs_bytes <= size_t(kDecodeStageBytes))
    hipLaunchKernelGGL((decode_fc1_kernel<FMT, true>), dim3(grid1), dim3(kF1Threads), table + xs_bytes, stream, p);
  else
    hipLaunchKernelGGL((decode_fc1_kernel<FMT, false>), dim3(grid1), dim3(kF1Threads), table, stream, p);
  if (marks) (void)hipEventRecord(marks[0], stream);
  const size_t lds2 = size_t(p.cap_blocks) * 4 + size_t(p.cap_blocks) * kBlockM * 4;
  hipLaunchKernelGGL((decode_fc2_kernel<FMT>), dim3(g.n2_groups), dim3(kF2Threads), lds2, stream, p);
  if (marks) {
    (void)hipEventRecord(marks[1], stream);
    (void)hipEventRecord(marks[2], stream);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const FusedParams& p, int num_cus, hipStream_t stream, hipEvent_t* marks) {
  return p.g.fmt == FMT_NVFP4 ? launch_decode_fmt<FMT_NVFP4>(p, num_cus, stream, marks)
                              : launch_decode_fmt<FMT_MXFP4>(p, num_cus, stream, marks);
}

}  // namespace moe
