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
//  * FC1: one workgroup (8 waves) per CU owns one (route block, 16 or 32 FC1 columns) item
//    at a time; its K blocks are dealt to the waves in slices, partial sums meet in LDS, and
//    wave 0 applies the FC1 global scale, the activation, the router weight and the FC2
//    global scale and stores the bf16 row slice of each route. The activation rows of
//    all m tokens sit in LDS, staged by DMA. (Two 4-wave workgroups per CU shared the CU's
//    bandwidth unevenly: the older one streamed its items ~25% faster, so the younger ones
//    set the launch's end.)
//  * FC2 (K split): a workgroup owns a few hidden row groups and one pair of intermediate
//    K blocks for every route block, with that K slice of every route staged in LDS; route
//    results go into per-wave, per-token LDS sums (the top-k sum), and the last K split of
//    a row group to finish adds the splits in a fixed order and stores bf16 once --
//    deterministic, no atomics on data.
//  * FC2 (one pass, when the staged rows do not fit): a workgroup (16 waves) owns 16 hidden
//    rows for every route block and full K, with the same per-token LDS sums.
//  * W4A8 (MXFP4 weights): the K-split FC2 rounds the staged slice of every route from FC1's
//    fp32 rows to MXFP8 itself and runs the block-scaled FP4 x FP8 MFMA on the codes.
#include <hip/hip_runtime.h>

#include "device.hpp"
#include "kernels.hpp"
#include "layout.hpp"

namespace moe {

namespace {

constexpr int kF1Threads = 512;  // one 8-wave workgroup per CU (two 4-wave ones shared a CU unevenly)
constexpr int kF1Waves = kF1Threads / 64;
constexpr int kF1Slice = 4;          // K blocks per FC1 unit
constexpr int kF2Threads = 1024;
constexpr int kF2Waves = kF2Threads / 64;
constexpr int kF2Slice = 2;          // K blocks per FC2 unit
constexpr int kF1PackRoutes = 256;   // FC1 packs the routes itself up to this many (one per thread of the first four waves)
constexpr int kF1PackExperts = 2048; // and this many local experts (their counts share the partial-sum area)
constexpr int kF1StaticLds = 2 * (kF1Waves - 1) * 2 * 64 * 16;   // the partial-sum area
constexpr int kLdsPerCU = 163840;
static_assert(kF1PackRoutes <= kF1Threads, "one route per thread");
// Rows + pack tables of the FC1 launch that packs its own routes (m <= 8 at hidden 4096)
constexpr size_t kF1PackRowsBudget = 69632;

// Route blocks the pack of R routes over E experts can produce: at most one per route, and
// at most one per touched expert plus R / 16 more.
__host__ __device__ inline int f1_pack_blocks(int routes, int E) {
  const int t = routes < E ? routes : E;
  const int b = t + (routes + kBlockM - 1) / kBlockM;
  return routes < b ? routes : b;
}
// LDS of the pack tables: slot -> route (int16), block -> expert, route -> weight, token (int16).
__host__ __device__ inline size_t f1_pack_lds_bytes(int routes, int E) {
  const int nb = f1_pack_blocks(routes, E);
  return size_t(nb) * kBlockM * 2 + size_t(nb) * 4 + size_t(routes) * 4 + (size_t(routes) * 2 + 15) / 16 * 16;
}

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Workgroup barrier over LDS only: this wave's LDS operations have completed (lgkmcnt 0),
// while its loads into LDS by DMA may still be in flight (a release fence would wait for
// them too).
__device__ __forceinline__ void pack_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ----------------------------------------------------------------------------- FC1

static_assert(kF1Slice == kScaleChunkKB, "one 16-byte scale load per fragment per FC1 unit");

struct F1Unit {
  u32x4 q0[kF1Slice], q1[kF1Slice];  // nibbles of the two row groups, one 1 KiB block per K block
  u32x4 s0, s1;                      // their scales: dword j = the four MFMA steps of K block j
  int2 info;                         // (token, router weight) of this lane's route column
};

template <int FMT, bool STAGED, bool PACK>
__global__ __launch_bounds__(kF1Threads, 1) void decode_fc1_kernel(FusedParams p) {
  extern __shared__ __align__(16) uint8_t dyn[];
  // Partial sums of waves 1..3 for the item epilogue, double-buffered by item parity so that
  // one barrier per item suffices: a wave refills a buffer only after the next item's
  // barrier, which wave 0 reaches only after it has read that buffer. The route pack (PACK)
  // uses the same area for its counts before the first item.
  __shared__ f32x4 red[2][kF1Waves - 1][2][64];
  static_assert(sizeof(red) >= (kF1PackExperts + 16) * 4 + kF1PackRoutes * 2, "pack scratch fits the partial-sum area");
  const PreparedGeom& g = p.g;
  const int tid = threadIdx.x, lane = tid & 63, wave = uniform(tid >> 6);
  const int q = lane >> 4, col = lane & 15;
  const int H = g.H;
  const int xp = int(p.xs_pitch);                            // elements per staged row
  uint16_t* xs = reinterpret_cast<uint16_t*>(dyn);           // [m][xp], chunk-swizzled
  int* sp = reinterpret_cast<int*>(dyn + size_t(p.m) * xp * 2);   // [64] per-token exponent p
  // PACK: the route tables after the exponents (f1_pack_lds_bytes).
  const int R = int(p.m) * p.topk;
  const int nbmax = f1_pack_blocks(R, g.E);
  int16_t* sroute = reinterpret_cast<int16_t*>(dyn + size_t(p.m) * xp * 2 + 256);   // [nbmax * 16] slot -> route
  int* sbe = reinterpret_cast<int*>(sroute + nbmax * kBlockM);                       // [nbmax] block -> expert
  float* sw = reinterpret_cast<float*>(sbe + nbmax);                                 // [R] router weight
  int16_t* stk = reinterpret_cast<int16_t*>(sw + R);                                 // [R] token

  const int n_it = int(g.n1_groups / 2);                      // items per block: two row groups
  const int nsl = int((g.kb1 + kF1Slice - 1) / kF1Slice);     // K slices per item
  const int spw = (nsl + kF1Waves - 1) / kF1Waves;            // slices per wave per item
  const int kb1 = int(g.kb1);
  const int sc_lane = FMT == FMT_NVFP4 ? ((lane >> 5) * 16 + col) * 16 : col * 16;
  // FC2's per-group arrival counts start at zero in every call.
  if (blockIdx.x == 0 && p.f2_count)
    for (int i = tid; i < int(g.n2_groups); i += kF1Threads) p.f2_count[i] = 0;
  int live_blocks = PACK ? 0 : p.live[2];
  if (!PACK && live_blocks * n_it <= int(blockIdx.x)) return;   // no item for this workgroup

  // NVFP4 runs on the f16 MFMA: E2M1 x E4M3 weights are exact in f16, and each token's row
  // is staged times a power of two 2^-p (exact) with its largest magnitude in [2^14, 2^15)
  // as f16 (converted by the route-pack launch, or here in LDS when this launch packs); the
  // epilogue multiplies by 2^p again.
  constexpr bool F16 = STAGED && FMT == FMT_NVFP4;
  if constexpr (STAGED) {
    // Activation rows into LDS by DMA, zero-padded to xp. Chunk j of row t sits at chunk
    // j ^ (t & 7) (hp is a multiple of 128, so every group of 8 chunks is complete): lanes
    // reading the same K of different tokens hit different banks. Lane i of a DMA row writes
    // LDS chunk 64c + i, so it fetches source chunk (64c + i) ^ (t & 7).
    // PACK: waves 1..3 stage the rows while wave 0 loads the routes (the pack waits on no DMA).
    const __amdgpu_buffer_rsrc_t xr = buffer_rsrc(F16 && !PACK ? p.x16 : p.x, uint32_t(p.m * H * 2));
    const int per_row = xp / 512;
    constexpr int kDmaWaves = PACK ? kF1Waves - 1 : kF1Waves;
    for (int n = PACK ? wave - 1 : wave; n >= 0 && n < int(p.m) * per_row; n += kDmaWaves) {
      const int t = n / per_row, c = n % per_row;
      const int j = (64 * c + lane) ^ (t & 7);
      dma16(xr, reinterpret_cast<const uint8_t*>(xs + t * xp + 512 * c), j * 8 < H ? uint32_t(t * H * 2 + j * 16) : kOutOfRange);
    }
    if (F16 && !PACK && wave == 0) dma4(buffer_rsrc(p.xexp, uint32_t(p.m * 4)), sp, uint32_t(lane * 4));
  }

  // The staged bf16 rows to f16 times 2^-p in place (NVFP4 with the routes packed here), one
  // wave per row.
  auto convert_rows = [&]() {
    const int nch = xp / 8;
    for (int t = wave; t < int(p.m); t += kF1Waves) {
      u32x4* row = reinterpret_cast<u32x4*>(xs + t * xp);
      float mx = 0.f;
      for (int c = lane; c < nch; c += 64) {
        const u32x4 v = row[c];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          mx = fmaxf(mx, fmaxf(fabsf(__uint_as_float(v[i] << 16)), fabsf(__uint_as_float(v[i] & 0xFFFF0000u))));
      }
#pragma unroll
      for (int d = 32; d >= 1; d >>= 1) mx = fmaxf(mx, __shfl_xor(mx, d, 64));
      const int pe = (mx > 0.f && mx <= 3.4e38f) ? __builtin_amdgcn_frexp_expf(mx) - 15 : 0;
      for (int c = lane; c < nch; c += 64) {
        const u32x4 v = row[c];
        u32x4 o;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const f16x2 h = f16x2{(_Float16)ldexpf(__uint_as_float(v[i] << 16), -pe),
                                (_Float16)ldexpf(__uint_as_float(v[i] & 0xFFFF0000u), -pe)};
          o[i] = __builtin_bit_cast(uint32_t, h);
        }
        row[c] = o;
      }
      if (lane == 0) sp[t] = pe;
    }
  };
  // A unit's weight loads: K slice `sl` of row groups 2 it, 2 it + 1 of expert eb (fragment
  // blocks and their scale dwords). Base addresses are wave-uniform (scalar registers); lanes
  // add a 32-bit offset.
  auto load_unit = [&](int eb, int it, int sl, F1Unit& r) {
    const int64_t gi = int64_t(eb) * g.n1_groups + 2 * it;
    const uint8_t* nb0 = p.nib1 + gi * g.kb1 * kFragBytes;
    const uint8_t* nb1 = nb0 + g.kb1 * kFragBytes;
#pragma unroll
    for (int j = 0; j < kF1Slice; ++j) {
      const int kb = min(sl * kF1Slice + j, kb1 - 1);
      r.q0[j] = *reinterpret_cast<const u32x4*>(nb0 + int64_t(kb) * kFragBytes + lane * 16);
      r.q1[j] = *reinterpret_cast<const u32x4*>(nb1 + int64_t(kb) * kFragBytes + lane * 16);
    }
    const uint8_t* sg0 = p.sc1 + gi * g.sc1_per_group + int64_t(sl) * g.sc_chunk_bytes;
    r.s0 = *reinterpret_cast<const u32x4*>(sg0 + sc_lane);
    r.s1 = *reinterpret_cast<const u32x4*>(sg0 + g.sc1_per_group + sc_lane);
  };
  F1Unit ra, rb;
  bool early = false;          // unit 0's weight loads already issued (PACK)

  if constexpr (PACK) {
    // The route pack of these few routes (R <= 256, one per thread), done by every workgroup
    // in its own LDS so that no launch waits for another: local expert ids, counts, padded
    // segment offsets (exclusive scan over the experts), block -> expert, and stable slots
    // (rank among the lower routes of the same expert), exactly as the route-pack kernel
    // orders them. Workgroup 0 also writes the tables FC2 reads.
    int* cnt = reinterpret_cast<int*>(&red[0][0][0][0]);     // [E] counts, then offsets
    int* scr = cnt + kF1PackExperts;                          // [16] scan scratch
    int16_t* sl = reinterpret_cast<int16_t*>(scr + 16);       // [256] local expert ids (-1 past R)
    // Barriers here order LDS only (lgkmcnt, no release fence): waves 1..3 keep their row
    // DMA in flight until the wait before the last one.
    for (int e = tid; e < g.E; e += kF1Threads) cnt[e] = 0;
    for (int s = tid; s < nbmax * kBlockM; s += kF1Threads) sroute[s] = -1;
    if (wave == 0) {
      const int rl = int(routes_in_use(p, p.m, p.topk));   // routes past rl are dropped
      int gid[kF1PackRoutes / 64];
      float wt[kF1PackRoutes / 64];
#pragma unroll
      for (int i = 0; i < kF1PackRoutes / 64; ++i) {
        const int r = lane + 64 * i;
        gid[i] = r < rl ? p.topk_ids[r] : -1;
        wt[i] = r < R ? p.topk_weights[r] : 0.f;
      }
#pragma unroll
      for (int i = 0; i < kF1PackRoutes / 64; ++i) {
        const int r = lane + 64 * i;
        int l = -1;
        if (gid[i] >= 0 && gid[i] < p.num_global_experts) {
          const int v = p.expert_map ? p.expert_map[gid[i]] : gid[i];
          l = (v >= 0 && v < g.E) ? v : -1;
        }
        sl[r] = int16_t(l);
        if (r < R) {
          sw[r] = wt[i];
          stk[r] = int16_t(r / p.topk);
        }
      }
    }
    pack_barrier();
    // The weights of each wave's first unit go out now, before the rest of the pack: with at
    // most 64 routes (one per lane) and at most 16 routes on each of the experts up to the
    // unit's block, that block's expert is the (block)-th smallest distinct local id, found by
    // repeated wave minima -- the block the pack below assigns it. Otherwise the loads wait
    // for the pack as usual. A wave that staged rows waits for them first (they left first and
    // have landed by now), so that no later wait counts these loads.
    {
      const int blk0 = int(blockIdx.x) / n_it;
      if (R <= 64 && blk0 < 8) {
        const int li = lane < R ? int(sl[lane]) : -1;
        int prev = -1, v = -1;
        bool ok = true;
        for (int k = 0; k <= blk0 && ok; ++k) {
          int cand = li > prev ? li : INT32_MAX;
#pragma unroll
          for (int d = 32; d >= 1; d >>= 1) cand = min(cand, __shfl_xor(cand, d, 64));
          v = uniform(cand);
          ok = v != INT32_MAX && __popcll(__ballot(li == v)) <= kBlockM;
          prev = v;
        }
        if (ok) {
          early = true;
          wait_vmcnt<0>();
          load_unit(v, int(blockIdx.x) % n_it, min(wave, nsl - 1), ra);
        }
      }
    }
    const int l = tid < kF1PackRoutes ? int(sl[tid]) : -1;
    if (l >= 0) atomicAdd(&cnt[l], 1);
    pack_barrier();
    constexpr int kPer = kF1PackExperts / kF1Threads;
    const int e0 = tid * kPer;
    int c[kPer], padded = 0, valid = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      c[i] = e0 + i < g.E ? cnt[e0 + i] : 0;
      padded += (c[i] + kBlockM - 1) / kBlockM * kBlockM;
      valid += c[i];
    }
    int x = padded, vx = valid;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int y = __shfl_up(x, d, 64), vy = __shfl_up(vx, d, 64);
      if (lane >= d) { x += y; vx += vy; }
    }
    if (lane == 63) { scr[wave] = x; scr[kF1Waves + wave] = vx; }
    pack_barrier();
    int off = x - padded, total = 0, nvalid = 0;
#pragma unroll
    for (int w = 0; w < kF1Waves; ++w) {
      off += w < wave ? scr[w] : 0;
      total += scr[w];
      nvalid += scr[kF1Waves + w];
    }
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      if (e0 + i < g.E) {
        cnt[e0 + i] = off;                                    // only this thread read these counts
        const int pb = (c[i] + kBlockM - 1) / kBlockM;
        for (int b = 0; b < pb; ++b) sbe[off / kBlockM + b] = e0 + i;
        off += pb * kBlockM;
      }
    }
    pack_barrier();
    if (l >= 0) {
      int rank = 0;
      for (int j = 0; j < R; j += 8) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(sl + j);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int li = int(int16_t(v[i >> 1] >> (16 * (i & 1))));
          rank += (j + i < tid) & (li == l);
        }
      }
      const int slot = cnt[l] + rank;
      sroute[slot] = int16_t(tid);
      if (blockIdx.x == 0) p.route_slot[tid] = slot;
    } else if (tid < R && blockIdx.x == 0) {
      p.route_slot[tid] = -1;
    }
    if (!early) wait_vmcnt<0>();                              // the rows (waves 1..3) have landed
    pack_barrier();
    live_blocks = total / kBlockM;
    if (blockIdx.x == 0) {
      for (int s = tid; s < live_blocks * kBlockM; s += kF1Threads) {
        const int r = sroute[s];
        p.sorted_route_ids[s] = r;
        p.slot_info[s] = make_int2(r >= 0 ? int(stk[r]) : -1, r >= 0 ? __float_as_int(sw[r]) : 0);
      }
      for (int b = tid; b < live_blocks; b += kF1Threads) p.block_expert[b] = sbe[b];
      if (tid == 0) {
        p.live[0] = nvalid;
        p.live[1] = total;
        p.live[2] = live_blocks;
        p.live[3] = int(routes_in_use(p, p.m, p.topk) / p.topk);
      }
    }
    if (live_blocks * n_it <= int(blockIdx.x)) return;        // no item for this workgroup
  }
  const int n_items = live_blocks * n_it;
  const int my_items = (n_items - int(blockIdx.x) + int(gridDim.x) - 1) / int(gridDim.x);
  const int U = my_items * spw;

  // Loads are unconditional so that the wait counters stay exact: units past the end and
  // K blocks past kb1 re-read a valid block (an L2 hit) whose contribution is skipped. The
  // block's expert comes through the scalar cache, so it waits on no vector load. `loads`
  // false: only the unit's route column (its loads went out early).
  auto issue = [&](int u, F1Unit& r, bool loads = true) {
    const int uu = min(u, U - 1);
    const int item = int(blockIdx.x) + (uu / spw) * int(gridDim.x);
    const int sl = min(wave + kF1Waves * (uu % spw), nsl - 1);
    const int blk = item / n_it, it = item % n_it;
    int eb;
    if constexpr (PACK) {
      const int rr = sroute[blk * kBlockM + col];
      r.info = make_int2(rr >= 0 ? int(stk[rr]) : -1, rr >= 0 ? __float_as_int(sw[rr]) : 0);
      eb = uniform(sbe[blk]);
    } else {
      r.info = p.slot_info[blk * kBlockM + col];
      eb = scalar_load(p.block_expert, blk);
    }
    if (loads) load_unit(eb, it, sl, r);
  };

  // Two register sets: the next unit's loads stay in flight while this one is computed. The
  // first unit goes out right behind the activation DMA; the rows (landed before the pack's
  // last barrier) are converted while its weights are in flight, and only then is the second
  // unit issued: with both issued first, the conversion waited behind a full load queue and
  // held up every wave at the barrier below (m = 8: FC1 75.6 -> 73.9 us).
  issue(0, ra, !early);
  if constexpr (PACK && F16) convert_rows();
  issue(1, rb);

  if constexpr (STAGED && !PACK) wait_vmcnt<0>();
  lds_barrier();

  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  auto compute = [&](int u, const F1Unit& r) {
    if (u >= U) return;
    const int sl = wave + kF1Waves * (u % spw);
    if (sl >= nsl) return;
    const int tok = r.info.x;
    const int t = max(tok, 0);                                // padding columns read row 0; masked later
    int xoff[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) xoff[s] = t * xp + (((4 * s + q) ^ (t & 7)) << 3);
#pragma unroll
    for (int j = 0; j < kF1Slice; ++j) {
      const int kb = sl * kF1Slice + j;
      if (kb < kb1) {
        float sa[4], sb[4];
        NvScalesF16 ha, hb;
        if constexpr (F16) {
          ha = nv_scales_f16(r.s0[j]);
          hb = nv_scales_f16(r.s1[j]);
        } else {
          decode_scales<FMT>(r.s0[j], sa);
          decode_scales<FMT>(r.s1[j], sb);
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          if constexpr (F16) {
            const f16x8 xb = __builtin_bit_cast(f16x8, *reinterpret_cast<const u32x4*>(xs + xoff[s] + kb * kKBlock));
            acc0 = mfma16h(dq8_nv_f16(r.q0[j][s], ha.step(s)), xb, acc0);
            acc1 = mfma16h(dq8_nv_f16(r.q1[j][s], hb.step(s)), xb, acc1);
          } else {
            bf16x8 xb;
            if (STAGED) xb = load_bf16x8(xs + xoff[s] + kb * kKBlock);
            else {
              const int k = kb * kKBlock + 32 * s + 8 * q;
              xb = (tok >= 0 && k < H) ? load_bf16x8(p.x + int64_t(tok) * H + k) : zero_bf16x8();
            }
            acc0 = mfma16(dq8<FMT>(r.q0[j][s], sa[s]), xb, acc0);
            acc1 = mfma16(dq8<FMT>(r.q1[j][s], sb[s]), xb, acc1);
          }
        }
      }
    }
  };

  auto finish = [&](int u, const int2 info) {
    if (u >= U || u % spw != spw - 1) return;                 // not the item's last slice
    const int item = int(blockIdx.x) + (u / spw) * int(gridDim.x);
    const int blk = item / n_it, it = item % n_it;
    const int par = (u / spw) & 1;
    const int e = PACK ? uniform(sbe[blk]) : scalar_load(p.block_expert, blk);
    float g13 = scalar_load(p.g13, e);
    const float g2 = scalar_load(p.g2, e);
    if (wave != 0) {
      red[par][wave - 1][0][lane] = acc0;
      red[par][wave - 1][1][lane] = acc1;
    }
    lds_barrier();
    if (wave == 0) {
      f32x4 h0 = acc0, h1 = acc1;
#pragma unroll
      for (int w = 0; w < kF1Waves - 1; ++w) {
        h0 += red[par][w][0][lane];
        h1 += red[par][w][1][lane];
      }
      const int tok = info.x;
      if constexpr (F16) g13 = ldexpf(g13, tok >= 0 ? sp[tok] : 0);
      // W4A8: the router weight and FC2 global scale come after FC2 (outside the quantisation)
      const float rw = (tok >= 0) ? (p.w4a8 ? 1.f : __int_as_float(info.y) * g2) : 0.f;
      const int64_t slot = int64_t(blk) * kBlockM + col;
      const int r0 = 4 * q;
      if (g.act == ACT_SWIGLU) {
        float a[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = silu_f32(h0[i] * g13) * (h1[i] * g13) * rw;
        store_inter4(p, slot, it * 16 + r0, a);
      } else {
        float a[4], b[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float x0 = fmaxf(h0[i] * g13, 0.f), x1 = fmaxf(h1[i] * g13, 0.f);
          a[i] = x0 * x0 * rw;
          b[i] = x1 * x1 * rw;
        }
        store_inter4(p, slot, 32 * it + r0, a);
        store_inter4(p, slot, 32 * it + 16 + r0, b);
      }
    }
    acc0 = f32x4{0.f, 0.f, 0.f, 0.f};
    acc1 = f32x4{0.f, 0.f, 0.f, 0.f};
  };

  // A unit's register set is refilled right after its MFMAs, before the item's epilogue and
  // its barrier, so the weight stream keeps flowing while waves wait there.
  // (Loading only units that exist in the last iterations, as FC2 does, made this kernel's
  // code larger and its m = 8 time bimodal, 74.6 or 76.2 us; the re-reads stay here.)
  const int U2 = (U + 1) & ~1;                                // even: units are taken in pairs
  for (int u = 0; u < U2; u += 2) {
    compute(u, ra);
    const int2 ia = ra.info;
    issue(u + 2, ra);
    finish(u, ia);
    compute(u + 1, rb);
    const int2 ib = rb.info;
    issue(u + 3, rb);
    finish(u + 1, ib);
  }
}

// ----------------------------------------------------------------------------- FC2

struct F2Unit {
  u32x4 q[kF2Slice];                 // 1 KiB fragment blocks
  uint2 s;                           // their scale dwords
  bf16x8 b[kF2Slice][4];             // the route column's intermediate values for the MFMA steps
};

template <int FMT>
__global__ __launch_bounds__(kF2Threads, 1) void decode_fc2_kernel(FusedParams p) {
  extern __shared__ __align__(16) uint8_t dyn[];
  __shared__ float tacc[kF2Waves][kDecodeMaxM][16];
  const PreparedGeom& g = p.g;
  const int tid = threadIdx.x, lane = tid & 63, wave = uniform(tid >> 6);
  const int q = lane >> 4, col = lane & 15;
  const int64_t ht = blockIdx.x;                             // 16 hidden rows per workgroup
  const int live_blocks = p.live[2];
  int* be = reinterpret_cast<int*>(dyn);                     // block -> expert
  int* stok = be + p.cap_blocks;                             // slot -> token (-1 = padding)
  static_assert(kScaleChunkKB % kF2Slice == 0, "an FC2 unit never straddles a scale chunk");
  const int kb2 = int(g.kb2);
  const int nsl = (kb2 + kF2Slice - 1) / kF2Slice;
  const int units = live_blocks * nsl;                        // (route block, K slice) pairs
  const int U = units > wave ? (units - wave + kF2Waves - 1) / kF2Waves : 0;
  const int U2 = (U + 1) & ~1;
  const int sc_lane = FMT == FMT_NVFP4 ? ((lane >> 5) * 16 + col) * 16 : col * 16;

  // Weight loads are unconditional (units past the end re-read the last one, skipped);
  // intermediate rows are loaded only for live route columns, so L2 traffic follows the
  // routes, not the padded blocks.
  auto issue = [&](int u, F2Unit& r, bool prologue) {
    const int unit = wave + min(u, U - 1) * kF2Waves;
    const int blk = unit / nsl, sl = unit % nsl;
    const int64_t gi = int64_t(uniform(prologue ? p.block_expert[blk] : be[blk])) * g.n2_groups + ht;
    const uint8_t* nb = p.nib2 + gi * g.kb2 * kFragBytes;
#pragma unroll
    for (int j = 0; j < kF2Slice; ++j) {
      const int kb = min(sl * kF2Slice + j, kb2 - 1);
      r.q[j] = *reinterpret_cast<const u32x4*>(nb + int64_t(kb) * kFragBytes + lane * 16);
    }
    const int kb0 = sl * kF2Slice;
    r.s = *reinterpret_cast<const uint2*>(p.sc2 + gi * g.sc2_per_group + int64_t(kb0 / kScaleChunkKB) * g.sc_chunk_bytes +
                                          sc_lane + (kb0 % kScaleChunkKB) * 4);
    const int slot = blk * kBlockM + col;
    const bool valid = (prologue ? p.slot_info[slot].x : stok[slot]) >= 0;
    const uint16_t* irow = p.inter + int64_t(slot) * g.ip + 8 * q;
#pragma unroll
    for (int j = 0; j < kF2Slice; ++j) {
      const int kb = min(sl * kF2Slice + j, kb2 - 1);
#pragma unroll
      for (int s = 0; s < 4; ++s) r.b[j][s] = valid ? load_bf16x8(irow + kb * kKBlock + 32 * s) : zero_bf16x8();
    }
  };
  // The first two units' loads go out before the table staging below. Two register sets:
  // the next unit's loads stay in flight while this one is computed.
  F2Unit ra, rb;
  if (U > 0) {
    issue(0, ra, true);
    issue(1, rb, true);
  }

  for (int b = tid; b < live_blocks; b += kF2Threads) be[b] = p.block_expert[b];
  for (int s = tid; s < live_blocks * kBlockM; s += kF2Threads) stok[s] = p.slot_info[s].x;
  for (int i = tid; i < kF2Waves * kDecodeMaxM * 16; i += kF2Threads) (&tacc[0][0][0])[i] = 0.f;
  lds_barrier();

  auto compute = [&](int u, const F2Unit& r) {
    if (u >= U) return;
    const int unit = wave + u * kF2Waves;
    const int blk = unit / nsl, sl = unit % nsl;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < kF2Slice; ++j) {
      if (sl * kF2Slice + j < kb2) {
        float sc[4];
        decode_scales<FMT>(j == 0 ? r.s.x : r.s.y, sc);
#pragma unroll
        for (int s = 0; s < 4; ++s) acc = mfma16(dq8<FMT>(r.q[j][s], sc[s]), r.b[j][s], acc);
      }
    }
    const int tok = stok[blk * kBlockM + col];
    if (tok >= 0) {
      const float wt = p.w4a8 ? __int_as_float(p.slot_info[blk * kBlockM + col].y) * scalar_load(p.g2, uniform(be[blk])) : 1.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) atomicAdd(&tacc[wave][tok][4 * q + i], acc[i] * wt);
    }
  };

  for (int u = 0; u < U2; u += 2) {
    compute(u, ra);
    issue(u + 2, ra, false);
    compute(u + 1, rb);
    issue(u + 3, rb, false);
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

// ----------------------------------------------------------------------------- FC2, K split
//
// Workgroup (z, G) owns RG row groups (16 RG hidden rows) and K blocks 2z, 2z + 1 of the
// intermediate for every route block. That K slice of every valid route's intermediate row
// is staged in LDS once (by DMA, row index = route id), so each LDS read of an MFMA B
// fragment feeds RG MFMAs and the weight stream carries no other loads. Units are route
// blocks (RG row groups x 2 K blocks = 2 RG KiB of nibbles), dealt to the 8 waves in turn;
// a unit's route results are added into per-wave, per-token LDS sums. The workgroup's
// fixed-order sum over waves is one fp32 partial per (K split, token, hidden row); the last
// K split of a row group to finish (one arrival count per group) adds the partials in split
// order and stores the bf16 rows: deterministic for any arrival order.

constexpr int kF3Threads = 512;
constexpr int kF3Waves = kF3Threads / 64;
constexpr int kF3KB = 2;             // K blocks per workgroup
constexpr int kF3RowGroups = 2;      // row groups per workgroup
constexpr int kF3MaxLds = 81920;     // two workgroups per CU
constexpr int kF3RowBytes = kF3KB * kKBlock * 2;   // staged bytes per route row
constexpr int kF3MaxRowDma = 8;      // 1 KiB row DMAs per wave: at most 64 KiB of staged rows

template <int RG>
struct F3Unit {
  u32x4 q[RG][kF3KB];                // 1 KiB fragment blocks: row group, K block
  uint32_t s[RG][kF3KB];             // their scale dwords
};

__host__ __device__ inline size_t f3_rows_bytes(int64_t routes) { return (size_t(routes) * kF3RowBytes + 1023) / 1024 * 1024; }
__host__ __device__ inline size_t f3_table_bytes(int64_t cap_blocks) { return (size_t(cap_blocks) * kBlockM * 4 + 255) / 256 * 256; }
__host__ __device__ inline size_t f3_exp_bytes(int64_t routes) { return (size_t(routes) * 4 + 15) / 16 * 16; }
template <int RG>
__host__ __device__ inline size_t f3_lds_bytes(int64_t m, int64_t topk, int64_t cap_blocks) {
  return f3_rows_bytes(m * topk) + f3_table_bytes(cap_blocks) + f3_exp_bytes(m * topk) + size_t(kF3Waves) * m * 16 * RG * 4;
}

// W8 (W4A8, block-scaled MFMA): each route's K slice as MXFP8 codes (256 B) and its 8 E8M0
// bytes.
constexpr int kF8RowBytes = kF3KB * kKBlock;
__host__ __device__ inline size_t f8_rows_bytes(int64_t routes) { return (size_t(routes) * kF8RowBytes + 1023) / 1024 * 1024; }
__host__ __device__ inline size_t f8_scale_bytes(int64_t routes) { return (size_t(routes) * 8 + 15) / 16 * 16; }
template <int RG>
__host__ __device__ inline size_t f8_lds_bytes(int64_t m, int64_t topk, int64_t cap_blocks) {
  return f8_rows_bytes(m * topk) + f8_scale_bytes(m * topk) + f3_table_bytes(cap_blocks) +
         f3_exp_bytes(m * topk) + size_t(kF3Waves) * m * 16 * RG * 4;
}

template <int FMT, int RG, bool W8>
__global__ __launch_bounds__(kF3Threads, 4) void decode_fc2_split_kernel(FusedParams p) {
  static_assert(!W8 || kF3KB == 2, "the block-scaled FC2 takes one 128-K block pair (256 codes) per workgroup");
  extern __shared__ __align__(16) uint8_t dyn[];
  const PreparedGeom& g = p.g;
  const int tid = threadIdx.x, lane = tid & 63, wave = uniform(tid >> 6);
  const int q = lane >> 4, col = lane & 15;
  const int nb = p.live[2];
  const int m = int(p.m), topk = p.topk, routes = m * topk;
  const int kb2 = int(g.kb2), groups = int(g.n2_groups);
  // Workgroups come in pairs (K splits 2p, 2p + 1 of one row-group set) that run on the same
  // XCD (workgroup i runs on XCD i % 8): the pair reads the two halves of the same 16-byte
  // scale chunks and adjacent weight blocks, so the second read of each scale line is an L2
  // hit. Pair L sits at workgroups 16 (L / 8) + L % 8 and 8 more.
  const int nsplit = (kb2 + kF3KB - 1) / kF3KB, npair = (nsplit + 1) / 2;
  const int ngroup = (groups + RG - 1) / RG;
  const int pair = (int(blockIdx.x) >> 4) * 8 + (int(blockIdx.x) & 7);
  const int z = 2 * (pair % npair) + ((int(blockIdx.x) >> 3) & 1), G = pair / npair;
  if (G >= ngroup || z >= nsplit) return;
  const int kq0 = z * kF3KB;
  uint8_t* bs = dyn;                                                        // [routes][kF3RowBytes] (W8: kF8RowBytes)
  // W8: E8M0 bytes [routes][8] after the code rows
  uint32_t* ssc = reinterpret_cast<uint32_t*>(dyn + f8_rows_bytes(routes));
  int* sroute = reinterpret_cast<int*>(dyn + (W8 ? f8_rows_bytes(routes) + f8_scale_bytes(routes)
                                                  : f3_rows_bytes(routes)));   // [nb * 16] slot -> route
  int* sexp = reinterpret_cast<int*>(reinterpret_cast<uint8_t*>(sroute) + f3_table_bytes(p.cap_blocks));    // [routes] f16 exponents
  float* tacc = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(sexp) + f3_exp_bytes(routes));          // [waves][m][16 RG]
  const int U = nb > wave ? (nb - wave + kF3Waves - 1) / kF3Waves : 0;
  const int sc_lane = FMT == FMT_NVFP4 ? ((lane >> 5) * 16 + col) * 16 : col * 16;

  // Staging: the slot -> route table and each route's K slice by DMA (dropped routes, the
  // table's tail and K blocks past kb2 read as zeros).
  for (int i = tid; i < kF3Waves * m * 16 * RG; i += kF3Threads) tacc[i] = 0.f;
  if (!(FMT == FMT_NVFP4) && p.w4a8)
    for (int r = tid; r < routes; r += kF3Threads) sexp[r] = __float_as_int(p.topk_weights[r]);
  const __amdgpu_buffer_rsrc_t tr = buffer_rsrc(p.sorted_route_ids, uint32_t(nb * kBlockM * 4));
  for (int n = wave; n * 64 < nb * kBlockM; n += kF3Waves) dma4(tr, sroute + 64 * n, uint32_t((64 * n + lane) * 4));
  // W8: this split's K slice of every route rounded to MXFP8 here, from FC1's fp32 rows: task
  // t covers 8 values, quarter t % 4 of MX group (t / 4) % 8 of route t / 32, so the four tasks
  // of a group sit in adjacent lanes. Dropped routes and K blocks past kb2 give zero codes.
  // The first tasks' loads go out ahead of the weight loads below.
  constexpr int kPre = 2;                                    // tasks per thread loaded ahead
  const int ntask = routes * 32;
  f32x4 pre[kPre][2];
  auto load_task = [&](int t, f32x4* v) {
    v[0] = v[1] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (t < ntask) {
      const int r = t >> 5, kblk = kq0 + ((t >> 4) & 1);
      const int sl = p.route_slot[r];
      if (sl >= 0 && kblk < kb2) {
        const float* src = p.inter32 + int64_t(sl) * g.ip + int64_t(kq0) * kKBlock + (t & 31) * 8;
        v[0] = *reinterpret_cast<const f32x4*>(src);
        v[1] = *reinterpret_cast<const f32x4*>(src + 4);
      }
    }
  };
  auto round_task = [&](int t, const f32x4* v) {
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) amax = fmaxf(amax, fmaxf(fabsf(v[0][i]), fabsf(v[1][i])));
    amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
    amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
    const int e = amax > 0.f ? mx8_exponent(amax) : 0;
    const float lo[4] = {v[0][0], v[0][1], v[0][2], v[0][3]}, hi[4] = {v[1][0], v[1][1], v[1][2], v[1][3]};
    if (t < ntask) {
      *reinterpret_cast<uint2*>(bs + (t >> 5) * kF8RowBytes + (t & 31) * 8) =
          make_uint2(mx8_codes4(lo, e, amax), mx8_codes4(hi, e, amax));
      if ((t & 3) == 0) reinterpret_cast<uint8_t*>(ssc)[(t >> 5) * 8 + ((t >> 2) & 7)] = uint8_t(amax > 0.f ? e + 127 : 0);
    }
  };
  if constexpr (W8) {
#pragma unroll
    for (int i = 0; i < kPre; ++i) load_task(i * kF3Threads + tid, pre[i]);
  } else {
    // The route -> slot lookups of all of a wave's rows go out together, then the row DMAs.
    const __amdgpu_buffer_rsrc_t ir = buffer_rsrc(p.inter, uint32_t(p.cap_blocks * kBlockM * g.ip * 2));
    const int nchunk = int(f3_rows_bytes(routes) / 1024);
    int slot[kF3MaxRowDma];
#pragma unroll
    for (int i = 0; i < kF3MaxRowDma; ++i) {
      const int n = wave + kF3Waves * i, r = (n * 1024 + lane * 16) / kF3RowBytes;
      slot[i] = n < nchunk && r < routes ? p.route_slot[r] : -1;
    }
#pragma unroll
    for (int i = 0; i < kF3MaxRowDma; ++i) {
      const int n = wave + kF3Waves * i, o = (n * 1024 + lane * 16) % kF3RowBytes;
      const bool ok = slot[i] >= 0 && kq0 + o / (kKBlock * 2) < kb2;
      if (n < nchunk) dma16(ir, bs + n * 1024, ok ? uint32_t((slot[i] * g.ip + kq0 * kKBlock) * 2 + o) : kOutOfRange);
    }
  }

  // Loads are unconditional so that the wait counters stay exact: units past the end re-read
  // the last unit, row groups past the end the last group, K blocks past kb2 the last block;
  // none of these is used.
  auto issue = [&](int u, F3Unit<RG>& r) {
    const int blk = wave + min(u, U - 1) * kF3Waves;
    const int64_t e = scalar_load(p.block_expert, blk);
#pragma unroll
    for (int rr = 0; rr < RG; ++rr) {
      const int64_t gi = e * groups + min(G * RG + rr, groups - 1);
      const uint8_t* nbp = p.nib2 + gi * kb2 * kFragBytes;
#pragma unroll
      for (int j = 0; j < kF3KB; ++j)
        r.q[rr][j] = *reinterpret_cast<const u32x4*>(nbp + int64_t(min(kq0 + j, kb2 - 1)) * kFragBytes + lane * 16);
      const uint8_t* sp = p.sc2 + gi * g.sc2_per_group + int64_t(kq0 / kScaleChunkKB) * g.sc_chunk_bytes + sc_lane + (kq0 % kScaleChunkKB) * 4;
      if constexpr (kF3KB == 4) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(sp);
#pragma unroll
        for (int j = 0; j < 4; ++j) r.s[rr][j] = v[j];
      } else {
        const uint2 v = *reinterpret_cast<const uint2*>(sp);
        r.s[rr][0] = v.x;
        r.s[rr][1] = v.y;
      }
    }
  };
  static_assert(kScaleChunkKB % kF3KB == 0 && (kF3KB == 2 || kF3KB == 4), "a workgroup's K blocks never straddle a scale chunk");

  F3Unit<RG> ra, rb;
  if (U > 0) issue(0, ra);
  if (U > 1) issue(1, rb);
  if constexpr (W8) {
#pragma unroll
    for (int i = 0; i < kPre; ++i) round_task(i * kF3Threads + tid, pre[i]);
    for (int t0 = kPre * kF3Threads; t0 < ntask; t0 += kF3Threads) {
      f32x4 v[2];
      load_task(t0 + tid, v);
      round_task(t0 + tid, v);
    }
  }
  wait_vmcnt<0>();
  lds_barrier();

  // NVFP4 runs on the f16 MFMA: E2M1 x E4M3 weights are exact in f16, and each staged route
  // row is rescaled in place by a power of two 2^-p (exact) with its largest magnitude in
  // [2^14, 2^15) before the f16 cast; the unit results are multiplied by 2^p again. The
  // exponent is per (route, K split), and the K splits meet only in fp32 sums.
  constexpr bool F16 = FMT == FMT_NVFP4;
  if constexpr (F16) {
    for (int r = wave; r < routes; r += kF3Waves) {
      uint32_t* rw = reinterpret_cast<uint32_t*>(bs + r * kF3RowBytes) + lane * kF3KB;
      uint32_t v[kF3KB];
      float mx = 0.f;
#pragma unroll
      for (int d = 0; d < kF3KB; ++d) {
        v[d] = rw[d];
        mx = fmaxf(mx, fmaxf(fabsf(__uint_as_float(v[d] << 16)), fabsf(__uint_as_float(v[d] & 0xFFFF0000u))));
      }
#pragma unroll
      for (int d = 32; d >= 1; d >>= 1) mx = fmaxf(mx, __shfl_xor(mx, d, 64));
      const int pe = (mx > 0.f && mx <= 3.4e38f) ? __builtin_amdgcn_frexp_expf(mx) - 15 : 0;
#pragma unroll
      for (int d = 0; d < kF3KB; ++d) {
        const f16x2 h = f16x2{(_Float16)ldexpf(__uint_as_float(v[d] << 16), -pe), (_Float16)ldexpf(__uint_as_float(v[d] & 0xFFFF0000u), -pe)};
        rw[d] = __builtin_bit_cast(uint32_t, h);
      }
      if (lane == 0) sexp[r] = pe;
    }
    lds_barrier();
  }

  auto compute = [&](int u, const F3Unit<RG>& r) {
    if (u >= U) return;
    const int blk = wave + u * kF3Waves;
    const int route = sroute[blk * kBlockM + col];
    const uint8_t* brow = bs + max(route, 0) * (W8 ? kF8RowBytes : kF3RowBytes) + q * 16;
    f32x4 acc[RG];
#pragma unroll
    for (int rr = 0; rr < RG; ++rr) acc[rr] = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (W8) {
      // Block-scaled FP4 x FP8 MFMA, one per (row group, K block). B (the routes' MXFP8 row):
      // lane (col, q) holds K 16 q .. 16 q + 15 and 64 + 16 q .. 64 + 16 q + 15 of route col; its
      // scale byte is block q of that route. A (the weights): lane (col, q) must hold the 32
      // consecutive K of block q of row col, while the fragment layout deals them out in
      // 8-K chunks over the four lane quarters (chunk 4 s + q in dword s): a 4 x 4 dword
      // transpose across the quarters (gfx950 lane swaps).
#pragma unroll
      for (int j = 0; j < kF3KB; ++j) {
        if (kq0 + j < kb2) {
          const u32x4 blo = route >= 0 ? *reinterpret_cast<const u32x4*>(brow + j * kKBlock) : u32x4{0u, 0u, 0u, 0u};
          const u32x4 bhi = route >= 0 ? *reinterpret_cast<const u32x4*>(brow + j * kKBlock + 64) : u32x4{0u, 0u, 0u, 0u};
          const i32x8 bop = i32x8{int(blo[0]), int(blo[1]), int(blo[2]), int(blo[3]), int(bhi[0]), int(bhi[1]), int(bhi[2]), int(bhi[3])};
          const int sb = route >= 0 ? int((ssc[route * 2 + j] >> (8 * q)) & 0xFFu) : 127;
#pragma unroll
          for (int rr = 0; rr < RG; ++rr) {
            const u32x4 a = transpose_quarters(r.q[rr][j]);
            const i32x8 aop = i32x8{int(a[0]), int(a[1]), int(a[2]), int(a[3]), 0, 0, 0, 0};
            const int sa = int((r.s[rr][j] >> (8 * q)) & 0xFFu);
            acc[rr] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aop, bop, acc[rr], 4, 0, 0, sa, 0, sb);
          }
        }
      }
    } else {
#pragma unroll
    for (int j = 0; j < kF3KB; ++j) {
      if (kq0 + j < kb2) {
        float sc[RG][4];
        NvScalesF16 sh[RG];
#pragma unroll
        for (int rr = 0; rr < RG; ++rr) {
          if constexpr (F16) sh[rr] = nv_scales_f16(r.s[rr][j]);
          else decode_scales<FMT>(r.s[rr][j], sc[rr]);
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          if constexpr (F16) {
            const f16x8 b = route >= 0 ? *reinterpret_cast<const f16x8*>(brow + j * kKBlock * 2 + s * 64) : zero_f16x8();
#pragma unroll
            for (int rr = 0; rr < RG; ++rr) acc[rr] = mfma16h(dq8_nv_f16(r.q[rr][j][s], sh[rr].step(s)), b, acc[rr]);
          } else {
            const bf16x8 b = route >= 0 ? *reinterpret_cast<const bf16x8*>(brow + j * kKBlock * 2 + s * 64) : zero_bf16x8();
#pragma unroll
            for (int rr = 0; rr < RG; ++rr) acc[rr] = mfma16(dq8<FMT>(r.q[rr][j][s], sc[rr][s]), b, acc[rr]);
          }
        }
      }
    }
    }
    if (route >= 0) {
      float* ta = tacc + (wave * m + route / topk) * (16 * RG) + 4 * q;
      const int pe = F16 ? sexp[route] : 0;
      // W4A8 (MXFP4 only, so the exponent area is free): router weight x FC2 global scale
      const float wt = !F16 && p.w4a8 ? __int_as_float(sexp[route]) * scalar_load(p.g2, scalar_load(p.block_expert, blk)) : 1.f;
#pragma unroll
      for (int rr = 0; rr < RG; ++rr)
#pragma unroll
        for (int i = 0; i < 4; ++i) atomicAdd(ta + 16 * rr + i, F16 ? ldexpf(acc[rr][i], pe) : acc[rr][i] * wt);
    }
  };

  // The last (up to three) units issue loads only for units that exist: re-reading a unit
  // for exact wait counts there only kept the launch waiting for loads nobody uses (m = 1:
  // FC2 17.0 -> 15.5 us).
  int u = 0;
  for (; u + 3 < U; u += 2) {
    compute(u, ra);
    issue(u + 2, ra);
    compute(u + 1, rb);
    issue(u + 3, rb);
  }
  if (u < U) {
    compute(u, ra);
    if (u + 2 < U) issue(u + 2, ra);
  }
  if (u + 1 < U) compute(u + 1, rb);
  if (u + 2 < U) compute(u + 2, ra);
  lds_barrier();
  // Fixed-order sum over the waves: the partial of K split z for rows of this group.
  for (int i = tid; i < m * 16 * RG; i += kF3Threads) {
    const int t = i / (16 * RG), row = i % (16 * RG);
    const int64_t h = int64_t(G) * 16 * RG + row;
    float sum = 0.f;
    for (int w = 0; w < kF3Waves; ++w) sum += tacc[(w * m + t) * (16 * RG) + row];
    if (h < g.H) __hip_atomic_store(p.part + (int64_t(z) * m + t) * g.H + h, sum, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // The last of the group's K splits to finish adds the partials in split order and stores
  // the bf16 output rows. The partials are written and read as device-scope (relaxed
  // atomic) accesses, which are coherent across the XCDs' L2s without flushing them; each
  // thread waits for its stores to complete before the workgroup's count goes up. The
  // counts were zeroed by the FC1 launch of the same call.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  __shared__ int last;
  if (tid == 0) last = __hip_atomic_fetch_add(p.f2_count + G, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == nsplit - 1;
  __syncthreads();
  if (!last) return;
  for (int i = tid; i < m * 16 * RG; i += kF3Threads) {
    const int t = i / (16 * RG), row = i % (16 * RG);
    const int64_t h = int64_t(G) * 16 * RG + row;
    if (h < g.H) {
      // batches of 8 loads in flight, added in split order
      float sum = 0.f;
      for (int z0 = 0; z0 < nsplit; z0 += 8) {
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
          v[j] = z0 + j < nsplit ? __hip_atomic_load(p.part + (int64_t(z0 + j) * m + t) * g.H + h, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (z0 + j < nsplit) sum += v[j];
      }
      bf16x2 v;
      v[0] = (__bf16)sum;
      p.out[int64_t(t) * g.H + h] = __builtin_bit_cast(uint16_t, v[0]);
    }
  }
}

template <typename K>
hipError_t allow_lds(K kernel, int bytes) {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
}

template <int FMT>
hipError_t launch_decode_fmt(const FusedParams& p0, int num_cus, hipStream_t stream, LaunchMarks* marks) {
  static const hipError_t lds_ok = [] {
    // dynamic LDS: FC1 staged rows + exponents (+ pack tables); FC2 block table + slot tokens
    hipError_t e = allow_lds(&decode_fc1_kernel<FMT, true, false>, kDecodeStageBytes + 256);
    if (e == hipSuccess) e = allow_lds(&decode_fc1_kernel<FMT, true, true>, kLdsPerCU - kF1StaticLds);
    if (e == hipSuccess) e = allow_lds(&decode_fc2_kernel<FMT>, 98304);
    if (e == hipSuccess) e = allow_lds(&decode_fc2_split_kernel<FMT, kF3RowGroups, false>, kF3MaxLds);
    if (FMT == FMT_MXFP4 && e == hipSuccess) e = allow_lds(&decode_fc2_split_kernel<FMT_MXFP4, kF3RowGroups, true>, kF3MaxLds);
    return e;
  }();
  if (lds_ok != hipSuccess) return lds_ok;
  FusedParams p = p0;
  const PreparedGeom& g = p.g;
  p.xs_pitch = decode_x_pitch(g);
  const int64_t items = p.cap_blocks * (g.n1_groups / 2);
  const bool pack = p.topk_ids != nullptr;                     // FC1 packs the routes (decode_fc1_packs)
  const size_t lds1 = size_t(p.m) * p.xs_pitch * 2 + 256 + (pack ? f1_pack_lds_bytes(int(p.m) * p.topk, g.E) : 0);
  const int64_t grid1 = max(int64_t(1), min(items, int64_t(num_cus)));   // one workgroup per CU
  if (pack)
    hipLaunchKernelGGL((decode_fc1_kernel<FMT, true, true>), dim3(grid1), dim3(kF1Threads), lds1, stream, p);
  else if (decode_stages_x(g, p.m))
    hipLaunchKernelGGL((decode_fc1_kernel<FMT, true, false>), dim3(grid1), dim3(kF1Threads), lds1, stream, p);
  else
    hipLaunchKernelGGL((decode_fc1_kernel<FMT, false, false>), dim3(grid1), dim3(kF1Threads), 0, stream, p);
  if (marks) marks->after(stream, KID_FC1);
  constexpr int RG = kF3RowGroups;
  const size_t lds3 = f3_lds_bytes<RG>(p.m, p.topk, p.cap_blocks);
  // (the intermediate rows are addressed through a buffer resource: 32-bit offsets)
  const bool split = lds3 <= size_t(kF3MaxLds) && f3_rows_bytes(p.m * p.topk) <= size_t(kF3MaxRowDma) * kF3Waves * 1024 &&
                     p.cap_blocks * kBlockM * g.ip * 2 <= int64_t(INT32_MAX);
  // W4A8: the K-split FC2 runs the block-scaled FP4 x FP8 MFMA on the MXFP8 codes; otherwise
  // FC2 multiplies their exact values in bf16
  const bool w8 = FMT == FMT_MXFP4 && p.w4a8 && p.inter8 != nullptr && split &&
                  f8_lds_bytes<RG>(p.m, p.topk, p.cap_blocks) <= size_t(kF3MaxLds);
  if (p.w4a8 && !w8) {
    // (the block-scaled FC2 rounds its own slices; the bf16 fallback needs the rounding pass)
    if (hipError_t e = launch_mxfp8_requant(p, stream); e != hipSuccess) return e;
    if (marks) marks->after(stream, KID_REQUANT);
  }
  if (split) {
    const int nsplit = int((g.kb2 + kF3KB - 1) / kF3KB);
    const int64_t pairs = ((g.n2_groups + RG - 1) / RG) * ((nsplit + 1) / 2);
    if (w8)
      hipLaunchKernelGGL((decode_fc2_split_kernel<FMT_MXFP4, RG, true>), dim3((pairs + 7) / 8 * 16), dim3(kF3Threads),
                         f8_lds_bytes<RG>(p.m, p.topk, p.cap_blocks), stream, p);
    else
      hipLaunchKernelGGL((decode_fc2_split_kernel<FMT, RG, false>), dim3((pairs + 7) / 8 * 16), dim3(kF3Threads), lds3, stream, p);
    if (marks) marks->after(stream, KID_FC2);
  } else {
    const size_t lds2 = size_t(p.cap_blocks) * 4 + size_t(p.cap_blocks) * kBlockM * 4;
    hipLaunchKernelGGL((decode_fc2_kernel<FMT>), dim3(g.n2_groups), dim3(kF2Threads), lds2, stream, p);
    if (marks) marks->after(stream, KID_FC2);
  }
  return hipGetLastError();
}

}  // namespace

bool decode_fc1_packs(const PreparedGeom& g, int64_t m, int topk) {
  // Only up to about 64 KiB of staged rows (m <= 8 at hidden 4096): with more rows the
  // separate route-pack launch, which also converts the rows once, was measured faster
  // (small shape, m = 16: 127.8 against 129.1 us per layer).
  const int64_t routes = m * topk;
  return m >= 1 && routes <= kF1PackRoutes && g.E <= kF1PackExperts && decode_stages_x(g, m) &&
         size_t(m) * decode_x_pitch(g) * 2 + 256 + f1_pack_lds_bytes(int(routes), g.E) <= kF1PackRowsBudget;
}

hipError_t launch_decode(const FusedParams& p, int num_cus, hipStream_t stream, LaunchMarks* marks) {
  return p.g.fmt == FMT_NVFP4 ? launch_decode_fmt<FMT_NVFP4>(p, num_cus, stream, marks)
                              : launch_decode_fmt<FMT_MXFP4>(p, num_cus, stream, marks);
}

}  // namespace moe
