// Grouped-GEMM (prefill) path of the fused W4A16 MoE layer on gfx950.
//
// FlashInfer PR 4255, Description: cooperative persistent launches for the fused FC1/FC2
// kernel with occupancy-aware tiles; Performance: at m = 2048 the old kernel stalled on
// grid-wide barriers because it was not launched cooperatively. Here FC1 -> FC2 -> combine
// are ordered by stream order between persistent launches, so no workgroup ever waits for
// another one that might not be resident.
//
// Items are (M tile, N tile) pairs: an M tile is up to 8 route blocks (128 rows) of one
// expert, an N tile 16 row groups (256 weight rows). One 8-wave workgroup per CU, two waves
// per SIMD, so that one wave's waits on loads and LDS reads are covered by the other's MFMAs
// (at about one VALU op per MFMA the dequantisation hides behind the other wave's MFMAs; at
// three per MFMA it costs a fifth of the rate; the activation reads from LDS, one per two
// MFMAs, are what bounds the loop). The tile's activation K blocks stream through a ring of LDS
// stages filled by buffer loads that write LDS directly; each wave streams its own two row
// groups' E2M1 fragments and scales into a register ring of the same depth, dequantises them
// in registers into MFMA A operands and reads activation fragments (B operands) from the stage.
//  * FC1 epilogue: expert FC1 global scale, SiLU-SwiGLU (gate and up fragments sit in the
//    same lanes) or relu2, times router weight and the expert's FC2 global scale, bf16 store
//    into the intermediate row of the route's slot (W4A8: rounded to MXFP8 codes instead).
//  * FC2 epilogue: the weighted row of each route rounded to bf16; the combine pass sums each
//    token's top-k rows in fp32 in a fixed order (deterministic, no atomics) and casts to bf16.
//  * W4A8 FC2: the block-scaled FP4 x FP8 MFMA on FC1's MXFP8 codes (gemm_item_w8).
// NVFP4 runs on f16 operands in both GEMMs: FC1 on activations pre-scaled per token by a power
// of two, FC2 on intermediate rows stored as f16 times a per-slot power of two; E2M1 x E4M3
// products are exact in f16 (half the dequantisation work of the bf16 route).
#include <hip/hip_runtime.h>

#include "device.hpp"
#include "kernels.hpp"
#include "layout.hpp"

namespace moe {

namespace {

constexpr int kGemmThreads = 512;                       // 8 waves, two per SIMD
constexpr int kRowBytes = kKBlock * 2;                  // one activation row of a K block: 256 B
constexpr int kBlockBytes = kBlockM * kRowBytes;        // one route block of a K block: 4 KiB
constexpr int kLdsBytes = 131072;                       // the activation stage ring
constexpr int kW8AmaxOffset = 98304;                    // W4A8 FC1 epilogue: per-wave group maxima (4 KiB)
constexpr int kEarlyTicketKB = 32;                      // items up to this many K blocks take their successor's ticket early
constexpr int kEpilogueStage = kW8AmaxOffset + 4096;    // the epilogue's per-route values (16 B per route slot)

// Wave layout and pipeline depth for tiles of NB route blocks: the 8 waves split the N tile,
// 2 row groups x NB blocks each, so every fragment is loaded and dequantised by exactly one
// wave, straight into its registers. The activation K block of the tile goes through a ring
// of LDS stages (layout at the activation loads below).
template <int NB>
struct Plan {
  static constexpr int FR = 2;                                      // row groups per wave
  static constexpr int BW = NB;                                     // route blocks per wave
  static constexpr int XD = NB >= 2 ? NB / 2 : 1;                   // activation loads per wave (NB 1: waves 4-7 repeat 0-3)
  static constexpr int kStage = NB * kBlockBytes;
  // 3 stages for 8-block tiles (measured ~2% faster FC1 than 4: fewer ring registers), else up
  // to 6 below the W4A8 exchange area (4 for 6-block tiles)
  static constexpr int kDepth = NB == 8 ? 3 : (kW8AmaxOffset / kStage < 6 ? kW8AmaxOffset / kStage : 6);
  static constexpr int kLoads = XD + 2 * FR;                        // vector loads a wave issues per stage
  static_assert(kDepth >= 3 && (kDepth - 1) * kLoads < 64, "ring too shallow or vmcnt out of range");
  static_assert(XD <= 2 * FR, "the stage wait relies on at least as many register loads as LDS loads");
};

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

// Four consecutive columns of a route's weighted FC2 row, rounded to bf16 (the combine pass sums
// a token's rows in fp32).
__device__ __forceinline__ void store_row4(uint16_t* dst, const f32x4& v) {
  *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
}

// Four consecutive values of an intermediate row times 2^-q, rounded to f16.
__device__ __forceinline__ void store_f16x4(uint16_t* dst, const float* v, int q) {
  const f16x2 a = f16x2{(_Float16)ldexpf(v[0], -q), (_Float16)ldexpf(v[1], -q)};
  const f16x2 b = f16x2{(_Float16)ldexpf(v[2], -q), (_Float16)ldexpf(v[3], -q)};
  *reinterpret_cast<uint2*>(dst) = make_uint2(__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b));
}

__device__ __forceinline__ f32x4 ldexp4(const f32x4& a, int q) {
  return f32x4{ldexpf(a[0], q), ldexpf(a[1], q), ldexpf(a[2], q), ldexpf(a[3], q)};
}

// Exponent q of a route's f16 intermediate row on the NVFP4 grouped GEMM. FC1 output j of the
// route is a_j = g13 <x, W_j> (u_j likewise with the up rows); by Cauchy-Schwarz
// |a_j| <= |g13| |x| n_gate and |u_j| <= |g13| |x| n_up, where |x|^2 = xss 2^(2 px) (xss: the
// sum of squares of the token's f16 row scaled by 2^-px), and |silu(a)| <= |a|. So every value
// of the row, silu(a) u w g2 (relu2: max(a, 0)^2 w g2), is below
// B = g13^2 xss 2^(2 px) n_gate n_up |w g2|. Each factor is m 2^e with 1/2 <= m < 1, so
// 2^(E-7) <= B < 2^E with E the sum of the exponents, and q = E - 14 keeps every value below
// 2^14 (a quarter of the f16 range, ample for the fp32 rounding of the factors): nothing
// overflows, and each value is stored within 2^-11 of itself plus 2^-25 2^q <= 2^-32 B (bf16:
// 2^-9 of itself; on real data B exceeds the row maximum by about the reduction length). A
// zero factor (a zero row or weight) or a non-finite one gives q = 0.
__device__ __forceinline__ int f16_row_exponent(float g13, float xss, int px, float n_gate, float n_up, float w,
                                                float g2) {
  const float f[6] = {g13, xss, n_gate, n_up, w, g2};
  int e_sum = 2 * px;
  bool finite = true;
#pragma unroll
  for (int i = 0; i < 6; ++i) {
    const float a = fabsf(f[i]);
    finite = finite && a > 0.f && a <= 3.4028235e38f;
    e_sum += (i == 0 ? 2 : 1) * __builtin_amdgcn_frexp_expf(a);
  }
  return finite ? e_sum - 14 : 0;
}

// Per-launch constants shared by every item of a workgroup.
struct GemmCtx {
  int groups, kbs;
  int64_t sc_per_group;
  const uint8_t* nib;
  const uint8_t* scb;
  __amdgpu_buffer_rsrc_t act;        // activations (x, its f16 copy, or the intermediate rows), bounds-checked
  int act_row_bytes, k_bytes;        // row pitch of that buffer and its K extent, in bytes
};

// Dequantisation of one wave's fragment dword for MFMA step s, for the three routes:
// NVFP4 to f16 (the FP4 convert, then one packed f16 multiply by the scale), NVFP4 to
// bf16 through f32, MXFP4 to bf16 (the scaled convert alone).
// The bf16 routes keep the raw scale dword and decode the scale of step s on use (fewer live
// registers than four decoded scales); the f16 route decodes the four scales at once, two per
// convert.
template <int FMT, bool F16>
struct Deq {
  typedef bf16x8 T;
  uint32_t w;
  __device__ __forceinline__ void set(uint32_t v) { w = v; }
  __device__ __forceinline__ T operator()(uint32_t q, int s) const {
    if (FMT == FMT_NVFP4) {
      const f32x2 pr = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(s >= 2 ? w >> 16 : w, 1.0f, false);
      return dq8<FMT>(q, pr[s & 1]);
    }
    return dq8<FMT>(q, __uint_as_float(((w >> (8 * s)) & 0xFFu) << 23));
  }
};
template <>
struct Deq<FMT_NVFP4, true> {
  typedef f16x8 T;
  NvScalesF16 sc;
  __device__ __forceinline__ void set(uint32_t v) { sc = nv_scales_f16(v); }
  __device__ __forceinline__ T operator()(uint32_t q, int s) const { return dq8_nv_f16(q, sc.step(s)); }
};

__device__ __forceinline__ f32x4 mma(const bf16x8& a, const bf16x8& b, const f32x4& c) { return mfma16(a, b, c); }
__device__ __forceinline__ f32x4 mma(const f16x8& a, const f16x8& b, const f32x4& c) { return mfma16h(a, b, c); }

// One item: NB route blocks (16 NB rows) of one expert x 256 weight rows, full K.
// KT: the activation K extent is not a multiple of the 256-byte K block (hidden size not a
// multiple of 128): every activation load checks its lane's offset against the row end.
template <int FMT, int PHASE, int NB, bool KT, typename Hook>
__device__ __forceinline__ void gemm_item(const FusedParams& p, const GemmCtx& c, uint8_t* lds, int mt, int nt,
                                          Hook&& take_ticket) {
  using P = Plan<NB>;
  constexpr int D = P::kDepth, FR = P::FR, BW = P::BW, XD = P::XD;
  // NVFP4 runs on f16 operands in both GEMMs: FC1 on the per-token scaled activations, FC2 on
  // the intermediate rows that FC1 stores as f16 times a per-slot power of two.
  constexpr bool F16 = FMT == FMT_NVFP4;
  using Dq = Deq<FMT, F16>;
  using T = typename Dq::T;
  const PreparedGeom& g = p.g;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int2 tile = p.tiles[mt];
  const int64_t fb = tile.x;
  const int nb = __builtin_amdgcn_readfirstlane(tile.y & 0xFF);
  const int e = __builtin_amdgcn_readfirstlane(tile.y >> 8);
  const int kbs = c.kbs;

  // The epilogue's per-route values -- FC1: token, router weight and (f16 route) the token's
  // exponent and sum of squares; FC2: route id and row exponent. Tiles of 4 or more blocks
  // load them now (thread s for slot s of the tile) and stage them in LDS past the stage ring
  // after the K loop, so that their epilogue waits on no global round trip (the token gathers
  // go out once the first stage has landed, which the slot loads, issued before it, have
  // too): prefill FC1 -1 %. Smaller tiles, whose epilogue is short, load them there (the
  // staging barrier cost them more than it saved).
  static_assert(kEpilogueStage + NB * kBlockM * 16 <= kLdsBytes, "epilogue staging fits in LDS");
  const bool staged_epi = NB >= 4 && (PHASE == 1 ? !p.w4a8 : !p.atomic_bf16);
  const bool stager = staged_epi && tid < NB * kBlockM;
  int4 epi = make_int4(-1, 0, 0, 0);
  if (stager) {
    const int64_t sslot = (fb + min(tid / kBlockM, nb - 1)) * kBlockM + (tid % kBlockM);
    if (PHASE == 1) {
      const int2 v = p.slot_info[sslot];
      epi.x = v.x;
      epi.y = v.y;
    } else {
      epi.x = p.sorted_route_ids[sslot];
      epi.y = F16 ? p.sexp[sslot] : 0;
    }
  }
  auto gather_tokens = [&]() {
    if (PHASE == 1 && F16 && stager) {
      const int t = max(epi.x, 0);
      epi.z = p.xexp[t];
      epi.w = __float_as_int(p.xss[t]);
    }
  };

  // Activation loads. A route block's K block (16 rows x 256 B) sits in LDS as 32 half-row
  // slots of 128 B: row r = 8 r3 + r7, half h goes to slot 4 r7 + 2 h + r3, and its 16-byte
  // chunk c to position c ^ r7 inside the slot. Load q (1 KiB) of a stage fills slots
  // 8 (q % 4) .. +7 of block q / 4 -- four whole rows, so every load reads eight full 128-byte
  // lines -- and the 16 lanes that later read one chunk column of 16 rows hit 16 distinct
  // bank groups. Padding slots and blocks past the tile read 0 through the bounds check, so no
  // load is predicated.
  uint32_t rowoff[XD], gofs[XD];
  int qdst[XD];
#pragma unroll
  for (int j = 0; j < XD; ++j) {
    const int q = NB >= 2 ? wave * XD + j : (wave & 3);
    const int hslot = 8 * (q & 3) + (lane >> 3);            // half-row slot of this lane
    const int r7 = hslot >> 2, h = (hslot >> 1) & 1, r3 = hslot & 1;
    const int row = (q >> 2) * kBlockM + 8 * r3 + r7;
    const int64_t slot = fb * kBlockM + row;
    const int t = row < nb * kBlockM ? p.slot_info[slot].x : -1;
    const int64_t src_row = PHASE == 1 ? int64_t(t) : slot;   // x row of the token, or the slot's own row
    qdst[j] = q * 1024;
    gofs[j] = uint32_t(8 * h + ((lane & 7) ^ r7)) << 4;
    rowoff[j] = t >= 0 ? uint32_t(src_row * c.act_row_bytes) : kOutOfRange;
  }
  // This wave's row groups 2w, 2w+1 of the N tile: fragment blocks and scale rows through
  // buffer resources over the tile's groups, so groups past the end (last N tile only) read
  // 0 and are never stored.
  const int tile_groups = min(16, c.groups - nt * 16);
  const int64_t g0 = int64_t(e) * c.groups + nt * 16;
  const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc(
      uniform_ptr(c.nib + g0 * kbs * kFragBytes), 0,
      __builtin_amdgcn_readfirstlane(tile_groups * kbs * kFragBytes), 0x00020000);
  const __amdgpu_buffer_rsrc_t sres = __builtin_amdgcn_make_buffer_rsrc(
      uniform_ptr(c.scb + g0 * c.sc_per_group), 0,
      __builtin_amdgcn_readfirstlane(int(tile_groups * c.sc_per_group)), 0x00020000);
  const int rg_base = nt * 16 + wave * FR;
  const int sc_lane = FMT == FMT_NVFP4 ? ((lane >> 5) * 16 + (lane & 15)) * 16 : (lane & 15) * 16;
  // the lane's constant parts of the weight and scale offsets (the K block's part goes in the
  // scalar offset of each load)
  int wvoff[FR], svoff[FR];
#pragma unroll
  for (int f = 0; f < FR; ++f) {
    wvoff[f] = (wave * FR + f) * kbs * kFragBytes + lane * 16;
    svoff[f] = int((wave * FR + f) * c.sc_per_group) + sc_lane;
  }

  // One stage: the activation K block into LDS slot `slot`, this wave's fragment dwords and
  // scale dwords into registers. Blocks past K are clamped (weights) or read 0 (activations):
  // every stage issues the same P::kLoads loads per wave, so the vmcnt arithmetic below is
  // exact. The loads are issued in four parts, one ahead of each MFMA K-step of the stage
  // being computed, so that a load queue that is still full stalls a wave between MFMA
  // groups instead of ahead of all of them.
  u32x4 wr[D][FR];
  uint32_t sc[D][FR];
  auto issue_part = [&](int part, int kb, int slot, u32x4* wd, uint32_t* scd) {
    uint8_t* st = lds + slot * P::kStage;
    const uint32_t k = uint32_t(kb) * kRowBytes;
    const int kc = min(kb, kbs - 1);
#pragma unroll
    // Order within a stage: scales, fragments (both needed first), then the activations.
    for (int l = 0; l < P::kLoads; ++l) {
      if (l * 4 / P::kLoads != part) continue;
      if (l < FR) {
        scd[l] = __builtin_amdgcn_raw_buffer_load_b32(sres, svoff[l], int((kc >> 2) * g.sc_chunk_bytes + (kc & 3) * 4), 0);
      } else if (l < 2 * FR) {
        const int f = l - FR;
        wd[f] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wres, wvoff[f], kc * kFragBytes, 0));
      } else {
        const int j = l - 2 * FR;
        if constexpr (KT)
          dma16(c.act, st + qdst[j], (rowoff[j] + k + gofs[j]) | (k + gofs[j] < uint32_t(c.k_bytes) ? 0u : kOutOfRange));
        else
          dma16s(c.act, st + qdst[j], rowoff[j] | gofs[j], k);     // whole K blocks: no row-end check
      }
    }
  };
  auto issue = [&](int kb, int slot, u32x4* wd, uint32_t* scd) {
#pragma unroll
    for (int part = 0; part < 4; ++part) issue_part(part, kb, slot, wd, scd);
    __builtin_amdgcn_sched_barrier(0);            // stages leave in order
  };

  f32x4 acc[FR][BW];
#pragma unroll
  for (int f = 0; f < FR; ++f)
#pragma unroll
    for (int b = 0; b < BW; ++b) acc[f][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  // One K block: four MFMA K-steps.
  auto compute = [&](int slot, const u32x4* wq, const uint32_t* scd, int kb_next, int slot_next, u32x4* wd_next,
                     uint32_t* scd_next) {
    const uint8_t* st = lds + slot * P::kStage;
    Dq dq[FR];
#pragma unroll
    for (int f = 0; f < FR; ++f) dq[f].set(scd[f]);
    // Lane l reads chunk 4 s + l / 16 of row l % 16: slot 4 r7 + 2 (s / 2) + r3, position
    // (4 (s % 2) + l / 16) ^ r7 -- two lane bases (even and odd s) plus immediates.
    const int r7 = lane & 7, r3 = (lane >> 3) & 1, q4 = lane >> 4;
    const uint8_t* xb_even = st + r7 * 512 + r3 * 128 + ((q4 ^ r7) << 4);
    const uint8_t* xb_odd = st + r7 * 512 + r3 * 128 + (((4 + q4) ^ r7) << 4);
    auto xread = [&](int b, int s) {
      return __builtin_bit_cast(T, *reinterpret_cast<const u32x4*>((s & 1 ? xb_odd : xb_even) + b * kBlockBytes +
                                                                   (s >> 1) * 256));
    };
    // The activation fragments of K-step s + 1 are read while K-step s runs its MFMAs (two
    // register sets inside the stage; the first K-step's reads wait at the stage start).
    // The scheduling barrier after each K-step keeps the compiler from hoisting further
    // reads (register pressure).
    T xb2[2][BW];
#pragma unroll
    for (int b = 0; b < BW; ++b) xb2[0][b] = xread(b, 0);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      issue_part(s, kb_next, slot_next, wd_next, scd_next);
      if (s < 3) {
#pragma unroll
        for (int b = 0; b < BW; ++b) xb2[(s + 1) & 1][b] = xread(b, s + 1);
      }
      T a[FR];
#pragma unroll
      for (int f = 0; f < FR; ++f) a[f] = dq[f](wq[f][s], s);
#pragma unroll
      for (int b = 0; b < BW; ++b)
#pragma unroll
        for (int f = 0; f < FR; ++f) acc[f][b] = mma(a[f], xb2[s & 1][b], acc[f][b]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Pipeline: stages 0 .. D-2 in flight before the loop; step kb waits until its own stage has
  // landed, meets the other waves at a barrier (their loads have landed too, and all are done
  // with slot (kb-1) % D), then computes stage kb while refilling that slot with stage kb+D-1.
  // Loads that write LDS and loads that write registers complete in order within each kind
  // but not with respect to each other (measured on gfx950: counting both kinds let a stage's
  // activation rows be read before they landed). So the wait leaves at most the later
  // stages' LDS loads, (D-2) * XD, outstanding: then this stage's LDS loads have landed, and
  // so have its register loads (at least 4 (D-2) >= (D-2) * XD register loads follow them).
  // The hook takes the next item's queue ticket: once the first stage has landed for items of
  // up to kEarlyTicketKB K blocks (edge and small shapes -3 %), after the K loop for longer
  // ones (taken early in a 56-block prefill FC1 item it cost 2.6 %).
  const bool early_ticket = kbs <= kEarlyTicketKB;
  auto step = [&](int kb, int j) {
    wait_vmcnt<(D - 2) * XD>();
    stage_barrier();
    if (kb == 0) {
      if (early_ticket) take_ticket();
      gather_tokens();
    }
    __builtin_amdgcn_sched_barrier(0);
    const int jn = (j + D - 1) % D;
    compute(j, wr[j], sc[j], kb + D - 1, jn, wr[jn], sc[jn]);
  };
#pragma unroll
  for (int j = 0; j < D - 1; ++j) issue(j, j, wr[j], sc[j]);
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
  if (!early_ticket) take_ticket();
  const int4* epi_lds = reinterpret_cast<const int4*>(lds + kEpilogueStage);
  if (staged_epi) {
    if (stager) reinterpret_cast<int4*>(lds + kEpilogueStage)[tid] = epi;
    lds_barrier();
  }

  // Epilogue. Lane (r0 = 4 (lane / 16), col = lane % 16) holds rows r0..r0+3 of each
  // 16-row group, route column col of each block.
  const int r0 = 4 * (lane >> 4), col = lane & 15;
  if constexpr (PHASE == 1 && FMT == FMT_MXFP4) {
    if (p.w4a8) {
      // W4A8: the activation output (without the router weight, which FC2 applies) rounded to
      // MXFP8 right here -- E4M3 codes into the route slot's code row, one E8M0 byte per 32
      // columns. With SiLU-SwiGLU a wave holds 16 columns of each route (one gate/up pair) and
      // the other half of their MX block sits in the neighbouring wave: the two exchange their
      // halves' maxima through LDS. With relu2 a wave's two row groups are one whole block.
      static_assert(P::kDepth * P::kStage <= kW8AmaxOffset, "the exchange area lies past the stage ring");
      const float g13 = p.g13[e];
      const bool swiglu = g.act == ACT_SWIGLU;
      float v[BW][FR][4], am[BW];
#pragma unroll
      for (int bb = 0; bb < BW; ++bb) {
        float a = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (swiglu) {
            v[bb][0][i] = silu_f32(acc[0][bb][i] * g13) * (acc[1][bb][i] * g13);
            v[bb][1][i] = 0.f;
          } else {
#pragma unroll
            for (int f = 0; f < FR; ++f) {
              const float u = fmaxf(acc[f][bb][i] * g13, 0.f);
              v[bb][f][i] = u * u;
            }
          }
#pragma unroll
          for (int f = 0; f < FR; ++f) a = fmaxf(a, fabsf(v[bb][f][i]));
        }
        a = fmaxf(a, __shfl_xor(a, 16, 64));
        am[bb] = fmaxf(a, __shfl_xor(a, 32, 64));
      }
      if (swiglu) {
        float* xam = reinterpret_cast<float*>(lds + kW8AmaxOffset);      // [waves][BW][16]
        if (lane < 16) {
#pragma unroll
          for (int bb = 0; bb < BW; ++bb) xam[(wave * BW + bb) * 16 + col] = am[bb];
        }
        lds_barrier();
#pragma unroll
        for (int bb = 0; bb < BW; ++bb) am[bb] = fmaxf(am[bb], xam[((wave ^ 1) * BW + bb) * 16 + col]);
      }
      const int64_t ip = g.ip;
      int tok[BW];
#pragma unroll
      for (int bb = 0; bb < BW; ++bb) tok[bb] = p.slot_info[(fb + min(bb, nb - 1)) * kBlockM + col].x;
#pragma unroll
      for (int bb = 0; bb < BW; ++bb) {
        if (bb < nb && rg_base < c.groups) {
          const int64_t slot = (fb + bb) * kBlockM + col;
          if (tok[bb] >= 0) {
            const float amax = am[bb];
            const int ex = amax > 0.f ? mx8_exponent(amax) : 0;
            const uint8_t sbyte = uint8_t(amax > 0.f ? ex + 127 : 0);
            uint8_t* crow = p.inter8 + slot * ip;
            if (swiglu) {
              const int64_t icol = int64_t(rg_base >> 1) * 16 + r0;
              *reinterpret_cast<uint32_t*>(crow + icol) = mx8_codes4(v[bb][0], ex, amax);
              if ((wave & 1) == 0 && r0 == 0) p.sc8[slot * (ip / 32) + icol / 32] = sbyte;
            } else {
#pragma unroll
              for (int f = 0; f < FR; ++f)
                *reinterpret_cast<uint32_t*>(crow + int64_t(rg_base + f) * 16 + r0) = mx8_codes4(v[bb][f], ex, amax);
              if (r0 == 0) p.sc8[slot * (ip / 32) + rg_base / 2] = sbyte;
            }
          }
        }
      }
      return;
    }
  }
  if (PHASE == 1) {
    const float g13 = p.g13[e], g2 = p.g2[e];
    const float n_gate = F16 ? p.n13[2 * e] : 0.f, n_up = F16 ? p.n13[2 * e + 1] : 0.f;
    // The per-route values: staged in LDS above, or loaded all together here (one round trip
    // for the slots, one for their tokens' exponents and sums of squares) from clamped
    // addresses, so that no load is predicated and none waits behind another.
    int2 info[BW];
    int xe[BW];
    float xs[BW];
    if constexpr (NB >= 4) {
#pragma unroll
      for (int bb = 0; bb < BW; ++bb) {
        const int4 v = epi_lds[bb * kBlockM + col];
        info[bb] = make_int2(v.x, v.y);
        xe[bb] = v.z;
        xs[bb] = __int_as_float(v.w);
      }
    } else {
#pragma unroll
      for (int bb = 0; bb < BW; ++bb) info[bb] = p.slot_info[(fb + min(bb, nb - 1)) * kBlockM + col];
      if constexpr (F16) {
#pragma unroll
        for (int bb = 0; bb < BW; ++bb) {
          const int t = max(info[bb].x, 0);
          xe[bb] = p.xexp[t];
          xs[bb] = p.xss[t];
        }
      }
    }
#pragma unroll
    for (int bb = 0; bb < BW; ++bb) {
      const int b = bb;
      if (b < nb) {
        const int64_t slot = (fb + b) * kBlockM + col;
        const bool valid = info[bb].x >= 0;
        // W4A8: the router weight and FC2 global scale come after FC2 (outside the quantisation)
        const float rw = valid ? (p.w4a8 ? 1.f : __int_as_float(info[bb].y) * g2) : 0.f;
        float s13 = g13;
        // f16 rows: the route's row times 2^-q, q from a bound on the row (the same in every N
        // tile of the route, so FC2 undoes it with one multiply per route)
        int q = 0;
        if constexpr (F16) {
          s13 = valid ? ldexpf(g13, xe[bb]) : g13;
          q = valid ? f16_row_exponent(g13, xs[bb], xe[bb], n_gate, n_up, __int_as_float(info[bb].y), g2) : 0;
          if (nt == 0 && wave == 0 && r0 == 0) p.sexp[slot] = q;
        }
        if (g.act == ACT_SWIGLU) {
#pragma unroll
          for (int pr = 0; pr < FR / 2; ++pr) {
            if (rg_base + 2 * pr < c.groups) {
              float v[4];
#pragma unroll
              for (int i = 0; i < 4; ++i)
                v[i] = silu_f32(acc[2 * pr][bb][i] * s13) * (acc[2 * pr + 1][bb][i] * s13) * rw;
              const int64_t icol = int64_t((rg_base + 2 * pr) >> 1) * 16 + r0;
              if constexpr (F16) store_f16x4(p.inter + slot * g.ip + icol, v, q);
              else store_inter4(p, slot, icol, v);
            }
          }
        } else {
#pragma unroll
          for (int f = 0; f < FR; ++f) {
            if (rg_base + f < c.groups) {
              float v[4];
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const float u = fmaxf(acc[f][bb][i] * s13, 0.f);
                v[i] = u * u * rw;
              }
              const int64_t icol = int64_t(rg_base + f) * 16 + r0;
              if constexpr (F16) store_f16x4(p.inter + slot * g.ip + icol, v, q);
              else store_inter4(p, slot, icol, v);
            }
          }
        }
      }
    }
  } else if (p.atomic_bf16) {
    // Opt-in approximate top-k sum: each route's row (router weight and FC2 global scale
    // already folded in by FC1) rounded to bf16 and added into its token's output row by
    // packed-bf16 atomics; the sum's rounding and order vary from run to run.
#pragma unroll
    for (int bb = 0; bb < BW; ++bb) {
      const int b = bb;
      if (b < nb) {
        const int tok = p.slot_info[(fb + b) * kBlockM + col].x;
        if (tok >= 0) {
          const int q = F16 ? p.sexp[(fb + b) * kBlockM + col] : 0;
#pragma unroll
          for (int f = 0; f < FR; ++f) {
            const int64_t h = int64_t(rg_base + f) * 16 + r0;
            if (h < g.H) {
              f32x4 a = acc[f][bb];
              if constexpr (F16) a = ldexp4(a, q);
              bf16x2* dst = reinterpret_cast<bf16x2*>(p.out + int64_t(tok) * g.H + h);
              __builtin_amdgcn_global_atomic_fadd_v2bf16(dst, __builtin_bit_cast(bf16x2, pack_bf16x2(a[0], a[1])));
              __builtin_amdgcn_global_atomic_fadd_v2bf16(dst + 1, __builtin_bit_cast(bf16x2, pack_bf16x2(a[2], a[3])));
            }
          }
        }
      }
    }
  } else {
    // (route ids and row exponents: staged in LDS above, or loaded together here)
    int rid[BW], qv[BW];
#pragma unroll
    for (int bb = 0; bb < BW; ++bb) {
      if constexpr (NB >= 4) {
        const int4 v = epi_lds[bb * kBlockM + col];
        rid[bb] = v.x;
        qv[bb] = v.y;
      } else {
        const int64_t slot = (fb + min(bb, nb - 1)) * kBlockM + col;
        rid[bb] = p.sorted_route_ids[slot];
        qv[bb] = F16 ? p.sexp[slot] : 0;
      }
    }
#pragma unroll
    for (int bb = 0; bb < BW; ++bb) {
      const int b = bb;
      if (b < nb) {
        const int r = rid[bb];
        if (r >= 0) {
          const float wt = p.w4a8 ? __int_as_float(p.slot_info[(fb + b) * kBlockM + col].y) * p.g2[e] : 1.f;
          const int q = qv[bb];
#pragma unroll
          for (int f = 0; f < FR; ++f) {
            const int64_t h = int64_t(rg_base + f) * 16 + r0;
            if (h < g.H) store_row4(p.y + int64_t(r) * g.H + h, F16 ? ldexp4(acc[f][bb], q) : acc[f][bb] * wt);
          }
        }
      }
    }
  }
}

// W4A8 FC2: the block-scaled FP4 x FP8 MFMA (v_mfma_scale_f32_16x16x128_f8f6f4), one per
// (row group, route block, K block), E8M0 scales applied by the matrix core -- no
// dequantisation. Operand lanes: A (weights) lane (c, q) holds the 32 consecutive K of MX block
// q of row c, made from the prepared fragment (8-K chunks dealt over the lane quarters) by a
// 4 x 4 dword transpose across the quarters; B (the routes' MXFP8 codes, written by FC1) lane
// (c, q) holds K 16 q .. +15 and 64 + 16 q .. +15 of route c; each lane passes the scale byte
// of MX block q of its row or route. The activation codes of a K block (128 B per route, the
// 16-byte chunk j of route row r at position j ^ (r % 8): the 16 lanes reading one chunk column
// hit distinct banks) and their scale dwords stream through the LDS stage ring as in the
// W4A16 item; each wave's fragments and scale dwords through its register ring.
template <int NB>
struct PlanW8 {
  static constexpr int FR = 2;                                       // row groups per wave
  static constexpr int XD = NB >= 4 ? NB / 4 : 1;                    // 1 KiB code loads per wave and stage
  static constexpr int kCodes = NB * kBlockM * kKBlock;              // codes of a stage
  static constexpr int kStage = kCodes + 512;                        // + up to 128 routes' scale dwords
  static constexpr int kDepth = NB >= 4 ? 3 : 5;   // (deeper rings spill registers)
  static constexpr int kLds = XD + 1;                                // loads into LDS per wave and stage
  static constexpr int kLoads = kLds + 2 * FR;
  static_assert(kDepth >= 3 && (kDepth - 1) * kLoads < 64, "ring too shallow or vmcnt out of range");
  static_assert(kLds <= 2 * FR, "the stage wait relies on at least as many register loads as LDS loads");
  static_assert(kDepth * kStage <= kLdsBytes, "stage ring larger than the LDS");
};

template <int NB, typename Hook>
__device__ __forceinline__ void gemm_item_w8(const FusedParams& p, const GemmCtx& c, uint8_t* lds, int mt, int nt,
                                             Hook&& take_ticket) {
  using P = PlanW8<NB>;
  constexpr int D = P::kDepth, FR = P::FR, XD = P::XD;
  const PreparedGeom& g = p.g;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q = lane >> 4, col = lane & 15;
  const int2 tile = p.tiles[mt];
  const int64_t fb = tile.x;
  const int nb = __builtin_amdgcn_readfirstlane(tile.y & 0xFF);
  const int e = __builtin_amdgcn_readfirstlane(tile.y >> 8);
  const int kbs = c.kbs;
  const int ip = int(g.ip);

  // Code loads: load j of this wave brings routes 8 qd .. 8 qd + 7 of the tile (qd below; with
  // fewer than 4 blocks several waves repeat the same load into the same place), lane i route
  // 8 qd + i / 8, stored chunk i % 8 = source chunk (i % 8) ^ (route % 8). Routes past the
  // tile's blocks read 0. Scale load: routes 64 h + lane, dword K block kb of the route's scale
  // row.
  uint32_t coff[XD];
  int cdst[XD];
#pragma unroll
  for (int j = 0; j < XD; ++j) {
    const int qd = NB >= 4 ? wave * XD + j : (wave % (2 * NB));
    const int row = 8 * qd + (lane >> 3);
    const uint32_t chunk = uint32_t((lane & 7) ^ (row & 7));
    cdst[j] = qd * 1024;
    coff[j] = row < nb * kBlockM ? uint32_t((fb * kBlockM + row) * ip) + chunk * 16 : kOutOfRange;
  }
  const int h = NB == 8 ? (wave & 1) : 0;
  const int srow = 64 * h + lane;
  const uint32_t soff = srow < nb * kBlockM ? uint32_t((fb * kBlockM + srow) * (ip / 32)) : kOutOfRange;
  const __amdgpu_buffer_rsrc_t cres = buffer_rsrc(p.inter8, uint32_t(p.cap_blocks * kBlockM * ip));
  const __amdgpu_buffer_rsrc_t bsres = buffer_rsrc(p.sc8, uint32_t(p.cap_blocks * kBlockM * (ip / 32)));

  const int tile_groups = min(16, c.groups - nt * 16);
  const int64_t g0 = int64_t(e) * c.groups + nt * 16;
  const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc(
      uniform_ptr(c.nib + g0 * kbs * kFragBytes), 0,
      __builtin_amdgcn_readfirstlane(tile_groups * kbs * kFragBytes), 0x00020000);
  const __amdgpu_buffer_rsrc_t sres = __builtin_amdgcn_make_buffer_rsrc(
      uniform_ptr(c.scb + g0 * c.sc_per_group), 0,
      __builtin_amdgcn_readfirstlane(int(tile_groups * c.sc_per_group)), 0x00020000);
  const int rg_base = nt * 16 + wave * FR;
  const int sc_lane = col * 16;

  u32x4 wr[D][FR];
  uint32_t sc[D][FR];
  // One stage (K block kb, clamped for the weights; stages past K are issued and never used):
  // scale dwords and fragments into registers, then codes and scale dwords into LDS.
  auto issue = [&](int kb, int slot, u32x4* wd, uint32_t* scd) {
    uint8_t* st = lds + slot * P::kStage;
    const int kc = min(kb, kbs - 1);
#pragma unroll
    for (int f = 0; f < FR; ++f)
      scd[f] = __builtin_amdgcn_raw_buffer_load_b32(
          sres, int((wave * FR + f) * c.sc_per_group + (kc >> 2) * g.sc_chunk_bytes) + sc_lane + (kc & 3) * 4, 0, 0);
#pragma unroll
    for (int f = 0; f < FR; ++f)
      wd[f] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
          wres, ((wave * FR + f) * kbs + kc) * kFragBytes + lane * 16, 0, 0));
#pragma unroll
    for (int j = 0; j < XD; ++j) dma16(cres, st + cdst[j], coff[j] + uint32_t(kc) * kKBlock);
    dma4(bsres, st + P::kCodes + 256 * h, soff + uint32_t(kc) * 4);
    __builtin_amdgcn_sched_barrier(0);            // stages leave in order
  };

  f32x4 acc[FR][NB];
#pragma unroll
  for (int f = 0; f < FR; ++f)
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[f][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  // lane (col, q): route col of each block, chunks q and q + 4 of its row (swizzled)
  const int olo = col * kKBlock + ((q ^ (col & 7)) << 4);
  const int ohi = olo ^ 64;
  auto compute = [&](int slot, const u32x4* wq, const uint32_t* scd) {
    const uint8_t* st = lds + slot * P::kStage;
    i32x8 a[FR];
    int sa[FR];
#pragma unroll
    for (int f = 0; f < FR; ++f) {
      const u32x4 t = transpose_quarters(wq[f]);
      a[f] = i32x8{int(t[0]), int(t[1]), int(t[2]), int(t[3]), 0, 0, 0, 0};
      sa[f] = int(scd[f] >> (8 * q));
    }
    // B operands one block ahead of the MFMAs (two register sets; the scheduling barriers keep
    // the compiler from hoisting every block's reads)
    auto bread = [&](int b, i32x8& bop, uint32_t& sbw) {
      const u32x4 lo = *reinterpret_cast<const u32x4*>(st + (b * kBlockM + col) * kKBlock + (olo - col * kKBlock));
      const u32x4 hi = *reinterpret_cast<const u32x4*>(st + (b * kBlockM + col) * kKBlock + (ohi - col * kKBlock));
      bop = i32x8{int(lo[0]), int(lo[1]), int(lo[2]), int(lo[3]), int(hi[0]), int(hi[1]), int(hi[2]), int(hi[3])};
      sbw = *reinterpret_cast<const uint32_t*>(st + P::kCodes + 4 * (b * kBlockM + col));
    };
    i32x8 bop[2];
    uint32_t sbw[2];
    bread(0, bop[0], sbw[0]);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      if (b + 1 < NB) bread(b + 1, bop[(b + 1) & 1], sbw[(b + 1) & 1]);
      const int sb = int(sbw[b & 1] >> (8 * q));
#pragma unroll
      for (int f = 0; f < FR; ++f)
        acc[f][b] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[f], bop[b & 1], acc[f][b], 4, 0, 0, sa[f], 0, sb);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // The same ring as the W4A16 item (loads into LDS and into registers complete in order within
  // each kind): the wait leaves only the later stages' LDS loads outstanding.
  const bool early_ticket = kbs <= kEarlyTicketKB;    // (the next item's ticket, as in the W4A16 item)
  auto step = [&](int kb, int j) {
    wait_vmcnt<(D - 2) * P::kLds>();
    stage_barrier();
    if (kb == 0 && early_ticket) take_ticket();
    __builtin_amdgcn_sched_barrier(0);
    const int jn = (j + D - 1) % D;
    issue(kb + D - 1, jn, wr[jn], sc[jn]);
    compute(j, wr[j], sc[j]);
    __builtin_amdgcn_sched_barrier(0);
  };
#pragma unroll
  for (int j = 0; j < D - 1; ++j) issue(j, j, wr[j], sc[j]);
  int kb = 0;
  for (; kb + D <= kbs; kb += D) {
#pragma unroll
    for (int j = 0; j < D; ++j) step(kb + j, j);
  }
#pragma unroll
  for (int j = 0; j < D - 1; ++j)
    if (kb + j < kbs) step(kb + j, j);
  wait_vmcnt<0>();
  if (!early_ticket) take_ticket();

  // Epilogue: the weighted bf16 row of each route (router weight x FC2 global scale, outside
  // the quantisation), summed over top-k by the combine pass.
  const int r0 = 4 * q;
  // (route ids and router weights of all blocks loaded together first, from clamped slots)
  const float g2 = p.g2[e];
  int rid[NB];
  float rwt[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int64_t slot = (fb + min(b, nb - 1)) * kBlockM + col;
    rid[b] = p.sorted_route_ids[slot];
    rwt[b] = __int_as_float(p.slot_info[slot].y);
  }
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    if (b < nb) {
      const int r = rid[b];
      if (r >= 0) {
        const float wt = rwt[b] * g2;
#pragma unroll
        for (int f = 0; f < FR; ++f) {
          const int64_t hh = int64_t(rg_base + f) * 16 + r0;
          if (hh < g.H) store_row4(p.y + int64_t(r) * g.H + hh, acc[f][b] * wt);
        }
      }
    }
  }
}

template <int FMT, int PHASE, bool W8>
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
    const uint16_t* src = FMT == FMT_NVFP4 ? p.x16 : p.x;
    c.act_row_bytes = g.H * 2;
    c.k_bytes = g.H * 2;
    c.act = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(src), 0, int(p.m * g.H * 2), 0x00020000);
  } else {
    c.act_row_bytes = int(g.ip * 2);
    c.k_bytes = int(g.ip * 2);
    c.act = __builtin_amdgcn_make_buffer_rsrc(p.inter, 0, int(p.cap_blocks * kBlockM * g.ip * 2), 0x00020000);
  }
  if (PHASE == 1 && p.atomic_bf16) {
    // FC2 accumulates into the output with atomics: zero it first (m * H * 2 bytes, H % 8 == 0;
    // FC2 runs after this launch in stream order).
    const int64_t n16 = p.m * g.H / 8;
    u32x4* o = reinterpret_cast<u32x4*>(p.out);
    for (int64_t i = int64_t(blockIdx.x) * kGemmThreads + threadIdx.x; i < n16; i += int64_t(gridDim.x) * kGemmThreads)
      o[i] = u32x4{0u, 0u, 0u, 0u};
  }
  const int n_mt = p.live[4];
  const int n_nt = (c.groups + 15) / 16;
  // Persistent workgroups take items from per-XCD queues (reset by the route packer).
  // Workgroups are dealt to the XCDs round robin; queue x holds the full M tiles and the
  // partial (tail) M tiles whose table index is x mod 8, alternating one full and one partial
  // tile, each as its N tiles in a row. So the ~32 workgroups of an XCD run two M tiles at a
  // time and fetch each activation K block into their shared L2 once, and an MFMA-bound full
  // tile runs beside a weight-stream-bound partial one, so that HBM and the matrix cores are
  // busy together. The same expert's M tiles on the other XCDs read its weight tiles at the
  // same time, which the Infinity Cache serves. An exhausted queue sends a workgroup on to
  // the next one, so the load stays balanced to the end.
  int* queues = p.live + (PHASE == 1 ? 8 : 16);
  const int n_full = p.live[5], n_part = n_mt - n_full;
  int q = blockIdx.x & 7, tried = 0;                 // thread 0's queue cursor
  // Thread 0: the item that ticket i of queue q stands for, or, when that queue is exhausted,
  // the next queue's (one more ticket each, -1 when every queue is).
  auto take = [&](int i) {
    for (;;) {
      const int fq = n_full > q ? (n_full - 1 - q) / 8 + 1 : 0;
      const int pq = n_part > q ? (n_part - 1 - q) / 8 + 1 : 0;
      if (i < (fq + pq) * n_nt) {
        const int m = i / n_nt, both = min(fq, pq);
        bool full;
        int ord;
        if (m < 2 * both) {
          full = (m & 1) == 0;
          ord = m >> 1;
        } else {
          full = fq > pq;
          ord = m - both;
        }
        const int mt = full ? q + 8 * ord : n_full + q + 8 * ord;
        return mt * n_nt + i % n_nt;
      }
      q = (q + 1) & 7;
      if (++tried == 8) return -1;
      i = atomicAdd(&queues[q], 1);
    }
  };
  // The next item's ticket is taken while the current item runs (see gemm_item), so that its
  // round trip is off the path between items; s_item alternates between the current item and
  // the one taken during it.
  __shared__ int s_item[2];
  if (threadIdx.x == 0) s_item[0] = take(atomicAdd(&queues[q], 1));
  lds_barrier();
  for (int par = 0;; par ^= 1) {
    const int item = __builtin_amdgcn_readfirstlane(s_item[par]);
    if (item < 0) break;
    int ticket = 0;
    auto reserve = [&]() {
      if (threadIdx.x == 0 && tried < 8) ticket = atomicAdd(&queues[q], 1);
    };
    const int mt = item / n_nt, nt = item % n_nt;
    const int nb = __builtin_amdgcn_readfirstlane(p.tiles[mt].y & 0xFF);
    // Tiles are compiled for 1, 2, 4, 6 or 8 route blocks so that the MFMA loop is straight-line
    // (6: the W4A16 kernel only; five- and six-block tiles ran as eight, prefill FC1 -1.6 %).
    if constexpr (W8) {
      if (nb <= 1) gemm_item_w8<1>(p, c, lds, mt, nt, reserve);
      else if (nb <= 2) gemm_item_w8<2>(p, c, lds, mt, nt, reserve);
      else if (nb <= 4) gemm_item_w8<4>(p, c, lds, mt, nt, reserve);
      else gemm_item_w8<8>(p, c, lds, mt, nt, reserve);
    } else if (c.k_bytes % kRowBytes) {
      if (nb <= 1) gemm_item<FMT, PHASE, 1, true>(p, c, lds, mt, nt, reserve);
      else if (nb <= 2) gemm_item<FMT, PHASE, 2, true>(p, c, lds, mt, nt, reserve);
      else if (nb <= 4) gemm_item<FMT, PHASE, 4, true>(p, c, lds, mt, nt, reserve);
      else if (nb <= 6) gemm_item<FMT, PHASE, 6, true>(p, c, lds, mt, nt, reserve);
      else gemm_item<FMT, PHASE, 8, true>(p, c, lds, mt, nt, reserve);
    } else {
      if (nb <= 1) gemm_item<FMT, PHASE, 1, false>(p, c, lds, mt, nt, reserve);
      else if (nb <= 2) gemm_item<FMT, PHASE, 2, false>(p, c, lds, mt, nt, reserve);
      else if (nb <= 4) gemm_item<FMT, PHASE, 4, false>(p, c, lds, mt, nt, reserve);
      else if (nb <= 6) gemm_item<FMT, PHASE, 6, false>(p, c, lds, mt, nt, reserve);
      else gemm_item<FMT, PHASE, 8, false>(p, c, lds, mt, nt, reserve);
    }
    if (threadIdx.x == 0) s_item[par ^ 1] = tried < 8 ? take(ticket) : -1;
    lds_barrier();
  }
}

// out[t] = bf16(sum over the token's valid routes of y[route]) in route order j = 0..k-1, the
// sum in fp32 over the routes' bf16 rows. A thread owns 8 columns of a token; the rows of up
// to 8 routes are loaded together, then added in order.
__global__ void combine_kernel(const uint16_t* __restrict__ y, const int32_t* __restrict__ route_slot,
                               uint16_t* __restrict__ out, int64_t m, int topk, int64_t H) {
  const int64_t q = H / 8;
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < m * q; i += int64_t(gridDim.x) * blockDim.x) {
    const int64_t t = i / q, c8 = (i % q) * 8;
    float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int j0 = 0; j0 < topk; j0 += 8) {
      u32x4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int64_t r = t * topk + j0 + u;
        v[u] = j0 + u < topk && route_slot[r] >= 0 ? *reinterpret_cast<const u32x4*>(y + r * H + c8) : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (j0 + u < topk) {
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            s[2 * w] += __uint_as_float(v[u][w] << 16);
            s[2 * w + 1] += __uint_as_float(v[u][w] & 0xFFFF0000u);
          }
        }
      }
    }
    *reinterpret_cast<u32x4*>(out + t * H + c8) =
        u32x4{pack_bf16x2(s[0], s[1]), pack_bf16x2(s[2], s[3]), pack_bf16x2(s[4], s[5]), pack_bf16x2(s[6], s[7])};
  }
}

}  // namespace

template <int FMT, int PHASE, bool W8>
hipError_t allow_large_lds(size_t lds) {
  // The stage ring needs more than the 64 KiB default of dynamic LDS.
  static hipError_t once = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_kernel<FMT, PHASE, W8>),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
  return once;
}

hipError_t launch_gemm(const FusedParams& p, int num_cus, hipStream_t stream, LaunchMarks* marks) {
  // One 8-wave workgroup per CU (two waves per SIMD, up to 256 registers each).
  const int grid = num_cus;
  const size_t lds = kLdsBytes;
  const bool nv = p.g.fmt == FMT_NVFP4;
  // W4A8 (MXFP4 weights only): FC1 rounds its activation output to MXFP8 codes in its epilogue
  // and FC2 runs the block-scaled MFMA on them.
  const bool w8 = !nv && p.w4a8;
  hipError_t e = nv ? allow_large_lds<FMT_NVFP4, 1, false>(lds) : allow_large_lds<FMT_MXFP4, 1, false>(lds);
  if (e == hipSuccess)
    e = nv ? allow_large_lds<FMT_NVFP4, 2, false>(lds)
           : (w8 ? allow_large_lds<FMT_MXFP4, 2, true>(lds) : allow_large_lds<FMT_MXFP4, 2, false>(lds));
  if (e != hipSuccess) return e;
  if (nv) hipLaunchKernelGGL((gemm_kernel<FMT_NVFP4, 1, false>), dim3(grid), dim3(kGemmThreads), lds, stream, p);
  else hipLaunchKernelGGL((gemm_kernel<FMT_MXFP4, 1, false>), dim3(grid), dim3(kGemmThreads), lds, stream, p);
  if (marks) marks->after(stream, KID_FC1);
  if (nv) hipLaunchKernelGGL((gemm_kernel<FMT_NVFP4, 2, false>), dim3(grid), dim3(kGemmThreads), lds, stream, p);
  else if (w8) hipLaunchKernelGGL((gemm_kernel<FMT_MXFP4, 2, true>), dim3(grid), dim3(kGemmThreads), lds, stream, p);
  else hipLaunchKernelGGL((gemm_kernel<FMT_MXFP4, 2, false>), dim3(grid), dim3(kGemmThreads), lds, stream, p);
  if (marks) marks->after(stream, KID_FC2);
  if (!p.atomic_bf16) {
    launch_combine(p, stream);
    if (marks) marks->after(stream, KID_COMBINE);
  }
  return hipGetLastError();
}

void launch_combine(const FusedParams& p, hipStream_t stream) {
  const int64_t n = p.m * p.g.H / 8;
  int64_t cb = (n + 255) / 256;
  if (cb < 1) cb = 1;
  if (cb > 8192) cb = 8192;
  hipLaunchKernelGGL(combine_kernel, dim3(cb), dim3(256), 0, stream, p.y, p.route_slot, p.out, p.m, p.topk, int64_t(p.g.H));
}

}  // namespace moe
