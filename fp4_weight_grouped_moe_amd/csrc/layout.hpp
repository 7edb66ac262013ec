// Geometry of the prepared weight buffer and of the fused-layer workspace.
// Host and device code both use these plain structs; every size is computed here once.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace moe {

constexpr int kRowGroup = 16;     // rows per MFMA fragment (v_mfma_f32_16x16x32_bf16: M = 16)
constexpr int kKBlock = 128;      // K elements per fragment block: 4 MFMA K-steps of 32
constexpr int kFragBytes = 1024;  // one 16 x 128 fragment block of E2M1 nibbles (64 lanes x 16 B)
constexpr int kScaleChunkKB = 4;  // K-blocks whose scales one lane reads with a 128-bit load
constexpr int kBlockM = 16;       // route block used by the fused layer
constexpr int kTileBlocks = 8;    // route blocks per grouped-GEMM M tile (128 rows)
constexpr int kMaxExperts = 2048; // LDS histogram bound of the single-workgroup route packer
constexpr int kMaxTopk = 64;

enum Fmt : int32_t { FMT_NVFP4 = 1, FMT_MXFP4 = 2 };
enum Act : int32_t { ACT_SWIGLU = 1, ACT_RELU2 = 2 };

__host__ __device__ constexpr inline int64_t round_up(int64_t a, int64_t b) { return (a + b - 1) / b * b; }
__host__ __device__ constexpr inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
__host__ __device__ constexpr inline size_t align256(size_t a) { return (a + 255) & ~size_t(255); }

// Prepared weights. Region order: FC1 nibbles, FC1 scales, FC2 nibbles, FC2 scales, g13, g2,
// FC1 row-norm bounds.
//  FC1 nibbles [E][n1_groups][hp/128][64 lanes][16 B]; lane l of a block holds, in dword s
//  (s = 0..3), the 8 codes of row 16*rg + l%16 at K = 128*kb + 32*s + 8*(l/16) + j, code j
//  in bits 4j..4j+3 -- exactly the A/B operand order of a 16x16x32 MFMA step s.
//  FC1 scales [E][n1_groups][ceil(kb/4)][...]: per chunk of 4 K-blocks,
//    NVFP4: 512 B = [h 2][row 16][kb%4][s 4], byte = scale of group 8*kb + 2*s + h;
//    MXFP4: 256 B = [row 16][kb%4][s 4],     byte = scale of group 4*kb + s.
//  SwiGLU row groups are interleaved: rg 2g = gate rows 16g.., rg 2g+1 = up rows 16g...
//  FC1 row-norm bounds [E][2] fp32 (NVFP4; zero for MXFP4): the largest Euclidean norm of a
//  dequantised gate row and of an up row (global scale excluded); relu2 stores its largest row
//  norm in both.
struct PreparedGeom {
  int32_t fmt, act, E, H, I;
  int64_t hp, ip;           // H and I rounded up to 128
  int64_t n1_groups;        // FC1 row groups: 2*ip/16 (SwiGLU) or ip/16 (relu2)
  int64_t n2_groups;        // FC2 row groups: hp/16
  int64_t kb1, kb2;         // K blocks of FC1 (hp/128) and FC2 (ip/128)
  int64_t sc_chunk_bytes;   // 512 (NVFP4) or 256 (MXFP4)
  int64_t sc1_per_group, sc2_per_group;  // scale bytes per row group
  size_t off_nib1, off_sc1, off_nib2, off_sc2, off_g13, off_g2, off_n13, total;
};

__host__ __device__ inline PreparedGeom make_prepared_geom(int32_t fmt, int32_t act, int32_t E, int32_t H,
                                                           int32_t I) {
  PreparedGeom g{};
  g.fmt = fmt; g.act = act; g.E = E; g.H = H; g.I = I;
  g.hp = round_up(H, kKBlock);
  g.ip = round_up(I, kKBlock);
  g.n1_groups = (act == ACT_SWIGLU ? 2 : 1) * g.ip / kRowGroup;
  g.n2_groups = g.hp / kRowGroup;
  g.kb1 = g.hp / kKBlock;
  g.kb2 = g.ip / kKBlock;
  g.sc_chunk_bytes = (fmt == FMT_NVFP4) ? 512 : 256;
  g.sc1_per_group = ceil_div(g.kb1, kScaleChunkKB) * g.sc_chunk_bytes;
  g.sc2_per_group = ceil_div(g.kb2, kScaleChunkKB) * g.sc_chunk_bytes;
  size_t o = 0;
  g.off_nib1 = o; o = align256(o + size_t(E) * g.n1_groups * g.kb1 * kFragBytes);
  g.off_sc1 = o;  o = align256(o + size_t(E) * g.n1_groups * g.sc1_per_group);
  g.off_nib2 = o; o = align256(o + size_t(E) * g.n2_groups * g.kb2 * kFragBytes);
  g.off_sc2 = o;  o = align256(o + size_t(E) * g.n2_groups * g.sc2_per_group);
  g.off_g13 = o;  o = align256(o + size_t(E) * 4);
  g.off_g2 = o;   o = align256(o + size_t(E) * 4);
  g.off_n13 = o;  o = align256(o + size_t(E) * 8);
  g.total = o;
  return g;
}

// Route-pack capacities for a token capacity.
struct PackGeom {
  int64_t cap, k, E, B;
  int64_t cap_routes, cap_blocks;
  size_t off_counts, off_offsets, off_sorted, off_block_expert, off_live, off_route_slot;
  size_t off_tiles, off_tok_of_slot, total;
};

__host__ __device__ inline PackGeom make_pack_geom(int64_t cap, int64_t k, int64_t E, int64_t B) {
  PackGeom p{};
  p.cap = cap; p.k = k; p.E = E; p.B = B;
  int64_t routes = cap * k;
  int64_t bound = routes + (E < routes ? E : routes) * (B - 1);
  p.cap_routes = round_up(bound, B);
  if (p.cap_routes < B) p.cap_routes = B;
  p.cap_blocks = p.cap_routes / B;
  size_t o = 0;
  p.off_counts = o;       o = align256(o + size_t(E) * 4);
  p.off_offsets = o;      o = align256(o + size_t(E + 1) * 4);
  p.off_sorted = o;       o = align256(o + size_t(p.cap_routes) * 4);
  p.off_block_expert = o; o = align256(o + size_t(p.cap_blocks) * 4);
  p.off_live = o;         o = align256(o + 64 * 4);  // [0..3] public, [4] M tiles, [5] full ones, [8..23] GEMM queues
  p.off_route_slot = o;   o = align256(o + size_t(routes) * 4);
  // fused-layer extras: M-tile table (first block, block count) and token + weight per slot
  p.off_tiles = o;        o = align256(o + size_t(p.cap_blocks) * 8);
  p.off_tok_of_slot = o;  o = align256(o + size_t(p.cap_routes) * 8);
  p.total = o;
  return p;
}

constexpr int kDecodeMaxM = 16;          // token columns of the decode path
constexpr int kDecodeStageBytes = 131072; // LDS for the decode FC1 staged activation rows (128 KiB)

// Decode FC1 keeps the activation rows in LDS when they fit, at a pitch of hp rounded up to
// 512 elements (whole 1 KiB rows of LDS DMA); up to 64 KiB of rows two workgroups share a
// CU, beyond that one. With NVFP4 weights the staged rows are the f16 copy made by the
// route-pack launch.
inline int64_t decode_x_pitch(const PreparedGeom& g) { return (g.hp + 511) / 512 * 512; }
inline bool decode_stages_x(const PreparedGeom& g, int64_t m) { return m * decode_x_pitch(g) * 2 <= kDecodeStageBytes; }

// Fused-layer workspace: route pack (block 16), 16-bit intermediate rows per packed slot (bf16;
// f16 times a per-slot power of two on the NVFP4 grouped-GEMM path), the f16 copy of the
// activations with per-token exponents and sums of squares (NVFP4), for the grouped-GEMM path
// the bf16 FC2 row of every route, summed over top-k by the combine pass, and for the
// decode path the fp32 FC2 partial sums of each K split with their arrival counts.
struct FusedGeom {
  PackGeom pack;
  size_t off_pack, off_inter, off_inter32, off_inter8, off_sc8, off_x16, off_xexp, off_xss, off_sexp, off_y, off_part,
      off_count, total;
};

__host__ __device__ inline FusedGeom make_fused_geom(const PreparedGeom& w, int64_t cap, int64_t k) {
  FusedGeom f{};
  f.pack = make_pack_geom(cap, k, w.E, kBlockM);
  size_t o = 0;
  f.off_pack = o;  o = align256(o + f.pack.total);
  f.off_inter = o; o = align256(o + size_t(f.pack.cap_routes) * w.ip * 2);
  // W4A8 (MXFP4 weights) on the decode path: FC1's fp32 activation output, rounded to MXFP8
  // after FC1
  const bool dec = cap <= kDecodeMaxM;
  f.off_inter32 = o; o = align256(o + (w.fmt == FMT_MXFP4 && dec ? size_t(f.pack.cap_routes) * w.ip * 4 : 0));
  // W4A8: the MXFP8 codes and E8M0 scale bytes that the block-scaled FC2 multiplies
  const bool w8 = w.fmt == FMT_MXFP4;
  f.off_inter8 = o; o = align256(o + (w8 ? size_t(f.pack.cap_routes) * w.ip : 0));
  f.off_sc8 = o;    o = align256(o + (w8 ? size_t(f.pack.cap_routes) * (w.ip / 32) : 0));
  f.off_x16 = o;   o = align256(o + size_t(cap) * w.H * 2);
  f.off_xexp = o;  o = align256(o + size_t(cap) * 4);
  // NVFP4 grouped GEMM: each f16 row's sum of squares, and the exponent of each slot's f16
  // intermediate row
  f.off_xss = o;   o = align256(o + size_t(cap) * 4);
  f.off_sexp = o;  o = align256(o + size_t(f.pack.cap_routes) * 4);
  f.off_y = o;     o = align256(o + size_t(cap) * k * w.H * 2);
  // decode FC2 partial sums: one fp32 [cap, H] slab per pair of intermediate K blocks
  f.off_part = o;  o = align256(o + (cap <= kDecodeMaxM ? size_t((w.kb2 + 1) / 2) * cap * w.H * 4 : 0));
  f.off_count = o; o = align256(o + (cap <= kDecodeMaxM ? size_t(w.n2_groups) * 4 : 0));
  f.total = o;
  return f;
}

}  // namespace moe
