// pc_kernels.h -- launchers of the gfx950 kernels (host side).
#pragma once
#include <hip/hip_runtime.h>

#include "pc_device.h"
#include "pc_launch.h"

namespace pc {

enum Epi { EPI_FWD = 0, EPI_ELEM = 1, EPI_PARAM = 2, EPI_VSTORE = 3 };

// Arguments of the MFMA product kernel (see k_gemm.hip).
struct GemmArgs {
  int32_t B, B_pad, B_padK;
  int64_t rowsA, rowsB;        // panel rows of the kept operands (parameter flows)
  int32_t ntiles;               // tiles along the batch (forward / element flows)
  int32_t splitk;               // workgroups sharing one tile's K range (forward / element flows)
  int32_t ngroups;              // groups of the layer, or blocks (parameter flows)
  const GroupRec* groups;
  const BlockRec* blocks;
  const int32_t* chblocks;      // the layer's child-block starts
  const uint16_t* opA;
  int64_t planeA;
  const uint16_t* opB;
  int64_t planeB;
  int32_t ldb;                  // row stride of the batch-major operand (forward / element flows)
  float* vals;                  // node values (written by forward, read by element flows)
  float* flows;                 // node flows
  float* scratch;               // element-flow scratch of overlapping layers
  const uint32_t* mkeys;        // column-max keys
  uint32_t* mkeys_out;          // the same keys, published by a product epilogue
  float* ssum;                  // scaled sums kept by the forward
  int32_t store;                // element flows: store instead of add
  const float* params;
  float* pflows;
  float* partials;              // split-K partial tiles
  uint32_t* counters;           // split-K arrival counters, zero between launches
  // parameter flows: tied copies [copy_lo, copy_hi) of each block; the launch
  // covers product tiles tile0 .. tile0 + grid - 1 of the block sequence
  int32_t copy_lo, copy_hi, tile0;
  // forward: the following affine two-child product layer evaluated in the
  // epilogue (ep_on).  Output node n is child ep_qs of product node
  // i = n - ep_base_s when 0 <= i < ep_pcount; i's other child is
  // ep_base_o + i; node i is stored at ep_pstart + i, and the column maxima of
  // the product nodes go to keys row ep_mrow.
  int32_t ep_on, ep_qs, ep_base_s, ep_base_o, ep_pstart, ep_pcount, ep_mrow;
  // element flows: the scaled-flow packing of the sum layer below the
  // following product layer, done in the epilogue (gp_on).  Output row j (a
  // product node, child j of this layer) passes its flow f to node
  // gp_out_start + j of that sum layer (child gp_qs of the product node) and to
  // node gp_other + j (its other child); g = f / S (S at row gp_s_row + j of
  // the kept scaled sums) goes to node-major rows gp_g_row + j (gp_np_direct
  // planes) and to batch-major columns gp_g_koff + j (gp_np_trans planes).
  int32_t gp_on, gp_qs, gp_out_start, gp_other, gp_np_direct, gp_np_trans, gp_g_koff;
  int64_t gp_s_row, gp_g_row, gp_direct_rows, gp_direct_plane, gp_trans_plane;
  uint16_t* gp_direct;
  uint16_t* gp_trans;
  // plain-store products of the LowRank "sum_exp" virtual batch (EPI_VSTORE):
  // the one group's weights (vs_elem 0: theta, rows M, K = N; 1: theta^T,
  // rows N, K = M) times the batch-major operand whose B (= 2 Q) rows are the
  // virtual columns q' = b * k + r (q' < Q) and Q + b * k + r; output (row,
  // q') goes to vs_lo (q' < Q) or vs_hi at [b][row][r] (rows of the product,
  // rank vs_rank)
  int32_t vs_elem, vs_rank, vs_half;
  float* vs_lo;
  float* vs_hi;
};

// The LowRank "sum_exp" parameter-flow products from e4m3 operands
// (k_f8gemm.hip): node-major operand panels of 64-byte K blocks, one E8M0
// scale per row and 32 consecutive K, 128 x 128 output tiles counted by the
// blocks' pt128 prefix, the contraction over every tied copy (copy s of a
// block at rows g_base + s * M_pad of A and e_base + s * N_pad of B).
struct F8Args {
  const uint8_t* A;
  const uint8_t* sA;
  int64_t rowsA;
  const uint8_t* B;
  const uint8_t* sB;
  int64_t rowsB;
  int32_t QK;                   // K of one copy (a multiple of 64)
  int32_t nblocks;
  const BlockRec* blocks;
  const float* params;          // F+ = theta * product; null: W = product
  float* out;                   // accumulated at each block's param_offset, rows of N
  int32_t splitk;
  float* partials;              // [tiles][splitk][128 x 128]
  uint32_t* counters;           // one per tile, zero between launches
};
void launch_f8param(const F8Args& a, int tiles, hipStream_t s);

// Output tile shapes of the product kernel (M x N per workgroup).
enum GemmTile { TILE_AUTO = 0, TILE_128x128 = 1, TILE_256x128 = 2, TILE_256x256 = 3, TILE_128x256 = 4, TILE_128x64 = 5, TILE_64x128 = 6 };

struct GemmShape {
  int tile;      // GemmTile
  int mt, nt;    // tile rows / columns
  int splitk;    // workgroups sharing one tile's K range (forward / element flows)
  int tiles;     // output tiles of the launch
};

// K slice width: 32.  Narrow slices give the ring more stages, so more bytes
// are in flight per CU (measured faster than 64-wide slices on every product
// of the HMM-4096 step: the loads, not the matrix instructions, set the pace).
constexpr int gemm_kt(int pa, int pb, int mt, int nt) { return 32; }
// LDS ring stages (at most 6) that fit 160 KB with 2 KB to spare.
constexpr int gemm_stages(int pa, int pb, int mt, int nt) {
  return ((160 - 2) * 1024) / ((pa * mt + pb * nt) * gemm_kt(pa, pb, mt, nt) * 2) > 6
             ? 6
             : ((160 - 2) * 1024) / ((pa * mt + pb * nt) * gemm_kt(pa, pb, mt, nt) * 2);
}

// Ring stages when the weights go straight to registers (forward, element-flow
// and virtual-batch products): the ring holds B only, and the registers hold
// one slice of weights per stage (pa * fm * 8 per lane: at most about 128 in
// all); 3 to 8 stages, within 160 KB of LDS.
constexpr int gemm_stages_direct(int pa, int pb, int mt, int nt, int fm) {
  const int by_regs = 16 / (pa * fm) < 3 ? 3 : 16 / (pa * fm) > 8 ? 8 : 16 / (pa * fm);
  const int by_lds = ((160 - 2) * 1024) / (pb * nt * gemm_kt(pa, pb, mt, nt) * 2);
  return by_regs < by_lds ? by_regs : by_lds;
}

// Shape of a forward / element-flow launch over a layer whose outputs span
// `rows256` 256-row blocks, batch padded to B_pad, largest padded K `kpad`.
// Automatic: 8192-output tiles, 64 x 128 when the first operand has more
// planes than the second, else 128 x 64 (the shape of every automatic
// split).  A tile loads pa * MT + pb * NT elements per K step, least at
// MT / NT = pb / pa, and the per-CU request rate, not the matrix
// instructions, sets the pace (measured with both operands staged in LDS,
// 4096-node HMM layers at batch 512: 128 x 64 3% faster per step than
// 128 x 128 split in two, and at batch 128 split in four 8% faster than
// 128 x 128 split in eight; with the weights in registers the HCLT step ran
// as fast on 128 x 64 tiles as on 128 x 128 tiles for its wide levels).  The K split
// (a power of two up to split_max) grows until the launch has 256 workgroups,
// keeping >= 4 slices per split.
// Columns (samples) of the tile a forward / element-flow launch uses.
inline int layer_tile_nt(int pa, int pb, int opt_tile) {
  if (opt_tile == TILE_AUTO) opt_tile = pa > pb ? TILE_64x128 : TILE_128x64;
  return opt_tile == TILE_128x256 ? 256 : opt_tile == TILE_128x64 ? 64 : 128;
}

inline GemmShape layer_shape(int rows256, int B_pad, int kpad, int pa, int pb, int opt_tile, int split_max) {
  GemmShape g{};
  if (opt_tile == TILE_AUTO) opt_tile = pa > pb ? TILE_64x128 : TILE_128x64;
  g.tile = opt_tile == TILE_256x128 ? TILE_256x128
         : opt_tile == TILE_128x256 ? TILE_128x256
         : opt_tile == TILE_128x64 ? TILE_128x64
         : opt_tile == TILE_64x128 ? TILE_64x128 : TILE_128x128;
  g.mt = g.tile == TILE_256x128 ? 256 : g.tile == TILE_64x128 ? 64 : 128;
  g.nt = g.tile == TILE_128x256 ? 256 : g.tile == TILE_128x64 ? 64 : 128;
  g.tiles = rows256 * (256 / g.mt) * (B_pad / g.nt);
  const int ksteps = kpad / gemm_kt(pa, pb, g.mt, g.nt);
  int S = 1;
  while (g.tiles * S < 256 && S * 2 <= split_max && ksteps / (S * 2) >= 4) S *= 2;
  g.splitk = S;
  return g;
}

// Launch the product kernel with the given operand split and shape.
void launch_gemm(int epi, int pa, int pb, const GemmShape& shape, const GemmArgs& a, hipStream_t s);

}  // namespace pc
