// pc_device.h -- records and argument blocks shared by the host runtime and
// the gfx950 kernels.  Every table here is batch-independent: offsets that
// scale with the batch are stored in rows (or columns) and multiplied by the
// batch-dependent strides passed as kernel arguments.
#pragma once
#include <stdint.h>

#ifndef __HIPCC__
#ifndef __host__
#define __host__
#define __device__
#endif
#endif

namespace pc {

// Padding of every bfloat16 operand kept in the workspace: rows (the M / N
// dimensions of the products) to ROW_PAD, the contraction dimension to K_PAD.
// Operands are therefore tile-aligned and the product kernels need no bounds
// checks in their main loop; pads hold zeros.
constexpr int ROW_PAD = 256;
constexpr int K_PAD = 64;
// Operands are stored as K-blocked panels: element (r, k) of an operand with
// R (padded) rows lives at ((k / KB) * R + r) * KB + k % KB.  The rows of one
// K block are contiguous, so a tile's K slice is one contiguous run and every
// 1 KB load instruction of the product kernel reads whole cache lines.
constexpr int KB = 32;

inline int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }
__host__ __device__ inline int64_t panel(int64_t r, int64_t k, int64_t R) { return ((k >> 5) * R + r) * KB + (k & 31); }
// The weight operands of the forward and element-flow products are stored in
// matrix-instruction fragment order instead: 32-row x 32-K blocks of 1024
// elements, row-block major (ks K blocks per row block), and inside a block
// the two 16-wide K steps one after the other, each as 64 lanes x 8 values:
// lane (r % 32) + 32 h of K step s holds K s*16 + h*8 .. + 7 of row r, the A
// operand of v_mfma_f32_32x32x16_bf16.  A wave loads its 32 rows of one K
// step with one contiguous 1 KB instruction, straight into registers.
__host__ __device__ inline int64_t frag_major(int64_t r, int64_t k, int64_t ks) {
  return ((r >> 5) * ks + (k >> 5)) * 1024 + ((k >> 4) & 1) * 512 + ((r & 31) + ((k >> 3) & 1) * 32) * 8 + (k & 7);
}

// One sum group (node block) of a sum layer.
struct GroupRec {
  int32_t out_start;     // first output node
  int32_t M;             // number of sum nodes
  int32_t N;             // number of children
  int32_t cbs;           // child block size
  int32_t blk_off;       // first entry of this group's child-block starts in the layer's block array
  int32_t nblk;          // number of child blocks
  int64_t param_offset;  // row-major [M, N] weights
  int32_t block;         // distinct weight block id
  int32_t m_row;         // row of the per-sample column-max keys
  int32_t e_koff;        // column offset of the group's slice of the layer's batch-major E
  int32_t g_koff;        // column offset of the group's slice of the layer's batch-major G
  int64_t e_row;         // first row of the group's node-major E (kept for parameter flows)
  int64_t g_row;         // first row of the group's node-major G (kept for parameter flows)
  int32_t mt_start;      // prefix of 256-row output blocks over the layer's groups (forward)
  int32_t ct_start;      // prefix of 256-row child blocks over the layer's groups (element flows)
  int32_t pk_start;      // prefix of 64-row child tiles over the layer's groups (column max, exp)
  int32_t pg_start;      // prefix of 64-row output tiles over the layer's groups (scaled flows)
  int32_t scratch_row;   // first row in the element-flow scratch (-1: write node flows directly)
  int32_t lowrank;       // LowRank slot or -1
  int32_t share_src;     // group whose E slice this group reuses (SHARED layers), or itself
  int32_t share_next;    // next group sharing this group's children (its E rows get a copy), or -1
  int32_t ch_start;      // child k is node ch_start + k when the child blocks are consecutive, else -1
  int64_t s_row;         // first row of the group's scaled sums S (kept from the forward), -1 if none
};

// One distinct weight block (tied copies share it).
struct BlockRec {
  int64_t param_offset;
  int32_t M, N;
  int64_t th_off;        // element offset of the [M_pad, N_padK] split weights (forward operand)
  int64_t tht_off;       // element offset of the [N_pad, M_padK] transposed split weights (element flows)
  int32_t ncopies;       // tied copies; copy s keeps its G rows at g_base + s*M_pad and
  int64_t g_base;        // its E rows at e_base + s*N_pad, so the parameter-flow product
  int64_t e_base;        // walks all copies as one contraction with affine addressing
  int32_t pk_start;      // prefix of 64x64 packing tiles over blocks
  int32_t pt256;         // prefix of 256x256 product tiles over blocks (parameter flows)
  int32_t pt128;         // prefix of 128x128 product tiles over blocks (parameter flows)
  int32_t pad_;
};

// Parameter row run normalised by EM.
struct RowSeg {
  int64_t offset;
  int32_t nrows;
  int32_t rlen;
  int32_t row_start;     // prefix of rows over segments
  int32_t lowrank;       // 1: a LowRank weight block (conditional M-step rows)
};

// Node range [start, start + count) with one fill value (flow seeding).
struct FillRange {
  int32_t start;
  int32_t count;
  float value;
  int32_t pad_;
};

// Batch-dependent strides and bases of the workspace, filled per call.
struct WsView {
  uint16_t* theta;      // split weights arena (planes at theta + p * theta_plane)
  uint16_t* thetaT;
  int64_t theta_plane, thetaT_plane;
  uint16_t* ebt;        // batch-major E of the current layer [B_pad, ebt_cols] per plane
  uint16_t* gbt;        // batch-major G of the current layer [B_pad, gbt_cols] per plane
  uint16_t* gbt2;       // the second G buffer (element-flow product epilogues)
  int64_t ebt_plane, gbt_plane;
  int32_t ebt_cols, gbt_cols;
  uint16_t* earena;     // node-major E rows [rows, B_padK] per plane (kept)
  uint16_t* garena;     // node-major G rows [rows, B_padK] per plane (kept)
  int64_t earena_plane, garena_plane;
  uint32_t* mkeys;      // [m_rows, B] order-preserving keys of the column maxima
  float* ssum;          // [s_rows, B] scaled sums S = sum_j theta e of every plain sum node
  float* scratch;       // [rows, B] element-flow contributions of overlapping layers
  int32_t* tokT;        // [num_vars, B] tokens transposed
  int32_t* bucket_ptr;  // [num_vars, K_max + 1]
  int32_t* bucket_idx;  // [num_vars, B]
  float* partials;      // split-K partial tiles of the current product
  uint32_t* counters;   // split-K arrival counters
  int32_t ncounters;
  int32_t B, B_pad, B_padK;
};

}  // namespace pc
