// pc_elem.h -- argument blocks and launchers of the memory-bound kernels.
#pragma once
#include <hip/hip_runtime.h>

#include "pc_device.h"
#include "pc_launch.h"

namespace pc {

struct InputArgs {
  int32_t B, node_start, num_nodes, K, num_rows, Kmax, max_row_nodes;
  int32_t num_vars, max_var_nodes;
  const int32_t* var_ptr;       // variable -> layer-local nodes (CSR, ascending)
  const int32_t* var_nodes;
  int64_t param_offset;
  const int32_t* var;
  const int32_t* row;
  const int32_t* row_ptr;
  const int32_t* row_nodes;
  const int32_t* tokT;
  const int32_t* bptr;
  const int32_t* bidx;
  const float* params;
  float* vals;
  const float* flows;
  float* pflows;
};

struct ProdArgs {
  int32_t B, node_start, num_nodes, nuniq, store;
  int32_t affine, deg;          // affine layer: child q of node i is abase[q] + i
  int32_t abase[8];
  const int32_t* ch_ptr;
  const int32_t* ch_ids;
  const int32_t* uchild;
  const int32_t* pptr;
  const int32_t* parents;
  float* vals;
  float* flows;
};

struct SumArgs {
  int32_t B, B_pad, B_padK, btiles, ngroups;
  const GroupRec* groups;
  GroupRec group0;          // a copy of the layer's only group when ngroups == 1 (no table read)
  const int32_t* pk_group;  // group of each 64-row child tile (column maxima, exp packing)
  const int32_t* pg_group;  // group of each 64-row output tile (scaled-flow packing)
  const int32_t* chblocks;
  const float* vals;
  const float* flows;
  uint32_t* mkeys;
  const float* ssum;
  // packed outputs: node-major ("direct", rows x B_padK) and batch-major ("trans")
  uint16_t* direct;
  int64_t direct_plane;
  int32_t np_direct;
  uint16_t* trans;
  int64_t trans_plane;
  int64_t direct_rows;      // panel rows of the node-major output
  int32_t np_trans;
  // overlapping-children reduction
  int32_t nuniq, store;
  const int32_t* red_child;
  const int32_t* red_ptr;
  const int32_t* red_src;
  const float* scratch;
  float* out_flows;
  // A product layer computed in the same launch.  Forward (column maxima):
  // children of the sum layer inside [fp_start, fp_start + fp_count) are that
  // layer's nodes, summed from their own children (fp_ptr / fp_ids = its
  // child CSR, at most fp_maxdeg each) and written to wvals.  Backward
  // (scaled flows): output row r of the packing tiles takes its flow from the
  // product layer's parents when fp_up[r] >= 0 (the single parent node when
  // fp_single, else a distinct-child index into the parent CSR fp_ptr /
  // fp_ids over fp_uchild; stored to wflows, added to the old flow unless
  // fp_store), and the workgroups past the fp_tiles packing tiles handle the
  // fp_nrest other distinct children fp_rest (child node with its parent
  // fp_rest_par when fp_single, else distinct-child indices).  fp_affine:
  // the product layer is affine (child q of node i at fp_abase[q] + i).
  int32_t fp_on, fp_start, fp_count, fp_maxdeg, fp_store, fp_nrest, fp_tiles, fp_affine, fp_single;
  int32_t fp_abase[8];
  const int32_t* fp_ptr;
  const int32_t* fp_ids;
  const int32_t* fp_uchild;
  const int32_t* fp_up;
  const int32_t* fp_rest;
  const int32_t* fp_rest_par;
  float* wvals;
  float* wflows;
};

struct ThetaArgs {
  int32_t nblocks, np_fwd, np_elem;
  const BlockRec* blocks;
  const float* params;
  uint16_t* theta;
  int64_t theta_plane;
  uint16_t* thetaT;
  int64_t thetaT_plane;
};

struct EmArgs {
  int32_t nsegs;
  const RowSeg* segs;
  float* params;
  const float* pflows;
  const float* zflows;   // LowRank denominator statistic (conditional M-step), or null
  float step, pseudo;
};

// One LowRank exp_sum group (k_lowrank.hip).  Row-major weights theta [M, N];
// factors A [B, M, krank], Bf [B, krank, N] (the slot's tensors); Z, S: [B, M]
// kept by the forward; U, W: [B, M, krank] kept by the forward; C1, C2: [B, M
// rounded up to 32] (zero past M); P: the group's block of ceil(B/8)
// parameter-flow partials [ceil(B/8), M, N]; pk: the group's fragment records
// of the factors (lr_pack_bytes), made by the forward's pack launch.
struct LRArgs {
  int32_t B, M, N, krank;
  int32_t out_start, m_row, cbs, blk_off, scratch_row, store;
  // coefficients: the following product layer's backward first (fp_on): the
  // flow of product node fp_pstart + i goes to output i and to node fp_other + i
  int32_t fp_on, fp_pstart, fp_other;
  // forward: the following affine two-child product layer evaluated with the
  // node values (ep_on): output node n is child ep_qs of product node
  // q = n - ep_base_s when 0 <= q < ep_pcount, whose other child is
  // ep_base_o + q; the product value goes to node ep_pstart + q and its
  // per-sample maximum to keys row ep_mrow (the next sum layer's shift)
  int32_t ep_on, ep_qs, ep_base_s, ep_base_o, ep_pstart, ep_pcount, ep_mrow;
  uint32_t* mkeys_out;
  int32_t sumexp;        // the "sum_exp" form (records of exp(A), exp(B))
  const int32_t* chblocks;
  const float* theta;
  const float* A;
  const float* Bf;
  const uint32_t* mkeys;
  float* vals;
  const float* flows;
  float* out_flows;
  float* scratch;
  float* Z;
  float* S;
  float* U;
  float* W;
  float* C1;
  float* C2;
  float* P;
  float* dA;
  float* dB;
  uint16_t* pk;
};

// Fragment packing of up to kMaxPackGroups LowRank groups in one launch:
// group g takes workgroups [wg0[g], wg0[g + 1]).
constexpr int kMaxPackGroups = 48;
struct LRPackArgs {
  int32_t B, krank, ngroups;
  int32_t sumexp;                  // records of exp(A), exp(B) ("sum_exp" form)
  int32_t M[kMaxPackGroups], N[kMaxPackGroups];
  int32_t wg0[kMaxPackGroups + 1];
  const float* A[kMaxPackGroups];
  const float* Bf[kMaxPackGroups];
  uint16_t* pk[kMaxPackGroups];
};

// Bytes of the fragment records of one group's factors.
int64_t lr_pack_bytes(int B, int M, int N, int krank, int fp32);
// Workgroups of one group's packing.
int lr_pack_workgroups(int B, int M, int N, int krank);
void launch_lr_pack(const LRPackArgs& pa, int fp32, hipStream_t s);
// Backward per layer: c1, c2 and dLL/dA.
void launch_lr_coef(const LRArgs& a, hipStream_t s);
void launch_lr_fwd(const LRArgs& a, int fp32, hipStream_t s);
void launch_lr_bwd(const LRArgs& a, int fp32, hipStream_t s);
// The denominator statistic W of the conditional M-step into the partials at a.P.
void launch_lr_zstat(const LRArgs& a, int fp32, hipStream_t s);
void launch_lr_fplus(const float* P, int nsg, int64_t elems, float* pflows, hipStream_t s);

// One LowRank "sum_exp" group on the virtual batch (k_vbatch.hip): Q = B k
// virtual columns q = b k + r; the batch-major operand vbt has Qpad rows
// (rows [0, Q) and [Q, 2Q) the two halves) and the node-major arenas
// nlo / nhi (X / C forward, Y1 / Y2 backward) rows n_row0 + node of n_rows,
// K = q padded to QK; np_bt / np_n bfloat16 planes (np_n = 0: not kept).
struct VBArgs {
  int32_t B, M, N, krank, Q, Qpad, QK;
  int32_t out_start, m_row, cbs, blk_off, scratch_row, store;
  const int32_t* chblocks;
  const float* A;          // [B, M, k]
  const float* Bf;         // [B, k, N]
  const uint32_t* mkeys;
  float* vals;
  float* out_flows;
  float* scratch;
  uint16_t* vbt;
  int64_t vbt_plane;
  int32_t np_bt;
  uint16_t* nlo;
  uint16_t* nhi;
  int64_t n_plane, n_rows, n_row0;
  int32_t np_n;
  // e4m3 node-major operands instead of the bf16 planes (f8 = 1): bytes in
  // 64-wide K-blocked panels of n_rows rows, one power-of-two scale byte per
  // row and 32 consecutive K at (k / 32) * n_rows + row
  int32_t f8;
  uint8_t* n8lo;
  uint8_t* n8hi;
  uint8_t* s8lo;
  uint8_t* s8hi;
  const float* C1;         // [B, M rounded up to 32] f / S, f / Z
  const float* C2;
  float* S;                // [B, M]
  float* Z;
  const float* U;          // [B, M, k] theta X^T, theta C^T (kept: the coefficient kernel's U, W)
  const float* W;
  const float* R1;         // [B, N, k] theta^T Y1^T, theta^T Y2^T
  const float* R2;
  float* dB;               // [B, k, N]
};
void launch_vb_fwd_pack(const VBArgs& a, hipStream_t s);
void launch_vb_fwd_reduce(const VBArgs& a, hipStream_t s);
void launch_vb_bwd_pack(const VBArgs& a, hipStream_t s);
void launch_vb_bwd_reduce(const VBArgs& a, hipStream_t s);

void launch_fill_u32(uint32_t* p, int64_t n, uint32_t v, hipStream_t s);
void launch_fill_ranges(float* flows, const FillRange* d_ranges, int nranges, int64_t max_count, int B,
                        hipStream_t s);
void launch_copy_row(const float* src, float* dst, int B, hipStream_t s);
void launch_tokens_t(const int32_t* tok, int32_t* tokT, int B, int V, hipStream_t s);
void launch_input_fwd(const InputArgs& a, hipStream_t s);
void launch_bucket(const int32_t* tokT, int V, int B, int Kmax, int32_t* bptr, int32_t* bidx, hipStream_t s);
void launch_input_bwd(const InputArgs& a, hipStream_t s);
void launch_prod_fwd(const ProdArgs& a, hipStream_t s);
void launch_prod_bwd(const ProdArgs& a, hipStream_t s);
void launch_colmax(const SumArgs& a, int row_tiles, hipStream_t s);     // row_tiles: 64-child packing tiles
void launch_exp_pack(const SumArgs& a, int row_tiles, hipStream_t s);
void launch_g_pack(const SumArgs& a, int row_tiles, hipStream_t s);
void launch_theta_pack(const ThetaArgs& a, int tiles, hipStream_t s);
void launch_elem_reduce(const SumArgs& a, hipStream_t s);
void launch_em(const EmArgs& a, int rows, hipStream_t s);

}  // namespace pc
