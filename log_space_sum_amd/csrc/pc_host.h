// pc_host.h -- the compiled layout held by a pc_handle, and the host-side
// helpers shared by the layout compiler, the pass scheduler and the kernel
// launchers.
#pragma once
#include <stdint.h>

#include <string>
#include <vector>

#include "../../include/pc.h"
#include "pc_device.h"

namespace pc {

// Error raised inside the library; converted to a status code at the C ABI.
struct Error {
  int code;
  std::string msg;
};
[[noreturn]] void fail(int code, const std::string& msg);

// Product kinds whose operand split is configurable.
enum GemmKind { GK_FWD = 0, GK_ELEM = 1, GK_PARAM = 2 };

struct InputPlan {
  int layer;
  int32_t node_start, num_nodes, num_cats, num_rows;
  int64_t param_offset;
  std::vector<int32_t> var, row;
  std::vector<int32_t> row_ptr, row_nodes;  // row -> nodes using it (ascending)
  int32_t max_row_nodes = 0;                 // most nodes sharing one parameter row
  std::vector<int32_t> var_ptr, var_nodes;   // variable -> layer-local node indices (ascending)
  int32_t max_var_nodes = 0;
  int32_t* d_var_ptr = nullptr;
  int32_t* d_var_nodes = nullptr;
  int32_t* d_var = nullptr;
  int32_t* d_row = nullptr;
  int32_t* d_row_ptr = nullptr;
  int32_t* d_row_nodes = nullptr;
};

struct ProductPlan {
  int layer;
  int32_t node_start, num_nodes;
  std::vector<int32_t> ch_ptr, ch_ids;
  std::vector<int32_t> uchild, pptr, parents;  // distinct children, their parents (CSR)
  bool store = false;                          // flows: first writer of every child
  int32_t max_deg = 0;                         // most children of one node
  // Affine layer: every node has max_deg <= 8 children, child q of node i is
  // abase[q] + i, and the max_deg child ranges are disjoint (so each child
  // has exactly one parent); addresses then need no index loads.
  bool affine = false;
  int32_t abase[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  bool single_parent = false;                  // every distinct child has exactly one parent here
  bool fwd_fused = false;                      // forward computed by the next sum layer's column-max kernel
  bool bwd_fused = false;                      // backward computed by the previous sum layer's flow packing
  int32_t* d_ch_ptr = nullptr;
  int32_t* d_ch_ids = nullptr;
  int32_t* d_uchild = nullptr;
  int32_t* d_pptr = nullptr;
  int32_t* d_parents = nullptr;
};

struct SumPlan {
  int layer;
  int cls;
  std::vector<GroupRec> groups;
  std::vector<int32_t> blocks;                 // concatenated child-block starts
  bool overlap = false;                        // a child is used by several groups
  bool store = false;                          // flows: first writer of every child
  bool lowrank = false;
  int32_t ebt_cols = 0, gbt_cols = 0;          // widths of the batch-major operands
  int32_t mtiles = 0, ctiles = 0;              // 128-row tiles over outputs / children
  int32_t pktiles = 0, pgtiles = 0;            // 64-row tiles over source children / outputs
  int32_t scratch_rows = 0;
  int32_t max_npk = 0, max_mpk = 0;            // widest contraction of the forward / element flows
  std::vector<int32_t> red_child, red_ptr, red_src;   // overlap reduction CSR
  std::vector<int64_t> lr_row;                 // LowRank: first row of each group's Z/S/U/W records
  std::vector<int32_t> lr_gidx;                // LowRank: index of each group among all LowRank groups
  // Adjacent product layers computed inside this layer's memory-bound kernels:
  // the one before it in the column-max kernel (forward), the one after it in
  // the scaled-flow packing (backward).
  int fwd_prod = -1, bwd_prod = -1;
  // Forward product epilogue: this layer's forward product (LowRank layers:
  // the kernel that writes their node values) also evaluates the
  // affine product layer epi_prod that follows it (its nodes i take child
  // epi_qs, abase[epi_qs] + i, from this layer's outputs; their other
  // children come from earlier layers) and publishes the column maxima of the
  // next sum layer, whose one group's children are exactly those product
  // nodes (keys row epi_mrow).  That layer then skips its column-max launch
  // (epi_max).
  int epi_prod = -1, epi_qs = -1, epi_mrow = -1;
  bool epi_max = false;
  int epi_src = -1;                                // the sum layer publishing this layer's maxima
  // Element-flow product epilogue: this layer's element-flow product also does
  // the scaled-flow packing of sum layer gp_sum (the backward of the affine
  // two-child product layer gp_prod between them: the product node's flow
  // goes to both its children, g = f / S of gp_sum's nodes into both operand
  // layouts).  gp_sum's own packing launch is then skipped (gp_done), when the
  // batch is a multiple of 256 (no padded samples in either layout).
  int gp_sum = -1, gp_prod = -1, gp_qs = -1;
  bool gp_done = false;
  // LowRank layer: the affine two-child product layer lr_prod after it, fed by
  // its outputs as child lr_qs, runs its backward in this layer's coefficient
  // kernel (the node's flow copied to both children before f / S, f / Z).
  int lr_prod = -1, lr_qs = -1;
  // Batch-major G buffer of the layer while those epilogues run: a layer whose
  // G is written during the next layer's element-flow product uses the other
  // buffer than that product's operand.
  int gbt_slot = 0;
  // Per 64-row output tile row: the parent node in bwd_prod when that layer
  // gives each child a single parent, else the distinct-child index; -1 when
  // the output is not a child of bwd_prod.
  std::vector<int32_t> up_idx;
  // bwd_prod's distinct children that are not outputs of this layer: child
  // node and its single parent, or the distinct-child index (and -1).
  std::vector<int32_t> up_rest, up_rest_par;
  // Per 64-row child tile / output tile: its group (the last group whose
  // pk_start / pg_start is at most the tile), so kernels need no search.
  std::vector<int32_t> pk_group, pg_group;
  int32_t* d_pk_group = nullptr;
  int32_t* d_pg_group = nullptr;
  int32_t* d_up_idx = nullptr;
  int32_t* d_up_rest = nullptr;
  int32_t* d_up_rest_par = nullptr;
  GroupRec* d_groups = nullptr;
  int32_t* d_blocks = nullptr;
  int32_t* d_red_child = nullptr;
  int32_t* d_red_ptr = nullptr;
  int32_t* d_red_src = nullptr;
};

struct LayerRef {
  int kind;
  int idx;   // index into inputs / prods / sums (-1 for external)
};

struct Handle {
  int device = -1;
  int mode = PC_PREC_AUTO;
  // planes[mode][gemm kind][0: first operand, 1: second operand]
  // auto: forward (2,2), element flows (2,2), parameter flows (2,1); fp32-level (3,3)
  int planes[2][3][2] = {{{2, 2}, {2, 2}, {2, 1}}, {{3, 3}, {3, 3}, {3, 3}}};
  int opt_layer_tile = 0, opt_param_tile = 0, opt_split_max = 8, opt_fuse = 1;   // pc_set_option
  int opt_param_chunk = -1;            // tied copies per parameter-flow launch (0: one launch at the end, -1: automatic)
  int opt_lr_pack = 0;                 // LowRank fragment records: 0 once per forward, 1 per layer and pass
  std::vector<std::vector<int32_t>> copy_layer;   // per weight block: the layer of each tied copy
  void* side_stream = nullptr;         // parameter-flow chunks run here, beside the element flows
  std::vector<void*> chunk_events;
  int32_t num_nodes = 0, num_vars = 0, root = -1, lowrank_rank = 0;
  int32_t lowrank_form = PC_LOWRANK_EXP_SUM;
  int64_t num_params = 0;
  std::vector<LayerRef> layers;
  std::vector<InputPlan> inputs;
  std::vector<ProductPlan> prods;
  std::vector<SumPlan> sums;
  std::vector<BlockRec> blocks;
  int32_t pk_block_tiles = 0;          // 64x64 tiles over all blocks (weight split)
  int32_t param_tiles256 = 0, param_tiles128 = 0;   // product tiles over all blocks (parameter flows)
  int64_t min_block_dim = 1 << 30;     // smallest M or N of a plain block
  int32_t max_sum_groups = 0;
  int64_t theta_elems = 0, thetaT_elems = 0;
  int64_t earena_rows = 0, garena_rows = 0, s_rows = 0;
  int32_t m_rows = 0;
  int32_t max_ebt_cols = 0, max_gbt_cols = 0, max_scratch_rows = 0;
  int gbt_slots = 1;                                   // 2 when an element-flow product epilogue packs G
  int32_t max_cats = 0;
  int32_t lowrank_slots = 0;
  int64_t lr_rows = 0;                 // LowRank: rows of the kept Z/S/U/W records (sum of group M)
  int32_t lr_max_m = 0;                // LowRank: largest group M (per-layer coefficients)
  int32_t lr_max_n = 0;                // LowRank: largest group N
  int32_t lr_groups = 0;               // LowRank: number of LowRank groups
  int64_t lr_p_elems = 0;              // LowRank: elements of the distinct LowRank weight blocks
  std::vector<int64_t> lr_p_off;       // per weight block: offset of its LowRank partials, -1 if none
  // LowRank "sum_exp" on a virtual batch (used unless opt_sumexp_fused):
  // one block record per distinct LowRank weight block, with its weight
  // planes after the plain blocks' (th_off, tht_off), the node-major rows of
  // its copies' virtual operands (X = exp(B) e and C = exp(B) at e_base +
  // copy * N_pad; Y1 = exp(A) c1 and Y2 = exp(A) c2 at g_base + copy * M_pad)
  // and its parameter-flow tile prefixes; and one group record per LowRank
  // group (index lr_gidx): that copy's block and operand rows.
  std::vector<BlockRec> vblocks;
  std::vector<GroupRec> vgroups;
  std::vector<std::vector<int32_t>> vcopy_layer;   // per virtual block: the layer of each copy
  int32_t v_pk_tiles = 0, v_param_tiles256 = 0, v_param_tiles128 = 0;
  int64_t vx_rows = 0, vy_rows = 0;                // node-major rows of the X / C and Y1 / Y2 arenas
  int32_t v_max_k = 0;                             // widest contraction of the two per-layer products
  int opt_sumexp_fused = 0;                        // 1: "sum_exp" through the fused LowRank kernels
  int opt_flow_fp8 = 0;                            // 1: "sum_exp" end products from e4m3 operands (auto)
  BlockRec* d_vblocks = nullptr;
  GroupRec* d_vgroups = nullptr;
  std::vector<RowSeg> rowsegs;
  int32_t total_rows = 0;
  std::vector<int32_t> outputs;
  std::vector<FillRange> zero_ranges;   // flows cleared before the backward
  std::vector<FillRange> seed_ranges;   // output flows without caller seeds: root 1, others 0
  int64_t max_zero_count = 0, max_seed_count = 0;
  bool has_plain_sums = false;
  // device copies of handle-wide tables
  BlockRec* d_blocks = nullptr;
  RowSeg* d_rowsegs = nullptr;
  FillRange* d_zero = nullptr;
  FillRange* d_seed = nullptr;
  // timing
  bool timing = false;
  bool no_events = false;              // set during a call that records no timing events (pc_forward_static)
  struct Ev {
    int kind;
    void* start;
    void* stop;
  };
  std::vector<Ev> events;
  size_t events_used = 0;
};

// Layout compiler (host only).
Handle* compile_layout(const pc_circuit_desc* d);
// Upload the handle's index tables to `device`.
void upload_tables(Handle* h, int device);
void free_tables(Handle* h);

// Effective precision mode for a batch (batches below 16 run fp32-level).
inline int effective_mode(const Handle* h, int B) { return B < 16 ? PC_PREC_FP32 : h->mode; }

// Element-flow product epilogues pack the next layer's G when fusion is on and
// the batch is a multiple of 64 (the node-major G has no padded samples; the
// epilogue masks the batch-major layout's padded ones).
inline bool gp_batch_ok(int B) { return B % 64 == 0; }
inline bool gp_active(const Handle* h, int B) { return h->opt_fuse && h->gbt_slots > 1 && gp_batch_ok(B); }

// Workspace plan for a batch: byte offsets of every region.
struct WsPlan {
  int B, B_pad, B_padK, mode;
  bool fwd_only;                                     // forward-only plan: no region the backward alone reads
  int pl[3][2];
  size_t theta, thetaT, ebt, gbt, gbt2, earena, garena, mkeys, ssum, scratch, tokT, bptr, bidx, lowrank;
  size_t lrE, lrZ, lrS, lrU, lrW, lrC1, lrC2, lrP;   // LowRank regions (float32)
  size_t lrPz;                                       // partials of the denominator statistic W
  size_t lrPK;                                       // LowRank fragment records of every LowRank group
  // LowRank "sum_exp" virtual batch: the batch-major operand of the layer's two
  // products ([Qpad rows = 2 B k padded, K] per plane), the node-major X, C, Y1,
  // Y2 arenas ([rows, QK = B k padded to 64] per plane), the backward's
  // products R1, R2 ([B, N, k] float32 each)
  bool vsum;
  int32_t Qv, Qpad, QK;
  size_t vbt, vX, vC, vY1, vY2, vR;
  bool vf8;                                        // e4m3 end products: the node-major operands below
  size_t vX8, vC8, vY18, vY28, vXs, vCs, vY1s, vY2s;
  std::vector<int64_t> lr_pk_off;                    // per LowRank group: byte offset of its records
  int lr_nsg;                                        // LowRank parameter-flow partials: ceil(B/8)
  size_t partials, counters;
  int64_t partial_elems;
  int32_t ncounters;
  // split-K state of the parameter-flow products (their own: those can run on
  // the second stream beside split-K per-layer products)
  size_t ppartials, pcounters;
  int32_t npcounters;
  size_t lowrank_bytes;
  size_t total;
};
WsPlan plan_workspace(const Handle* h, int B, bool fwd_only = false);
WsView make_view(const Handle* h, const WsPlan& p, void* ws);

}  // namespace pc
