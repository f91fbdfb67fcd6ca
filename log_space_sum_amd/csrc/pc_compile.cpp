// pc_compile.cpp -- host-side layout compiler.
//
// Checks a circuit descriptor, classifies every sum layer after the PyJuice
// pull request #62, Summary item 2 (layers whose blocks share their children
// are exponentiated once; evenly strided groups run as one batched product;
// anything else is a general block-sparse layer), finds tied weight blocks,
// and plans where every operand lives in the workspace and how the backward
// pass writes element flows (first writer stores, later writers add; several
// groups sharing a child go through a scratch buffer and a fixed-order
// reduction, so the flows are deterministic).
#include <algorithm>
#include <climits>
#include <map>
#include <numeric>
#include <string>
#include <vector>

#include "pc_host.h"

namespace pc {

[[noreturn]] void fail(int code, const std::string& msg) { throw Error{code, msg}; }

static void need(bool ok, const std::string& msg) {
  if (!ok) fail(PC_ERR_INVALID_ARG, msg);
}

static std::string L(int i) { return "layer " + std::to_string(i) + ": "; }

Handle* compile_layout(const pc_circuit_desc* d) {
  need(d != nullptr, "null descriptor");
  need(d->num_nodes >= 1, "num_nodes must be >= 1");
  need(d->num_vars >= 0, "num_vars must be >= 0");
  need(d->num_params >= 0, "num_params must be >= 0");
  need(d->num_layers >= 1 && d->layers != nullptr, "need at least one layer");
  need(d->root >= -1 && d->root < d->num_nodes, "root out of range");
  if (d->lowrank_rank < 0 || d->lowrank_rank > 64)
    fail(PC_ERR_UNSUPPORTED, "LowRank rank must be in 1..64 (the fused LowRank kernels)");
  if (d->lowrank_form != PC_LOWRANK_EXP_SUM && d->lowrank_form != PC_LOWRANK_SUM_EXP)
    fail(PC_ERR_UNSUPPORTED, "LowRank form must be PC_LOWRANK_EXP_SUM or PC_LOWRANK_SUM_EXP");

  Handle* h = new Handle();
  h->num_nodes = d->num_nodes;
  h->num_vars = d->num_vars;
  h->num_params = d->num_params;
  h->root = d->root;
  h->lowrank_rank = d->lowrank_rank;
  h->lowrank_form = d->lowrank_form;
  const int64_t NN = d->num_nodes;

  std::vector<int32_t> defined_at(NN, -1);
  std::vector<int32_t> last_parent(NN, -1);     // last layer (topological) using the node as a child
  std::vector<int32_t> stamp(NN, -1);
  int stamp_id = 0;

  auto define = [&](int li, int64_t s, int64_t n) {
    need(n >= 0 && s >= 0 && s + n <= NN, L(li) + "node range out of bounds");
    for (int64_t i = s; i < s + n; ++i) {
      need(defined_at[i] < 0, L(li) + "node " + std::to_string(i) + " defined twice");
      defined_at[i] = li;
    }
  };
  auto use = [&](int li, int64_t c) {
    need(c >= 0 && c < NN, L(li) + "child id out of range");
    need(defined_at[c] >= 0 && defined_at[c] < li,
         L(li) + "child " + std::to_string(c) + " not defined by an earlier layer");
    last_parent[c] = li;
  };
  auto param_range = [&](int li, int64_t off, int64_t len) {
    need(off >= 0 && len >= 0 && off + len <= d->num_params, L(li) + "parameters out of range");
  };

  // ---- pass 1: check every layer, build per-kind plans ----------------------
  std::map<int64_t, std::pair<int32_t, int32_t>> block_shape;   // param_offset -> (M, N)
  std::map<int64_t, int> block_id;
  std::vector<std::pair<int64_t, int64_t>> param_intervals;      // distinct [off, off+len)
  std::map<int64_t, std::pair<int32_t, int32_t>> table_shape;   // input tables
  int lowrank_slots = 0;

  for (int li = 0; li < d->num_layers; ++li) {
    const pc_layer_desc& ly = d->layers[li];
    LayerRef ref{ly.kind, -1};
    if (ly.kind == PC_LAYER_INPUT_CAT) {
      need(ly.num_nodes >= 1 && ly.num_cats >= 1 && ly.num_rows >= 1, L(li) + "empty input layer");
      need(ly.var && ly.row, L(li) + "null var/row");
      need(d->num_vars >= 1, L(li) + "categorical input needs num_vars >= 1");
      define(li, ly.node_start, ly.num_nodes);
      param_range(li, ly.param_offset, (int64_t)ly.num_rows * ly.num_cats);
      InputPlan ip;
      ip.layer = li;
      ip.node_start = ly.node_start;
      ip.num_nodes = ly.num_nodes;
      ip.num_cats = ly.num_cats;
      ip.num_rows = ly.num_rows;
      ip.param_offset = ly.param_offset;
      ip.var.assign(ly.var, ly.var + ly.num_nodes);
      ip.row.assign(ly.row, ly.row + ly.num_nodes);
      for (int32_t i = 0; i < ly.num_nodes; ++i) {
        need(ip.var[i] >= 0 && ip.var[i] < d->num_vars, L(li) + "var out of range");
        need(ip.row[i] >= 0 && ip.row[i] < ly.num_rows, L(li) + "row out of range");
      }
      // row -> nodes CSR (ascending node order)
      ip.row_ptr.assign(ly.num_rows + 1, 0);
      for (int32_t i = 0; i < ly.num_nodes; ++i) ip.row_ptr[ip.row[i] + 1]++;
      for (int32_t r = 0; r < ly.num_rows; ++r) {
        ip.max_row_nodes = std::max(ip.max_row_nodes, ip.row_ptr[r + 1]);
        ip.row_ptr[r + 1] += ip.row_ptr[r];
      }
      ip.row_nodes.assign(ly.num_nodes, 0);
      std::vector<int32_t> fillp(ip.row_ptr.begin(), ip.row_ptr.end() - 1);
      for (int32_t i = 0; i < ly.num_nodes; ++i) ip.row_nodes[fillp[ip.row[i]]++] = ly.node_start + i;
      // nodes of each variable (ascending), for the input flows of layers whose rows have one node each
      ip.var_ptr.assign(d->num_vars + 1, 0);
      for (int32_t i = 0; i < ly.num_nodes; ++i) ip.var_ptr[ip.var[i] + 1]++;
      for (int32_t v = 0; v < d->num_vars; ++v) {
        ip.max_var_nodes = std::max(ip.max_var_nodes, ip.var_ptr[v + 1]);
        ip.var_ptr[v + 1] += ip.var_ptr[v];
      }
      ip.var_nodes.assign(ly.num_nodes, 0);
      std::vector<int32_t> fillv(ip.var_ptr.begin(), ip.var_ptr.end() - 1);
      for (int32_t i = 0; i < ly.num_nodes; ++i) ip.var_nodes[fillv[ip.var[i]]++] = i;
      auto it = table_shape.find(ly.param_offset);
      if (it == table_shape.end()) {
        table_shape[ly.param_offset] = {ly.num_rows, ly.num_cats};
        param_intervals.push_back({ly.param_offset, ly.param_offset + (int64_t)ly.num_rows * ly.num_cats});
      } else {
        need(it->second == std::make_pair(ly.num_rows, ly.num_cats),
             L(li) + "input tables sharing parameters differ in shape");
      }
      h->max_cats = std::max(h->max_cats, ly.num_cats);
      ref.idx = (int)h->inputs.size();
      h->inputs.push_back(std::move(ip));
    } else if (ly.kind == PC_LAYER_INPUT_EXTERNAL) {
      need(ly.num_nodes >= 1, L(li) + "empty external layer");
      define(li, ly.node_start, ly.num_nodes);
    } else if (ly.kind == PC_LAYER_PRODUCT) {
      need(ly.num_nodes >= 1 && ly.ch_ptr && ly.ch_ids, L(li) + "empty product layer");
      need(ly.ch_ptr[0] == 0, L(li) + "ch_ptr[0] must be 0");
      for (int32_t i = 0; i < ly.num_nodes; ++i)
        need(ly.ch_ptr[i + 1] > ly.ch_ptr[i], L(li) + "product node without children");
      ProductPlan pp;
      pp.layer = li;
      pp.node_start = ly.node_start;
      pp.num_nodes = ly.num_nodes;
      pp.ch_ptr.assign(ly.ch_ptr, ly.ch_ptr + ly.num_nodes + 1);
      pp.ch_ids.assign(ly.ch_ids, ly.ch_ids + ly.ch_ptr[ly.num_nodes]);
      for (int32_t c : pp.ch_ids) use(li, c);
      for (int32_t i = 0; i < ly.num_nodes; ++i) pp.max_deg = std::max(pp.max_deg, pp.ch_ptr[i + 1] - pp.ch_ptr[i]);
      define(li, ly.node_start, ly.num_nodes);
      // parent CSR over distinct children
      std::vector<std::pair<int32_t, int32_t>> cp;
      cp.reserve(pp.ch_ids.size());
      for (int32_t i = 0; i < ly.num_nodes; ++i)
        for (int32_t k = pp.ch_ptr[i]; k < pp.ch_ptr[i + 1]; ++k) cp.push_back({pp.ch_ids[k], ly.node_start + i});
      std::sort(cp.begin(), cp.end());
      pp.pptr.push_back(0);
      for (size_t k = 0; k < cp.size(); ++k) {
        if (k == 0 || cp[k].first != cp[k - 1].first) {
          if (k) pp.pptr.push_back((int32_t)k);
          pp.uchild.push_back(cp[k].first);
        }
        pp.parents.push_back(cp[k].second);
      }
      pp.pptr.push_back((int32_t)cp.size());
      pp.single_parent = pp.parents.size() == pp.uchild.size();
      {   // affine: uniform degree, child q of node i at abase[q] + i, disjoint ranges
        const int32_t D = pp.ch_ptr[1] - pp.ch_ptr[0];
        bool af = D <= 8 && pp.single_parent;
        for (int32_t i = 0; af && i < ly.num_nodes; ++i) {
          af = pp.ch_ptr[i + 1] - pp.ch_ptr[i] == D;
          for (int32_t q = 0; af && q < D; ++q) af = pp.ch_ids[(int64_t)i * D + q] == pp.ch_ids[q] + i;
        }
        if (af) {
          pp.affine = true;
          for (int32_t q = 0; q < D; ++q) pp.abase[q] = pp.ch_ids[q];
        }
      }
      ref.idx = (int)h->prods.size();
      h->prods.push_back(std::move(pp));
    } else if (ly.kind == PC_LAYER_SUM) {
      need(ly.num_groups >= 1 && ly.groups, L(li) + "empty sum layer");
      SumPlan sp;
      sp.layer = li;
      int n_lr = 0;
      for (int32_t g = 0; g < ly.num_groups; ++g) {
        const pc_sum_group& G = ly.groups[g];
        std::string gs = L(li) + "group " + std::to_string(g) + ": ";
        need(G.num_nodes >= 1 && G.num_ch_blocks >= 1 && G.ch_block_size >= 1 && G.ch_block_start,
             gs + "empty group");
        int64_t N = (int64_t)G.num_ch_blocks * G.ch_block_size;
        need(N <= (1 << 30) && G.num_nodes <= (1 << 30), gs + "group too large");
        ++stamp_id;
        for (int32_t k = 0; k < G.num_ch_blocks; ++k) {
          int64_t s = G.ch_block_start[k];
          need(s >= 0 && s + G.ch_block_size <= NN, gs + "child block out of range");
          for (int64_t c = s; c < s + G.ch_block_size; ++c) {
            use(li, c);
            need(stamp[c] != stamp_id, gs + "child " + std::to_string(c) + " listed twice");
            stamp[c] = stamp_id;
          }
        }
        param_range(li, G.param_offset, (int64_t)G.num_nodes * N);
        need(G.lowrank_slot >= -1, gs + "bad lowrank slot");
        if (G.lowrank_slot >= 0) {
          if (d->lowrank_rank < 1) fail(PC_ERR_UNSUPPORTED, gs + "LowRank group needs lowrank_rank in 1..64");
          ++n_lr;
          lowrank_slots = std::max(lowrank_slots, G.lowrank_slot + 1);
        }
        auto it = block_shape.find(G.param_offset);
        if (it == block_shape.end()) {
          block_shape[G.param_offset] = {G.num_nodes, (int32_t)N};
          param_intervals.push_back({G.param_offset, G.param_offset + (int64_t)G.num_nodes * N});
        } else {
          need(it->second == std::make_pair(G.num_nodes, (int32_t)N), gs + "tied groups differ in shape");
        }
        GroupRec r{};
        r.out_start = G.out_start;
        r.M = G.num_nodes;
        r.N = (int32_t)N;
        r.cbs = G.ch_block_size;
        r.blk_off = (int32_t)sp.blocks.size();
        r.nblk = G.num_ch_blocks;
        r.param_offset = G.param_offset;
        r.lowrank = G.lowrank_slot;
        r.ch_start = G.num_ch_blocks > 0 ? G.ch_block_start[0] : -1;
        for (int32_t b = 1; b < G.num_ch_blocks && r.ch_start >= 0; ++b)
          if (G.ch_block_start[b] != G.ch_block_start[0] + (int64_t)b * G.ch_block_size) r.ch_start = -1;
        sp.blocks.insert(sp.blocks.end(), G.ch_block_start, G.ch_block_start + G.num_ch_blocks);
        sp.groups.push_back(r);
      }
      need(n_lr == 0 || n_lr == ly.num_groups, L(li) + "a sum layer is either all LowRank or none");
      sp.lowrank = n_lr > 0;
      for (auto& r : sp.groups) define(li, r.out_start, r.M);
      ref.idx = (int)h->sums.size();
      h->sums.push_back(std::move(sp));
    } else {
      fail(PC_ERR_INVALID_ARG, L(li) + "unknown layer kind");
    }
    h->layers.push_back(ref);
  }
  for (int64_t i = 0; i < NN; ++i) need(defined_at[i] >= 0, "node " + std::to_string(i) + " is not defined");
  h->lowrank_slots = lowrank_slots;

  // distinct parameter blocks must not overlap
  std::sort(param_intervals.begin(), param_intervals.end());
  for (size_t k = 1; k < param_intervals.size(); ++k)
    need(param_intervals[k].first >= param_intervals[k - 1].second, "parameter blocks overlap");

  // ---- pass 2: sum-layer classification and operand placement -------------
  int64_t s_rows = 0;
  int32_t m_rows = 0;
  for (auto& sp : h->sums) {
    const int G = (int)sp.groups.size();
    auto same_children = [&](const GroupRec& a, const GroupRec& b) {
      if (a.cbs != b.cbs || a.nblk != b.nblk) return false;
      for (int k = 0; k < a.nblk; ++k)
        if (sp.blocks[a.blk_off + k] != sp.blocks[b.blk_off + k]) return false;
      return true;
    };
    bool shared = true;
    for (int g = 1; g < G; ++g) shared = shared && same_children(sp.groups[0], sp.groups[g]);
    bool strided = G >= 2;
    if (strided) {
      const GroupRec& a = sp.groups[0];
      const GroupRec& b = sp.groups[1];
      int64_t d_out = b.out_start - a.out_start;
      int64_t d_ch = (int64_t)sp.blocks[b.blk_off] - sp.blocks[a.blk_off];
      int64_t d_par = b.param_offset - a.param_offset;
      for (int g = 0; g < G && strided; ++g) {
        const GroupRec& c = sp.groups[g];
        strided = c.M == a.M && c.N == a.N && c.nblk == 1 &&
                  c.out_start == a.out_start + g * d_out &&
                  sp.blocks[c.blk_off] == sp.blocks[a.blk_off] + g * d_ch &&
                  c.param_offset == a.param_offset + g * d_par;
      }
      strided = strided && d_ch != 0;
    }
    sp.cls = sp.lowrank ? PC_CLASS_LOWRANK : shared ? PC_CLASS_SHARED : strided ? PC_CLASS_STRIDED : PC_CLASS_GENERAL;

    // overlap: does any child belong to two groups of this layer?
    ++stamp_id;
    sp.overlap = false;
    for (auto& r : sp.groups)
      for (int k = 0; k < r.nblk && !sp.overlap; ++k)
        for (int64_t c = sp.blocks[r.blk_off + k]; c < sp.blocks[r.blk_off + k] + r.cbs; ++c) {
          if (stamp[c] == stamp_id) { sp.overlap = true; break; }
          stamp[c] = stamp_id;
        }

    int32_t ekoff = 0, gkoff = 0, mt = 0, ct = 0, pk = 0, pg = 0, srow = 0;
    for (int g = 0; g < G; ++g) {
      GroupRec& r = sp.groups[g];
      r.share_src = (sp.cls == PC_CLASS_SHARED) ? 0 : g;
      const int64_t Mp = round_up(r.M, ROW_PAD), Np = round_up(r.N, ROW_PAD);
      const int64_t MpK = round_up(r.M, K_PAD), NpK = round_up(r.N, K_PAD);
      auto bit = block_id.find(r.param_offset);
      if (bit == block_id.end()) {
        int id = (int)h->blocks.size();
        block_id[r.param_offset] = id;
        BlockRec b{};
        b.param_offset = r.param_offset;
        b.M = r.M;
        b.N = r.N;
        h->blocks.push_back(b);
        r.block = id;
      } else {
        r.block = bit->second;
      }
      r.share_next = -1;
      if (r.share_src == g) {
        r.m_row = m_rows++;
        r.e_koff = ekoff;
        ekoff += (int32_t)NpK;
        r.pk_start = pk;
        pk += (int32_t)(Np / 64);
      } else {
        GroupRec& s = sp.groups[r.share_src];
        r.m_row = s.m_row;
        r.e_koff = s.e_koff;
        r.pk_start = pk;          // empty range: the source group's tiles write this group's E rows too
        int q = r.share_src;      // append to the source's chain of sharers
        while (sp.groups[q].share_next >= 0) q = sp.groups[q].share_next;
        sp.groups[q].share_next = g;
      }
      r.e_row = r.g_row = -1;     // placed per weight block below
      r.s_row = sp.lowrank ? -1 : s_rows;
      if (!sp.lowrank) s_rows += r.M;
      r.g_koff = gkoff;
      gkoff += (int32_t)MpK;
      r.mt_start = mt;
      mt += (int32_t)(Mp / ROW_PAD);
      r.ct_start = ct;
      ct += (int32_t)(Np / ROW_PAD);
      r.pg_start = pg;
      pg += (int32_t)(Mp / 64);
      if (sp.overlap) {
        r.scratch_row = srow;
        srow += r.N;
      } else {
        r.scratch_row = -1;
      }
    }
    for (auto& r : sp.groups) {
      sp.max_npk = std::max<int32_t>(sp.max_npk, (int32_t)round_up(r.N, K_PAD));
      sp.max_mpk = std::max<int32_t>(sp.max_mpk, (int32_t)round_up(r.M, K_PAD));
    }
    sp.ebt_cols = ekoff;
    sp.gbt_cols = gkoff;
    sp.mtiles = mt;
    sp.ctiles = ct;
    sp.pktiles = pk;
    sp.pgtiles = pg;
    sp.pk_group.assign(pk, 0);
    sp.pg_group.assign(pg, 0);
    for (int32_t q = 0; q < (int32_t)sp.groups.size(); ++q) {   // later groups win ties (empty ranges)
      for (int32_t t = sp.groups[q].pk_start; t < pk; ++t) sp.pk_group[t] = q;
      for (int32_t t = sp.groups[q].pg_start; t < pg; ++t) sp.pg_group[t] = q;
    }
    sp.scratch_rows = srow;
    h->max_ebt_cols = std::max(h->max_ebt_cols, ekoff);
    h->max_gbt_cols = std::max(h->max_gbt_cols, gkoff);
    h->max_scratch_rows = std::max(h->max_scratch_rows, srow);
    if (!sp.lowrank) h->has_plain_sums = true;

    if (sp.overlap) {   // reduction CSR: distinct child -> scratch rows (group order)
      std::vector<std::pair<int32_t, int32_t>> cs;
      for (auto& r : sp.groups)
        for (int k = 0; k < r.nblk; ++k)
          for (int j = 0; j < r.cbs; ++j)
            cs.push_back({sp.blocks[r.blk_off + k] + j, r.scratch_row + k * r.cbs + j});
      std::stable_sort(cs.begin(), cs.end(),
                       [](const std::pair<int32_t, int32_t>& a, const std::pair<int32_t, int32_t>& b) {
                         return a.first < b.first;
                       });
      sp.red_ptr.push_back(0);
      for (size_t k = 0; k < cs.size(); ++k) {
        if (k == 0 || cs[k].first != cs[k - 1].first) {
          if (k) sp.red_ptr.push_back((int32_t)k);
          sp.red_child.push_back(cs[k].first);
        }
        sp.red_src.push_back(cs[k].second);
      }
      sp.red_ptr.push_back((int32_t)cs.size());
    }
  }
  h->s_rows = s_rows;
  h->m_rows = m_rows;

  // Tied copies of each block, in layer order: copy s keeps its node-major G
  // rows at g_base + s*M_pad and its E rows at e_base + s*N_pad.
  {
    std::vector<std::vector<std::pair<int, int>>> per(h->blocks.size());
    for (int si = 0; si < (int)h->sums.size(); ++si) {
      if (h->sums[si].lowrank) continue;
      for (int g = 0; g < (int)h->sums[si].groups.size(); ++g) per[h->sums[si].groups[g].block].push_back({si, g});
    }
    int64_t th = 0, tht = 0, erow = 0, grow = 0;
    int32_t pk = 0, p256 = 0, p128 = 0;
    h->copy_layer.assign(h->blocks.size(), {});
    for (size_t b = 0; b < h->blocks.size(); ++b) {
      BlockRec& B = h->blocks[b];
      const int64_t Mp = round_up(B.M, ROW_PAD), Np = round_up(B.N, ROW_PAD);
      const int64_t MpK = round_up(B.M, K_PAD), NpK = round_up(B.N, K_PAD);
      B.ncopies = (int32_t)per[b].size();
      B.g_base = grow;
      B.e_base = erow;
      h->copy_layer[b].clear();
      for (int c = 0; c < B.ncopies; ++c) h->copy_layer[b].push_back(h->sums[per[b][c].first].layer);
      for (int c = 0; c < B.ncopies; ++c) {
        GroupRec& r = h->sums[per[b][c].first].groups[per[b][c].second];
        r.g_row = grow + c * Mp;
        r.e_row = erow + c * Np;
      }
      grow += B.ncopies * Mp;
      erow += B.ncopies * Np;
      B.pk_start = pk;
      B.pt256 = p256;
      B.pt128 = p128;
      if (B.ncopies > 0) {
        B.th_off = th;
        th += Mp * NpK;
        B.tht_off = tht;
        tht += Np * MpK;
        pk += (int32_t)((Mp / 64) * (Np / 64));
        p256 += (int32_t)((Mp / 256) * (Np / 256));
        p128 += (int32_t)((Mp / 128) * (Np / 128));
        h->min_block_dim = std::min<int64_t>(h->min_block_dim, std::min(B.M, B.N));
      } else {
        B.th_off = B.tht_off = -1;
      }
    }
    h->theta_elems = th;
    h->thetaT_elems = tht;
    h->pk_block_tiles = pk;
    h->param_tiles256 = p256;
    h->param_tiles128 = p128;
    h->earena_rows = erow;
    h->garena_rows = grow;
    for (auto& sp : h->sums) h->max_sum_groups = std::max<int32_t>(h->max_sum_groups, (int32_t)sp.groups.size());
  }

  // LowRank groups: rows of their kept forward records, and the parameter-flow
  // partials of each distinct LowRank weight block
  h->lr_p_off.assign(h->blocks.size(), -1);
  for (auto& sp : h->sums) {
    if (!sp.lowrank) continue;
    for (auto& r : sp.groups) {
      sp.lr_row.push_back(h->lr_rows);
      sp.lr_gidx.push_back(h->lr_groups++);
      h->lr_rows += r.M;
      h->lr_max_m = std::max(h->lr_max_m, r.M);
      h->lr_max_n = std::max(h->lr_max_n, r.N);
      if (h->lr_p_off[r.block] < 0) {
        h->lr_p_off[r.block] = h->lr_p_elems;
        h->lr_p_elems += (int64_t)r.M * r.N;
      }
    }
  }

  // LowRank "sum_exp" on a virtual batch (pyjuice.parameterizations.LowRank,
  // definition: sum_exp "is k matmuls with the shared parameters"): a block
  // record per distinct LowRank weight block, placed after the plain blocks
  // in the weight-plane arenas, with its copies' node-major operand rows and
  // its own parameter-flow tile prefixes; a group record per LowRank group.
  if (h->lowrank_form == PC_LOWRANK_SUM_EXP && h->lr_groups > 0) {
    std::map<int32_t, int> vid;                       // block -> virtual block
    std::vector<std::vector<std::pair<int, int>>> per;  // virtual block -> (sum layer, group)
    h->vgroups.assign(h->lr_groups, GroupRec{});
    for (int si = 0; si < (int)h->sums.size(); ++si) {
      SumPlan& sp = h->sums[si];
      if (!sp.lowrank) continue;
      for (int g = 0; g < (int)sp.groups.size(); ++g) {
        const GroupRec& r = sp.groups[g];
        auto it = vid.find(r.block);
        if (it == vid.end()) {
          it = vid.emplace(r.block, (int)h->vblocks.size()).first;
          BlockRec b{};
          b.param_offset = h->blocks[r.block].param_offset;
          b.M = r.M;
          b.N = r.N;
          h->vblocks.push_back(b);
          per.emplace_back();
        }
        per[it->second].push_back({si, g});
      }
    }
    int64_t th = h->theta_elems, tht = h->thetaT_elems, xr = 0, yr = 0;
    int32_t pk = 0, p256 = 0, p128 = 0;
    h->vcopy_layer.assign(h->vblocks.size(), {});
    for (size_t v = 0; v < h->vblocks.size(); ++v) {
      BlockRec& B = h->vblocks[v];
      const int64_t Mp = round_up(B.M, ROW_PAD), Np = round_up(B.N, ROW_PAD);
      const int64_t MpK = round_up(B.M, K_PAD), NpK = round_up(B.N, K_PAD);
      B.ncopies = (int32_t)per[v].size();
      B.g_base = yr;
      B.e_base = xr;
      B.th_off = th;
      th += Mp * NpK;
      B.tht_off = tht;
      tht += Np * MpK;
      B.pk_start = pk;
      pk += (int32_t)((Mp / 64) * (Np / 64));
      B.pt256 = p256;
      p256 += (int32_t)((Mp / 256) * (Np / 256));
      B.pt128 = p128;
      p128 += (int32_t)((Mp / 128) * (Np / 128));
      for (int c = 0; c < B.ncopies; ++c) {
        const SumPlan& sp = h->sums[per[v][c].first];
        const GroupRec& r = sp.groups[per[v][c].second];
        GroupRec q{};
        q.out_start = r.out_start;
        q.M = r.M;
        q.N = r.N;
        q.cbs = r.cbs;
        q.blk_off = r.blk_off;
        q.nblk = r.nblk;
        q.param_offset = r.param_offset;
        q.block = (int32_t)v;
        q.m_row = r.m_row;
        q.mt_start = q.ct_start = q.pk_start = q.pg_start = 0;
        q.e_koff = q.g_koff = 0;
        q.e_row = xr + c * Np;
        q.g_row = yr + c * Mp;
        q.scratch_row = r.scratch_row;
        q.lowrank = r.lowrank;
        q.share_src = 0;
        q.share_next = -1;
        q.ch_start = r.ch_start;
        q.s_row = -1;
        h->vgroups[sp.lr_gidx[per[v][c].second]] = q;
        h->vcopy_layer[v].push_back(sp.layer);
        h->v_max_k = std::max<int32_t>(h->v_max_k, (int32_t)std::max(MpK, NpK));
      }
      xr += B.ncopies * Np;
      yr += B.ncopies * Mp;
    }
    h->theta_elems = th;
    h->thetaT_elems = tht;
    h->v_pk_tiles = pk;
    h->v_param_tiles256 = p256;
    h->v_param_tiles128 = p128;
    h->vx_rows = xr;
    h->vy_rows = yr;
  }

  // EM row segments: every distinct block and input table
  {
    std::map<int64_t, RowSeg> segs;
    for (size_t bi = 0; bi < h->blocks.size(); ++bi) {
      const BlockRec& B = h->blocks[bi];
      segs[B.param_offset] = RowSeg{B.param_offset, B.M, B.N, 0, h->lr_p_off[bi] >= 0 ? 1 : 0};
    }
    for (auto& kv : table_shape) segs[kv.first] = RowSeg{kv.first, kv.second.first, kv.second.second, 0, 0};
    int32_t rows = 0;
    for (auto& kv : segs) {
      RowSeg s = kv.second;
      s.row_start = rows;
      rows += s.nrows;
      h->rowsegs.push_back(s);
    }
    h->total_rows = rows;
  }

  // ---- pass 3: element-flow write plan --------------------------------------
  // A layer stores (instead of adding) the flows of its children when it is
  // the first writer of each of them in reverse order, i.e. the last layer in
  // topological order that uses them.  Children whose first writer adds are
  // cleared before the backward starts.
  std::vector<char> zero(NN, 0);
  for (auto& pp : h->prods) {
    bool st = true;
    for (int32_t c : pp.uchild) st = st && last_parent[c] == pp.layer;
    pp.store = st;
    if (!st)
      for (int32_t c : pp.uchild)
        if (last_parent[c] == pp.layer) zero[c] = 1;
  }
  for (auto& sp : h->sums) {
    bool st = true;
    for (auto& r : sp.groups)
      for (int k = 0; k < r.nblk; ++k)
        for (int j = 0; j < r.cbs; ++j) st = st && last_parent[sp.blocks[r.blk_off + k] + j] == sp.layer;
    sp.store = st;
    if (!st)
      for (auto& r : sp.groups)
        for (int k = 0; k < r.nblk; ++k)
          for (int j = 0; j < r.cbs; ++j) {
            int32_t c = sp.blocks[r.blk_off + k] + j;
            if (last_parent[c] == sp.layer) zero[c] = 1;
          }
  }
  for (int64_t i = 0; i < NN; ++i)
    if (last_parent[i] < 0) h->outputs.push_back((int32_t)i);
  // runs of cleared nodes
  for (int64_t i = 0; i < NN;) {
    if (!zero[i]) { ++i; continue; }
    int64_t j = i;
    while (j < NN && zero[j]) ++j;
    h->zero_ranges.push_back(FillRange{(int32_t)i, (int32_t)(j - i), 0.0f, 0});
    h->max_zero_count = std::max<int64_t>(h->max_zero_count, j - i);
    i = j;
  }
  // seeds without caller seeds: the root gets 1, every other output 0
  for (size_t k = 0; k < h->outputs.size();) {
    size_t q = k;
    while (q + 1 < h->outputs.size() && h->outputs[q + 1] == h->outputs[q] + 1 &&
           h->outputs[q + 1] != h->root && h->outputs[k] != h->root)
      ++q;
    const int32_t s0 = h->outputs[k], n = (int32_t)(q - k + 1);
    h->seed_ranges.push_back(FillRange{s0, n, (s0 == h->root) ? 1.0f : 0.0f, 0});
    h->max_seed_count = std::max<int64_t>(h->max_seed_count, n);
    k = q + 1;
  }

  // ---- pass 4: product layers computed inside an adjacent sum layer's kernels --
  // Forward: a product layer directly followed by a sum layer whose column-max
  // tiles cover each of its nodes exactly once is evaluated by those tiles
  // (each tile row sums its product node's children, stores it and takes the
  // maximum), saving a launch and a re-read.  Backward: a product layer
  // directly after a plain sum layer runs inside that layer's scaled-flow
  // packing, which comes next in reverse order; the packing rows of the sum
  // layer's outputs gather their parents' flows, the other distinct children
  // of the product layer get extra workgroups.  Both keep every sum in the
  // product kernels' order, so the results are the same bits.
  for (size_t li = 0; li + 1 < h->layers.size(); ++li) {
    const LayerRef a = h->layers[li], b = h->layers[li + 1];
    if (a.kind == PC_LAYER_PRODUCT && b.kind == PC_LAYER_SUM) {
      ProductPlan& pp = h->prods[a.idx];
      SumPlan& sp = h->sums[b.idx];
      std::vector<int32_t> cnt(pp.num_nodes, 0);
      for (size_t g = 0; g < sp.groups.size(); ++g) {
        const GroupRec& r = sp.groups[g];
        if (r.share_src != (int32_t)g) continue;   // sharing groups have no column-max tiles
        for (int k = 0; k < r.nblk; ++k)
          for (int64_t c = sp.blocks[r.blk_off + k]; c < sp.blocks[r.blk_off + k] + r.cbs; ++c) {
            const int64_t q = c - pp.node_start;
            if (q >= 0 && q < pp.num_nodes) ++cnt[q];
          }
      }
      bool once = true;
      for (int32_t x : cnt) once = once && x == 1;
      if (once) {
        pp.fwd_fused = true;
        sp.fwd_prod = a.idx;
      }
    }
    if (a.kind == PC_LAYER_SUM && b.kind == PC_LAYER_PRODUCT && !h->sums[a.idx].lowrank) {
      SumPlan& sp = h->sums[a.idx];
      ProductPlan& pp = h->prods[b.idx];
      sp.up_idx.assign((size_t)sp.pgtiles * 64, -1);
      std::vector<char> is_out(pp.uchild.size(), 0);
      for (const GroupRec& r : sp.groups)
        for (int32_t k = 0; k < r.M; ++k) {
          const int32_t n = r.out_start + k;
          auto it = std::lower_bound(pp.uchild.begin(), pp.uchild.end(), n);
          if (it == pp.uchild.end() || *it != n) continue;
          const int32_t u = (int32_t)(it - pp.uchild.begin());
          sp.up_idx[(size_t)r.pg_start * 64 + k] = pp.single_parent ? pp.parents[pp.pptr[u]] : u;
          is_out[u] = 1;
        }
      for (size_t u = 0; u < pp.uchild.size(); ++u)
        if (!is_out[u]) {
          sp.up_rest.push_back(pp.single_parent ? pp.uchild[u] : (int32_t)u);
          sp.up_rest_par.push_back(pp.single_parent ? pp.parents[pp.pptr[u]] : -1);
        }
      pp.bwd_fused = true;
      sp.bwd_prod = b.idx;
    }
  }
  // Forward product epilogues (see SumPlan::epi_prod): sum layer L1 (its
  // product kernel's epilogue, or for a LowRank layer the kernel that writes
  // its node values), affine product layer P of two children per node
  // evaluated by the next sum layer's column maxima (fwd_fused), sum layer L3
  // with a single group whose children are exactly P's nodes.  P's child
  // range q_s must be L1's outputs node for node, its other child ranges must
  // avoid L1's outputs.
  for (size_t li = 0; li + 2 < h->layers.size(); ++li) {
    const LayerRef a = h->layers[li], b = h->layers[li + 1], c = h->layers[li + 2];
    if (a.kind != PC_LAYER_SUM || b.kind != PC_LAYER_PRODUCT || c.kind != PC_LAYER_SUM) continue;
    SumPlan& s1 = h->sums[a.idx];
    ProductPlan& pp = h->prods[b.idx];
    SumPlan& s3 = h->sums[c.idx];
    if (!pp.affine || pp.max_deg != 2 || !pp.fwd_fused || s3.fwd_prod != b.idx) continue;
    if (s3.groups.size() != 1 || s3.groups[0].N != pp.num_nodes) continue;
    {   // L3's children: P's nodes, each once
      const GroupRec& r = s3.groups[0];
      std::vector<char> seen(pp.num_nodes, 0);
      bool ok = true;
      for (int k = 0; ok && k < r.nblk; ++k)
        for (int64_t ch = s3.blocks[r.blk_off + k]; ok && ch < s3.blocks[r.blk_off + k] + r.cbs; ++ch) {
          const int64_t q = ch - pp.node_start;
          ok = q >= 0 && q < pp.num_nodes && !seen[q];
          if (ok) seen[q] = 1;
        }
      if (!ok) continue;
    }
    // L1's outputs as a node mask
    int32_t lo = INT32_MAX, hi = -1;
    for (const GroupRec& r : s1.groups) {
      lo = std::min(lo, r.out_start);
      hi = std::max(hi, r.out_start + r.M);
    }
    std::vector<char> out((size_t)(hi - lo), 0);
    for (const GroupRec& r : s1.groups)
      for (int32_t k = 0; k < r.M; ++k) out[(size_t)(r.out_start + k - lo)] = 1;
    auto is_out = [&](int64_t n) { return n >= lo && n < hi && out[(size_t)(n - lo)]; };
    int qs = -1;
    bool ok = true;
    for (int32_t q = 0; ok && q < pp.max_deg; ++q) {
      int64_t inside = 0;
      for (int32_t i = 0; i < pp.num_nodes; ++i) inside += is_out((int64_t)pp.abase[q] + i);
      if (inside == pp.num_nodes && qs < 0) qs = q;
      else if (inside != 0) ok = false;
    }
    if (!ok || qs < 0) continue;
    s1.epi_prod = b.idx;
    s1.epi_qs = qs;
    s1.epi_mrow = s3.groups[0].m_row;
    s3.epi_max = true;
    s3.epi_src = a.idx;
  }
  // Element-flow product epilogues (see SumPlan::gp_sum): plain single-group
  // sum layer A (M a multiple of 64), affine two-child product layer P fused
  // into A's scaled-flow packing (every child of P with P as its only parent,
  // P the first writer of their flows), plain single-group sum layer C whose
  // children are P's nodes in order, C the only writer of their flows.  P's
  // child range q_s must be A's outputs in order.
  for (size_t li = 0; li + 2 < h->layers.size(); ++li) {
    const LayerRef a = h->layers[li], b = h->layers[li + 1], c = h->layers[li + 2];
    if (a.kind != PC_LAYER_SUM || b.kind != PC_LAYER_PRODUCT || c.kind != PC_LAYER_SUM) continue;
    SumPlan& sa = h->sums[a.idx];
    ProductPlan& pp = h->prods[b.idx];
    SumPlan& sc = h->sums[c.idx];
    if (sa.lowrank || sc.lowrank || sa.groups.size() != 1 || sc.groups.size() != 1) continue;
    if (!pp.affine || pp.max_deg != 2 || !pp.single_parent || !pp.store || sa.bwd_prod != b.idx) continue;
    const GroupRec& ra = sa.groups[0];
    const GroupRec& rc = sc.groups[0];
    if (ra.M % 64 != 0 || pp.num_nodes != ra.M) continue;
    int qs = -1;
    for (int q = 0; q < 2; ++q)
      if (pp.abase[q] == ra.out_start) qs = q;
    if (qs < 0) continue;
    const int32_t ob = pp.abase[1 - qs];
    if (ob < ra.out_start + ra.M && ob + pp.num_nodes > ra.out_start) continue;   // other child range overlaps A
    if (!sc.store || sc.overlap || rc.scratch_row >= 0 || rc.N != pp.num_nodes) continue;
    bool inorder = true;
    for (int32_t j = 0; inorder && j < rc.N; ++j)
      inorder = sc.blocks[rc.blk_off + j / rc.cbs] + j % rc.cbs == pp.node_start + j;
    if (!inorder) continue;
    if (ra.s_row < 0) continue;
    sc.gp_sum = a.idx;
    sc.gp_prod = b.idx;
    sc.gp_qs = qs;
    sa.gp_done = true;
    h->gbt_slots = 2;
  }
  // LowRank coefficient kernels with the product backward (see
  // SumPlan::lr_prod): single-group LowRank layer A, affine two-child product
  // layer P right after it whose child range q_s is A's outputs in order, P
  // the single parent and first writer of every child.
  for (size_t li = 0; li + 1 < h->layers.size(); ++li) {
    const LayerRef a = h->layers[li], b = h->layers[li + 1];
    if (a.kind != PC_LAYER_SUM || b.kind != PC_LAYER_PRODUCT) continue;
    SumPlan& sa = h->sums[a.idx];
    ProductPlan& pp = h->prods[b.idx];
    if (!sa.lowrank || sa.groups.size() != 1 || pp.bwd_fused) continue;
    if (!pp.affine || pp.max_deg != 2 || !pp.single_parent || !pp.store) continue;
    const GroupRec& ra = sa.groups[0];
    if (pp.num_nodes != ra.M) continue;
    int qs = -1;
    for (int q = 0; q < 2; ++q)
      if (pp.abase[q] == ra.out_start) qs = q;
    if (qs < 0) continue;
    const int32_t ob = pp.abase[1 - qs];
    if (ob < ra.out_start + ra.M && ob + pp.num_nodes > ra.out_start) continue;
    sa.lr_prod = b.idx;
    sa.lr_qs = qs;
    pp.bwd_fused = true;
  }
  // G buffers, from the last layer down: a layer packed by the element-flow
  // product of the layer after it takes the other buffer.
  int next_slot = 0;
  for (int li = (int)h->layers.size() - 1; li >= 0; --li) {
    if (h->layers[li].kind != PC_LAYER_SUM) continue;
    SumPlan& sp = h->sums[h->layers[li].idx];
    sp.gbt_slot = sp.gp_done ? 1 - next_slot : 0;
    next_slot = sp.gbt_slot;
  }
  return h;
}

}  // namespace pc
