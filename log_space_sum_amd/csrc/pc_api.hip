// pc_api.hip -- the C ABI: handles, workspace plan, and the launch schedule of
// the forward pass, the backward pass (element flows, then the deferred
// parameter-flow products of every weight block with all its tied copies as
// one contraction) and the EM update.  Every launch goes on the caller's
// stream; nothing here allocates device memory or synchronises, except
// pc_compile_layout (index tables) and pc_kernel_times (waits on its events).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "pc_elem.h"
#include "pc_host.h"
#include "pc_kernels.h"

using namespace pc;

namespace {

thread_local std::string g_err;

int set_error(int code, const std::string& msg) {
  g_err = msg;
  return code;
}

#define HIPCHECK(x)                                                                       \
  do {                                                                                    \
    hipError_t e_ = (x);                                                                  \
    if (e_ != hipSuccess) fail(PC_ERR_HIP, std::string(#x) + ": " + hipGetErrorString(e_)); \
  } while (0)

template <typename T>
T* upload(const std::vector<T>& v) {
  if (v.empty()) return nullptr;
  T* d = nullptr;
  HIPCHECK(hipMalloc((void**)&d, v.size() * sizeof(T)));
  HIPCHECK(hipMemcpy(d, v.data(), v.size() * sizeof(T), hipMemcpyHostToDevice));
  return d;
}

template <typename T>
void release(T*& p) {
  if (p) (void)hipFree(p);
  p = nullptr;
}

struct DeviceGuard {
  int prev = -1;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) != hipSuccess) prev = -1;
    if (prev != dev) HIPCHECK(hipSetDevice(dev));
  }
  ~DeviceGuard() {
    int cur = -1;
    if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
  }
};

enum KernelKind {
  KK_FWD = 0, KK_ELEM, KK_PARAM, KK_SPLIT, KK_COLMAX, KK_EXP, KK_GPACK, KK_INFWD, KK_INBWD,
  KK_PRODFWD, KK_PRODBWD, KK_EM, KK_LRFWD, KK_LRBWD, KK_OTHER, KK_LRCOEF
};

}  // namespace

EventSink*& pc::event_sink() {
  static thread_local EventSink* sink = nullptr;
  return sink;
}

namespace {

// Times the launches made in its scope under one kernel kind when the handle
// times kernels: each launch stamps an event pair of its own (pc_launch.h).
struct Timed : EventSink {
  Handle* h;
  int kind;
  EventSink* prev = nullptr;
  bool on;
  Timed(Handle* h_, int kind_, hipStream_t) : h(h_), kind(kind_), on(h_->timing && !h_->no_events) {
    if (on) {
      prev = event_sink();
      event_sink() = this;
    }
  }
  ~Timed() override {
    if (on) event_sink() = prev;
  }
  void acquire(hipEvent_t* start, hipEvent_t* stop) override {
    if (h->events_used == h->events.size()) {
      Handle::Ev ev{kind, nullptr, nullptr};
      HIPCHECK(hipEventCreate((hipEvent_t*)&ev.start));
      HIPCHECK(hipEventCreate((hipEvent_t*)&ev.stop));
      h->events.push_back(ev);
    }
    Handle::Ev& ev = h->events[h->events_used++];
    ev.kind = kind;
    *start = (hipEvent_t)ev.start;
    *stop = (hipEvent_t)ev.stop;
  }
};

void check_launch() {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) fail(PC_ERR_HIP, std::string("kernel launch: ") + hipGetErrorString(e));
}

bool planes_ok(int pa, int pb) {
  return (pa == 1 && pb == 1) || (pa == 2 && pb == 1) || (pa == 1 && pb == 2) || (pa == 2 && pb == 2) ||
         (pa == 3 && pb == 3);
}

}  // namespace

namespace pc {

void upload_tables(Handle* h, int device) {
  HIPCHECK(hipSetDevice(device));
  h->device = device;
  for (auto& ip : h->inputs) {
    ip.d_var = upload(ip.var);
    ip.d_row = upload(ip.row);
    ip.d_row_ptr = upload(ip.row_ptr);
    ip.d_row_nodes = upload(ip.row_nodes);
    ip.d_var_ptr = upload(ip.var_ptr);
    ip.d_var_nodes = upload(ip.var_nodes);
  }
  for (auto& pp : h->prods) {
    pp.d_ch_ptr = upload(pp.ch_ptr);
    pp.d_ch_ids = upload(pp.ch_ids);
    pp.d_uchild = upload(pp.uchild);
    pp.d_pptr = upload(pp.pptr);
    pp.d_parents = upload(pp.parents);
  }
  for (auto& sp : h->sums) {
    sp.d_groups = upload(sp.groups);
    sp.d_blocks = upload(sp.blocks);
    sp.d_red_child = upload(sp.red_child);
    sp.d_red_ptr = upload(sp.red_ptr);
    sp.d_red_src = upload(sp.red_src);
    sp.d_up_idx = upload(sp.up_idx);
    sp.d_up_rest = upload(sp.up_rest);
    sp.d_up_rest_par = upload(sp.up_rest_par);
    sp.d_pk_group = upload(sp.pk_group);
    sp.d_pg_group = upload(sp.pg_group);
  }
  h->d_blocks = upload(h->blocks);
  h->d_vblocks = upload(h->vblocks);
  h->d_vgroups = upload(h->vgroups);
  h->d_rowsegs = upload(h->rowsegs);
  h->d_zero = upload(h->zero_ranges);
  h->d_seed = upload(h->seed_ranges);
}

void free_tables(Handle* h) {
  if (h->device < 0) return;
  int prev = -1;
  (void)hipGetDevice(&prev);
  (void)hipSetDevice(h->device);
  for (auto& ip : h->inputs) {
    release(ip.d_var);
    release(ip.d_row);
    release(ip.d_row_ptr);
    release(ip.d_row_nodes);
    release(ip.d_var_ptr);
    release(ip.d_var_nodes);
  }
  for (auto& pp : h->prods) {
    release(pp.d_ch_ptr);
    release(pp.d_ch_ids);
    release(pp.d_uchild);
    release(pp.d_pptr);
    release(pp.d_parents);
  }
  for (auto& sp : h->sums) {
    release(sp.d_groups);
    release(sp.d_blocks);
    release(sp.d_red_child);
    release(sp.d_red_ptr);
    release(sp.d_red_src);
    release(sp.d_up_idx);
    release(sp.d_up_rest);
    release(sp.d_up_rest_par);
    release(sp.d_pk_group);
    release(sp.d_pg_group);
  }
  release(h->d_blocks);
  release(h->d_vblocks);
  release(h->d_vgroups);
  release(h->d_rowsegs);
  release(h->d_zero);
  release(h->d_seed);
  for (auto& ev : h->events) {
    if (ev.start) (void)hipEventDestroy((hipEvent_t)ev.start);
    if (ev.stop) (void)hipEventDestroy((hipEvent_t)ev.stop);
  }
  h->events.clear();
  if (prev >= 0) (void)hipSetDevice(prev);
}

GemmShape layer_gemm_shape(const Handle* h, const SumPlan& sp, int kind, int B_pad, int pa, int pb) {
  const int rows256 = kind == GK_FWD ? sp.mtiles : sp.ctiles, kpad = kind == GK_FWD ? sp.max_npk : sp.max_mpk;
  // (wide levels of strided groups keep the automatic 128 x 64 tiles too: with
  // the weights in registers, 128 x 128 tiles ran the HCLT step no faster)
  return layer_shape(rows256, B_pad, kpad, pa, pb, h->opt_layer_tile, h->opt_split_max);
}

// The LowRank "sum_exp" virtual batch runs (no fused kernels asked for).
bool vsum_active(const Handle* h) {
  return h->lowrank_form == PC_LOWRANK_SUM_EXP && !h->vblocks.empty() && !h->opt_sumexp_fused;
}

// Shape of a virtual-batch product over one LowRank group: rows M (forward,
// weights) or N (element side, transposed weights), Qpad virtual columns, K
// the other dimension; the automatic tiles only.
GemmShape vb_gemm_shape(const Handle* h, const GroupRec& r, bool elem, int Qpad, int pa, int pb) {
  const int rows = elem ? r.N : r.M, K = elem ? r.M : r.N;
  return layer_shape((int)(round_up(rows, ROW_PAD) / ROW_PAD), Qpad, (int)round_up(K, K_PAD), pa, pb, TILE_AUTO,
                     h->opt_split_max);
}

GemmShape param_gemm_shape_tiles(const Handle* h, int pa, int pb, int tiles256, int tiles128);

// K split of a parameter-flow launch with `tiles` output tiles over
// `kslices` 32-wide K slices (its copies' samples): a power of two up to 8
// until the launch has 256 workgroups, keeping >= 8 slices per split.
int param_splitk(int tiles, int64_t kslices) {
  int S = 1;
  while (tiles * S < 256 && S * 2 <= 8 && kslices / (S * 2) >= 8) S *= 2;
  return S;
}

// K split of an e4m3 parameter-flow launch with `tiles` 128 x 128 tiles over
// `ksteps` 64-wide K steps: a power of two up to 16 until the launch has 256
// workgroups (one per CU; measured: 1024^2 outputs over 64512 K take 185 us
// with 4 splits, 215 us with 8, 346 us with 16), keeping >= 8 steps per split.
int f8_splitk(int tiles, int64_t ksteps) {
  int S = 1;
  while (tiles * S < 256 && S * 2 <= 16 && ksteps / (S * 2) >= 8) S *= 2;
  return S;
}

GemmShape param_gemm_shape(const Handle* h, int pa, int pb) {
  return param_gemm_shape_tiles(h, pa, pb, h->param_tiles256, h->param_tiles128);
}

GemmShape param_gemm_shape_tiles(const Handle* h, int pa, int pb, int tiles256, int tiles128) {
  GemmShape g{};
  // Automatic: 128 x 256 when the first operand (G) has more planes than the
  // second, else 128 x 128: fewer bytes per output at the same K (HMM-4096
  // parameter flows, G split in two: 128 x 256 7% faster than 128 x 128, which
  // was faster than 256 x 256, whose one long tile per CU leaves a tail)
  const bool big = pa + pb <= 3 && h->opt_param_tile == TILE_256x256;   // rows are padded to 256
  const bool wide = !big && (h->opt_param_tile == TILE_128x256 || (h->opt_param_tile == TILE_AUTO && pa > pb));
  g.tile = big ? TILE_256x256 : wide ? TILE_128x256 : TILE_128x128;
  g.mt = big ? 256 : 128;
  g.nt = big || wide ? 256 : 128;
  g.splitk = 1;
  g.tiles = big ? tiles256 : wide ? 2 * tiles256 : tiles128;
  return g;
}

WsPlan plan_workspace(const Handle* h, int B, bool fwd_only) {
  WsPlan p{};
  p.B = B;
  p.fwd_only = fwd_only;
  p.B_padK = (int)round_up(B, K_PAD);
  p.mode = effective_mode(h, B);
  for (int k = 0; k < 3; ++k)
    for (int j = 0; j < 2; ++j) p.pl[k][j] = h->planes[p.mode][k][j];
  // the batch-major operands hold whole column tiles of the per-layer
  // products (and whole 64-sample packing tiles), no more
  {
    const int nt = std::max(layer_tile_nt(p.pl[GK_FWD][0], p.pl[GK_FWD][1], h->opt_layer_tile),
                            layer_tile_nt(p.pl[GK_ELEM][0], p.pl[GK_ELEM][1], h->opt_layer_tile));
    p.B_pad = (int)round_up(B, std::max(nt, 64));
  }
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = (size_t)round_up((int64_t)(off + bytes), 256);
    return o;
  };
  const size_t Bp = p.B_pad, BpK = p.B_padK, Bs = B;
  // regions only the backward reads (the transposed weights, the operands
  // kept for the parameter flows, the scaled sums, the element-flow scratch,
  // the input-flow buckets) are left out of a forward-only plan
  const size_t bw = fwd_only ? 0 : 1;
  p.theta = take((size_t)p.pl[GK_FWD][0] * h->theta_elems * 2);
  p.thetaT = take(bw * p.pl[GK_ELEM][0] * h->thetaT_elems * 2);
  p.ebt = take((size_t)p.pl[GK_FWD][1] * Bp * h->max_ebt_cols * 2);
  p.gbt = take(bw * p.pl[GK_ELEM][1] * Bp * h->max_gbt_cols * 2);
  p.gbt2 = take(bw * (h->gbt_slots > 1 && gp_batch_ok(B) ?   // independent of the fusion option
                        (size_t)p.pl[GK_ELEM][1] * Bp * h->max_gbt_cols * 2 : 0));
  p.earena = take(bw * p.pl[GK_PARAM][1] * h->earena_rows * BpK * 2);
  p.garena = take(bw * p.pl[GK_PARAM][0] * h->garena_rows * BpK * 2);
  p.mkeys = take((size_t)h->m_rows * Bs * 4);
  p.ssum = take(bw * h->s_rows * Bs * 4);
  p.scratch = take(bw * h->max_scratch_rows * Bs * 4);
  const bool inp = !h->inputs.empty();
  p.tokT = take(inp ? (size_t)h->num_vars * Bs * 4 : 0);
  p.bptr = take(inp ? bw * h->num_vars * (h->max_cats + 1) * 4 : 0);
  p.bidx = take(inp ? bw * h->num_vars * Bs * 4 : 0);
  // split-K partial tiles and arrival counters (forward / element flows)
  {
    int64_t pel = 0;
    int32_t nct = 0;
    for (const auto& sp : h->sums) {
      if (sp.lowrank) continue;
      for (int e = 0; e < 2; ++e) {
        const GemmShape g = layer_gemm_shape(h, sp, e, p.B_pad, p.pl[e][0], p.pl[e][1]);
        if (g.splitk > 1) pel = std::max<int64_t>(pel, (int64_t)g.tiles * g.splitk * g.mt * g.nt);
        nct = std::max(nct, g.tiles);
      }
    }
    if (vsum_active(h)) {
      const int Qv = B * h->lowrank_rank;
      const int nt = std::max(layer_tile_nt(p.pl[GK_FWD][0], p.pl[GK_FWD][1], TILE_AUTO),
                              layer_tile_nt(p.pl[GK_ELEM][0], p.pl[GK_ELEM][1], TILE_AUTO));
      const int Qpad = (int)round_up(2 * (int64_t)Qv, std::max(nt, 64));
      for (const auto& r : h->vgroups)
        for (int e = 0; e < 2; ++e) {
          const GemmShape g = vb_gemm_shape(h, r, e == 1, Qpad, p.pl[e][0], p.pl[e][1]);
          if (g.splitk > 1) pel = std::max<int64_t>(pel, (int64_t)g.tiles * g.splitk * g.mt * g.nt);
          nct = std::max(nct, g.tiles);
        }
    }
    p.partial_elems = pel;
    p.ncounters = nct;
    p.partials = take((size_t)pel * 4);
    p.counters = take((size_t)nct * 4);
    // the parameter-flow launches: every plain block at once, one block
    // (chunks on the second stream), the LowRank "sum_exp" blocks
    int64_t ppel = 0;
    int32_t pct = 0;
    auto consider = [&](const GemmShape& g, int64_t kslices) {
      const int S = param_splitk(g.tiles, kslices);
      if (S > 1) ppel = std::max<int64_t>(ppel, (int64_t)g.tiles * S * g.mt * g.nt);
      pct = std::max(pct, g.tiles);
    };
    if (!bw) {
    } else if (h->has_plain_sums) {
      const GemmShape g = param_gemm_shape(h, p.pl[GK_PARAM][0], p.pl[GK_PARAM][1]);
      int64_t kmin = INT64_MAX;
      for (const BlockRec& bl : h->blocks)
        if (bl.ncopies > 0) {
          kmin = std::min<int64_t>(kmin, (int64_t)bl.ncopies * (p.B_padK / 32));
          GemmShape gb = g;
          gb.tiles = (int)((round_up(bl.M, ROW_PAD) / g.mt) * (round_up(bl.N, ROW_PAD) / g.nt));
          consider(gb, (int64_t)bl.ncopies * (p.B_padK / 32));   // a chunk of all its copies at most
        }
      if (kmin != INT64_MAX) consider(g, kmin);
    }
    if (bw && vsum_active(h)) {
      const int QK = (int)round_up((int64_t)B * h->lowrank_rank, K_PAD);
      const GemmShape g = param_gemm_shape_tiles(h, p.pl[GK_PARAM][0], p.pl[GK_PARAM][1], h->v_param_tiles256,
                                                 h->v_param_tiles128);
      int64_t kmin = INT64_MAX;
      for (const BlockRec& bl : h->vblocks) kmin = std::min<int64_t>(kmin, (int64_t)bl.ncopies * (QK / 32));
      if (kmin == INT64_MAX) {
      } else if (h->opt_flow_fp8 && p.mode == PC_PREC_AUTO) {
        const int S = f8_splitk(h->v_param_tiles128, kmin / 2);
        if (S > 1) ppel = std::max<int64_t>(ppel, (int64_t)h->v_param_tiles128 * S * 128 * 128);
        pct = std::max(pct, h->v_param_tiles128);
      } else {
        consider(g, kmin);
      }
    }
    p.npcounters = pct;
    p.ppartials = take((size_t)ppel * 4);
    p.pcounters = take((size_t)pct * 4);
  }
  // LowRank: exp of the children (per layer), kept Z/S/U/W, per-layer
  // coefficients, parameter-flow partials (ceil(B/8) copies of each block)
  p.lr_nsg = (B + 7) / 8;
  const bool lr = h->lowrank_slots > 0;
  const size_t kr = (size_t)h->lowrank_rank;
  const size_t lr0 = off;
  p.lrZ = take(lr ? (size_t)h->lr_rows * Bs * 4 : 0);
  p.lrS = take(lr ? (size_t)h->lr_rows * Bs * 4 : 0);
  p.lrU = take(lr ? (size_t)h->lr_rows * Bs * kr * 4 : 0);
  p.lrW = take(lr ? (size_t)h->lr_rows * Bs * kr * 4 : 0);
  p.lrC1 = take(lr ? bw * round_up(h->lr_max_m, 32) * Bs * 4 : 0);   // rows padded to 32 (zeros)
  p.lrC2 = take(lr ? bw * round_up(h->lr_max_m, 32) * Bs * 4 : 0);
  // the fused kernels' parameter-flow partials and fragment records (not
  // used by the "sum_exp" virtual batch)
  p.vsum = vsum_active(h);
  const size_t fz = p.vsum ? 0 : 1;
  p.lrP = take(lr ? fz * bw * p.lr_nsg * h->lr_p_elems * 4 : 0);
  p.lrPz = take(lr ? fz * bw * p.lr_nsg * h->lr_p_elems * 4 : 0);
  {
    size_t pk = 0;
    for (const auto& sp : h->sums)
      for (const auto& r : sp.groups)
        if (r.lowrank >= 0) {
          p.lr_pk_off.push_back((int64_t)pk);
          pk += fz * (size_t)round_up(lr_pack_bytes(B, r.M, r.N, (int)kr, p.mode == PC_PREC_FP32), 256);
        }
    p.lrPK = take(pk);
  }
  // "sum_exp" virtual batch: batch-major operand, node-major arenas, backward products
  if (p.vsum) {
    p.Qv = B * (int)kr;
    p.QK = (int)round_up(p.Qv, K_PAD);
    const int nt = std::max(layer_tile_nt(p.pl[GK_FWD][0], p.pl[GK_FWD][1], TILE_AUTO),
                            layer_tile_nt(p.pl[GK_ELEM][0], p.pl[GK_ELEM][1], TILE_AUTO));
    p.Qpad = (int)round_up(2 * (int64_t)p.Qv, std::max(nt, 64));
    const size_t npb = (size_t)std::max(p.pl[GK_FWD][1], p.pl[GK_ELEM][1]);
    p.vbt = take(npb * p.Qpad * h->v_max_k * 2);
    // the end products' node-major operands: bf16 planes, or e4m3 bytes and
    // scales (PC_OPT_FLOW_FP8 in auto mode)
    p.vf8 = bw && h->opt_flow_fp8 && p.mode == PC_PREC_AUTO;
    const size_t b16 = bw && !p.vf8 ? 1 : 0, b8 = p.vf8 ? 1 : 0;
    p.vX = take(b16 * p.pl[GK_PARAM][1] * h->vx_rows * p.QK * 2);
    p.vC = take(b16 * p.pl[GK_PARAM][1] * h->vx_rows * p.QK * 2);
    p.vY1 = take(b16 * p.pl[GK_PARAM][0] * h->vy_rows * p.QK * 2);
    p.vY2 = take(b16 * p.pl[GK_PARAM][0] * h->vy_rows * p.QK * 2);
    p.vX8 = take(b8 * h->vx_rows * p.QK);
    p.vC8 = take(b8 * h->vx_rows * p.QK);
    p.vY18 = take(b8 * h->vy_rows * p.QK);
    p.vY28 = take(b8 * h->vy_rows * p.QK);
    p.vXs = take(b8 * h->vx_rows * (p.QK / 32));
    p.vCs = take(b8 * h->vx_rows * (p.QK / 32));
    p.vY1s = take(b8 * h->vy_rows * (p.QK / 32));
    p.vY2s = take(b8 * h->vy_rows * (p.QK / 32));
    p.vR = take(bw * 2 * (size_t)B * h->lr_max_n * kr * 4);
  }
  p.lowrank = lr0;
  p.lowrank_bytes = off - lr0;
  p.total = off;
  return p;
}

WsView make_view(const Handle* h, const WsPlan& p, void* ws) {
  char* base = (char*)ws;
  WsView v{};
  v.theta = (uint16_t*)(base + p.theta);
  v.thetaT = (uint16_t*)(base + p.thetaT);
  v.theta_plane = h->theta_elems;
  v.thetaT_plane = h->thetaT_elems;
  v.ebt = (uint16_t*)(base + p.ebt);
  v.gbt = (uint16_t*)(base + p.gbt);
  v.gbt2 = (uint16_t*)(base + p.gbt2);
  v.ebt_plane = (int64_t)p.B_pad * h->max_ebt_cols;
  v.gbt_plane = (int64_t)p.B_pad * h->max_gbt_cols;
  v.earena = (uint16_t*)(base + p.earena);
  v.garena = (uint16_t*)(base + p.garena);
  v.earena_plane = h->earena_rows * p.B_padK;
  v.garena_plane = h->garena_rows * p.B_padK;
  v.mkeys = (uint32_t*)(base + p.mkeys);
  v.ssum = (float*)(base + p.ssum);
  v.scratch = (float*)(base + p.scratch);
  v.tokT = (int32_t*)(base + p.tokT);
  v.bucket_ptr = (int32_t*)(base + p.bptr);
  v.bucket_idx = (int32_t*)(base + p.bidx);
  v.partials = (float*)(base + p.partials);
  v.counters = (uint32_t*)(base + p.counters);
  v.ncounters = p.ncounters;
  v.B = p.B;
  v.B_pad = p.B_pad;
  v.B_padK = p.B_padK;
  return v;
}

}  // namespace pc

// ---------------------------------------------------------------------------
// schedule helpers
// ---------------------------------------------------------------------------
namespace {

Handle* checked(pc_handle hh) {
  if (!hh) fail(PC_ERR_INVALID_ARG, "null handle");
  return reinterpret_cast<Handle*>(hh);
}

struct Call {
  Handle* h;
  WsPlan p;
  WsView v;
  hipStream_t s;
  void* ws;
};

Call begin_call(pc_handle hh, int B, void* ws, size_t ws_bytes, void* stream, bool fwd_only = false) {
  Handle* h = checked(hh);
  if (h->device < 0) fail(PC_ERR_NO_DEVICE, "handle was compiled without a device");
  if (B < 1) fail(PC_ERR_INVALID_ARG, "batch must be >= 1");
  if (!h->inputs.empty() && (size_t)(h->max_cats + 1 + B) * 4 > 65536)
    fail(PC_ERR_UNSUPPORTED, "categories + batch too large for the input-flow bucketing (limit 16383)");
  Call c{h, plan_workspace(h, B, fwd_only), {}, (hipStream_t)stream, ws};
  if (c.p.total > 0 && !ws) fail(PC_ERR_INVALID_ARG, "null workspace");
  if (ws_bytes < c.p.total)
    fail(PC_ERR_WORKSPACE, "workspace too small: need " + std::to_string(c.p.total) + " bytes, got " +
                               std::to_string(ws_bytes));
  c.v = make_view(h, c.p, ws);
  return c;
}

GemmArgs gemm_common(const Call& c) {
  GemmArgs a{};
  a.B = c.v.B;
  a.B_pad = c.v.B_pad;
  a.B_padK = c.v.B_padK;
  a.rowsA = c.h->garena_rows;
  a.rowsB = c.h->earena_rows;
  a.ntiles = c.v.B_pad / 128;
  a.blocks = c.h->d_blocks;
  a.partials = c.v.partials;
  a.counters = c.v.counters;
  a.copy_lo = 0;
  a.copy_hi = 1 << 30;
  a.tile0 = 0;
  return a;
}

SumArgs sum_common(const Call& c, const SumPlan& sp) {
  SumArgs a{};
  a.B = c.v.B;
  a.B_pad = c.v.B_pad;
  a.B_padK = c.v.B_padK;
  a.btiles = c.v.B_pad / 64;
  a.ngroups = (int)sp.groups.size();
  a.groups = sp.d_groups;
  a.pk_group = sp.d_pk_group;
  a.pg_group = sp.d_pg_group;
  if (sp.groups.size() == 1) a.group0 = sp.groups[0];
  a.chblocks = sp.d_blocks;
  a.mkeys = c.v.mkeys;
  return a;
}

InputArgs input_args(const Call& c, const InputPlan& ip, const float* params) {
  InputArgs a{};
  a.B = c.v.B;
  a.node_start = ip.node_start;
  a.num_nodes = ip.num_nodes;
  a.K = ip.num_cats;
  a.num_rows = ip.num_rows;
  a.Kmax = c.h->max_cats;
  a.max_row_nodes = ip.max_row_nodes;
  a.param_offset = ip.param_offset;
  a.var = ip.d_var;
  a.row = ip.d_row;
  a.row_ptr = ip.d_row_ptr;
  a.row_nodes = ip.d_row_nodes;
  a.var_ptr = ip.d_var_ptr;
  a.var_nodes = ip.d_var_nodes;
  a.num_vars = c.h->num_vars;
  a.max_var_nodes = ip.max_var_nodes;
  a.tokT = c.v.tokT;
  a.bptr = c.v.bucket_ptr;
  a.bidx = c.v.bucket_idx;
  a.params = params;
  return a;
}

void check_lowrank_io(const Handle* h, const pc_lowrank_io* io, bool backward) {
  if (h->lowrank_slots == 0) return;
  if (!io) fail(PC_ERR_INVALID_ARG, "the circuit has LowRank groups: lowrank factors are required");
  if (io->num_slots < h->lowrank_slots || !io->A || !io->B)
    fail(PC_ERR_INVALID_ARG, "lowrank: need A and B for " + std::to_string(h->lowrank_slots) + " slots");
  if (backward && (!io->dA || !io->dB)) fail(PC_ERR_INVALID_ARG, "lowrank: pc_backward needs dA and dB");
  for (const auto& sp : h->sums)
    for (const auto& r : sp.groups)
      if (r.lowrank >= 0) {
        if (!io->A[r.lowrank] || !io->B[r.lowrank]) fail(PC_ERR_INVALID_ARG, "lowrank: null factor");
        if (backward && (!io->dA[r.lowrank] || !io->dB[r.lowrank])) fail(PC_ERR_INVALID_ARG, "lowrank: null gradient");
      }
}

LRArgs lr_args(const Call& c, const SumPlan& sp, int g, const pc_lowrank_io* io, const float* params, float* vals,
               float* flows) {
  const Handle* h = c.h;
  const GroupRec& r = sp.groups[g];
  char* base = (char*)c.ws;
  const int64_t B = c.v.B, kr = h->lowrank_rank;
  LRArgs a{};
  a.B = c.v.B;
  a.M = r.M;
  a.N = r.N;
  a.krank = h->lowrank_rank;
  a.sumexp = h->lowrank_form == PC_LOWRANK_SUM_EXP ? 1 : 0;
  a.out_start = r.out_start;
  a.m_row = r.m_row;
  a.cbs = r.cbs;
  a.blk_off = r.blk_off;
  a.scratch_row = r.scratch_row;
  a.store = sp.store ? 1 : 0;
  a.chblocks = sp.d_blocks;
  a.theta = params + r.param_offset;
  a.A = io->A[r.lowrank];
  a.Bf = io->B[r.lowrank];
  a.mkeys = c.v.mkeys;
  a.vals = vals;
  a.flows = flows;
  a.out_flows = flows;
  a.scratch = c.v.scratch;
  a.Z = (float*)(base + c.p.lrZ) + sp.lr_row[g] * B;
  a.S = (float*)(base + c.p.lrS) + sp.lr_row[g] * B;
  a.U = (float*)(base + c.p.lrU) + sp.lr_row[g] * B * kr;
  a.W = (float*)(base + c.p.lrW) + sp.lr_row[g] * B * kr;
  a.C1 = (float*)(base + c.p.lrC1);
  a.C2 = (float*)(base + c.p.lrC2);
  a.P = (float*)(base + c.p.lrP) + h->lr_p_off[r.block] * c.p.lr_nsg;
  a.pk = (uint16_t*)(base + c.p.lrPK + c.p.lr_pk_off[sp.lr_gidx[g]]);
  if (io->dA) a.dA = io->dA[r.lowrank];
  if (io->dB) a.dB = io->dB[r.lowrank];
  return a;
}

// Fragment records of LowRank group g of `sp`, in its own launch.
void lr_pack_group(const Call& c, const SumPlan& sp, int g, const pc_lowrank_io* io) {
  const GroupRec& r = sp.groups[g];
  LRPackArgs pa{};
  pa.B = c.v.B;
  pa.krank = c.h->lowrank_rank;
  pa.sumexp = c.h->lowrank_form == PC_LOWRANK_SUM_EXP ? 1 : 0;
  pa.ngroups = 1;
  pa.M[0] = r.M;
  pa.N[0] = r.N;
  pa.A[0] = io->A[r.lowrank];
  pa.Bf[0] = io->B[r.lowrank];
  pa.pk[0] = (uint16_t*)((char*)c.ws + c.p.lrPK + c.p.lr_pk_off[sp.lr_gidx[g]]);
  pa.wg0[0] = 0;
  pa.wg0[1] = lr_pack_workgroups(c.v.B, r.M, r.N, c.h->lowrank_rank);
  launch_lr_pack(pa, c.p.mode == PC_PREC_FP32, c.s);
}

// One LowRank group's virtual-batch arguments (forward: X / C operands;
// backward: Y1 / Y2).
VBArgs vb_args(const Call& c, const SumPlan& sp, int g, const pc_lowrank_io* io, float* vals, float* flows,
               bool bwd) {
  const Handle* h = c.h;
  const GroupRec& r = sp.groups[g];
  const GroupRec& vr = h->vgroups[sp.lr_gidx[g]];
  char* base = (char*)c.ws;
  const int64_t B = c.v.B, kr = h->lowrank_rank;
  VBArgs a{};
  a.B = c.v.B;
  a.M = r.M;
  a.N = r.N;
  a.krank = h->lowrank_rank;
  a.Q = c.p.Qv;
  a.Qpad = c.p.Qpad;
  a.QK = c.p.QK;
  a.out_start = r.out_start;
  a.m_row = r.m_row;
  a.cbs = r.cbs;
  a.blk_off = r.blk_off;
  a.scratch_row = r.scratch_row;
  a.store = sp.store ? 1 : 0;
  a.chblocks = sp.d_blocks;
  a.A = io->A[r.lowrank];
  a.Bf = io->B[r.lowrank];
  a.mkeys = c.v.mkeys;
  a.vals = vals;
  a.out_flows = flows;
  a.scratch = c.v.scratch;
  a.vbt = (uint16_t*)(base + c.p.vbt);
  a.vbt_plane = (int64_t)c.p.Qpad * h->v_max_k;
  a.np_bt = c.p.pl[bwd ? GK_ELEM : GK_FWD][1];
  const int npn = c.p.pl[GK_PARAM][bwd ? 0 : 1];
  a.np_n = c.p.fwd_only ? 0 : npn;
  a.nlo = (uint16_t*)(base + (bwd ? c.p.vY1 : c.p.vX));
  a.nhi = (uint16_t*)(base + (bwd ? c.p.vY2 : c.p.vC));
  a.n_rows = bwd ? h->vy_rows : h->vx_rows;
  a.n_plane = a.n_rows * c.p.QK;
  a.n_row0 = bwd ? vr.g_row : vr.e_row;
  if (c.p.vf8) {
    a.f8 = 1;
    a.np_n = 0;
    a.n8lo = (uint8_t*)(base + (bwd ? c.p.vY18 : c.p.vX8));
    a.n8hi = (uint8_t*)(base + (bwd ? c.p.vY28 : c.p.vC8));
    a.s8lo = (uint8_t*)(base + (bwd ? c.p.vY1s : c.p.vXs));
    a.s8hi = (uint8_t*)(base + (bwd ? c.p.vY2s : c.p.vCs));
  }
  a.C1 = (const float*)(base + c.p.lrC1);
  a.C2 = (const float*)(base + c.p.lrC2);
  a.Z = (float*)(base + c.p.lrZ) + sp.lr_row[g] * B;
  a.S = (float*)(base + c.p.lrS) + sp.lr_row[g] * B;
  a.U = (const float*)(base + c.p.lrU) + sp.lr_row[g] * B * kr;
  a.W = (const float*)(base + c.p.lrW) + sp.lr_row[g] * B * kr;
  a.R1 = (const float*)(base + c.p.vR);
  a.R2 = (const float*)(base + c.p.vR) + (size_t)B * h->lr_max_n * kr;
  if (io->dB) a.dB = io->dB[r.lowrank];
  return a;
}

// The virtual-batch product of one LowRank group: weights (forward) or
// transposed weights (backward) times the batch-major operand, stored to
// lo / hi in [B, rows, k].
void vb_product(const Call& c, const SumPlan& sp, int g, bool elem, float* lo, float* hi) {
  const Handle* h = c.h;
  const int gi = sp.lr_gidx[g];
  const GroupRec& vr = h->vgroups[gi];
  const int kind = elem ? GK_ELEM : GK_FWD;
  const int pa = c.p.pl[kind][0], pb = c.p.pl[kind][1];
  GemmArgs a = gemm_common(c);
  a.B = 2 * c.p.Qv;
  a.B_pad = c.p.Qpad;
  a.ngroups = 1;
  a.groups = h->d_vgroups + gi;
  a.blocks = h->d_vblocks;
  a.opA = elem ? c.v.thetaT : c.v.theta;
  a.planeA = elem ? c.v.thetaT_plane : c.v.theta_plane;
  a.opB = (const uint16_t*)((const char*)c.ws + c.p.vbt);
  a.planeB = (int64_t)c.p.Qpad * h->v_max_k;
  a.vs_elem = elem ? 1 : 0;
  a.vs_rank = h->lowrank_rank;
  a.vs_half = c.p.Qv;
  a.vs_lo = lo;
  a.vs_hi = hi;
  const GemmShape shp = vb_gemm_shape(h, vr, elem, c.p.Qpad, pa, pb);
  a.ntiles = c.p.Qpad / shp.nt;
  a.splitk = shp.splitk;
  launch_gemm(EPI_VSTORE, pa, pb, shp, a, c.s);
}

ProdArgs prod_args(const Call& c, const ProductPlan& pp) {
  ProdArgs a{};
  a.B = c.v.B;
  a.node_start = pp.node_start;
  a.num_nodes = pp.num_nodes;
  a.nuniq = (int)pp.uchild.size();
  a.store = pp.store ? 1 : 0;
  a.ch_ptr = pp.d_ch_ptr;
  a.ch_ids = pp.d_ch_ids;
  a.uchild = pp.d_uchild;
  a.pptr = pp.d_pptr;
  a.parents = pp.d_parents;
  a.affine = pp.affine ? 1 : 0;
  a.deg = pp.max_deg;
  for (int q = 0; q < 8; ++q) a.abase[q] = pp.abase[q];
  return a;
}

}  // namespace

namespace {

// Scratch of pc_forward_static, for callers that cannot allocate device
// memory.  Each device holds its own copy until the process ends.  Host code
// must not use the array's name as an address: the device address of each
// device's copy is resolved once per device (with that device current) by
// hipGetSymbolAddress and kept in g_static.
__device__ __align__(256) unsigned char scratch[PC_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
struct StaticScratch {
  std::mutex mu;
  bool tried[kMaxDevices] = {};
  hipError_t err[kMaxDevices] = {};
  void* ptr[kMaxDevices] = {};
};
StaticScratch g_static;

// Resolve `scratch` on `device`, which must be current (once per device).
void resolve_static_scratch(int device) {
  if (device < 0 || device >= kMaxDevices) return;
  std::lock_guard<std::mutex> lk(g_static.mu);
  if (g_static.tried[device]) return;
  g_static.tried[device] = true;
  void* ptr = nullptr;
  g_static.err[device] = hipGetSymbolAddress((void**)&ptr, HIP_SYMBOL(scratch));
  g_static.ptr[device] = g_static.err[device] == hipSuccess ? ptr : nullptr;
}

void* static_scratch(int device) {
  if (device < 0 || device >= kMaxDevices) fail(PC_ERR_UNSUPPORTED, "device id too large for the static scratch table");
  std::lock_guard<std::mutex> lk(g_static.mu);
  if (!g_static.tried[device]) fail(PC_ERR_HIP, "static scratch was not resolved for this device");
  if (g_static.err[device] != hipSuccess)
    fail(PC_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(g_static.err[device]));
  return g_static.ptr[device];
}

// Clears Handle::no_events when the call ends (however it ends).
struct NoEvents {
  Handle* h;
  explicit NoEvents(Handle* h_) : h(h_) { h->no_events = true; }
  ~NoEvents() { h->no_events = false; }
};

// The forward pass of one call: every launch on c.s, nothing allocated.  A
// forward-only call (c.p.fwd_only) writes none of what only the backward
// reads: the transposed weight planes, the kept E planes and the scaled sums.
void run_forward(const Call& c, const int32_t* tokens, const float* params, float* node_vals, float* ll,
                 const pc_lowrank_io* lowrank) {
  Handle* h = c.h;
  check_lowrank_io(h, lowrank, false);
  if (!params || !node_vals) fail(PC_ERR_INVALID_ARG, "null params or node_vals");
  if (!h->inputs.empty() && !tokens) fail(PC_ERR_INVALID_ARG, "null tokens");
  if (ll && h->root < 0) fail(PC_ERR_INVALID_ARG, "ll requested but the circuit has no root");
  DeviceGuard dg(h->device);
  const int B = c.v.B;
  const WsPlan& p = c.p;
  const WsView& v = c.v;
  if (h->has_plain_sums) {
    ThetaArgs ta{};
    ta.nblocks = (int)h->blocks.size();
    ta.np_fwd = p.pl[GK_FWD][0];
    ta.np_elem = p.fwd_only ? 0 : p.pl[GK_ELEM][0];   // the transposed weights serve the backward only
    ta.blocks = h->d_blocks;
    ta.params = params;
    ta.theta = v.theta;
    ta.theta_plane = v.theta_plane;
    ta.thetaT = v.thetaT;
    ta.thetaT_plane = v.thetaT_plane;
    Timed t(h, KK_SPLIT, c.s);
    launch_theta_pack(ta, h->pk_block_tiles, c.s);
  }
  if (p.vsum) {
    // weight planes of the LowRank "sum_exp" blocks (virtual-batch products)
    ThetaArgs ta{};
    ta.nblocks = (int)h->vblocks.size();
    ta.np_fwd = p.pl[GK_FWD][0];
    ta.np_elem = p.fwd_only ? 0 : p.pl[GK_ELEM][0];
    ta.blocks = h->d_vblocks;
    ta.params = params;
    ta.theta = v.theta;
    ta.theta_plane = v.theta_plane;
    ta.thetaT = v.thetaT;
    ta.thetaT_plane = v.thetaT_plane;
    Timed t(h, KK_SPLIT, c.s);
    launch_theta_pack(ta, h->v_pk_tiles, c.s);
  }
  if (!h->inputs.empty()) {
    Timed t(h, KK_OTHER, c.s);
    launch_tokens_t(tokens, v.tokT, B, h->num_vars, c.s);
  }
  if (h->m_rows > 0) {
    Timed t(h, KK_OTHER, c.s);
    launch_fill_u32(v.mkeys, (int64_t)h->m_rows * B, 0u, c.s);
  }
  if (p.ncounters > 0) {
    Timed t(h, KK_OTHER, c.s);
    launch_fill_u32(v.counters, p.ncounters, 0u, c.s);
  }
  if (h->lowrank_slots > 0 && h->opt_lr_pack == 0 && !p.vsum) {
    // the fragment records of every LowRank group's factors, kept for the backward
    LRPackArgs pa{};
    pa.B = B;
    pa.krank = h->lowrank_rank;
    pa.sumexp = h->lowrank_form == PC_LOWRANK_SUM_EXP ? 1 : 0;
    auto flush = [&]() {
      if (pa.ngroups == 0) return;
      Timed t(h, KK_SPLIT, c.s);
      launch_lr_pack(pa, p.mode == PC_PREC_FP32, c.s);
      pa.ngroups = 0;
    };
    for (const auto& sp : h->sums)
      for (size_t gi = 0; gi < sp.groups.size(); ++gi) {
        const GroupRec& r = sp.groups[gi];
        if (r.lowrank < 0) continue;
        const int q = pa.ngroups;
        if (q == 0) pa.wg0[0] = 0;
        pa.M[q] = r.M;
        pa.N[q] = r.N;
        pa.A[q] = lowrank->A[r.lowrank];
        pa.Bf[q] = lowrank->B[r.lowrank];
        pa.pk[q] = (uint16_t*)((char*)c.ws + p.lrPK + p.lr_pk_off[sp.lr_gidx[gi]]);
        pa.wg0[q + 1] = pa.wg0[q] + lr_pack_workgroups(B, r.M, r.N, h->lowrank_rank);
        if (++pa.ngroups == kMaxPackGroups) flush();
      }
    flush();
  }
  for (const LayerRef& r : h->layers) {
    if (r.kind == PC_LAYER_INPUT_CAT) {
      InputArgs a = input_args(c, h->inputs[r.idx], params);
      a.vals = node_vals;
      Timed t(h, KK_INFWD, c.s);
      launch_input_fwd(a, c.s);
    } else if (r.kind == PC_LAYER_PRODUCT) {
      if (h->opt_fuse && h->prods[r.idx].fwd_fused) continue;   // evaluated by the next layer's column maxima
      ProdArgs a = prod_args(c, h->prods[r.idx]);
      a.vals = node_vals;
      Timed t(h, KK_PRODFWD, c.s);
      launch_prod_fwd(a, c.s);
    } else if (r.kind == PC_LAYER_SUM) {
      const SumPlan& sp = h->sums[r.idx];
      SumArgs a = sum_common(c, sp);
      a.vals = node_vals;
      a.direct = v.earena;
      a.direct_plane = v.earena_plane;
      a.np_direct = p.fwd_only ? 0 : p.pl[GK_PARAM][1];   // node-major E is kept for the parameter flows
      a.trans = v.ebt;
      a.trans_plane = v.ebt_plane;
      a.direct_rows = h->earena_rows;
      a.np_trans = p.pl[GK_FWD][1];
      if (h->opt_fuse && sp.fwd_prod >= 0) {
        const ProductPlan& pp = h->prods[sp.fwd_prod];
        a.fp_on = 1;
        a.fp_start = pp.node_start;
        a.fp_count = pp.num_nodes;
        a.fp_maxdeg = pp.max_deg;
        a.fp_ptr = pp.d_ch_ptr;
        a.fp_ids = pp.d_ch_ids;
        a.fp_affine = pp.affine ? 1 : 0;
        for (int q = 0; q < 8; ++q) a.fp_abase[q] = pp.abase[q];
        a.wvals = node_vals;
      }
      // the column maxima are published by the previous layer when it has a
      // product epilogue: plain layers' forward products and the fused
      // LowRank forward kernels (not the "sum_exp" virtual batch)
      const bool published = h->opt_fuse && sp.epi_max && !(p.vsum && h->sums[sp.epi_src].lowrank);
      if (!published) {
        Timed t(h, KK_COLMAX, c.s);
        launch_colmax(a, sp.pktiles, c.s);
      }
      a.fp_on = 0;
      if (sp.lowrank) {
        for (int gi = 0; gi < (int)sp.groups.size(); ++gi) {
          if (p.vsum) {
            // "sum_exp" on the virtual batch: X, C operands; theta [X | C]^T
            // into U, W; the rank reduction and the node values
            VBArgs va = vb_args(c, sp, gi, lowrank, node_vals, nullptr, false);
            {
              Timed t(h, KK_EXP, c.s);
              launch_vb_fwd_pack(va, c.s);
            }
            {
              Timed t(h, KK_FWD, c.s);
              vb_product(c, sp, gi, false, const_cast<float*>(va.U), const_cast<float*>(va.W));
            }
            Timed t(h, KK_LRFWD, c.s);
            launch_vb_fwd_reduce(va, c.s);
            continue;
          }
          LRArgs la = lr_args(c, sp, gi, lowrank, params, node_vals, nullptr);
          if (h->opt_fuse && sp.epi_prod >= 0) {     // the product layer above and the next shift
            const ProductPlan& pp = h->prods[sp.epi_prod];
            la.ep_on = 1;
            la.ep_qs = sp.epi_qs;
            la.ep_base_s = pp.abase[sp.epi_qs];
            la.ep_base_o = pp.abase[1 - sp.epi_qs];
            la.ep_pstart = pp.node_start;
            la.ep_pcount = pp.num_nodes;
            la.ep_mrow = sp.epi_mrow;
            la.mkeys_out = v.mkeys;
          }
          if (h->opt_lr_pack == 1) {
            Timed t(h, KK_SPLIT, c.s);
            lr_pack_group(c, sp, gi, lowrank);
          }
          Timed t(h, KK_LRFWD, c.s);
          launch_lr_fwd(la, p.mode == PC_PREC_FP32, c.s);
        }
        continue;
      }
      {
        Timed t(h, KK_EXP, c.s);
        launch_exp_pack(a, sp.pktiles, c.s);
      }
      GemmArgs g = gemm_common(c);
      g.ngroups = (int)sp.groups.size();
      g.groups = sp.d_groups;
      g.chblocks = sp.d_blocks;
      g.opA = v.theta;
      g.planeA = v.theta_plane;
      g.opB = v.ebt;
      g.planeB = v.ebt_plane;
      g.ldb = sp.ebt_cols;
      g.vals = node_vals;
      g.mkeys = v.mkeys;
      g.mkeys_out = v.mkeys;
      g.ssum = p.fwd_only ? nullptr : v.ssum;           // S is kept for the backward
      if (h->opt_fuse && sp.epi_prod >= 0) {
        const ProductPlan& pp = h->prods[sp.epi_prod];
        g.ep_on = 1;
        g.ep_qs = sp.epi_qs;
        g.ep_base_s = pp.abase[sp.epi_qs];
        g.ep_base_o = pp.abase[1 - sp.epi_qs];
        g.ep_pstart = pp.node_start;
        g.ep_pcount = pp.num_nodes;
        g.ep_mrow = sp.epi_mrow;
      }
      const GemmShape shp = layer_gemm_shape(h, sp, GK_FWD, v.B_pad, p.pl[GK_FWD][0], p.pl[GK_FWD][1]);
      g.ntiles = v.B_pad / shp.nt;
      g.splitk = shp.splitk;
      Timed t(h, KK_FWD, c.s);
      launch_gemm(EPI_FWD, p.pl[GK_FWD][0], p.pl[GK_FWD][1], shp, g, c.s);
    }
  }
  if (ll) {
    Timed t(h, KK_OTHER, c.s);
    launch_copy_row(node_vals + (int64_t)h->root * B, ll, B, c.s);
  }
  check_launch();
}

}  // namespace

// ---------------------------------------------------------------------------
// C ABI
// ---------------------------------------------------------------------------
extern "C" {

const char* pc_last_error(void) { return g_err.c_str(); }

int pc_compile_layout(const pc_circuit_desc* desc, int device, pc_handle* out) {
  Handle* h = nullptr;
  try {
    if (!out) fail(PC_ERR_INVALID_ARG, "null output handle pointer");
    *out = nullptr;
    h = compile_layout(desc);
    if (device >= 0) {
      upload_tables(h, device);       // leaves `device` current
      resolve_static_scratch(device);
    }
    *out = reinterpret_cast<pc_handle>(h);
    return PC_OK;
  } catch (const Error& e) {
    if (h) {
      free_tables(h);
      delete h;
    }
    return set_error(e.code, e.msg);
  } catch (const std::exception& e) {
    if (h) {
      free_tables(h);
      delete h;
    }
    return set_error(PC_ERR_INVALID_ARG, e.what());
  }
}

int pc_destroy(pc_handle hh) {
  if (!hh) return PC_OK;
  Handle* h = reinterpret_cast<Handle*>(hh);
  if (h->device >= 0 && (h->side_stream || !h->chunk_events.empty())) {
    int prev = -1;
    (void)hipGetDevice(&prev);
    (void)hipSetDevice(h->device);
    if (h->side_stream) {
      (void)hipStreamSynchronize((hipStream_t)h->side_stream);
      (void)hipStreamDestroy((hipStream_t)h->side_stream);
    }
    for (void* e : h->chunk_events) (void)hipEventDestroy((hipEvent_t)e);
    if (prev >= 0) (void)hipSetDevice(prev);
  }
  free_tables(h);
  delete h;
  return PC_OK;
}

int pc_set_precision(pc_handle hh, int mode) {
  try {
    Handle* h = checked(hh);
    if (mode == PC_PREC_TF32)
      fail(PC_ERR_UNSUPPORTED, "precision 'tf32': gfx950 has no TF32 matrix instruction; use PC_PREC_AUTO or PC_PREC_FP32");
    if (mode != PC_PREC_AUTO && mode != PC_PREC_FP32) fail(PC_ERR_INVALID_ARG, "unknown precision mode " + std::to_string(mode));
    h->mode = mode;
    return PC_OK;
  } catch (const Error& e) {
    return set_error(e.code, e.msg);
  }
}

int pc_get_precision(pc_handle hh, int* mode) {
  try {
    Handle* h = checked(hh);
    if (!mode) fail(PC_ERR_INVALID_ARG, "null mode pointer");
    *mode = h->mode;
    return PC_OK;
  } catch (const Error& e) {
    return set_error(e.code, e.msg);
  }
}

int pc_set_split(pc_handle hh, int mode, int gemm_kind, int planes_a, int planes_b) {
  try {
    Handle* h = checked(hh);
    if (mode != PC_PREC_AUTO && mode != PC_PREC_FP32) fail(PC_ERR_INVALID_ARG, "unknown precision mode");
    if (gemm_kind < 0 || gemm_kind > 2) fail(PC_ERR_INVALID_ARG, "unknown product kind");
    if (!planes_ok(planes_a, planes_b)) fail(PC_ERR_INVALID_ARG, "unsupported plane counts");
    h->planes[mode][gemm_kind][0] = planes_a;
    h->planes[mode][gemm_kind][1] = planes_b;
    return PC_OK;
  } catch (const Error& e) {
    return set_error(e.code, e.msg);
  }
}

int pc_set_option(pc_handle hh, int option, int value) {
  try {
    Handle* h = checked(hh);
    if (option == PC_OPT_LAYER_TILE) {
      if (value < 0 || value > 5) fail(PC_ERR_INVALID_ARG, "layer tile must be 0, 1, 2, 3, 4 or 5");
      h->opt_layer_tile = value == 1 ? TILE_128x128 : value == 2 ? TILE_256x128 : value == 3 ? TILE_128x256
                        : value == 4 ? TILE_128x64 : value == 5 ? TILE_64x128 : TILE_AUTO;
    } else if (option == PC_OPT_PARAM_TILE) {
      if (value < 0 || value > 3) fail(PC_ERR_INVALID_ARG, "parameter tile must be 0, 1, 2 or 3");
      h->opt_param_tile = value == 3 ? TILE_128x256 : value == 2 ? TILE_256x256 : value == 1 ? TILE_128x128 : TILE_AUTO;
    } else if (option == PC_OPT_SPLIT_MAX) {
      if (value != 1 && value != 2 && value != 4 && value != 8) fail(PC_ERR_INVALID_ARG, "split must be 1, 2, 4 or 8");
      h->opt_split_max = value;
    } else if (option == PC_OPT_PARAM_CHUNK) {
      if (value < -1) fail(PC_ERR_INVALID_ARG, "parameter-flow chunk must be >= -1");
      h->opt_param_chunk = value;
    } else if (option == PC_OPT_LR_PACK) {
      if (value != 0 && value != 1) fail(PC_ERR_INVALID_ARG, "lr_pack must be 0 or 1");
      h->opt_lr_pack = value;
    } else if (option == PC_OPT_FUSE) {
      if (value != 0 && value != 1) fail(PC_ERR_INVALID_ARG, "fuse must be 0 or 1");
      h->opt_fuse = value;
    } else if (option == PC_OPT_SUMEXP_FUSED) {
      if (value != 0 && value != 1) fail(PC_ERR_INVALID_ARG, "sumexp_fused must be 0 or 1");
      h->opt_sumexp_fused = value;
    } else if (option == PC_OPT_FLOW_FP8) {
      if (value != 0 && value != 1) fail(PC_ERR_INVALID_ARG, "flow_fp8 must be 0 or 1");
      h->opt_flow_fp8 = value;
    } else {
      fail(PC_ERR_INVALID_ARG, "unknown option");
    }
    return PC_OK;
  } catch (const Error& e) {
    return set_error(e.code, e.msg);
  }
}

int pc_workspace_bytes(pc_handle hh, int batch, size_t* bytes) {
  try {
    Handle* h = checked(hh);
    if (batch < 1) fail(PC_ERR_INVALID_ARG, "batch must be >= 1");
    if (!bytes) fail(PC_ERR_INVALID_ARG, "null bytes pointer");
    *bytes = plan_workspace(h, batch).total;
    return PC_OK;
  } catch (const Error& e) {
    return set_error(e.code, e.msg);
  }
}

int pc_layout_info(pc_handle hh, pc_layout_summary* info) {
  try {
    Handle* h = checked(hh);
    if (!info) fail(PC_ERR_INVALID_ARG, "null info pointer");
    info->num_layers = (int32_t)h->layers.size();
    info->num_sum_layers = (int32_t)h->sums.size();
    info->num_param_blocks = (int32_t)h->blocks.size();
    info->num_row_segments = (int32_t)h->rowsegs.size();
    info->num_params = h->num_params;
    info->num_outputs = (int32_t)h->outputs.size();
    info->device = h->device;
    return PC_OK;
  } catch (const Error& e) {
    return set_error(e.code, e.msg);
  }
}

int pc_layer_class(pc_handle hh, int layer, int* cls) {
  try {
    Handle* h = checked(hh);
    if (!cls) fail(PC_ERR_INVALID_ARG, "null class pointer");
    if (layer < 0 || layer >= (int)h->layers.size()) fail(PC_ERR_INVALID_ARG, "layer out of range");
    const LayerRef& r = h->layers[layer];
    *cls = (r.kind == PC_LAYER_SUM) ? h->sums[r.idx].cls : -1;
    return PC_OK;
  } catch (const Error& e) {
    return set_error(e.code, e.msg);
  }
}

int pc_forward(pc_handle hh, int batch, const int32_t* tokens, const float* params, float* node_vals,
               float* ll, const pc_lowrank_io* lowrank, void* ws, size_t ws_bytes, void* stream) {
  try {
    Call c = begin_call(hh, batch, ws, ws_bytes, stream);
    run_forward(c, tokens, params, node_vals, ll, lowrank);
    return PC_OK;
  } catch (const Error& e) {
    return set_error(e.code, e.msg);
  }
}

int pc_forward_static(pc_handle hh, int batch, const int32_t* tokens, const float* params, float* node_vals,
                      float* ll, const pc_lowrank_io* lowrank, void* stream) {
  try {
    Handle* h = checked(hh);
    if (h->device < 0) fail(PC_ERR_NO_DEVICE, "handle was compiled without a device");
    if (batch < 1) fail(PC_ERR_INVALID_ARG, "batch must be >= 1");
    const WsPlan p = plan_workspace(h, batch, true);
    if (p.total > PC_STATIC_SCRATCH_BYTES)
      fail(PC_ERR_WORKSPACE, "pc_forward_static: the forward of " + std::to_string(batch) + " samples needs " +
                                 std::to_string(p.total) + " bytes of scratch, more than the static " +
                                 std::to_string((size_t)PC_STATIC_SCRATCH_BYTES) + " (use pc_forward with a workspace)");
    void* ws = static_scratch(h->device);
    Call c = begin_call(hh, batch, ws, PC_STATIC_SCRATCH_BYTES, stream, true);
    NoEvents ne(h);                      // no timing events: creating them could allocate
    run_forward(c, tokens, params, node_vals, ll, lowrank);
    return PC_OK;
  } catch (const Error& e) {
    return set_error(e.code, e.msg);
  }
}

int pc_backward(pc_handle hh, int batch, const int32_t* tokens, const float* params, const float* node_vals,
                float* node_flows, float* param_flows, int flags, const pc_lowrank_io* lowrank, void* ws,
                size_t ws_bytes, void* stream) {
  try {
    Call c = begin_call(hh, batch, ws, ws_bytes, stream);
    Handle* h = c.h;
    check_lowrank_io(h, lowrank, true);
    (void)tokens;
    if (!params || !node_vals || !node_flows || !param_flows) fail(PC_ERR_INVALID_ARG, "null buffer");
    if (flags & ~PC_BWD_SEEDED) fail(PC_ERR_INVALID_ARG, "unknown flags");
    const bool seeded = (flags & PC_BWD_SEEDED) != 0;
    if (!seeded && h->root < 0) fail(PC_ERR_INVALID_ARG, "no root: seed the output flows (PC_BWD_SEEDED)");
    DeviceGuard dg(h->device);
    const int B = batch;
    const WsPlan& p = c.p;
    const WsView& v = c.v;
    float* vals = const_cast<float*>(node_vals);
    const bool gp = gp_active(h, B);
    {
      Timed t(h, KK_OTHER, c.s);
      launch_fill_ranges(node_flows, h->d_zero, (int)h->zero_ranges.size(), h->max_zero_count, B, c.s);
    }
    if (!seeded) {
      Timed t(h, KK_OTHER, c.s);
      launch_fill_ranges(node_flows, h->d_seed, (int)h->seed_ranges.size(), h->max_seed_count, B, c.s);
    }
    if (p.ncounters > 0) {
      Timed t(h, KK_OTHER, c.s);
      launch_fill_u32(v.counters, p.ncounters, 0u, c.s);
    }
    if (p.npcounters > 0) {
      Timed t(h, KK_OTHER, c.s);
      launch_fill_u32((uint32_t*)((char*)c.ws + p.pcounters), p.npcounters, 0u, c.s);
    }
    if (!h->inputs.empty()) {
      Timed t(h, KK_OTHER, c.s);
      launch_bucket(v.tokT, h->num_vars, B, h->max_cats, v.bucket_ptr, v.bucket_idx, c.s);
    }
    // LowRank denominator statistic W of the conditional M-step (on request)
    const bool zstat = h->lowrank_slots > 0 && lowrank && lowrank->z_flows;
    if (h->lowrank_slots > 0 && !p.vsum) {
      Timed t(h, KK_OTHER, c.s);
      launch_fill_u32((uint32_t*)((char*)c.ws + p.lrP), (int64_t)p.lr_nsg * h->lr_p_elems, 0u, c.s);
      if (zstat) launch_fill_u32((uint32_t*)((char*)c.ws + p.lrPz), (int64_t)p.lr_nsg * h->lr_p_elems, 0u, c.s);
    }
    // Parameter flows: one product over every tied copy after the layers, or
    // (opt_param_chunk > 0) chunks of that many copies per weight block on a
    // second stream, each launched once the last of its copies has its
    // scaled flows packed, in a fixed order (chunks of a block add into its
    // parameter flows one after another), joined before returning.
    GemmArgs pg = gemm_common(c);
    pg.ngroups = (int)h->blocks.size();
    pg.opA = v.garena;
    pg.planeA = v.garena_plane;
    pg.opB = v.earena;
    pg.planeB = v.earena_plane;
    pg.params = params;
    pg.pflows = param_flows;
    pg.partials = (float*)((char*)c.ws + p.ppartials);
    pg.counters = (uint32_t*)((char*)c.ws + p.pcounters);
    GemmShape pshp = param_gemm_shape(h, p.pl[GK_PARAM][0], p.pl[GK_PARAM][1]);
    {
      int64_t kmin = INT64_MAX;
      for (const BlockRec& bl : h->blocks)
        if (bl.ncopies > 0) kmin = std::min<int64_t>(kmin, (int64_t)bl.ncopies * (p.B_padK / 32));
      pshp.splitk = kmin == INT64_MAX ? 1 : param_splitk(pshp.tiles, kmin);
      pg.splitk = pshp.splitk;
    }
    struct Chunk {
      int ready, block, lo, hi;
    };
    std::vector<Chunk> chunks;
    int CC = h->opt_param_chunk;
    if (CC < 0) {
      // automatic: with a few weight blocks of which some are tied (the HMM's
      // transition has a copy per position), one chunk of all its copies per
      // block, launched as soon as the last copy has its scaled flows, so
      // that the product overlaps the rest of the backward (HMM-4096 at batch
      // 512: 4.72 -> 4.47 ms per step); with many blocks (HCLT's 767 untied
      // blocks, 24.8 vs 41.9 ms) the one product after the layers
      int nb = 0, maxc = 0;
      for (const BlockRec& bl : h->blocks)
        if (bl.ncopies > 0) {
          ++nb;
          maxc = std::max(maxc, (int)bl.ncopies);
        }
      CC = (nb <= 8 && maxc >= 2) ? maxc : 0;
    }
    if (h->has_plain_sums && CC > 0) {
      for (size_t b = 0; b < h->blocks.size(); ++b)
        for (int lo = 0; lo < h->blocks[b].ncopies; lo += CC) {
          const int hi = std::min(lo + CC, (int)h->blocks[b].ncopies);
          int ready = 1 << 30;
          for (int q = lo; q < hi; ++q) ready = std::min(ready, h->copy_layer[b][q]);
          chunks.push_back(Chunk{ready, (int)b, lo, hi});
        }
      std::stable_sort(chunks.begin(), chunks.end(), [](const Chunk& x, const Chunk& y) { return x.ready > y.ready; });
      if (!h->side_stream) {
        hipStream_t ss;
        HIPCHECK(hipStreamCreateWithFlags(&ss, hipStreamNonBlocking));
        h->side_stream = ss;
      }
      while (h->chunk_events.size() < chunks.size() + 1) {
        hipEvent_t e;
        HIPCHECK(hipEventCreateWithFlags(&e, hipEventDisableTiming));
        h->chunk_events.push_back(e);
      }
    }
    hipStream_t side = (hipStream_t)h->side_stream;
    size_t next_chunk = 0;
    auto launch_ready_chunks = [&](int li) {
      while (next_chunk < chunks.size() && chunks[next_chunk].ready >= li) {
        const Chunk& ch = chunks[next_chunk];
        hipEvent_t e = (hipEvent_t)h->chunk_events[next_chunk];
        HIPCHECK(hipEventRecord(e, c.s));
        HIPCHECK(hipStreamWaitEvent(side, e, 0));
        const BlockRec& bl = h->blocks[ch.block];
        GemmArgs g = pg;
        g.copy_lo = ch.lo;
        g.copy_hi = ch.hi;
        GemmShape shp = pshp;
        const int64_t Mp = round_up(bl.M, ROW_PAD), Np = round_up(bl.N, ROW_PAD);
        g.tile0 = shp.mt == 256 ? bl.pt256 : shp.nt == 256 ? 2 * bl.pt256 : bl.pt128;
        shp.tiles = (int)((Mp / shp.mt) * (Np / shp.nt));
        shp.splitk = param_splitk(shp.tiles, (int64_t)(ch.hi - ch.lo) * (p.B_padK / 32));
        g.splitk = shp.splitk;
        Timed t(h, KK_PARAM, side);
        launch_gemm(EPI_PARAM, p.pl[GK_PARAM][0], p.pl[GK_PARAM][1], shp, g, side);
        ++next_chunk;
      }
    };
    for (int li = (int)h->layers.size() - 1; li >= 0; --li) {
      launch_ready_chunks(li + 1);
      const LayerRef& r = h->layers[li];
      if (r.kind == PC_LAYER_SUM && h->sums[r.idx].lowrank) {
        const SumPlan& sp = h->sums[r.idx];
        for (int gi = 0; gi < (int)sp.groups.size(); ++gi) {
          LRArgs la = lr_args(c, sp, gi, lowrank, params, vals, node_flows);
          if (h->opt_fuse && sp.lr_prod >= 0) {
            const ProductPlan& pp = h->prods[sp.lr_prod];
            la.fp_on = 1;
            la.fp_pstart = pp.node_start;
            la.fp_other = pp.abase[1 - sp.lr_qs];
          }
          if (p.vsum) {
            // "sum_exp" on the virtual batch: c1, c2 and dA; Y1, Y2 operands;
            // theta^T [Y1 | Y2]^T; child flows and dB
            {
              Timed t(h, KK_LRCOEF, c.s);
              launch_lr_coef(la, c.s);
            }
            VBArgs vb = vb_args(c, sp, gi, lowrank, vals, node_flows, true);
            {
              Timed t(h, KK_GPACK, c.s);
              launch_vb_bwd_pack(vb, c.s);
            }
            {
              Timed t(h, KK_ELEM, c.s);
              vb_product(c, sp, gi, true, const_cast<float*>(vb.R1), const_cast<float*>(vb.R2));
            }
            Timed t(h, KK_LRBWD, c.s);
            launch_vb_bwd_reduce(vb, c.s);
            continue;
          }
          if (h->opt_lr_pack == 1) {
            Timed t(h, KK_SPLIT, c.s);
            lr_pack_group(c, sp, gi, lowrank);
          }
          {
            Timed t(h, KK_LRCOEF, c.s);
            launch_lr_coef(la, c.s);
          }
          Timed t(h, KK_LRBWD, c.s);
          launch_lr_bwd(la, p.mode == PC_PREC_FP32, c.s);
          if (zstat) {   // W's partials, from this layer's c2 = f / Z before the next layer rewrites it
            LRArgs lz = la;
            lz.P = (float*)((char*)c.ws + p.lrPz) + h->lr_p_off[sp.groups[gi].block] * p.lr_nsg;
            launch_lr_zstat(lz, p.mode == PC_PREC_FP32, c.s);
          }
        }
        if (sp.overlap) {
          SumArgs ra = sum_common(c, sp);
          ra.nuniq = (int)sp.red_child.size();
          ra.store = sp.store ? 1 : 0;
          ra.red_child = sp.d_red_child;
          ra.red_ptr = sp.d_red_ptr;
          ra.red_src = sp.d_red_src;
          ra.scratch = v.scratch;
          ra.out_flows = node_flows;
          Timed t(h, KK_OTHER, c.s);
          launch_elem_reduce(ra, c.s);
        }
      } else if (r.kind == PC_LAYER_SUM) {
        const SumPlan& sp = h->sums[r.idx];
        uint16_t* gbt = gp && sp.gbt_slot ? v.gbt2 : v.gbt;
        SumArgs a = sum_common(c, sp);
        a.vals = vals;
        a.flows = node_flows;
        a.ssum = v.ssum;
        a.direct = v.garena;
        a.direct_plane = v.garena_plane;
        a.np_direct = p.pl[GK_PARAM][0];
        a.trans = gbt;
        a.trans_plane = v.gbt_plane;
        a.direct_rows = h->garena_rows;
        a.np_trans = p.pl[GK_ELEM][1];
        if (h->opt_fuse && sp.bwd_prod >= 0) {
          const ProductPlan& pp = h->prods[sp.bwd_prod];
          a.fp_on = 1;
          a.fp_store = pp.store ? 1 : 0;
          a.fp_nrest = (int)sp.up_rest.size();
          a.fp_ptr = pp.d_pptr;
          a.fp_ids = pp.d_parents;
          a.fp_uchild = pp.d_uchild;
          a.fp_up = sp.d_up_idx;
          a.fp_rest = sp.d_up_rest;
          a.fp_rest_par = sp.d_up_rest_par;
          a.fp_single = pp.single_parent ? 1 : 0;
          a.wflows = node_flows;
        }
        if (!(gp && sp.gp_done)) {   // else packed by the next layer's element-flow product
          Timed t(h, KK_GPACK, c.s);
          launch_g_pack(a, sp.pgtiles, c.s);
        }
        GemmArgs g = gemm_common(c);
        g.ngroups = (int)sp.groups.size();
        g.groups = sp.d_groups;
        g.chblocks = sp.d_blocks;
        g.opA = v.thetaT;
        g.planeA = v.thetaT_plane;
        g.opB = gbt;
        g.planeB = v.gbt_plane;
        g.ldb = sp.gbt_cols;
        if (gp && sp.gp_sum >= 0) {
          const SumPlan& sa = h->sums[sp.gp_sum];
          const ProductPlan& pp = h->prods[sp.gp_prod];
          const GroupRec& ra = sa.groups[0];
          g.gp_on = 1;
          g.gp_qs = sp.gp_qs;
          g.gp_out_start = ra.out_start;
          g.gp_other = pp.abase[1 - sp.gp_qs];
          g.gp_np_direct = p.pl[GK_PARAM][0];
          g.gp_np_trans = p.pl[GK_ELEM][1];
          g.gp_g_koff = ra.g_koff;
          g.gp_s_row = ra.s_row;
          g.gp_g_row = ra.g_row;
          g.gp_direct_rows = h->garena_rows;
          g.gp_direct_plane = v.garena_plane;
          g.gp_trans_plane = v.gbt_plane;
          g.gp_direct = v.garena;
          g.gp_trans = sa.gbt_slot ? v.gbt2 : v.gbt;
          g.ssum = v.ssum;   // the packed layer's kept scaled sums
          if (!g.ssum || !g.gp_direct || !g.gp_trans || !gp_batch_ok(B) || ra.s_row < 0)
            fail(PC_ERR_INVALID_ARG, "internal: element-flow product epilogue without its operands");
        }
        g.vals = vals;
        g.flows = node_flows;
        g.scratch = v.scratch;
        g.mkeys = v.mkeys;
        g.store = sp.store ? 1 : 0;
        {
          const GemmShape shp = layer_gemm_shape(h, sp, GK_ELEM, v.B_pad, p.pl[GK_ELEM][0], p.pl[GK_ELEM][1]);
          g.ntiles = v.B_pad / shp.nt;
          g.splitk = shp.splitk;
          Timed t(h, KK_ELEM, c.s);
          launch_gemm(EPI_ELEM, p.pl[GK_ELEM][0], p.pl[GK_ELEM][1], shp, g, c.s);
        }
        if (sp.overlap) {
          SumArgs ra = sum_common(c, sp);
          ra.nuniq = (int)sp.red_child.size();
          ra.store = sp.store ? 1 : 0;
          ra.red_child = sp.d_red_child;
          ra.red_ptr = sp.d_red_ptr;
          ra.red_src = sp.d_red_src;
          ra.scratch = v.scratch;
          ra.out_flows = node_flows;
          Timed t(h, KK_OTHER, c.s);
          launch_elem_reduce(ra, c.s);
        }
      } else if (r.kind == PC_LAYER_PRODUCT) {
        if (h->opt_fuse && h->prods[r.idx].bwd_fused) continue;   // runs in the previous layer's scaled-flow packing
        ProdArgs a = prod_args(c, h->prods[r.idx]);
        a.flows = node_flows;
        Timed t(h, KK_PRODBWD, c.s);
        launch_prod_bwd(a, c.s);
      } else if (r.kind == PC_LAYER_INPUT_CAT) {
        InputArgs a = input_args(c, h->inputs[r.idx], params);
        a.flows = node_flows;
        a.pflows = param_flows;
        Timed t(h, KK_INBWD, c.s);
        launch_input_bwd(a, c.s);
      }
    }
    for (size_t bi = 0; bi < h->blocks.size() && !p.vsum; ++bi) {
      if (h->lr_p_off[bi] < 0) continue;
      const BlockRec& bl = h->blocks[bi];
      Timed t(h, KK_LRBWD, c.s);
      launch_lr_fplus((float*)((char*)c.ws + p.lrP) + h->lr_p_off[bi] * p.lr_nsg, p.lr_nsg, (int64_t)bl.M * bl.N,
                      param_flows + bl.param_offset, c.s);
      if (zstat)
        launch_lr_fplus((float*)((char*)c.ws + p.lrPz) + h->lr_p_off[bi] * p.lr_nsg, p.lr_nsg, (int64_t)bl.M * bl.N,
                        lowrank->z_flows + bl.param_offset, c.s);
    }
    if (!chunks.empty()) {
      launch_ready_chunks(-(1 << 29));
      hipEvent_t e = (hipEvent_t)h->chunk_events[chunks.size()];
      HIPCHECK(hipEventRecord(e, side));
      HIPCHECK(hipStreamWaitEvent(c.s, e, 0));
    } else if (h->has_plain_sums) {
      Timed t(h, KK_PARAM, c.s);
      launch_gemm(EPI_PARAM, p.pl[GK_PARAM][0], p.pl[GK_PARAM][1], pshp, pg, c.s);
    }
    if (p.vsum) {
      // F+ = theta * (Y1 X^T) and W = Y2 C^T over every (copy, sample, rank)
      // of each LowRank block, one product each; after the plain blocks'
      // parameter flows (joined from the second stream above), whose split-K
      // partials and arrival counters they share
      GemmArgs pv = gemm_common(c);
      pv.B_padK = p.QK;
      pv.rowsA = h->vy_rows;
      pv.rowsB = h->vx_rows;
      pv.blocks = h->d_vblocks;
      pv.ngroups = (int)h->vblocks.size();
      pv.opA = (const uint16_t*)((char*)c.ws + p.vY1);
      pv.planeA = h->vy_rows * p.QK;
      pv.opB = (const uint16_t*)((char*)c.ws + p.vX);
      pv.planeB = h->vx_rows * p.QK;
      pv.params = params;
      pv.pflows = param_flows;
      pv.partials = (float*)((char*)c.ws + p.ppartials);
      pv.counters = (uint32_t*)((char*)c.ws + p.pcounters);
      GemmShape vshp = param_gemm_shape_tiles(h, p.pl[GK_PARAM][0], p.pl[GK_PARAM][1], h->v_param_tiles256,
                                              h->v_param_tiles128);
      {
        int64_t kmin = INT64_MAX;
        for (const BlockRec& bl : h->vblocks) kmin = std::min<int64_t>(kmin, (int64_t)bl.ncopies * (p.QK / 32));
        vshp.splitk = param_splitk(vshp.tiles, kmin);
        pv.splitk = vshp.splitk;
      }
      if (p.vf8) {
        // e4m3 operands (PC_OPT_FLOW_FP8): F+ from Y1, X; W from Y2, C
        char* base = (char*)c.ws;
        int64_t kmin = INT64_MAX;
        for (const BlockRec& bl : h->vblocks) kmin = std::min<int64_t>(kmin, (int64_t)bl.ncopies * (p.QK / 64));
        F8Args f{};
        f.A = (const uint8_t*)(base + p.vY18);
        f.sA = (const uint8_t*)(base + p.vY1s);
        f.rowsA = h->vy_rows;
        f.B = (const uint8_t*)(base + p.vX8);
        f.sB = (const uint8_t*)(base + p.vXs);
        f.rowsB = h->vx_rows;
        f.QK = p.QK;
        f.nblocks = (int)h->vblocks.size();
        f.blocks = h->d_vblocks;
        f.params = params;
        f.out = param_flows;
        f.splitk = f8_splitk(h->v_param_tiles128, kmin);
        f.partials = (float*)(base + p.ppartials);
        f.counters = (uint32_t*)(base + p.pcounters);
        {
          Timed t(h, KK_PARAM, c.s);
          launch_f8param(f, h->v_param_tiles128, c.s);
        }
        if (zstat) {
          f.A = (const uint8_t*)(base + p.vY28);
          f.sA = (const uint8_t*)(base + p.vY2s);
          f.B = (const uint8_t*)(base + p.vC8);
          f.sB = (const uint8_t*)(base + p.vCs);
          f.params = nullptr;                // no weights: W
          f.out = lowrank->z_flows;
          Timed t(h, KK_PARAM, c.s);
          launch_f8param(f, h->v_param_tiles128, c.s);
        }
      } else {
        {
          Timed t(h, KK_PARAM, c.s);
          launch_gemm(EPI_PARAM, p.pl[GK_PARAM][0], p.pl[GK_PARAM][1], vshp, pv, c.s);
        }
        if (zstat) {
          pv.opA = (const uint16_t*)((char*)c.ws + p.vY2);
          pv.opB = (const uint16_t*)((char*)c.ws + p.vC);
          pv.params = nullptr;                 // no weights: W
          pv.pflows = lowrank->z_flows;
          Timed t(h, KK_PARAM, c.s);
          launch_gemm(EPI_PARAM, p.pl[GK_PARAM][0], p.pl[GK_PARAM][1], vshp, pv, c.s);
        }
      }
    }
    check_launch();
    return PC_OK;
  } catch (const Error& e) {
    return set_error(e.code, e.msg);
  }
}

static int em_common(pc_handle hh, float* params, const float* param_flows, const float* z_flows, bool corrected,
                     float step_size, float pseudocount, void* stream) {
  try {
    Handle* h = checked(hh);
    if (h->device < 0) fail(PC_ERR_NO_DEVICE, "handle was compiled without a device");
    if (!params || !param_flows) fail(PC_ERR_INVALID_ARG, "null params or param_flows");
    if (corrected && !z_flows) fail(PC_ERR_INVALID_ARG, "null z_flows");
    if (!(step_size >= 0.0f && step_size <= 1.0f)) fail(PC_ERR_INVALID_ARG, "step_size must be in [0, 1]");
    if (!(pseudocount >= 0.0f)) fail(PC_ERR_INVALID_ARG, "pseudocount must be >= 0");
    DeviceGuard dg(h->device);
    EmArgs a{};
    a.nsegs = (int)h->rowsegs.size();
    a.segs = h->d_rowsegs;
    a.params = params;
    a.pflows = param_flows;
    a.zflows = corrected ? z_flows : nullptr;
    a.step = step_size;
    a.pseudo = pseudocount;
    hipStream_t s = (hipStream_t)stream;
    Timed t(h, KK_EM, s);
    launch_em(a, h->total_rows, s);
    check_launch();
    return PC_OK;
  } catch (const Error& e) {
    return set_error(e.code, e.msg);
  }
}

int pc_em_step(pc_handle hh, float* params, const float* param_flows, float step_size, float pseudocount,
               void* stream) {
  return em_common(hh, params, param_flows, nullptr, false, step_size, pseudocount, stream);
}

int pc_em_step_corrected(pc_handle hh, float* params, const float* param_flows, const float* z_flows,
                         float step_size, float pseudocount, void* stream) {
  return em_common(hh, params, param_flows, z_flows, true, step_size, pseudocount, stream);
}

int pc_set_timing(pc_handle hh, int enable) {
  try {
    Handle* h = checked(hh);
    h->timing = enable != 0;
    h->events_used = 0;
    return PC_OK;
  } catch (const Error& e) {
    return set_error(e.code, e.msg);
  }
}

int pc_kernel_times(pc_handle hh, int64_t* launches, double* ms) {
  try {
    Handle* h = checked(hh);
    if (!launches || !ms) fail(PC_ERR_INVALID_ARG, "null output arrays");
    for (int k = 0; k < PC_NUM_KERNEL_KINDS; ++k) {
      launches[k] = 0;
      ms[k] = 0.0;
    }
    for (size_t i = 0; i < h->events_used; ++i) {
      const Handle::Ev& ev = h->events[i];
      HIPCHECK(hipEventSynchronize((hipEvent_t)ev.stop));
      float t = 0.0f;
      HIPCHECK(hipEventElapsedTime(&t, (hipEvent_t)ev.start, (hipEvent_t)ev.stop));
      launches[ev.kind] += 1;
      ms[ev.kind] += t;
    }
    h->events_used = 0;
    return PC_OK;
  } catch (const Error& e) {
    return set_error(e.code, e.msg);
  }
}

}  // extern "C"
