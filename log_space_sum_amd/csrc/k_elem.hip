// k_elem.hip -- the memory-bound kernels around the sum-layer products:
// categorical input layer, product layer, per-group column maxima, the
// exponentiated children and scaled flows in bfloat16 operand planes, the
// weight planes, the overlapping-children reduction, the input-layer
// parameter flows and the EM update.  All reductions run in a fixed order, so
// every result is bitwise reproducible (the column maxima use integer atomic
// max on order-preserving keys, which is order independent).
#include <hip/hip_runtime.h>

#include "pc_elem.h"

namespace pc {

// ---- helpers ----------------------------------------------------------------
__device__ __forceinline__ uint32_t float_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_shift(uint32_t k) {
  const uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  const float m = __uint_as_float(u);
  return (m == m && fabsf(m) <= 3.0e38f) ? m : 0.0f;
}
// float32 -> bfloat16, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint16_t f2bf(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// Split x into `np` bfloat16 planes: x ~ p0 + p1 + p2, each the rounding of
// what the previous planes leave.
__device__ __forceinline__ void split_store(float x, int np, uint16_t* dst, int64_t plane) {
  float r = x;
  for (int p = 0; p < np; ++p) {
    const uint16_t h = f2bf(r);
    dst[p * plane] = h;
    r = r - bf2f(h);
  }
}

template <typename Rec, typename F>
__device__ __forceinline__ int last_le(const Rec* recs, int n, int x, F field) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (field(recs[mid]) <= x) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__device__ __forceinline__ int child_of(const GroupRec& g, const int32_t* blocks, int k) {
  return blocks[g.blk_off + k / g.cbs] + k % g.cbs;
}

// ---- fills, copies, transposes ----------------------------------------------
__global__ void k_fill_u32(uint32_t* p, int64_t n, uint32_t v) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

__global__ void k_fill_ranges(float* flows, const FillRange* rs, int B) {
  const FillRange r = rs[blockIdx.y];
  const int64_t n = (int64_t)r.count * B;
  float* base = flows + (int64_t)r.start * B;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    base[i] = r.value;
}

__global__ void k_copy_row(const float* src, float* dst, int B) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < B) dst[b] = src[b];
}

__global__ void k_tokens_t(const int32_t* tok, int32_t* tokT, int B, int V) {
  __shared__ int32_t t[32][33];
  const int v0 = blockIdx.x * 32, b0 = blockIdx.y * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;   // 256 threads: 32 x 8
  for (int y = ty; y < 32; y += 8) {
    const int b = b0 + y, v = v0 + tx;
    t[y][tx] = (b < B && v < V) ? tok[(int64_t)b * V + v] : 0;
  }
  __syncthreads();
  for (int y = ty; y < 32; y += 8) {
    const int v = v0 + y, b = b0 + tx;
    if (v < V && b < B) tokT[(int64_t)v * B + b] = t[tx][y];
  }
}

// ---- categorical input layer ---------------------------------------------------
// v[u,b] = log theta_in[row(u), x[b, var(u)]]; a token outside [0, K) gives NaN
// (and never an out-of-range read).
__global__ void k_input_fwd(InputArgs a) {
  const int64_t n = (int64_t)a.num_nodes * a.B;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const int u = (int)(i / a.B), b = (int)(i - (int64_t)u * a.B);
    const int x = a.tokT[(int64_t)a.var[u] * a.B + b];
    float v;
    if (x >= 0 && x < a.K) v = logf(a.params[a.param_offset + (int64_t)a.row[u] * a.K + x]);
    else v = __uint_as_float(0x7fc00000u);
    a.vals[(int64_t)(a.node_start + u) * a.B + b] = v;
  }
}

// Samples of each variable bucketed by category in ascending sample order
// (a stable counting sort), so the input flows are summed in a fixed order.
__global__ void k_bucket(const int32_t* tokT, int B, int Kmax, int32_t* bptr, int32_t* bidx) {
  extern __shared__ int32_t sm[];
  int32_t* cnt = sm;              // Kmax + 1
  int32_t* xs = sm + Kmax + 1;    // B
  const int v = blockIdx.x;
  const int32_t* x = tokT + (int64_t)v * B;
  for (int k = threadIdx.x; k <= Kmax; k += blockDim.x) cnt[k] = 0;
  for (int b = threadIdx.x; b < B; b += blockDim.x) xs[b] = x[b];
  __syncthreads();
  for (int b = threadIdx.x; b < B; b += blockDim.x) {
    const int c = xs[b];
    if (c >= 0 && c < Kmax) atomicAdd(&cnt[c + 1], 1);
  }
  __syncthreads();
  if (threadIdx.x == 0)
    for (int k = 0; k < Kmax; ++k) cnt[k + 1] += cnt[k];
  __syncthreads();
  int32_t* ptr = bptr + (int64_t)v * (Kmax + 1);
  for (int k = threadIdx.x; k <= Kmax; k += blockDim.x) ptr[k] = cnt[k];
  for (int b = threadIdx.x; b < B; b += blockDim.x) {
    const int c = xs[b];
    if (c < 0 || c >= Kmax) continue;
    int rank = 0;
    for (int bb = 0; bb < b; ++bb) rank += (xs[bb] == c);
    bidx[(int64_t)v * B + cnt[c] + rank] = b;
  }
}

// F_in[row, k] += sum over the row's nodes u (ascending) and the samples b
// with x[b, var(u)] = k (ascending) of f[u, b].
__global__ void k_input_bwd(InputArgs a) {
  const int64_t n = (int64_t)a.num_rows * a.K;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const int r = (int)(i / a.K), k = (int)(i - (int64_t)r * a.K);
    float acc = 0.0f;
    for (int q = a.row_ptr[r]; q < a.row_ptr[r + 1]; ++q) {
      const int node = a.row_nodes[q];
      const int v = a.var[node - a.node_start];
      const int32_t* ptr = a.bptr + (int64_t)v * (a.Kmax + 1);
      const int32_t* idx = a.bidx + (int64_t)v * a.B;
      const float* f = a.flows + (int64_t)node * a.B;
      for (int t = ptr[k]; t < ptr[k + 1]; ++t) acc += f[idx[t]];
    }
    a.pflows[a.param_offset + i] += acc;
  }
}

// ---- product layer -------------------------------------------------------------
__global__ void k_prod_fwd(ProdArgs a) {
  const int64_t n = (int64_t)a.num_nodes * a.B;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const int p = (int)(i / a.B), b = (int)(i - (int64_t)p * a.B);
    float s = 0.0f;
    for (int q = a.ch_ptr[p]; q < a.ch_ptr[p + 1]; ++q) s += a.vals[(int64_t)a.ch_ids[q] * a.B + b];
    a.vals[(int64_t)(a.node_start + p) * a.B + b] = s;
  }
}

// f[c] (=|+=) sum of the flows of c's parents in this layer (parent order).
__global__ void k_prod_bwd(ProdArgs a) {
  const int64_t n = (int64_t)a.nuniq * a.B;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const int k = (int)(i / a.B), b = (int)(i - (int64_t)k * a.B);
    float s = 0.0f;
    for (int q = a.pptr[k]; q < a.pptr[k + 1]; ++q) s += a.flows[(int64_t)a.parents[q] * a.B + b];
    float* dst = a.flows + (int64_t)a.uchild[k] * a.B + b;
    if (a.store) *dst = s; else *dst += s;
  }
}

// ---- sum layer: column maxima, exponentiated children, scaled flows -------------
// Tiles of 64 children x 64 samples over the source groups of a layer.
__global__ void k_colmax(SumArgs a) {
  __shared__ float red[4][64];
  const int t = blockIdx.x;
  const int rt = t / a.btiles, bt = t - rt * a.btiles;
  const int g = last_le(a.groups, a.ngroups, rt, [](const GroupRec& r) { return r.pk_start; });
  const GroupRec gr = a.groups[g];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int b = bt * 64 + lane;
  const int k0 = (rt - gr.pk_start) * 64 + w * 16;
  float m = -INFINITY;
  if (b < a.B)
    for (int k = k0; k < k0 + 16 && k < gr.N; ++k)
      m = fmaxf(m, a.vals[(int64_t)child_of(gr, a.chblocks, k) * a.B + b]);
  red[w][lane] = m;
  __syncthreads();
  if (w == 0 && b < a.B) {
    m = fmaxf(fmaxf(red[0][lane], red[1][lane]), fmaxf(red[2][lane], red[3][lane]));
    if (k0 < gr.N) atomicMax(a.mkeys + (int64_t)gr.m_row * a.B + b, float_key(m));
  }
}

// e[j,b] = exp(v[child j, b] - m[b]) split into planes, written node-major
// (kept for the parameter flows) and batch-major (forward operand).
__global__ void k_exp_pack(SumArgs a) {
  __shared__ float tile[64][65];
  const int t = blockIdx.x;
  const int rt = t / a.btiles, bt = t - rt * a.btiles;
  const int g = last_le(a.groups, a.ngroups, rt, [](const GroupRec& r) { return r.pk_start; });
  const GroupRec gr = a.groups[g];
  const int k0 = (rt - gr.pk_start) * 64, b0 = bt * 64;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int b = b0 + lane;
  const float sh = (b < a.B) ? key_shift(a.mkeys[(int64_t)gr.m_row * a.B + b]) : 0.0f;
  for (int r = w; r < 64; r += 4) {
    const int k = k0 + r;
    float e = 0.0f;
    if (k < gr.N && b < a.B) e = expf(a.vals[(int64_t)child_of(gr, a.chblocks, k) * a.B + b] - sh);
    tile[r][lane] = e;
    if (b < a.B_padK)     // node-major copy for every group sharing these children
      for (int q = g; q >= 0; q = a.groups[q].share_next)
        split_store(e, a.np_direct, a.direct + panel(a.groups[q].e_row + k, b, a.direct_rows), a.direct_plane);
  }
  __syncthreads();
  const int NpK = (gr.N + K_PAD - 1) / K_PAD * K_PAD;
  for (int r = w; r < 64; r += 4) {          // r = sample within the tile, lane = child
    const int bb = b0 + r, k = k0 + lane;
    if (k < NpK && bb < a.B_pad)
      split_store(tile[lane][r], a.np_trans, a.trans + panel(bb, gr.e_koff + k, a.B_pad), a.trans_plane);
  }
}

// g[i,b] = f[i,b] / S[i,b] = f[i,b] * exp(m[b] - v[i,b]) (0 where f = 0 or
// S = 0), with S the scaled sum kept by the forward (dividing by it avoids the
// rounding of the absolute log-value v), split into planes and written
// node-major (kept) and batch-major (element-flow operand).
__global__ void k_g_pack(SumArgs a) {
  __shared__ float tile[64][65];
  const int t = blockIdx.x;
  const int rt = t / a.btiles, bt = t - rt * a.btiles;
  const int g = last_le(a.groups, a.ngroups, rt, [](const GroupRec& r) { return r.pg_start; });
  const GroupRec gr = a.groups[g];
  const int i0 = (rt - gr.pg_start) * 64, b0 = bt * 64;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int b = b0 + lane;
  for (int r = w; r < 64; r += 4) {
    const int i = i0 + r;
    float gv = 0.0f;
    if (i < gr.M && b < a.B) {
      const float f = a.flows[(int64_t)(gr.out_start + i) * a.B + b];
      const float S = a.ssum[(gr.s_row + i) * a.B + b];
      gv = (f == 0.0f || !(S > 0.0f)) ? 0.0f : f / S;
    }
    tile[r][lane] = gv;
    if (b < a.B_padK)
      split_store(gv, a.np_direct, a.direct + panel(gr.g_row + i, b, a.direct_rows), a.direct_plane);
  }
  __syncthreads();
  const int MpK = (gr.M + K_PAD - 1) / K_PAD * K_PAD;
  for (int r = w; r < 64; r += 4) {
    const int bb = b0 + r, i = i0 + lane;
    if (i < MpK && bb < a.B_pad)
      split_store(tile[lane][r], a.np_trans, a.trans + panel(bb, gr.g_koff + i, a.B_pad), a.trans_plane);
  }
}

// Weights of every block split into planes, row-major [M_pad, N_padK] (forward
// operand) and transposed [N_pad, M_padK] (element-flow operand).
__global__ void k_theta_pack(ThetaArgs a) {
  __shared__ float tile[64][65];
  const int t = blockIdx.x;
  const int bi = last_le(a.blocks, a.nblocks, t, [](const BlockRec& r) { return r.pk_start; });
  const BlockRec bl = a.blocks[bi];
  const int ntj = (bl.N + ROW_PAD - 1) / ROW_PAD * (ROW_PAD / 64);
  const int lt = t - bl.pk_start;
  const int i0 = (lt / ntj) * 64, j0 = (lt % ntj) * 64;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int NpK = (bl.N + K_PAD - 1) / K_PAD * K_PAD, MpK = (bl.M + K_PAD - 1) / K_PAD * K_PAD;
  const int64_t Mp = (bl.M + ROW_PAD - 1) / ROW_PAD * ROW_PAD, Np = (bl.N + ROW_PAD - 1) / ROW_PAD * ROW_PAD;
  const int j = j0 + lane;
  for (int r = w; r < 64; r += 4) {
    const int i = i0 + r;
    const float x = (i < bl.M && j < bl.N) ? a.params[bl.param_offset + (int64_t)i * bl.N + j] : 0.0f;
    tile[r][lane] = x;
    if (j < NpK) split_store(x, a.np_fwd, a.theta + bl.th_off + panel(i, j, Mp), a.theta_plane);
  }
  __syncthreads();
  for (int r = w; r < 64; r += 4) {
    const int jj = j0 + r, i = i0 + lane;
    if (i < MpK) split_store(tile[lane][r], a.np_elem, a.thetaT + bl.tht_off + panel(jj, i, Np), a.thetaT_plane);
  }
}

// Overlapping children: f[c] (=|+=) sum of the scratch rows of c (group order).
__global__ void k_elem_reduce(SumArgs a) {
  const int64_t n = (int64_t)a.nuniq * a.B;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const int k = (int)(i / a.B), b = (int)(i - (int64_t)k * a.B);
    float s = 0.0f;
    for (int q = a.red_ptr[k]; q < a.red_ptr[k + 1]; ++q) s += a.scratch[(int64_t)a.red_src[q] * a.B + b];
    float* dst = a.out_flows + (int64_t)a.red_child[k] * a.B + b;
    if (a.store) *dst = s; else *dst += s;
  }
}

// ---- EM ------------------------------------------------------------------------
__global__ void k_em(EmArgs a) {
  __shared__ float red[256];
  const int row = blockIdx.x;
  const int s = last_le(a.segs, a.nsegs, row, [](const RowSeg& r) { return r.row_start; });
  const RowSeg sg = a.segs[s];
  const int64_t off = sg.offset + (int64_t)(row - sg.row_start) * sg.rlen;
  float acc = 0.0f;
  for (int j = threadIdx.x; j < sg.rlen; j += 256) acc += a.pflows[off + j];
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  const float tot = red[0] + a.pseudo;
  if (!(tot > 0.0f)) return;
  const float add = a.pseudo / (float)sg.rlen;
  for (int j = threadIdx.x; j < sg.rlen; j += 256) {
    const float nw = (a.pflows[off + j] + add) / tot;
    a.params[off + j] = (1.0f - a.step) * a.params[off + j] + a.step * nw;
  }
}

// ---- launchers -------------------------------------------------------------------
static int grid_for(int64_t n, int per = 256, int cap = 65536) {
  int64_t g = (n + per - 1) / per;
  if (g < 1) g = 1;
  return (int)(g > cap ? cap : g);
}

void launch_fill_u32(uint32_t* p, int64_t n, uint32_t v, hipStream_t s) {
  if (n > 0) hipLaunchKernelGGL(k_fill_u32, dim3(grid_for(n)), dim3(256), 0, s, p, n, v);
}
void launch_fill_ranges(float* flows, const FillRange* d_ranges, int nranges, int64_t max_count, int B, hipStream_t s) {
  if (nranges <= 0) return;
  const int gx = grid_for(max_count * B, 256, 4096);
  hipLaunchKernelGGL(k_fill_ranges, dim3(gx, nranges), dim3(256), 0, s, flows, d_ranges, B);
}
void launch_copy_row(const float* src, float* dst, int B, hipStream_t s) {
  hipLaunchKernelGGL(k_copy_row, dim3((B + 255) / 256), dim3(256), 0, s, src, dst, B);
}
void launch_tokens_t(const int32_t* tok, int32_t* tokT, int B, int V, hipStream_t s) {
  hipLaunchKernelGGL(k_tokens_t, dim3((V + 31) / 32, (B + 31) / 32), dim3(256), 0, s, tok, tokT, B, V);
}
void launch_input_fwd(const InputArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_input_fwd, dim3(grid_for((int64_t)a.num_nodes * a.B)), dim3(256), 0, s, a);
}
void launch_bucket(const int32_t* tokT, int V, int B, int Kmax, int32_t* bptr, int32_t* bidx, hipStream_t s) {
  const size_t sh = (size_t)(Kmax + 1 + B) * sizeof(int32_t);
  hipLaunchKernelGGL(k_bucket, dim3(V), dim3(256), sh, s, tokT, B, Kmax, bptr, bidx);
}
void launch_input_bwd(const InputArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_input_bwd, dim3(grid_for((int64_t)a.num_rows * a.K)), dim3(256), 0, s, a);
}
void launch_prod_fwd(const ProdArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_prod_fwd, dim3(grid_for((int64_t)a.num_nodes * a.B)), dim3(256), 0, s, a);
}
void launch_prod_bwd(const ProdArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_prod_bwd, dim3(grid_for((int64_t)a.nuniq * a.B)), dim3(256), 0, s, a);
}
void launch_colmax(const SumArgs& a, int tiles, hipStream_t s) {
  if (tiles > 0) hipLaunchKernelGGL(k_colmax, dim3(tiles), dim3(256), 0, s, a);
}
void launch_exp_pack(const SumArgs& a, int tiles, hipStream_t s) {
  if (tiles > 0) hipLaunchKernelGGL(k_exp_pack, dim3(tiles), dim3(256), 0, s, a);
}
void launch_g_pack(const SumArgs& a, int tiles, hipStream_t s) {
  if (tiles > 0) hipLaunchKernelGGL(k_g_pack, dim3(tiles), dim3(256), 0, s, a);
}
void launch_theta_pack(const ThetaArgs& a, int tiles, hipStream_t s) {
  if (tiles > 0) hipLaunchKernelGGL(k_theta_pack, dim3(tiles), dim3(256), 0, s, a);
}
void launch_elem_reduce(const SumArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_elem_reduce, dim3(grid_for((int64_t)a.nuniq * a.B)), dim3(256), 0, s, a);
}
void launch_em(const EmArgs& a, int rows, hipStream_t s) {
  if (rows > 0) hipLaunchKernelGGL(k_em, dim3(rows), dim3(256), 0, s, a);
}

}  // namespace pc
