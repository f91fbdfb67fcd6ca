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
  return g.ch_start >= 0 ? g.ch_start + k : blocks[g.blk_off + k / g.cbs] + k % g.cbs;
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

// ---- batch vectors -------------------------------------------------------------
// Element-wise kernels give each thread V consecutive samples of one row: V = 4
// (16-byte loads and stores) when the batch is a multiple of 4, so every row
// of a [nodes, B] array starts 16-byte aligned, else V = 1.
template <int V>
struct Row {
  float x[V];
  __device__ __forceinline__ void load(const float* p) {
    if constexpr (V == 4) {
      const float4 t = *(const float4*)p;
      x[0] = t.x; x[1] = t.y; x[2] = t.z; x[3] = t.w;
    } else if constexpr (V == 2) {
      const float2 t = *(const float2*)p;
      x[0] = t.x; x[1] = t.y;
    } else {
#pragma unroll
      for (int k = 0; k < V; ++k) x[k] = p[k];
    }
  }
  __device__ __forceinline__ void store(float* p) const {
    if constexpr (V == 4) *(float4*)p = make_float4(x[0], x[1], x[2], x[3]);
    else if constexpr (V == 2) *(float2*)p = make_float2(x[0], x[1]);
    else
#pragma unroll
      for (int k = 0; k < V; ++k) p[k] = x[k];
  }
};

// s += rows ids[q0..q1) of x at samples [b, b + V), added in q order; the
// loads of each chunk of 4 rows are all issued before the first add.
template <int V>
__device__ __forceinline__ void sum_rows(Row<V>& s, const float* x, const int32_t* ids, int q0, int q1, int B,
                                         int b) {
  for (int q = q0; q < q1; q += 4) {
    Row<V> c[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (q + u < q1) c[u].load(x + (int64_t)ids[q + u] * B + b);
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (q + u < q1)
#pragma unroll
        for (int e = 0; e < V; ++e) s.x[e] += c[u].x[e];
  }
}

// ---- categorical input layer ---------------------------------------------------
// v[u,b] = log theta_in[row(u), x[b, var(u)]]; a token outside [0, K) gives NaN
// (and never an out-of-range read).
template <int V>
__global__ void k_input_fwd(InputArgs a) {
  // U items (node, V samples) per thread per pass, every load of the pass
  // issued before the first log
  constexpr int U = 4;
  const uint32_t QB = (uint32_t)(a.B / V), n = (uint32_t)a.num_nodes * QB;
  const uint32_t stride = gridDim.x * blockDim.x;
  for (uint32_t i0 = blockIdx.x * blockDim.x + threadIdx.x; i0 < n; i0 += U * stride) {
    Row<V> xs[U];
    const float* th[U];
#pragma unroll
    for (int q = 0; q < U; ++q) {
      const uint32_t i = i0 + q * stride;
      th[q] = nullptr;
      if (i >= n) continue;
      const uint32_t u = i / QB, b = (i - u * QB) * V;
      xs[q].load((const float*)(a.tokT + (int64_t)a.var[u] * a.B + b));   // the V tokens, as raw 32-bit words
      th[q] = a.params + a.param_offset + (int64_t)a.row[u] * a.K;
    }
    float g[U][V];
#pragma unroll
    for (int q = 0; q < U; ++q)
#pragma unroll
      for (int k = 0; k < V; ++k) {
        const int x = __float_as_int(xs[q].x[k]);
        g[q][k] = (th[q] && x >= 0 && x < a.K) ? th[q][x] : -1.0f;
      }
#pragma unroll
    for (int q = 0; q < U; ++q) {
      const uint32_t i = i0 + q * stride;
      if (i >= n) continue;
      const uint32_t u = i / QB, b = (i - u * QB) * V;
      Row<V> r;
#pragma unroll
      for (int k = 0; k < V; ++k) {
        const int x = __float_as_int(xs[q].x[k]);
        r.x[k] = (x >= 0 && x < a.K) ? logf(g[q][k]) : __uint_as_float(0x7fc00000u);
      }
      r.store(a.vals + (int64_t)(a.node_start + u) * a.B + b);
    }
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

// F_in[row, k] += sum over the row's nodes u of n_u[k], with n_u[k] the sum
// over the samples b with x[b, var(u)] = k (ascending) of f[u, b].  One
// workgroup of NW waves per parameter row; wave w takes the row's nodes
// w, w + NW, ... on its own (no workgroup barrier between nodes): it stages
// the node's flow row and its variable's category buckets in its own LDS
// region and adds every bucket's sum to its per-category registers.  At the
// end the NW partial sums are added in wave order, so the result does not
// depend on timing.  Needs K <= 1024 and the LDS regions to fit (see
// launch_input_bwd).
template <int NW>
__global__ __launch_bounds__(64 * NW) void k_input_bwd(InputArgs a) {
  extern __shared__ float ib_sm[];
  constexpr int J = 1024 / 64;
  const int B = a.B, K = a.K;
  const int per = 2 * B + K + 1;              // f[B], idx[B], ptr[K + 1]
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  float* f = ib_sm + w * per;
  int32_t* idx = (int32_t*)(f + B);
  int32_t* ptr = idx + B;
  const int r = blockIdx.x, q0 = a.row_ptr[r], q1 = a.row_ptr[r + 1];
  float acc[J];
#pragma unroll
  for (int j = 0; j < J; ++j) acc[j] = 0.0f;
  for (int q = q0 + w; q < q1; q += NW) {
    const int node = a.row_nodes[q];
    const int v = a.var[node - a.node_start];
    const float* F = a.flows + (int64_t)node * B;
    const int32_t* I = a.bidx + (int64_t)v * B;
    const int32_t* P = a.bptr + (int64_t)v * (a.Kmax + 1);
    // a wave's LDS operations complete in order: the previous node's reads
    // are done before these writes land, and these writes before the reads below
    __builtin_amdgcn_wave_barrier();
#pragma unroll 4
    for (int b = lane; b < B; b += 64) {
      f[b] = F[b];
      idx[b] = I[b];
    }
#pragma unroll 4
    for (int k = lane; k <= K; k += 64) ptr[k] = P[k];
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int k = j * 64 + lane;
      if (k < K) {
        float t = 0.0f;
        for (int e = ptr[k]; e < ptr[k + 1]; ++e) t += f[idx[e]];
        acc[j] += t;
      }
    }
  }
  float* out = a.pflows + a.param_offset + (int64_t)r * K;
  if constexpr (NW == 1) {
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int k = j * 64 + lane;
      if (k < K) out[k] += acc[j];
    }
  } else {
    __syncthreads();                            // every wave done with its region
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int k = j * 64 + lane;
      if (k < K) f[k] = acc[j];                 // K <= per: the partial fits the region
    }
    __syncthreads();
    for (int k = tid; k < K; k += 64 * NW) {
      float t = 0.0f;
#pragma unroll
      for (int u = 0; u < NW; ++u) t += ib_sm[u * per + k];
      out[k] += t;
    }
  }
}

// The same sums when every parameter row has one node (an untied input
// layer): workgroup = one variable and a chunk of 64 of its nodes; the
// variable's category buckets are staged in LDS once, and each wave streams
// 16 of the nodes, one flow row at a time in its own LDS region, adding each
// category's bucket sum to its node's row.
constexpr int kVarChunk = 64;
__global__ __launch_bounds__(256) void k_input_bwd_var(InputArgs a) {
  extern __shared__ float ib_sm[];
  const int B = a.B, K = a.K;
  int32_t* idx = (int32_t*)ib_sm;             // [B]
  int32_t* ptr = idx + B;                     // [K + 1]
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  float* f = ib_sm + B + K + 1 + w * B;       // [B] per wave
  const int nchunk = (a.max_var_nodes + kVarChunk - 1) / kVarChunk;
  const int v = blockIdx.x / nchunk, c = blockIdx.x - v * nchunk;
  const int q0 = a.var_ptr[v] + c * kVarChunk, q1 = min(a.var_ptr[v + 1], q0 + kVarChunk);
  if (q0 >= q1) return;
  const int32_t* I = a.bidx + (int64_t)v * B;
  const int32_t* P = a.bptr + (int64_t)v * (a.Kmax + 1);
  for (int b = threadIdx.x; b < B; b += blockDim.x) idx[b] = I[b];
  for (int k = threadIdx.x; k <= K; k += blockDim.x) ptr[k] = P[k];
  __syncthreads();
  for (int q = q0 + w; q < q1; q += 4) {
    const int u = a.var_nodes[q];
    const float* F = a.flows + (int64_t)(a.node_start + u) * B;
    // a wave's LDS operations complete in order
    __builtin_amdgcn_wave_barrier();
#pragma unroll 4
    for (int b = lane; b < B; b += 64) f[b] = F[b];
    __builtin_amdgcn_wave_barrier();
    float* out = a.pflows + a.param_offset + (int64_t)a.row[u] * K;
    for (int k = lane; k < K; k += 64) {
      float t = 0.0f;
      for (int e = ptr[k]; e < ptr[k + 1]; ++e) t += f[idx[e]];
      out[k] += t;
    }
  }
}

// The two input-layer parameter-flow kernels above with the next node's rows
// loading into registers while the current node is summed, for batches of at
// most 512 and at most 512 categories (a lane's share: 8 samples, 9 bounds).
constexpr int kPfB = 8, kPfK = 9;
template <int NW>
__global__ __launch_bounds__(64 * NW) void k_input_bwd_pf(InputArgs a) {
  extern __shared__ float ib_sm[];
  constexpr int J = 512 / 64;
  const int B = a.B, K = a.K;
  const int per = 2 * B + K + 1;              // f[B], idx[B], ptr[K + 1]
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  float* f = ib_sm + w * per;
  int32_t* idx = (int32_t*)(f + B);
  int32_t* ptr = idx + B;
  const int r = blockIdx.x, q0 = a.row_ptr[r], q1 = a.row_ptr[r + 1];
  float nf[kPfB];
  int ni[kPfB], np[kPfK];
  auto fetch = [&](int q) {
    const int node = a.row_nodes[q];
    const int v = a.var[node - a.node_start];
    const float* F = a.flows + (int64_t)node * B;
    const int32_t* I = a.bidx + (int64_t)v * B;
    const int32_t* P = a.bptr + (int64_t)v * (a.Kmax + 1);
#pragma unroll
    for (int i = 0; i < kPfB; ++i) {
      const int b = lane + 64 * i;
      nf[i] = b < B ? F[b] : 0.0f;
      ni[i] = b < B ? I[b] : 0;
    }
#pragma unroll
    for (int i = 0; i < kPfK; ++i) {
      const int k = lane + 64 * i;
      np[i] = k <= K ? P[k] : 0;
    }
  };
  float acc[J];
#pragma unroll
  for (int j = 0; j < J; ++j) acc[j] = 0.0f;
  if (q0 + w < q1) fetch(q0 + w);
  for (int q = q0 + w; q < q1; q += NW) {
    // a wave's LDS operations complete in order: the previous node's reads
    // are done before these writes land, and these writes before the reads below
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int i = 0; i < kPfB; ++i) {
      const int b = lane + 64 * i;
      if (b < B) {
        f[b] = nf[i];
        idx[b] = ni[i];
      }
    }
#pragma unroll
    for (int i = 0; i < kPfK; ++i) {
      const int k = lane + 64 * i;
      if (k <= K) ptr[k] = np[i];
    }
    __builtin_amdgcn_wave_barrier();
    if (q + NW < q1) fetch(q + NW);
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int k = j * 64 + lane;
      if (k < K) {
        float t = 0.0f;
        for (int e = ptr[k]; e < ptr[k + 1]; ++e) t += f[idx[e]];
        acc[j] += t;
      }
    }
  }
  float* out = a.pflows + a.param_offset + (int64_t)r * K;
  __syncthreads();                            // every wave done with its region
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int k = j * 64 + lane;
    if (k < K) f[k] = acc[j];                 // K <= per: the partial fits the region
  }
  __syncthreads();
  for (int k = tid; k < K; k += 64 * NW) {
    float t = 0.0f;
#pragma unroll
    for (int u = 0; u < NW; ++u) t += ib_sm[u * per + k];
    out[k] += t;
  }
}

__global__ __launch_bounds__(256) void k_input_bwd_var_pf(InputArgs a) {
  extern __shared__ float ib_sm[];
  const int B = a.B, K = a.K;
  int32_t* idx = (int32_t*)ib_sm;             // [B]
  int32_t* ptr = idx + B;                     // [K + 1]
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  float* f = ib_sm + B + K + 1 + w * B;       // [B] per wave
  const int nchunk = (a.max_var_nodes + kVarChunk - 1) / kVarChunk;
  const int v = blockIdx.x / nchunk, c = blockIdx.x - v * nchunk;
  const int q0 = a.var_ptr[v] + c * kVarChunk, q1 = min(a.var_ptr[v + 1], q0 + kVarChunk);
  if (q0 >= q1) return;
  const int32_t* I = a.bidx + (int64_t)v * B;
  const int32_t* P = a.bptr + (int64_t)v * (a.Kmax + 1);
  float nf[kPfB];
  auto fetch = [&](int q) {
    const float* F = a.flows + (int64_t)(a.node_start + a.var_nodes[q]) * B;
#pragma unroll
    for (int i = 0; i < kPfB; ++i) {
      const int b = lane + 64 * i;
      nf[i] = b < B ? F[b] : 0.0f;
    }
  };
  if (q0 + w < q1) fetch(q0 + w);
  for (int b = threadIdx.x; b < B; b += blockDim.x) idx[b] = I[b];
  for (int k = threadIdx.x; k <= K; k += blockDim.x) ptr[k] = P[k];
  __syncthreads();
  for (int q = q0 + w; q < q1; q += 4) {
    const int u = a.var_nodes[q];
    // a wave's LDS operations complete in order
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int i = 0; i < kPfB; ++i) {
      const int b = lane + 64 * i;
      if (b < B) f[b] = nf[i];
    }
    __builtin_amdgcn_wave_barrier();
    if (q + 4 < q1) fetch(q + 4);
    float* out = a.pflows + a.param_offset + (int64_t)a.row[u] * K;
    for (int k = lane; k < K; k += 64) {
      float t = 0.0f;
      for (int e = ptr[k]; e < ptr[k + 1]; ++e) t += f[idx[e]];
      out[k] += t;
    }
  }
}

// The same sums for rows whose regions do not fit: the row's nodes one at a
// time, the flow row staged in LDS, buckets read from global memory.
__global__ void k_input_bwd_wide(InputArgs a) {
  extern __shared__ float frow[];   // [B]
  const int r = blockIdx.x, tid = threadIdx.x;
  const int q0 = a.row_ptr[r], q1 = a.row_ptr[r + 1];
  float* out = a.pflows + a.param_offset + (int64_t)r * a.K;
  for (int kc = 0; kc < a.K; kc += 1024) {
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int q = q0; q < q1; ++q) {
      const int node = a.row_nodes[q];
      const int v = a.var[node - a.node_start];
      const float* f = a.flows + (int64_t)node * a.B;
      __syncthreads();                          // previous row fully read
      for (int b = tid; b < a.B; b += blockDim.x) frow[b] = f[b];
      __syncthreads();
      const int32_t* ptr = a.bptr + (int64_t)v * (a.Kmax + 1);
      const int32_t* idx = a.bidx + (int64_t)v * a.B;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int k = kc + j * 256 + tid;
        if (k < a.K) {
          float t = 0.0f;
          for (int e = ptr[k]; e < ptr[k + 1]; ++e) t += frow[idx[e]];
          acc[j] += t;
        }
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int k = kc + j * 256 + tid;
      if (k < a.K) out[k] += acc[j];
    }
  }
}

// ---- product layer -------------------------------------------------------------
template <int V>
__global__ void k_prod_fwd(ProdArgs a) {
  const uint32_t QB = (uint32_t)(a.B / V), n = (uint32_t)a.num_nodes * QB;
  for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) {
    const uint32_t p = i / QB, b = (i - p * QB) * V;
    Row<V> s;
#pragma unroll
    for (int k = 0; k < V; ++k) s.x[k] = 0.0f;
    if (a.affine) {   // child q at abase[q] + p: every load issued before the first add
      Row<V> c[8];
#pragma unroll
      for (int q = 0; q < 8; ++q)
        if (q < a.deg) c[q].load(a.vals + (int64_t)(a.abase[q] + (int)p) * a.B + b);
#pragma unroll
      for (int q = 0; q < 8; ++q)
        if (q < a.deg)
#pragma unroll
          for (int e = 0; e < V; ++e) s.x[e] += c[q].x[e];
    } else {
      sum_rows<V>(s, a.vals, a.ch_ids, a.ch_ptr[p], a.ch_ptr[p + 1], a.B, b);
    }
    s.store(a.vals + (int64_t)(a.node_start + p) * a.B + b);
  }
}

// f[c] (=|+=) sum of the flows of c's parents in this layer (parent order).
template <int V>
__global__ void k_prod_bwd(ProdArgs a) {
  const uint32_t QB = (uint32_t)(a.B / V), n = (uint32_t)a.nuniq * QB;
  for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) {
    const uint32_t k = i / QB, b = (i - k * QB) * V;
    Row<V> s;
#pragma unroll
    for (int e = 0; e < V; ++e) s.x[e] = 0.0f;
    sum_rows<V>(s, a.flows, a.parents, a.pptr[k], a.pptr[k + 1], a.B, b);
    float* dst = a.flows + (int64_t)a.uchild[k] * a.B + b;
    if (!a.store) {
      Row<V> o;
      o.load(dst);
#pragma unroll
      for (int e = 0; e < V; ++e) s.x[e] = o.x[e] + s.x[e];
    }
    s.store(dst);
  }
}

// ---- sum layer: column maxima, exponentiated children, scaled flows -------------
// Column maxima: a workgroup takes 4*RW children (a part of one 64-child
// packing tile) x 64*V samples; each wave reduces RW children, the waves
// combine in LDS and one integer atomic max per sample publishes the
// workgroup's maximum.  With PROD the
// children that are nodes of the preceding product layer are evaluated here:
// each is the sum of its own children in child-list order (as the product
// kernel adds them), stored, and used for the maximum.  The loads of all 16
// rows go out together, one child slot at a time.
template <int V, bool PROD, int RW>
__global__ __launch_bounds__(256) void k_colmax(SumArgs a) {
  __shared__ float red[4][64 * V];
  constexpr int NSUB = 16 / RW;              // workgroups per 64-child tile
  const int sbt = (a.B + 64 * V - 1) / (64 * V);
  const int t = blockIdx.x;
  const int st = t % sbt, rs = t / sbt, sub = rs % NSUB, rt = rs / NSUB;
  const GroupRec gr = a.ngroups == 1 ? a.group0 : a.groups[a.pk_group[rt]];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int b = st * 64 * V + lane * V;
  const int kw = (rt - gr.pk_start) * 64 + sub * 4 * RW;   // the workgroup's first child
  const int k0 = kw + w * RW;
  Row<V> m;
#pragma unroll
  for (int e = 0; e < V; ++e) m.x[e] = -INFINITY;
  if (b < a.B) {
    Row<V> c[RW];
    if constexpr (!PROD) {
#pragma unroll
      for (int kk = 0; kk < RW; ++kk)      // every load in flight at once
        if (k0 + kk < gr.N) c[kk].load(a.vals + (int64_t)child_of(gr, a.chblocks, k0 + kk) * a.B + b);
    } else {
      int32_t node[RW], q0[RW], q1[RW];
      if (a.fp_affine) {   // child q of product node i at fp_abase[q] + i: no index loads
        bool isp[RW];
#pragma unroll
        for (int kk = 0; kk < RW; ++kk) {
          isp[kk] = false;
          if (k0 + kk < gr.N) {
            node[kk] = child_of(gr, a.chblocks, k0 + kk);
            const uint32_t p = (uint32_t)(node[kk] - a.fp_start);
            isp[kk] = p < (uint32_t)a.fp_count;
            q0[kk] = (int32_t)p;
            if (!isp[kk]) c[kk].load(a.vals + (int64_t)node[kk] * a.B + b);
          }
        }
        Row<V> u[RW][2];
#pragma unroll
        for (int q = 0; q < 2; ++q)      // the first two child slots of all RW rows at once
#pragma unroll
          for (int kk = 0; kk < RW; ++kk)
            if (isp[kk] && q < a.fp_maxdeg) u[kk][q].load(a.vals + (int64_t)(a.fp_abase[q] + q0[kk]) * a.B + b);
#pragma unroll
        for (int kk = 0; kk < RW; ++kk)
          if (isp[kk]) {
#pragma unroll
            for (int e = 0; e < V; ++e) c[kk].x[e] = 0.0f;
#pragma unroll
            for (int q = 0; q < 2; ++q)
              if (q < a.fp_maxdeg)
#pragma unroll
                for (int e = 0; e < V; ++e) c[kk].x[e] += u[kk][q].x[e];
          }
        for (int q = 2; q < a.fp_maxdeg; ++q) {
#pragma unroll
          for (int kk = 0; kk < RW; ++kk)
            if (isp[kk]) u[kk][0].load(a.vals + (int64_t)(a.fp_abase[q] + q0[kk]) * a.B + b);
#pragma unroll
          for (int kk = 0; kk < RW; ++kk)
            if (isp[kk])
#pragma unroll
              for (int e = 0; e < V; ++e) c[kk].x[e] += u[kk][0].x[e];
        }
#pragma unroll
        for (int kk = 0; kk < RW; ++kk)
          if (isp[kk]) c[kk].store(a.wvals + (int64_t)node[kk] * a.B + b);
      } else {
#pragma unroll
      for (int kk = 0; kk < RW; ++kk) {
        node[kk] = -1;
        q0[kk] = q1[kk] = 0;
        if (k0 + kk < gr.N) {
          node[kk] = child_of(gr, a.chblocks, k0 + kk);
          const uint32_t p = (uint32_t)(node[kk] - a.fp_start);
          if (p < (uint32_t)a.fp_count) {
            q0[kk] = a.fp_ptr[p];
            q1[kk] = a.fp_ptr[p + 1];
#pragma unroll
            for (int e = 0; e < V; ++e) c[kk].x[e] = 0.0f;
          } else {
            c[kk].load(a.vals + (int64_t)node[kk] * a.B + b);
          }
        }
      }
      for (int q = 0; q < a.fp_maxdeg; ++q) {
        Row<V> u[RW];
#pragma unroll
        for (int kk = 0; kk < RW; ++kk)
          if (q0[kk] + q < q1[kk]) u[kk].load(a.vals + (int64_t)a.fp_ids[q0[kk] + q] * a.B + b);
#pragma unroll
        for (int kk = 0; kk < RW; ++kk)
          if (q0[kk] + q < q1[kk])
#pragma unroll
            for (int e = 0; e < V; ++e) c[kk].x[e] += u[kk].x[e];
      }
#pragma unroll
      for (int kk = 0; kk < RW; ++kk)
        if (q1[kk] > q0[kk]) c[kk].store(a.wvals + (int64_t)node[kk] * a.B + b);
      }
    }
#pragma unroll
    for (int kk = 0; kk < RW; ++kk)
      if (k0 + kk < gr.N)
#pragma unroll
        for (int e = 0; e < V; ++e) m.x[e] = fmaxf(m.x[e], c[kk].x[e]);
  }
#pragma unroll
  for (int e = 0; e < V; ++e) red[w][lane * V + e] = m.x[e];
  __syncthreads();
  if (kw >= gr.N) return;   // past the group's children: nothing to publish
  for (int x = threadIdx.x; x < 64 * V; x += blockDim.x) {
    const int bb = st * 64 * V + x;
    if (bb < a.B) {
      const float mx = fmaxf(fmaxf(red[0][x], red[1][x]), fmaxf(red[2][x], red[3][x]));
      atomicMax(a.mkeys + (int64_t)gr.m_row * a.B + bb, float_key(mx));
    }
  }
}

// Split 8 values into np bfloat16 planes and store each plane as 16 bytes.
__device__ __forceinline__ void split_store8(const float (&x)[8], int np, uint16_t* dst, int64_t plane) {
  float r[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = x[e];
  for (int p = 0; p < np; ++p) {
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint16_t h0 = f2bf(r[2 * e]), h1 = f2bf(r[2 * e + 1]);
      r[2 * e] -= bf2f(h0);
      r[2 * e + 1] -= bf2f(h1);
      w[e] = (uint32_t)h0 | ((uint32_t)h1 << 16);
    }
    *(uint4*)(dst + p * plane) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// 8 consecutive samples [bs, bs + 8) of a row: two 16-byte accesses when the
// chunk is whole and 16-byte aligned (vec), else one by one within the batch
// (missing samples read as 0 and are not written).
__device__ __forceinline__ void load8(const float* p, bool vec, int bs, int B, float (&x)[8]) {
  if (vec) {
    const float4 t0 = *(const float4*)p, t1 = *(const float4*)(p + 4);
    x[0] = t0.x; x[1] = t0.y; x[2] = t0.z; x[3] = t0.w;
    x[4] = t1.x; x[5] = t1.y; x[6] = t1.z; x[7] = t1.w;
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = bs + e < B ? p[e] : 0.0f;
  }
}
__device__ __forceinline__ void store8(float* p, bool vec, int bs, int B, const float (&x)[8]) {
  if (vec) {
    *(float4*)p = make_float4(x[0], x[1], x[2], x[3]);
    *(float4*)(p + 4) = make_float4(x[4], x[5], x[6], x[7]);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (bs + e < B) p[e] = x[e];
  }
}

// Product-layer backward for the distinct children listed in fp_rest (the ones
// the packing tiles do not cover): f[c] (=|+=) its parents' flows, in parent
// order, 4 samples per item; workgroup `wg` of `nwg`.
__device__ __forceinline__ void prod_bwd_rest(const SumArgs& a, int wg, int nwg) {
  const int QB = (a.B + 3) / 4;
  const int64_t n = (int64_t)a.fp_nrest * QB;
  const bool vec = (a.B & 3) == 0;
  const int64_t step = (int64_t)nwg * blockDim.x;
  // two items per pass, the single-parent loads of both issued first
  for (int64_t i0 = (int64_t)wg * blockDim.x + threadIdx.x; i0 < n; i0 += 2 * step) {
    float s[2][4], o[2][4];
    int b[2], u[2];
    float* dst[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int64_t i = i0 + h * step;
#pragma unroll
      for (int e = 0; e < 4; ++e) s[h][e] = o[h][e] = 0.0f;
      dst[h] = nullptr;
      if (i >= n) continue;
      const int ri = (int)(i / QB);
      b[h] = (int)(i - (int64_t)ri * QB) * 4;
      u[h] = a.fp_rest[ri];
      dst[h] = a.wflows + (int64_t)(a.fp_single ? u[h] : a.fp_uchild[u[h]]) * a.B + b[h];
      if (a.fp_single) {
        const float* pf = a.wflows + (int64_t)a.fp_rest_par[ri] * a.B + b[h];
        if (vec) {
          const float4 y = *(const float4*)pf;
          s[h][0] = 0.0f + y.x; s[h][1] = 0.0f + y.y; s[h][2] = 0.0f + y.z; s[h][3] = 0.0f + y.w;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (b[h] + e < a.B) s[h][e] = 0.0f + pf[e];
        }
      }
      if (!a.fp_store) {
        if (vec) {
          const float4 y = *(const float4*)dst[h];
          o[h][0] = y.x; o[h][1] = y.y; o[h][2] = y.z; o[h][3] = y.w;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (b[h] + e < a.B) o[h][e] = dst[h][e];
        }
      }
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (!dst[h]) continue;
      if (!a.fp_single) {
        for (int q = a.fp_ptr[u[h]]; q < a.fp_ptr[u[h] + 1]; ++q) {
          const float* pf = a.wflows + (int64_t)a.fp_ids[q] * a.B + b[h];
          if (vec) {
            const float4 y = *(const float4*)pf;
            s[h][0] += y.x; s[h][1] += y.y; s[h][2] += y.z; s[h][3] += y.w;
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (b[h] + e < a.B) s[h][e] += pf[e];
          }
        }
      }
      if (!a.fp_store)
#pragma unroll
        for (int e = 0; e < 4; ++e) s[h][e] = o[h][e] + s[h][e];
      if (vec) {
        *(float4*)dst[h] = make_float4(s[h][0], s[h][1], s[h][2], s[h][3]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (b[h] + e < a.B) dst[h][e] = s[h][e];
      }
    }
  }
}

// Packing of a 64-row x 64-sample tile of an operand computed on the fly
// (KIND 0: e = exp(v[child] - m[b]); KIND 1: g = f / S) into
//   the node-major panel ("direct": rows drow0 + r, K = sample), 8 samples per
//   16-byte store, for every group in the sharing chain (exp only), and
//   the batch-major panel ("trans": rows = samples, K = tk0 + r), through an
//   LDS transpose, 8 rows per 16-byte store.
//
// With PROD (KIND 1 only) the backward of the product layer that follows the
// sum layer runs here too: an output row whose node is a child of that layer
// first gathers its parents' flows (parent order, then added to the old flow
// unless the layer stores), stores the flow and packs f / S; workgroups past
// the packing tiles push the flows of the product layer's other children.
template <int KIND, bool PROD>
__global__ __launch_bounds__(512) void k_pack(SumArgs a) {
  __shared__ float tile[64][65];
  const int t = blockIdx.x;
  if constexpr (PROD) {
    if (t >= a.fp_tiles) {
      prod_bwd_rest(a, t - a.fp_tiles, (int)gridDim.x - a.fp_tiles);
      return;
    }
  }
  const int rt = t / a.btiles, bt = t - rt * a.btiles;
  const int g = a.ngroups == 1 ? 0 : KIND == 0 ? a.pk_group[rt] : a.pg_group[rt];
  const GroupRec gr = a.ngroups == 1 ? a.group0 : a.groups[g];
  const int r0 = (rt - (KIND == 0 ? gr.pk_start : gr.pg_start)) * 64, b0 = bt * 64;
  const int nrows = KIND == 0 ? gr.N : gr.M;
  const int tid = threadIdx.x;
  // phase 1: item = (row, 8-sample chunk), 512 items, one per thread of the
  // 512-thread workgroup (16 waves per CU at two workgroups; two items per
  // thread on 256 threads measured slower): every load of the items is
  // issued before the first store (the stores could alias the loads, so the
  // compiler would not hoist a later item's loads)
  constexpr int U = 1;
  int kq[U], bsq[U], upq[U];
  bool okq[U], vq[U];
  float u0[U][8], u1[U][8], uo[U][8];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int it = tid + 512 * u, r = it >> 3, c = it & 7;
    const int k = r0 + r, bs = b0 + c * 8;
    kq[u] = k;
    bsq[u] = bs;
    okq[u] = k < nrows && bs < a.B;
    // the 8 samples' inputs: two 16-byte loads per array when the chunk is
    // whole and rows are 16-byte aligned (B % 4 == 0), else one by one
    vq[u] = (a.B & 3) == 0 && bs + 8 <= a.B;
    upq[u] = (PROD && okq[u]) ? a.fp_up[rt * 64 + r] : -1;
#pragma unroll
    for (int e = 0; e < 8; ++e) u0[u][e] = u1[u][e] = uo[u][e] = 0.0f;
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (!okq[u]) continue;
    const int k = kq[u], bs = bsq[u];
    if (KIND == 0) {
      load8(a.vals + (int64_t)child_of(gr, a.chblocks, k) * a.B + bs, vq[u], bs, a.B, u0[u]);
      load8((const float*)(a.mkeys + (int64_t)gr.m_row * a.B + bs), vq[u], bs, a.B, u1[u]);
    } else {
      if (PROD && upq[u] >= 0) {
        // single parent: its flow now; several: gathered below in parent order
        if (a.fp_single) load8(a.wflows + (int64_t)upq[u] * a.B + bs, vq[u], bs, a.B, u0[u]);
        if (!a.fp_store) load8(a.wflows + (int64_t)(gr.out_start + k) * a.B + bs, vq[u], bs, a.B, uo[u]);
      } else {
        load8(a.flows + (int64_t)(gr.out_start + k) * a.B + bs, vq[u], bs, a.B, u0[u]);
      }
      load8(a.ssum + (gr.s_row + k) * a.B + bs, vq[u], bs, a.B, u1[u]);
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int it = tid + 512 * u, r = it >> 3, c = it & 7;
    const int k = kq[u], bs = bsq[u];
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = 0.0f;
    if (okq[u]) {
      if (PROD && upq[u] >= 0) {
        // this output's flow: its parents in the product layer, in order,
        // added to the old flow unless the layer stores
        float f[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = 0.0f;
        if (a.fp_single) {
#pragma unroll
          for (int e = 0; e < 8; ++e) f[e] += u0[u][e];
        } else {
          const int up = upq[u];
          for (int q = a.fp_ptr[up]; q < a.fp_ptr[up + 1]; ++q) {
            float y[8];
            load8(a.wflows + (int64_t)a.fp_ids[q] * a.B + bs, vq[u], bs, a.B, y);
#pragma unroll
            for (int e = 0; e < 8; ++e) f[e] += y[e];
          }
        }
        if (!a.fp_store)
#pragma unroll
          for (int e = 0; e < 8; ++e) f[e] = uo[u][e] + f[e];
        store8(a.wflows + (int64_t)(gr.out_start + k) * a.B + bs, vq[u], bs, a.B, f);
#pragma unroll
        for (int e = 0; e < 8; ++e) u0[u][e] = f[e];
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (bs + e >= a.B) continue;
        if (KIND == 0) {
          x[e] = expf(u0[u][e] - key_shift(__float_as_uint(u1[u][e])));
        } else {
          const float fv = u0[u][e], sv = u1[u][e];
          x[e] = (fv == 0.0f || !(sv > 0.0f)) ? 0.0f : fv / sv;
        }
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) tile[r][c * 8 + e] = x[e];
    if (bs < a.B_padK) {
      if (KIND == 0) {
        // this group's rows from the record already in registers (a table
        // read after a store would wait for it), then the sharing chain's
        split_store8(x, a.np_direct, a.direct + panel(gr.e_row + k, bs, a.direct_rows), a.direct_plane);
        for (int q = gr.share_next; q >= 0; q = a.groups[q].share_next)
          split_store8(x, a.np_direct, a.direct + panel(a.groups[q].e_row + k, bs, a.direct_rows), a.direct_plane);
      } else {
        split_store8(x, a.np_direct, a.direct + panel(gr.g_row + k, bs, a.direct_rows), a.direct_plane);
      }
    }
  }
  __syncthreads();
  // phase 2: item = (sample, 8-row chunk); K columns up to the padded row count.
  // Four consecutive lanes take the four chunks of one sample's 32-row block,
  // so each store instruction writes whole 64-byte runs.
  const int kpad = (nrows + K_PAD - 1) / K_PAD * K_PAD;
  const int tk0 = KIND == 0 ? gr.e_koff : gr.g_koff;
  if (r0 >= kpad) return;
  for (int it = tid; it < 512; it += 512) {
    const int bl = (it >> 2) & 63, c = (it >> 8) * 4 + (it & 3);
    const int bb = b0 + bl;
    if (bb >= a.B_pad) continue;
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = tile[c * 8 + e][bl];
    split_store8(x, a.np_trans, a.trans + panel(bb, tk0 + r0 + c * 8, a.B_pad), a.trans_plane);
  }
}

// Split 4 values into np bfloat16 planes and store each plane as 8 bytes.
__device__ __forceinline__ void split_store4(const float (&x)[4], int np, uint16_t* dst, int64_t plane) {
  float r[4] = {x[0], x[1], x[2], x[3]};
  for (int p = 0; p < np; ++p) {
    uint32_t w[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const uint16_t h0 = f2bf(r[2 * e]), h1 = f2bf(r[2 * e + 1]);
      r[2 * e] -= bf2f(h0);
      r[2 * e + 1] -= bf2f(h1);
      w[e] = (uint32_t)h0 | ((uint32_t)h1 << 16);
    }
    *(uint2*)(dst + p * plane) = make_uint2(w[0], w[1]);
  }
}

// Weights of every block split into planes, [M_pad, N_padK] (forward operand)
// and transposed [N_pad, M_padK] (element-flow operand), both in fragment
// order (frag_major).  A 64 x 64
// tile per workgroup; each thread takes 4 consecutive columns of 4 rows (all
// four loads issued first, 16-byte loads when the block's rows are 16-byte
// aligned), and after the LDS transpose 4 consecutive rows of 4 columns, so
// every plane store is 8 bytes.
__global__ __launch_bounds__(256) void k_theta_pack(ThetaArgs a) {
  __shared__ float tile[64][65];
  const int t = blockIdx.x;
  const int bi = last_le(a.blocks, a.nblocks, t, [](const BlockRec& r) { return r.pk_start; });
  const BlockRec bl = a.blocks[bi];
  const int ntj = (bl.N + ROW_PAD - 1) / ROW_PAD * (ROW_PAD / 64);
  const int lt = t - bl.pk_start;
  const int i0 = (lt / ntj) * 64, j0 = (lt % ntj) * 64;
  const int NpK = (bl.N + K_PAD - 1) / K_PAD * K_PAD, MpK = (bl.M + K_PAD - 1) / K_PAD * K_PAD;
  const bool vec = ((bl.param_offset | (int64_t)bl.N) & 3) == 0;
  const int tid = threadIdx.x, rr = tid >> 4, c4 = (tid & 15) * 4;
  const int j = j0 + c4;
  float x[4][4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int i = i0 + rr + 16 * q;
    const float* src = a.params + bl.param_offset + (int64_t)i * bl.N + j;
    if (vec) {
      const float4 v = (i < bl.M && j < bl.N) ? *(const float4*)src : make_float4(0.f, 0.f, 0.f, 0.f);
      x[q][0] = v.x; x[q][1] = v.y; x[q][2] = v.z; x[q][3] = v.w;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) x[q][e] = (i < bl.M && j + e < bl.N) ? src[e] : 0.0f;
    }
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r = rr + 16 * q;
#pragma unroll
    for (int e = 0; e < 4; ++e) tile[r][c4 + e] = x[q][e];
    if (j < NpK) split_store4(x[q], a.np_fwd, a.theta + bl.th_off + frag_major(i0 + r, j, NpK >> 5), a.theta_plane);
  }
  __syncthreads();
  const int i = i0 + c4;                       // 4 consecutive rows of the block
  if (i >= MpK) return;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int jl = rr + 16 * q;
    const float y[4] = {tile[c4][jl], tile[c4 + 1][jl], tile[c4 + 2][jl], tile[c4 + 3][jl]};
    split_store4(y, a.np_elem, a.thetaT + bl.tht_off + frag_major(j0 + jl, i, MpK >> 5), a.thetaT_plane);
  }
}

// Overlapping children: f[c] (=|+=) sum of the scratch rows of c (group order).
template <int V>
__global__ void k_elem_reduce(SumArgs a) {
  const uint32_t QB = (uint32_t)(a.B / V), n = (uint32_t)a.nuniq * QB;
  for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) {
    const uint32_t k = i / QB, b = (i - k * QB) * V;
    Row<V> s;
#pragma unroll
    for (int e = 0; e < V; ++e) s.x[e] = 0.0f;
    sum_rows<V>(s, a.scratch, a.red_src, a.red_ptr[k], a.red_ptr[k + 1], a.B, b);
    float* dst = a.out_flows + (int64_t)a.red_child[k] * a.B + b;
    if (!a.store) {
      Row<V> o;
      o.load(dst);
#pragma unroll
      for (int e = 0; e < V; ++e) s.x[e] = o.x[e] + s.x[e];
    }
    s.store(dst);
  }
}

// ---- EM ------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_em(EmArgs a, int total_rows) {
  // one wave per parameter row, four rows per workgroup: the row sum is a
  // per-lane sum in index order then a fixed butterfly over the wave, so the
  // result does not depend on timing.  Rows of LowRank weight blocks under
  // the conditional M-step use R = F+ / W (theta > 0 and W > 0, else 0) in
  // place of F.
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= total_rows) return;
  const int s = last_le(a.segs, a.nsegs, row, [](const RowSeg& r) { return r.row_start; });
  const RowSeg sg = a.segs[s];
  const int64_t off = sg.offset + (int64_t)(row - sg.row_start) * sg.rlen;
  const bool vec = ((off | (int64_t)sg.rlen) & 3) == 0;   // 16-byte rows
  const bool corr = a.zflows != nullptr && sg.lowrank != 0;
  // the old weights enter only through the step's (1 - step) share and the
  // conditional M-step's test: a plain step of 1 writes without reading them
  // (0 stands in for them, which leaves the same bits for finite weights)
  const bool need_p = corr || a.step != 1.0f;
  auto ratio = [](float f, float w, float p) { return (p > 0.0f && w > 0.0f) ? f / w : 0.0f; };
  auto ratio4 = [&](float4 f, float4 w, float4 p) {
    return make_float4(ratio(f.x, w.x, p.x), ratio(f.y, w.y, p.y), ratio(f.z, w.z, p.z), ratio(f.w, w.w, p.w));
  };
  // rows of up to 1024 (16-byte aligned): the lane's four 16-byte chunks are
  // loaded at once and kept for the update, along with the parameters
  constexpr int RU = 4;
  const bool held = vec && sg.rlen <= RU * 256;
  float4 fh[RU], ph[RU];
  float acc = 0.0f;
  if (held) {
    float4 wh[RU];
#pragma unroll
    for (int u = 0; u < RU; ++u) {
      const int j = lane * 4 + u * 256;
      const bool in = j < sg.rlen;
      fh[u] = in ? *(const float4*)(a.pflows + off + j) : make_float4(0.f, 0.f, 0.f, 0.f);
      ph[u] = (in && need_p) ? *(const float4*)(a.params + off + j) : make_float4(0.f, 0.f, 0.f, 0.f);
      wh[u] = (in && corr) ? *(const float4*)(a.zflows + off + j) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    if (corr)
#pragma unroll
      for (int u = 0; u < RU; ++u) fh[u] = ratio4(fh[u], wh[u], ph[u]);
#pragma unroll
    for (int u = 0; u < RU; ++u)
      if (lane * 4 + u * 256 < sg.rlen) acc += ((fh[u].x + fh[u].y) + fh[u].z) + fh[u].w;
  } else if (vec) {
    for (int j = lane * 4; j < sg.rlen; j += 256) {
      float4 f = *(const float4*)(a.pflows + off + j);
      if (corr) f = ratio4(f, *(const float4*)(a.zflows + off + j), *(const float4*)(a.params + off + j));
      acc += ((f.x + f.y) + f.z) + f.w;
    }
  } else {
    for (int j = lane; j < sg.rlen; j += 64)
      acc += corr ? ratio(a.pflows[off + j], a.zflows[off + j], a.params[off + j]) : a.pflows[off + j];
  }
#pragma unroll
  for (int w = 32; w > 0; w >>= 1) acc += __shfl_xor(acc, w);
  const float tot = acc + a.pseudo;
  if (!(tot > 0.0f)) return;                    // a row without flow (and no pseudocount) keeps theta
  const float add = a.pseudo / (float)sg.rlen;
  const float keep = 1.0f - a.step;
  if (held) {
#pragma unroll
    for (int u = 0; u < RU; ++u) {
      const int j = lane * 4 + u * 256;
      if (j >= sg.rlen) continue;
      const float4 f = fh[u];
      float4 p = ph[u];
      p.x = keep * p.x + a.step * ((f.x + add) / tot);
      p.y = keep * p.y + a.step * ((f.y + add) / tot);
      p.z = keep * p.z + a.step * ((f.z + add) / tot);
      p.w = keep * p.w + a.step * ((f.w + add) / tot);
      *(float4*)(a.params + off + j) = p;
    }
  } else if (vec) {
    for (int j = lane * 4; j < sg.rlen; j += 256) {
      float4 f = *(const float4*)(a.pflows + off + j);
      float4 p = need_p ? *(const float4*)(a.params + off + j) : make_float4(0.f, 0.f, 0.f, 0.f);
      if (corr) f = ratio4(f, *(const float4*)(a.zflows + off + j), p);
      p.x = keep * p.x + a.step * ((f.x + add) / tot);
      p.y = keep * p.y + a.step * ((f.y + add) / tot);
      p.z = keep * p.z + a.step * ((f.z + add) / tot);
      p.w = keep * p.w + a.step * ((f.w + add) / tot);
      *(float4*)(a.params + off + j) = p;
    }
  } else {
    for (int j = lane; j < sg.rlen; j += 64) {
      const float f = corr ? ratio(a.pflows[off + j], a.zflows[off + j], a.params[off + j]) : a.pflows[off + j];
      const float nw = (f + add) / tot;
      a.params[off + j] = keep * (need_p ? a.params[off + j] : 0.0f) + a.step * nw;
    }
  }
}


// ---- launchers -------------------------------------------------------------------
static int grid_for(int64_t n, int per = 256, int cap = 65536) {
  int64_t g = (n + per - 1) / per;
  if (g < 1) g = 1;
  return (int)(g > cap ? cap : g);
}

void launch_fill_u32(uint32_t* p, int64_t n, uint32_t v, hipStream_t s) {
  if (n > 0) launch_kernel(k_fill_u32, dim3(grid_for(n)), dim3(256), 0, s, p, n, v);
}
void launch_fill_ranges(float* flows, const FillRange* d_ranges, int nranges, int64_t max_count, int B, hipStream_t s) {
  if (nranges <= 0) return;
  const int gx = grid_for(max_count * B, 256, 4096);
  launch_kernel(k_fill_ranges, dim3(gx, nranges), dim3(256), 0, s, flows, d_ranges, B);
}
void launch_copy_row(const float* src, float* dst, int B, hipStream_t s) {
  launch_kernel(k_copy_row, dim3((B + 255) / 256), dim3(256), 0, s, src, dst, B);
}
void launch_tokens_t(const int32_t* tok, int32_t* tokT, int B, int V, hipStream_t s) {
  launch_kernel(k_tokens_t, dim3((V + 31) / 32, (B + 31) / 32), dim3(256), 0, s, tok, tokT, B, V);
}
// V = 4 needs B % 4 == 0 (rows 16-byte aligned); the base pointers come
// from the caller's allocations, aligned far beyond 16 bytes.
#define PC_LAUNCH_V(kern, n_items, args, s)                                                       \
  do {                                                                                          \
    if ((args).B % 4 == 0)                                                                      \
      launch_kernel(kern<4>, dim3(grid_for((int64_t)(n_items) * ((args).B / 4))), dim3(256), 0, s, args); \
    else                                                                                        \
      launch_kernel(kern<1>, dim3(grid_for((int64_t)(n_items) * (args).B)), dim3(256), 0, s, args);       \
  } while (0)

void launch_input_fwd(const InputArgs& a, hipStream_t s) {
  // a lane takes the kernel's 4 items per pass (their loads in flight together)
  if ((a.B & 3) == 0)
    launch_kernel(k_input_fwd<4>, dim3(grid_for((int64_t)a.num_nodes * (a.B / 4), 256 * 4)), dim3(256), 0, s, a);
  else
    PC_LAUNCH_V(k_input_fwd, a.num_nodes, a, s);
}
void launch_bucket(const int32_t* tokT, int V, int B, int Kmax, int32_t* bptr, int32_t* bidx, hipStream_t s) {
  const size_t sh = (size_t)(Kmax + 1 + B) * sizeof(int32_t);
  launch_kernel(k_bucket, dim3(V), dim3(256), sh, s, tokT, B, Kmax, bptr, bidx);
}
void launch_input_bwd(const InputArgs& a, hipStream_t s) {
  if (a.num_rows <= 0) return;
  const size_t per = (size_t)(2 * a.B + a.K + 1) * sizeof(float);
  if (a.K <= 1024 && per * 4 <= 64 * 1024) {
    // rows of several nodes: the row's nodes over 4 waves; else one row per wave
    if (a.max_row_nodes >= 2) {
      if (a.B <= 64 * kPfB && a.K <= 512)
        launch_kernel(k_input_bwd_pf<4>, dim3(a.num_rows), dim3(256), per * 4, s, a);
      else
        launch_kernel(k_input_bwd<4>, dim3(a.num_rows), dim3(256), per * 4, s, a);
    } else {
      const size_t sh = (size_t)(5 * a.B + a.K + 1) * sizeof(float);
      const int nchunk = (a.max_var_nodes + kVarChunk - 1) / kVarChunk;
      if (a.B <= 64 * kPfB)
        launch_kernel(k_input_bwd_var_pf, dim3(a.num_vars * nchunk), dim3(256), sh, s, a);
      else
        launch_kernel(k_input_bwd_var, dim3(a.num_vars * nchunk), dim3(256), sh, s, a);
    }
  } else {
    launch_kernel(k_input_bwd_wide, dim3(a.num_rows), dim3(256), (size_t)a.B * sizeof(float), s, a);
  }
}
void launch_prod_fwd(const ProdArgs& a, hipStream_t s) { PC_LAUNCH_V(k_prod_fwd, a.num_nodes, a, s); }
void launch_prod_bwd(const ProdArgs& a, hipStream_t s) { PC_LAUNCH_V(k_prod_bwd, a.nuniq, a, s); }
// Column maxima (and the preceding product layer when a.fp_on): V samples per
// lane and RW children per wave, the first of (V, RW) = (4, 16) (16-byte
// accesses, batch a multiple of 4), (2, 16), (1, 16), (1, 4), (1, 1) that
// still gives 512 workgroups (two per CU), else (1, 1): a 4096-child layer
// at batch 512 is 64 tiles of 64 children, only 128 workgroups of 256
// samples; a 1024-child layer at batch 64 only 16 workgroups of 64 rows.
template <bool PROD>
static void launch_colmax_v(const SumArgs& a, int row_tiles, hipStream_t s) {
  const int g4 = row_tiles * ((a.B + 255) / 256), g2 = row_tiles * ((a.B + 127) / 128);
  const int g1 = row_tiles * ((a.B + 63) / 64);
  if (a.B % 4 == 0 && g4 >= 512)
    launch_kernel((k_colmax<4, PROD, 16>), dim3(g4), dim3(256), 0, s, a);
  else if (a.B % 2 == 0 && g2 >= 512)
    launch_kernel((k_colmax<2, PROD, 16>), dim3(g2), dim3(256), 0, s, a);
  else if (g1 >= 512)
    launch_kernel((k_colmax<1, PROD, 16>), dim3(g1), dim3(256), 0, s, a);
  // small layers: fewer workgroups with 16 children each rather than 256
  // with 4 (each workgroup publishes one atomic maximum per sample; on 1024
  // children x 64 samples: 4.6 us instead of 7.7)
  else if (g1 * 4 >= 64)
    launch_kernel((k_colmax<1, PROD, 4>), dim3(g1 * 4), dim3(256), 0, s, a);
  else
    launch_kernel((k_colmax<1, PROD, 1>), dim3(g1 * 16), dim3(256), 0, s, a);
}
void launch_colmax(const SumArgs& a, int row_tiles, hipStream_t s) {
  if (row_tiles <= 0) return;
  if (a.fp_on) launch_colmax_v<true>(a, row_tiles, s);
  else launch_colmax_v<false>(a, row_tiles, s);
}
void launch_exp_pack(const SumArgs& a, int row_tiles, hipStream_t s) {
  if (row_tiles > 0) launch_kernel((k_pack<0, false>), dim3(row_tiles * a.btiles), dim3(512), 0, s, a);
}
// Scaled flows; with a.fp_on also the following product layer's backward, its
// other children on up to 1024 extra workgroups.
void launch_g_pack(const SumArgs& a, int row_tiles, hipStream_t s) {
  if (row_tiles <= 0) return;
  if (!a.fp_on) {
    launch_kernel((k_pack<1, false>), dim3(row_tiles * a.btiles), dim3(512), 0, s, a);
    return;
  }
  SumArgs b = a;
  b.fp_tiles = row_tiles * a.btiles;
  // up to 16 workgroups per CU for the other children (2 items per lane per pass)
  const int rest = b.fp_nrest > 0 ? grid_for((int64_t)b.fp_nrest * ((a.B + 3) / 4), 256, 4096) : 0;
  launch_kernel((k_pack<1, true>), dim3(b.fp_tiles + rest), dim3(512), 0, s, b);
}
void launch_theta_pack(const ThetaArgs& a, int tiles, hipStream_t s) {
  if (tiles > 0) launch_kernel(k_theta_pack, dim3(tiles), dim3(256), 0, s, a);
}
void launch_elem_reduce(const SumArgs& a, hipStream_t s) { PC_LAUNCH_V(k_elem_reduce, a.nuniq, a, s); }
void launch_em(const EmArgs& a, int rows, hipStream_t s) {
  if (rows > 0) launch_kernel(k_em, dim3((rows + 3) / 4), dim3(256), 0, s, a, rows);
}

}  // namespace pc
