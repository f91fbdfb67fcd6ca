// k_vbatch.hip -- the LowRank "sum_exp" scaled sum layer as products with the
// shared weights on a virtual batch (pyjuice.parameterizations.LowRank,
// definition: "sum_exp" is k matmuls with the shared parameters; Note: it
// runs through the plain sum-layer kernels on a virtual batch).
//
// With a = exp(A_b) [M, k], c = exp(B_b) [k, N] and e = exp(child - m), the
// scale g_b = a c is a sum of k rank-one terms, so every sum over the
// children of theta * g_b * (something per child) is k products with the
// shared theta.  Virtual column q = b * k + r (Q = B k of them):
//
//   forward    X[q, j] = c[r, j] e[j],  C[q, j] = c[r, j]          (k_vb_fwd_pack)
//              Tx = theta X^T, Tc = theta C^T                        (one product, 2Q columns)
//              Sraw[i] = sum_r a[i, r] Tx[i, q],  Z[i] = sum_r a[i, r] Tc[i, q]
//              v[i] = m + log(Sraw / Z)                               (k_vb_fwd_reduce)
//   backward   c1 = f / Sraw, c2 = f / Z; dA = a (c1 Tx - c2 Tc)      (k_lr_coef, Tx, Tc kept as U, W)
//              Y1[q, i] = a[i, r] c1[i],  Y2[q, i] = a[i, r] c2[i]   (k_vb_bwd_pack)
//              R1 = theta^T Y1^T, R2 = theta^T Y2^T                  (one product, 2Q columns)
//              f[j] += e[j] sum_r c[r, j] R1[j, q]
//              dB[r, j] = c[r, j] (e[j] R1[j, q] - R2[j, q])          (k_vb_bwd_reduce)
//   parameter flows F+ = theta * (Y1 X^T) and the denominator statistic
//              W = Y2 C^T, each one product over every (copy, sample, rank)
//
// The pack kernels write each operand in both layouts: batch-major (rows =
// virtual columns, K = children or nodes; the per-layer product's second
// operand) and node-major (rows = children or nodes of the copy, K = q; the
// parameter-flow products' operands, kept for all copies), bf16 planes as the
// plain layers' operands.
#include <hip/hip_runtime.h>

#include "pc_elem.h"

namespace pc {

namespace {

__device__ __forceinline__ float key_shift_vb(uint32_t k) {
  const uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  const float m = __uint_as_float(u);
  return (m == m && fabsf(m) <= 3.0e38f) ? m : 0.0f;
}

__device__ __forceinline__ uint16_t f2bf_vb(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__device__ __forceinline__ float bf2f_vb(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// 8 values into np bfloat16 planes (each the rounding of what the previous
// planes leave), one 16-byte store per plane.
__device__ __forceinline__ void store8_planes(const float (&x)[8], int np, uint16_t* dst, int64_t plane) {
  float r[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = x[e];
  for (int p = 0; p < np; ++p) {
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint16_t h0 = f2bf_vb(r[2 * e]), h1 = f2bf_vb(r[2 * e + 1]);
      r[2 * e] -= bf2f_vb(h0);
      r[2 * e + 1] -= bf2f_vb(h1);
      w[e] = (uint32_t)h0 | ((uint32_t)h1 << 16);
    }
    *(uint4*)(dst + p * plane) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// float -> e4m3 (OCP FP8 E4M3: bias 7, 3 mantissa bits, largest finite 448,
// no infinities), round to nearest even; |x| < 464 (the caller scales to
// below 256).  Normal range by rounding the float's mantissa to 3 bits,
// subnormals (below 2^-6) as the nearest multiple of 2^-9.
__device__ __forceinline__ uint32_t f2e4m3(float x) {
  if (!(x == x)) return 0x7fu;
  const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
  const float ax = fabsf(x);
  uint32_t code;
  if (ax >= 0.015625f) {
    uint32_t u = __float_as_uint(ax);
    u += 0x7ffffu + ((u >> 20) & 1u);
    code = ((((u >> 23) & 0xffu) - 120u) << 3) | ((u >> 20) & 7u);
    code = code > 0x7eu ? 0x7eu : code;
  } else {
    code = (uint32_t)rintf(ax * 512.0f);
  }
  return sign | code;
}

// 8 consecutive K values of one row, a quarter of a 32-wide K block whose
// other quarters are held by the neighbouring lanes (lane & 3 = the quarter,
// all four lanes call this): the block's scale 2^e with e = floor(log2 max|x|)
// - 7 (the block's largest magnitude lands in [128, 256)), the values x 2^-e
// as e4m3 in one 8-byte store, and the scale byte 127 + e from quarter 0.
// `st` false: the lane takes part in the maximum but stores nothing.
__device__ __forceinline__ void store8_e4m3(const float (&x)[8], bool st, uint8_t* dst, uint8_t* sdst) {
  float m = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(x[e]));
  m = fmaxf(m, __shfl_xor(m, 1));
  m = fmaxf(m, __shfl_xor(m, 2));
  int e = 0;
  if (m >= 1.17549435e-38f && m <= 3.4e38f) {
    e = (int)((__float_as_uint(m) >> 23) & 0xffu) - 127 - 7;
    e = e < -127 ? -127 : e > 127 ? 127 : e;
  }
  if (!st) return;
  uint32_t w[2] = {0u, 0u};
#pragma unroll
  for (int k = 0; k < 8; ++k) w[k >> 2] |= f2e4m3(ldexpf(x[k], -e)) << (8 * (k & 3));
  *(uint2*)dst = make_uint2(w[0], w[1]);
  if ((threadIdx.x & 3) == 0) *sdst = (uint8_t)(127 + e);
}

__device__ __forceinline__ int64_t panel8(int64_t r, int64_t k, int64_t R) { return ((k >> 6) * R + r) * 64 + (k & 63); }
__device__ __forceinline__ int64_t scale8(int64_t r, int64_t k, int64_t R) { return (k >> 5) * R + r; }

__device__ __forceinline__ int child_vb(const VBArgs& a, int j) {
  return a.chblocks[a.blk_off + j / a.cbs] + j % a.cbs;
}

}  // namespace

// Forward operands: a workgroup packs a 64 (q) x 64 (j) tile of X and of C.
// Phase 1, item = (q, 8 children): c = exp(B_b[r, j]) (row q of B_b viewed as
// [Q, N]), e of the 8 children for the sample b = q / k; stores the
// batch-major rows q (X) and Q + q (C), 8 children per 16-byte store.
// Phase 2, through LDS, item = (j, 8 virtual columns): the node-major rows
// e_row + j of X and C, K = q.  Children past N and columns past Q are zeros
// (the K padding of both layouts); virtual rows past 2Q are left alone (the
// products' columns there are never stored).
__global__ __launch_bounds__(512) void k_vb_fwd_pack(VBArgs a) {
  __shared__ float tx[64][65], tc[64][65];
  __shared__ float te[64][65];     // e of the tile's children for its samples (q0 / k ..)
  const int nqt = (a.QK + 63) / 64;
  const int qt = blockIdx.x % nqt, jt = blockIdx.x / nqt;
  const int q0 = qt * 64, j0 = jt * 64;
  const int tid = threadIdx.x;
  // phase 0: e[j, b] = exp(child j - m[b]) once per (child, sample) of the
  // tile (its 64 virtual columns cover at most 64 samples), not once per rank
  {
    const int bfirst = q0 / a.krank;
    const int nb = min((q0 + 63) / a.krank, a.B - 1) - bfirst + 1;
    for (int it = tid; it < 64 * nb; it += 512) {
      const int jl = it & 63, bl = it >> 6, j = j0 + jl, b = bfirst + bl;
      float ev = 0.0f;
      if (j < a.N) ev = expf(a.vals[(int64_t)child_vb(a, j) * a.B + b] - key_shift_vb(a.mkeys[(int64_t)a.m_row * a.B + b]));
      te[bl][jl] = ev;
    }
  }
  __syncthreads();
  {
    const int r8 = tid >> 3, c8 = tid & 7;
    const int q = q0 + r8, jb = j0 + c8 * 8;
    float x[8], cc[8];
    const bool qv = q < a.Q;
    const int bl = qv ? q / a.krank - q0 / a.krank : 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int j = jb + e;
      float cv = 0.0f, ev = 0.0f;
      if (qv && j < a.N) {
        cv = expf(a.Bf[(int64_t)q * a.N + j]);
        ev = te[bl][c8 * 8 + e];
      }
      cc[e] = cv;
      x[e] = cv * ev;
      tx[r8][c8 * 8 + e] = x[e];
      tc[r8][c8 * 8 + e] = cc[e];
    }
    if (qv) {
      store8_planes(x, a.np_bt, a.vbt + panel(q, jb, a.Qpad), a.vbt_plane);
      store8_planes(cc, a.np_bt, a.vbt + panel(a.Q + q, jb, a.Qpad), a.vbt_plane);
    }
  }
  if (a.np_n == 0 && !a.f8) return;   // forward only: no node-major operands
  __syncthreads();
  {
    const int jl = tid >> 3, c8 = tid & 7;
    const int j = j0 + jl;
    if (j >= a.N) return;            // the four lanes of a K block share j
    float x[8], cc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      x[e] = tx[c8 * 8 + e][jl];
      cc[e] = tc[c8 * 8 + e][jl];
    }
    const int64_t row = a.n_row0 + j;
    const int k = q0 + c8 * 8;
    if (a.f8) {
      store8_e4m3(x, true, a.n8lo + panel8(row, k, a.n_rows), a.s8lo + scale8(row, k, a.n_rows));
      store8_e4m3(cc, true, a.n8hi + panel8(row, k, a.n_rows), a.s8hi + scale8(row, k, a.n_rows));
    } else {
      store8_planes(x, a.np_n, a.nlo + panel(row, k, a.n_rows), a.n_plane);
      store8_planes(cc, a.np_n, a.nhi + panel(row, k, a.n_rows), a.n_plane);
    }
  }
}

// Forward reduction over the rank, four lanes per (sample, node), lane l of
// the four taking ranks 4l .. 4l + 3 (+ 16 t): Sraw = sum_r a Tx, Z = sum_r a
// Tc (Tx, Tc stored as U, W [B, M, k]), v = m + log(Sraw / Z) (-inf unless
// both are positive).  The four lanes' sums are added in a fixed order.
__global__ __launch_bounds__(256) void k_vb_fwd_reduce(VBArgs a) {
  const int64_t x = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 2;
  const int l = threadIdx.x & 3;
  const bool live = x < (int64_t)a.B * a.M;
  const int kr = a.krank;
  float S = 0.0f, Z = 0.0f;
  if (live) {
    const float* Ar = a.A + x * kr;
    const float* Ur = a.U + x * kr;
    const float* Wr = a.W + x * kr;
    for (int r0 = 4 * l; r0 < kr; r0 += 16) {
      if ((kr & 3) == 0) {
        const float4 av = *(const float4*)(Ar + r0), uv = *(const float4*)(Ur + r0), wv = *(const float4*)(Wr + r0);
        const float e0 = expf(av.x), e1 = expf(av.y), e2 = expf(av.z), e3 = expf(av.w);
        S += e0 * uv.x + e1 * uv.y + e2 * uv.z + e3 * uv.w;
        Z += e0 * wv.x + e1 * wv.y + e2 * wv.z + e3 * wv.w;
      } else {
        for (int r = r0; r < r0 + 4 && r < kr; ++r) {
          const float e = expf(Ar[r]);
          S += e * Ur[r];
          Z += e * Wr[r];
        }
      }
    }
  }
  // lanes 0..3 of the row: (0 + 1) + (2 + 3)
  S += __shfl_xor(S, 1);
  Z += __shfl_xor(Z, 1);
  S += __shfl_xor(S, 2);
  Z += __shfl_xor(Z, 2);
  if (!live || l != 0) return;
  const int b = (int)(x / a.M), i = (int)(x - (int64_t)b * a.M);
  a.S[x] = S;
  a.Z[x] = Z;
  const float sh = key_shift_vb(a.mkeys[(int64_t)a.m_row * a.B + b]);
  a.vals[(int64_t)(a.out_start + i) * a.B + b] = (Z > 0.0f && S > 0.0f) ? sh + logf(S / Z) : -INFINITY;
}

// Backward operands: a workgroup packs a 64 (q) x 64 (i) tile of Y1 and Y2.
// Phase 1, item = (i, 8 virtual columns): a = exp(A_b[i, r]) and c1, c2 of
// (b, i); the node-major rows g_row + i (K = q).  Phase 2, through LDS, item =
// (q, 8 nodes): the batch-major rows q (Y1) and Q + q (Y2), K = i.  Zeros past
// M and past Q as for the forward operands.
__global__ __launch_bounds__(512) void k_vb_bwd_pack(VBArgs a) {
  __shared__ float t1[64][65], t2[64][65];
  const int nqt = (a.QK + 63) / 64;
  const int qt = blockIdx.x % nqt, it = blockIdx.x / nqt;
  const int q0 = qt * 64, i0 = it * 64;
  const int tid = threadIdx.x;
  const int ldC = (a.M + 31) / 32 * 32;
  {
    const int il = tid >> 3, c8 = tid & 7;
    const int i = i0 + il, qb = q0 + c8 * 8;
    float y1[8], y2[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int q = qb + e;
      float v1 = 0.0f, v2 = 0.0f;
      if (q < a.Q && i < a.M) {
        const int b = q / a.krank, r = q - b * a.krank;
        const float av = expf(a.A[((int64_t)b * a.M + i) * a.krank + r]);
        v1 = av * a.C1[(int64_t)b * ldC + i];
        v2 = av * a.C2[(int64_t)b * ldC + i];
      }
      y1[e] = v1;
      y2[e] = v2;
      t1[il][c8 * 8 + e] = v1;
      t2[il][c8 * 8 + e] = v2;
    }
    if (a.f8) {
      // rows past M (the four lanes of a K block share i) store nothing
      const int64_t row = a.n_row0 + i;
      store8_e4m3(y1, i < a.M, a.n8lo + panel8(row, qb, a.n_rows), a.s8lo + scale8(row, qb, a.n_rows));
      store8_e4m3(y2, i < a.M, a.n8hi + panel8(row, qb, a.n_rows), a.s8hi + scale8(row, qb, a.n_rows));
    } else if (i < a.M && a.np_n > 0) {
      store8_planes(y1, a.np_n, a.nlo + panel(a.n_row0 + i, qb, a.n_rows), a.n_plane);
      store8_planes(y2, a.np_n, a.nhi + panel(a.n_row0 + i, qb, a.n_rows), a.n_plane);
    }
  }
  __syncthreads();
  {
    const int ql = tid >> 3, c8 = tid & 7;
    const int q = q0 + ql, ib = i0 + c8 * 8;
    if (q >= a.Q) return;
    float y1[8], y2[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      y1[e] = t1[c8 * 8 + e][ql];
      y2[e] = t2[c8 * 8 + e][ql];
    }
    store8_planes(y1, a.np_bt, a.vbt + panel(q, ib, a.Qpad), a.vbt_plane);
    store8_planes(y2, a.np_bt, a.vbt + panel(a.Q + q, ib, a.Qpad), a.vbt_plane);
  }
}

// Backward reduction over the rank, four lanes per (sample, child), lane l
// taking ranks 4l .. 4l + 3 (+ 16 t): dLL/dB_b[r, j] = c (e R1 - R2) and the
// child flow e sum_r c R1 (the four lanes' sums added in a fixed order;
// stored, added, or into the layer's scratch rows when several groups share
// children).
__global__ __launch_bounds__(256) void k_vb_bwd_reduce(VBArgs a) {
  const int64_t x = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 2;
  const int l = threadIdx.x & 3;
  const bool live = x < (int64_t)a.B * a.N;
  const int kr = a.krank;
  int b = 0, j = 0, child = 0;
  float ev = 0.0f, t = 0.0f;
  if (live) {
    b = (int)(x / a.N);
    j = (int)(x - (int64_t)b * a.N);
    child = child_vb(a, j);
    const float sh = key_shift_vb(a.mkeys[(int64_t)a.m_row * a.B + b]);
    ev = expf(a.vals[(int64_t)child * a.B + b] - sh);
    const float* R1 = a.R1 + x * kr;
    const float* R2 = a.R2 + x * kr;
    for (int r0 = 4 * l; r0 < kr; r0 += 16) {
      float r1[4] = {0.0f, 0.0f, 0.0f, 0.0f}, r2[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      if ((kr & 3) == 0) {
        const float4 u = *(const float4*)(R1 + r0), w = *(const float4*)(R2 + r0);
        r1[0] = u.x; r1[1] = u.y; r1[2] = u.z; r1[3] = u.w;
        r2[0] = w.x; r2[1] = w.y; r2[2] = w.z; r2[3] = w.w;
      } else {
        for (int e = 0; e < 4 && r0 + e < kr; ++e) {
          r1[e] = R1[r0 + e];
          r2[e] = R2[r0 + e];
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = r0 + e;
        if (r >= kr) break;
        const int64_t o = ((int64_t)b * kr + r) * a.N + j;
        const float cv = expf(a.Bf[o]);
        t += cv * r1[e];
        a.dB[o] = cv * (ev * r1[e] - r2[e]);
      }
    }
  }
  t += __shfl_xor(t, 1);
  t += __shfl_xor(t, 2);
  if (!live || l != 0) return;
  const float fl = ev * t;
  if (a.scratch_row >= 0) {
    a.scratch[(int64_t)(a.scratch_row + j) * a.B + b] = fl;
  } else {
    float* dst = a.out_flows + (int64_t)child * a.B + b;
    *dst = a.store ? fl : *dst + fl;
  }
}

// ---- launchers ------------------------------------------------------------
void launch_vb_fwd_pack(const VBArgs& a, hipStream_t s) {
  const int tiles = ((a.QK + 63) / 64) * ((a.N + 63) / 64);
  launch_kernel(k_vb_fwd_pack, dim3(tiles), dim3(512), 0, s, a);
}
void launch_vb_fwd_reduce(const VBArgs& a, hipStream_t s) {
  const int64_t n = (int64_t)a.B * a.M * 4;
  launch_kernel(k_vb_fwd_reduce, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a);
}
void launch_vb_bwd_pack(const VBArgs& a, hipStream_t s) {
  const int tiles = ((a.QK + 63) / 64) * ((a.M + 63) / 64);
  launch_kernel(k_vb_bwd_pack, dim3(tiles), dim3(512), 0, s, a);
}
void launch_vb_bwd_reduce(const VBArgs& a, hipStream_t s) {
  const int64_t n = (int64_t)a.B * a.N * 4;
  launch_kernel(k_vb_bwd_reduce, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a);
}

}  // namespace pc
