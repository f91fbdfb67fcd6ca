// k_lowrank.hip -- the LowRank exp_sum scaled sum layer (pyjuice.parameterizations.LowRank,
// definition and Training), fused on gfx950 matrix cores.
//
// Per sample b a group's weights are theta_b = q_b / Z_b with
//   q_b[i, j] = theta[i, j] exp(h_b[i, j]),  h_b = A_b B_b  (A_b [M, k], B_b [k, N]),
//   Z_b[i]    = sum_j q_b[i, j],
// and the layer value is v[i, b] = m[b] + log(Sraw[i, b] / Z[i, b]) with
// Sraw = sum_j q_b[i, j] e[j, b], e = exp(child - m).  q is rebuilt tile by
// tile (h on the matrix cores, one exp2 per pair) and never stored.
//
// Backward, with f the flow of the sum node and c1 = f / Sraw, c2 = f / Z:
//   edge flow        eps[i, j] = q e[j] c1[i]               (theta_b e g, g = f / S)
//   child flows      f[j]     += sum_i eps[i, j]
//   parameter flows  F+[i, j] += sum_b eps[i, j]
//   dLL/dh           X[i, j]   = eps - f theta_b = q (e[j] c1[i] - c2[i])
//   dLL/dA_b = X B_b^T = c1 U - c2 W  with U = sum_j q e B^T, W = sum_j q B^T (kept by the forward)
//   dLL/dB_b = A_b^T X
// The forward walks a 32-row strip of one sample per wave over all children
// (computing h^T so that each lane sums its row over children in registers,
// and U, W with a second matrix product fed straight from the first one's
// accumulators); the backward walks a 32-child strip over all rows (h, so
// that the child flows and dB sum over rows in registers).  Parameter flows
// of a strip are summed over the workgroup's 8 samples and added to one of
// ceil(B/8) partial matrices, reduced in order after the last layer.
//
// Precision: h uses PH bfloat16 planes per operand (hi + lo [+ lo2]; the
// products of planes below order PH), the gradient products U, W, dB use PG.
#include <hip/hip_runtime.h>

#include "pc_elem.h"

namespace pc {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

namespace {

constexpr float kLog2e = 1.4426950408889634f;
// weight slabs staged in LDS: 512 columns (forward) or 448 rows (backward) of
// a 32-wide strip, so that two workgroups share a CU
constexpr int kChunkF = 512, kChunkB = 448;
constexpr int kSlabF = 32 * (kChunkF + 4), kSlabB = 32 * (kChunkB + 4);

__device__ __forceinline__ float key_to_shift_lr(uint32_t k) {
  const uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  const float m = __uint_as_float(u);
  return (m == m && fabsf(m) <= 3.0e38f) ? m : 0.0f;
}

// x ~ sum of P bfloat16 planes, each the rounding of what the previous leave.
template <int P>
__device__ __forceinline__ void split8(const float (&x)[8], bf16x8_t (&out)[P]) {
  float r[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = x[e];
#pragma unroll
  for (int p = 0; p < P; ++p)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const __bf16 h = (__bf16)r[e];
      out[p][e] = h;
      r[e] -= (float)h;
    }
}

// acc += sum over plane pairs of order below P (highest order first) of a_pa b_pb
template <int P>
__device__ __forceinline__ void mfma_planes(f32x16_t& acc, const bf16x8_t (&a)[P], const bf16x8_t (&b)[P]) {
#pragma unroll
  for (int o = P - 1; o >= 0; --o)
#pragma unroll
    for (int pa = 0; pa <= o; ++pa) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[pa], b[o - pa], acc, 0, 0, 0);
}

__device__ __forceinline__ float4 ld4(const float* p) { return *(const float4*)p; }
__device__ __forceinline__ float at4(const float4& v, int e) { return e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w; }

}  // namespace

// e[j, b] = exp(v[child j, b] - m[b]), float32, sample-major [B][ldE] at column
// e_koff + j (zero for N <= j < N rounded up to 32).  64 children x 64
// samples per workgroup through an LDS transpose.
__global__ void k_lr_exp(LRArgs a) {
  __shared__ float t[64][65];
  const int ncols = (a.N + 31) / 32 * 32, nj = (ncols + 63) / 64;
  const int jt = blockIdx.x % nj, bt = blockIdx.x / nj;
  const int j0 = jt * 64, b0 = bt * 64;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int b = b0 + lane;
  const float sh = b < a.B ? key_to_shift_lr(a.mkeys[(int64_t)a.m_row * a.B + b]) : 0.0f;
  for (int r = w; r < 64; r += 4) {
    const int j = j0 + r;
    float e = 0.0f;
    if (j < a.N && b < a.B) {
      const int child = a.chblocks[a.blk_off + j / a.cbs] + j % a.cbs;
      e = expf(a.vals[(int64_t)child * a.B + b] - sh);
    }
    t[r][lane] = e;
  }
  __syncthreads();
  for (int r = w; r < 64; r += 4) {
    const int bb = b0 + r, j = j0 + lane;
    if (bb < a.B && j < ncols) a.E[(int64_t)bb * a.ldE + a.e_koff + j] = t[lane][r];   // zeros past N
  }
}

// Forward: workgroup = 32 rows x 4 samples (one per wave), all children.
template <int PH, int PG, int KC>
__global__ __launch_bounds__(256) void k_lr_fwd(LRArgs a) {
  __shared__ __attribute__((aligned(16))) float slab[kSlabF];   // theta rows [32][C + 4]
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, h = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int mt = (a.M + 31) / 32;
  const int i0 = (blockIdx.x % mt) * 32, b = (blockIdx.x / mt) * 4 + wave;
  const bool act = b < a.B;
  const int M = a.M, N = a.N, kr = a.krank;
  const float* Bb = a.Bf + (int64_t)(act ? b : 0) * kr * N;
  const float* Eb = a.E + (int64_t)(act ? b : 0) * a.ldE + a.e_koff;

  // second operand of h^T: A_b[i, k] log2(e), i = i0 + l32, k = kc*16 + h*8 + e
  bf16x8_t bA[KC][PH];
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) {
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int k = kc * 16 + h * 8 + e;
      x[e] = (act && k < kr && i0 + l32 < M) ? a.A[((int64_t)b * M + i0 + l32) * kr + k] * kLog2e : 0.0f;
    }
    split8<PH>(x, bA[kc]);
  }
  float Zp = 0.0f, Sp = 0.0f;
  f32x16_t U, W;
#pragma unroll
  for (int r = 0; r < 16; ++r) U[r] = W[r] = 0.0f;

  for (int c0 = 0; c0 < N; c0 += kChunkF) {
    // weights of the strip, zero outside the block (rows >= M, columns >= N)
    const int cw = (min(kChunkF, N - c0) + 31) / 32 * 32, CP = cw + 4;
    __syncthreads();
    for (int base = tid; base < 32 * cw; base += 256 * 8) {   // 8 loads in flight per thread
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int idx = base + u * 256, r = idx / cw, c = idx - r * cw;
        v[u] = (idx < 32 * cw && i0 + r < M && c0 + c < N) ? a.theta[(int64_t)(i0 + r) * N + c0 + c] : 0.0f;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int idx = base + u * 256, r = idx / cw, c = idx - r * cw;
        if (idx < 32 * cw) slab[r * CP + c] = v[u];
      }
    }
    __syncthreads();
    if (!act) continue;
    // global operands of one 32-child block, loaded a block ahead
    struct Ld {
      float xh[KC][8];    // B_b[k, j] for h^T: row j = j0 + l32, k = kc*16 + h*8 + e
      float4 ev[4];       // e[j, b] at rows j0 + g*8 + h*4 .. +3
      float xb[2][8];     // B_b[k, j] for U, W: row k = l32, K chunk cc
    };
    auto load = [&](int j0, Ld& L) {
#pragma unroll
      for (int kc = 0; kc < KC; ++kc)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int k = kc * 16 + h * 8 + e;
          L.xh[kc][e] = (k < kr && j0 + l32 < N) ? Bb[(int64_t)k * N + j0 + l32] : 0.0f;
        }
#pragma unroll
      for (int g = 0; g < 4; ++g) L.ev[g] = ld4(Eb + j0 + g * 8 + h * 4);
#pragma unroll
      for (int cc = 0; cc < 2; ++cc)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int j = j0 + 16 * cc + (e / 4) * 8 + h * 4 + (e % 4);
          L.xb[cc][e] = (l32 < kr && j < N) ? Bb[(int64_t)l32 * N + j] : 0.0f;
        }
    };
    const int nb = cw / 32;
    // one 32-child block from the operands in `cur`, with the block two ahead
    // loaded into the other buffer meanwhile (ping-pong: no register copies)
    auto block = [&](int jb, const Ld& cur, Ld& fill) {
      const int j0 = c0 + jb * 32;
      if (jb + 1 < nb) load(j0 + 32, fill);
      // h^T[j, i] = sum_k B_b[k, j] A_b[i, k]: first operand rows j = j0 + l32
      f32x16_t H;
#pragma unroll
      for (int r = 0; r < 16; ++r) H[r] = 0.0f;
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        bf16x8_t pb[PH];
        split8<PH>(cur.xh[kc], pb);
        mfma_planes<PH>(H, pb, bA[kc]);
      }
      // register r: row j = j0 + (r/4)*8 + h*4 + r%4, column i = i0 + l32
      float q[16], qe[16];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int jr = g * 8 + h * 4;
        const float4 th = *(const float4*)&slab[l32 * CP + (j0 - c0) + jr];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = g * 4 + e;
          q[r] = at4(th, e) * __builtin_amdgcn_exp2f(H[r]);
          qe[r] = q[r] * at4(cur.ev[g], e);
          Zp += q[r];
          Sp += qe[r];
        }
      }
      // U[k, i] += sum_j B_b[k, j] qe[j, i], W[k, i] += sum_j B_b[k, j] q[j, i]:
      // the second operand is the accumulator itself (K index 8h + e of chunk cc
      // is register 8cc + e, row j0 + 16cc + (e/4)*8 + h*4 + e%4)
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        float xq[8], xw[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          xq[e] = qe[8 * cc + e];
          xw[e] = q[8 * cc + e];
        }
        bf16x8_t pb[PG], pq[PG], pw[PG];
        split8<PG>(cur.xb[cc], pb);
        split8<PG>(xq, pq);
        split8<PG>(xw, pw);
        mfma_planes<PG>(U, pb, pq);
        mfma_planes<PG>(W, pb, pw);
      }
    };
    Ld b0, b1;
    load(c0, b0);
    for (int jb = 0; jb < nb; jb += 2) {
      block(jb, b0, b1);
      if (jb + 1 < nb) block(jb + 1, b1, b0);
    }
  }
  const float Z = Zp + __shfl_xor(Zp, 32), S = Sp + __shfl_xor(Sp, 32);
  const int i = i0 + l32;
  if (!act || i >= M) return;
  if (h == 0) {
    const float sh = key_to_shift_lr(a.mkeys[(int64_t)a.m_row * a.B + b]);
    a.Z[(int64_t)b * M + i] = Z;
    a.S[(int64_t)b * M + i] = S;
    a.vals[(int64_t)(a.out_start + i) * a.B + b] = (Z > 0.0f && S > 0.0f) ? sh + logf(S / Z) : -INFINITY;
  }
  // accumulator register r: row k = (r/4)*8 + h*4 + r%4, column i
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int k = (r / 4) * 8 + h * 4 + (r % 4);
    if (k < kr) {
      a.U[((int64_t)b * M + i) * kr + k] = U[r];
      a.W[((int64_t)b * M + i) * kr + k] = W[r];
    }
  }
}

// c1 = f / Sraw, c2 = f / Z per (sample, row); zero where the flow is zero or
// the node's value is -inf (Sraw = 0 or Z = 0).
__global__ void k_lr_coef(LRArgs a) {
  const int64_t n = (int64_t)a.B * a.M;
  for (int64_t x = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; x < n; x += (int64_t)gridDim.x * blockDim.x) {
    const int b = (int)(x / a.M), i = (int)(x - (int64_t)b * a.M);
    const float f = a.flows[(int64_t)(a.out_start + i) * a.B + b];
    const float Z = a.Z[x], S = a.S[x];
    const bool ok = f != 0.0f && Z > 0.0f && S > 0.0f;
    a.C1[x] = ok ? f / S : 0.0f;
    a.C2[x] = ok ? f / Z : 0.0f;
  }
}

// Backward: workgroup = 32 children x 8 samples (two per wave), all rows.
template <int PH, int PG, int KC>
__global__ __launch_bounds__(256) void k_lr_bwd(LRArgs a) {
  __shared__ __attribute__((aligned(16))) float slab[kSlabB];   // theta^T [32][R + 4]
  __shared__ float xch[4][1024];                                 // parameter flows of a 32 x 32 tile per wave
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, h = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nt = (a.N + 31) / 32;
  const int j0 = (blockIdx.x % nt) * 32, sg = blockIdx.x / nt;
  const int M = a.M, N = a.N, kr = a.krank;
  int bs[2];
  bool act[2];
  bs[0] = sg * 8 + wave;
  bs[1] = sg * 8 + 4 + wave;
  act[0] = bs[0] < a.B;
  act[1] = bs[1] < a.B;
  // second operand of h, per sample: B_b[k, j], j = j0 + l32
  bf16x8_t bB[2][KC][PH];
  float ev[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const float* Bb = a.Bf + (int64_t)(act[s] ? bs[s] : 0) * kr * N;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int k = kc * 16 + h * 8 + e;
        x[e] = (act[s] && k < kr && j0 + l32 < N) ? Bb[(int64_t)k * N + j0 + l32] : 0.0f;
      }
      split8<PH>(x, bB[s][kc]);
    }
    ev[s] = act[s] ? a.E[(int64_t)bs[s] * a.ldE + a.e_koff + j0 + l32] : 0.0f;   // zero past N
  }
  float fcp[2] = {0.0f, 0.0f};
  f32x16_t dB[2];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int r = 0; r < 16; ++r) dB[s][r] = 0.0f;
  float* P = a.P + (int64_t)sg * M * N;

  for (int r0 = 0; r0 < M; r0 += kChunkB) {
    // transposed weights of the strip, zero outside the block
    const int rw = (min(kChunkB, M - r0) + 31) / 32 * 32, RP = rw + 4;
    __syncthreads();
    for (int base = tid; base < rw * 32; base += 256 * 8) {   // 8 loads in flight per thread
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int idx = base + u * 256, ii = idx >> 5, jj = idx & 31;
        v[u] = (idx < rw * 32 && r0 + ii < M && j0 + jj < N) ? a.theta[(int64_t)(r0 + ii) * N + j0 + jj] : 0.0f;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int idx = base + u * 256, ii = idx >> 5, jj = idx & 31;
        if (idx < rw * 32) slab[jj * RP + ii] = v[u];
      }
    }
    __syncthreads();
    // global operands of one (32-row block, sample) step, loaded a step ahead
    struct Ld {
      float xa[KC][8];    // A_b[i, k] log2(e) for h: row i = i0 + l32, k = kc*16 + h*8 + e
      float c1[16], c2[16];
      float xk[2][8];     // A_b[i, k] for dB: row k = l32, K chunk cc
    };
    auto load = [&](int i0, int s, Ld& L) {
      const int b = bs[s];
      const float* Ab = a.A + (int64_t)b * M * kr;
#pragma unroll
      for (int kc = 0; kc < KC; ++kc)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int k = kc * 16 + h * 8 + e;
          L.xa[kc][e] = (k < kr && i0 + l32 < M) ? Ab[(int64_t)(i0 + l32) * kr + k] * kLog2e : 0.0f;
        }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = i0 + (r / 4) * 8 + h * 4 + (r % 4);
        L.c1[r] = i < M ? a.C1[(int64_t)b * M + i] : 0.0f;
        L.c2[r] = i < M ? a.C2[(int64_t)b * M + i] : 0.0f;
      }
#pragma unroll
      for (int cc = 0; cc < 2; ++cc)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int i = i0 + 16 * cc + (e / 4) * 8 + h * 4 + (e % 4);
          L.xk[cc][e] = (l32 < kr && i < M) ? Ab[(int64_t)i * kr + l32] : 0.0f;
        }
    };
    // the wave's steps: (row block ib, sample s) for its active samples
    const int nsteps = (rw / 32) * (act[1] ? 2 : act[0] ? 1 : 0);
    const int per = act[1] ? 2 : 1;
    Ld buf[2];
    if (nsteps > 0) load(r0, 0, buf[0]);
    for (int ib = 0; ib < rw / 32; ++ib) {
      const int i0 = r0 + ib * 32;
      float fp[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) fp[r] = 0.0f;
#pragma unroll
      for (int s = 0; s < 2; ++s) {      // static sample index: the per-sample operands stay in registers
        if (s >= per || nsteps == 0) continue;
        const int t = ib * per + s;
        // ping-pong: step t reads buf[t & 1] and fills the other with step t + 1
        auto stepk = [&](const Ld& cur, Ld& fill) {
          if (t + 1 < nsteps) load(r0 + ((t + 1) / per) * 32, (t + 1) % per, fill);
          // h[i, j] = sum_k A_b[i, k] B_b[k, j]: first operand rows i = i0 + l32
          f32x16_t H;
#pragma unroll
          for (int r = 0; r < 16; ++r) H[r] = 0.0f;
#pragma unroll
          for (int kc = 0; kc < KC; ++kc) {
            bf16x8_t pa[PH];
            split8<PH>(cur.xa[kc], pa);
            mfma_planes<PH>(H, pa, bB[s][kc]);
          }
          // register r: row i = i0 + (r/4)*8 + h*4 + r%4, column j = j0 + l32
          float X[16];
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int ir = g * 8 + h * 4;
            const float4 th = *(const float4*)&slab[l32 * RP + (i0 - r0) + ir];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int r = g * 4 + e;
              const float q = at4(th, e) * __builtin_amdgcn_exp2f(H[r]);
              const float eps = q * ev[s] * cur.c1[r];
              X[r] = q * (ev[s] * cur.c1[r] - cur.c2[r]);
              fcp[s] += eps;
              fp[r] += eps;
            }
          }
          // dB[k, j] += sum_i A_b[i, k] X[i, j]: K index 8h + e of chunk cc is
          // register 8cc + e, row i0 + 16cc + (e/4)*8 + h*4 + e%4
#pragma unroll
          for (int cc = 0; cc < 2; ++cc) {
            float xx[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) xx[e] = X[8 * cc + e];
            bf16x8_t pa[PG], px[PG];
            split8<PG>(cur.xk[cc], pa);
            split8<PG>(xx, px);
            mfma_planes<PG>(dB[s], pa, px);
          }
        };
        if (t & 1) stepk(buf[1], buf[0]);
        else stepk(buf[0], buf[1]);
      }
      // parameter flows of the tile, summed over the waves in order
#pragma unroll
      for (int r = 0; r < 16; ++r) xch[wave][r * 64 + lane] = fp[r];
      __syncthreads();
      for (int x = tid; x < 1024; x += 256) {
        const int r = x >> 6, ll = x & 63;
        const float v = ((xch[0][x] + xch[1][x]) + xch[2][x]) + xch[3][x];
        const int i = i0 + (r / 4) * 8 + (ll >> 5) * 4 + (r % 4), j = j0 + (ll & 31);
        if (i < M && j < N) P[(int64_t)i * N + j] += v;
      }
      __syncthreads();
    }
  }
  // child flows, dB
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const float tot = fcp[s] + __shfl_xor(fcp[s], 32);
    const int b = bs[s], j = j0 + l32;
    if (!act[s] || j >= N) continue;
    if (h == 0) {
      if (a.scratch_row >= 0) {
        a.scratch[(int64_t)(a.scratch_row + j) * a.B + b] = tot;
      } else {
        const int child = a.chblocks[a.blk_off + j / a.cbs] + j % a.cbs;
        float* dst = a.out_flows + (int64_t)child * a.B + b;
        *dst = a.store ? tot : *dst + tot;
      }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int k = (r / 4) * 8 + h * 4 + (r % 4);
      if (k < kr) a.dB[((int64_t)b * kr + k) * N + j] = dB[s][r];
    }
  }
}

// dLL/dA_b[i, k] = c1[i] U[i, k] - c2[i] W[i, k]
__global__ void k_lr_dA(LRArgs a) {
  const int64_t n = (int64_t)a.B * a.M * a.krank;
  for (int64_t x = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; x < n; x += (int64_t)gridDim.x * blockDim.x) {
    const int64_t bi = x / a.krank;
    a.dA[x] = a.C1[bi] * a.U[x] - a.C2[bi] * a.W[x];
  }
}

// F+ += sum of the ceil(B/8) partial matrices, in order.
__global__ void k_lr_fplus(const float* P, int nsg, int64_t elems, float* pflows) {
  for (int64_t x = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; x < elems; x += (int64_t)gridDim.x * blockDim.x) {
    float s = 0.0f;
    for (int g = 0; g < nsg; ++g) s += P[(int64_t)g * elems + x];
    pflows[x] += s;
  }
}

// ---- launchers ------------------------------------------------------------------
static int grid_lr(int64_t n) {
  const int64_t g = (n + 255) / 256;
  return (int)(g < 1 ? 1 : g > 65536 ? 65536 : g);
}

void launch_lr_exp(const LRArgs& a, hipStream_t s) {
  const int ncols = (a.N + 31) / 32 * 32;
  hipLaunchKernelGGL(k_lr_exp, dim3(((ncols + 63) / 64) * ((a.B + 63) / 64)), dim3(256), 0, s, a);
}

template <int PH, int PG>
static void lr_fwd_k(const LRArgs& a, hipStream_t s) {
  const dim3 grid(((a.M + 31) / 32) * ((a.B + 3) / 4));
  if (a.krank <= 16) hipLaunchKernelGGL((k_lr_fwd<PH, PG, 1>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((k_lr_fwd<PH, PG, 2>), grid, dim3(256), 0, s, a);
}
template <int PH, int PG>
static void lr_bwd_k(const LRArgs& a, hipStream_t s) {
  const dim3 grid(((a.N + 31) / 32) * ((a.B + 7) / 8));
  if (a.krank <= 16) hipLaunchKernelGGL((k_lr_bwd<PH, PG, 1>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((k_lr_bwd<PH, PG, 2>), grid, dim3(256), 0, s, a);
}

void launch_lr_fwd(const LRArgs& a, int fp32, hipStream_t s) {
  if (fp32) lr_fwd_k<3, 3>(a, s);
  else lr_fwd_k<2, 1>(a, s);
}
void launch_lr_coef(const LRArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_lr_coef, dim3(grid_lr((int64_t)a.B * a.M)), dim3(256), 0, s, a);
}
void launch_lr_bwd(const LRArgs& a, int fp32, hipStream_t s) {
  if (fp32) lr_bwd_k<3, 3>(a, s);
  else lr_bwd_k<2, 1>(a, s);
}
void launch_lr_dA(const LRArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_lr_dA, dim3(grid_lr((int64_t)a.B * a.M * a.krank)), dim3(256), 0, s, a);
}
void launch_lr_fplus(const float* P, int nsg, int64_t elems, float* pflows, hipStream_t s) {
  hipLaunchKernelGGL(k_lr_fplus, dim3(grid_lr(elems)), dim3(256), 0, s, P, nsg, elems, pflows);
}

}  // namespace pc
