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
constexpr int kChunkF = 512, kChunkB = 512;
constexpr int kSlabF = 32 * (kChunkF + 4), kSlabB = 32 * (kChunkB + 4);

// Order-preserving 32-bit key of a float (integer atomic max = float max).
__device__ __forceinline__ uint32_t float_to_key_lr(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

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

// ---- per-layer preparation ---------------------------------------------------
// Fragment records: the factors of one sample and one 32-wide block of rows (A)
// or columns (B), split into bfloat16 planes and stored in the order the
// matrix instructions read them (64 lanes x 8 values, 16 bytes per lane), so
// that the fused kernels load each operand with one 16-byte access per lane:
//   A side, block ib of rows, per sample b:
//     h form, K chunk kc (PH planes): lane l: A[ib*32 + l%32][kc*16 + (l/32)*8 + e] * log2(e)
//     d form, rank block kb, chunk cc (PG planes):
//                                     lane l: A[ib*32 + 16cc + (e/4)*8 + (l/32)*4 + e%4][kb*32 + l%32]
//   B side, block jb of columns, per sample b:
//     h form, K chunk kc (PH planes): lane l: B[kc*16 + (l/32)*8 + e][jb*32 + l%32]
//     u form, rank block kb, chunk cc (PG planes):
//                                     lane l: B[kb*32 + l%32][jb*32 + 16cc + (e/4)*8 + (l/32)*4 + e%4]
// (zero outside the factor).  The h forms are the two operands of h = A B (or
// of its transpose); the d form is the first operand of dB = A^T X and the u
// form that of U^T, W^T = B (q e)^T, B q^T, whose second operands come from h's
// accumulator registers, hence the permuted order along the contraction.
// Records of a block: the h forms (kc, plane), then the d / u forms (kb, cc,
// plane).  KC chunks of 16 cover the rank in h; KB blocks of 32 cover it in
// the gradient products (KB = 1 up to rank 32, 2 up to rank 64).
constexpr int kFrag = 512;   // bfloat16 elements per record

template <int PH, int PG, int KC, int KB>
struct LrPack {
  static constexpr int FB = KC * PH + 2 * KB * PG;     // records per block
  static __device__ __forceinline__ const uint16_t* bside(const uint16_t* pk, int N, int b, int jb) {
    const int nJB = (N + 31) / 32;
    return pk + ((int64_t)b * nJB + jb) * FB * kFrag;
  }
  static __device__ __forceinline__ const uint16_t* aside(const uint16_t* pk, int Bn, int M, int N, int b, int ib) {
    const int nJB = (N + 31) / 32, nIB = (M + 31) / 32;
    return pk + ((int64_t)Bn * nJB + (int64_t)b * nIB + ib) * FB * kFrag;
  }
};

// One 16-byte fragment: `ub` is uniform over the wave (held in scalar
// registers), `lane_bytes` the lane's 32-bit offset.
__device__ __forceinline__ bf16x8_t ldfrag(const uint16_t* ub, uint32_t lane_bytes) {
  return *(const bf16x8_t*)((const char*)ub + lane_bytes);
}

// Round x into P bfloat16 planes (each the rounding of what the previous
// planes leave) and store plane p as 16 bytes at dst + p * kFrag.
template <int P>
__device__ __forceinline__ void split_store_frag(const float (&x)[8], uint16_t* dst) {
  bf16x8_t o[P];
  split8<P>(x, o);
#pragma unroll
  for (int p = 0; p < P; ++p) *(bf16x8_t*)(dst + p * kFrag) = o[p];
}

// The fragment records of every LowRank group of the circuit, made once per
// forward and kept for the backward: workgroups [wg0[g], wg0[g + 1]) pack
// group g, four record sets (64 lanes each) per workgroup.
template <int PH, int PG, int KC, int KB>
__global__ __launch_bounds__(256) void k_lr_pack(LRPackArgs pa) {
  using PK = LrPack<PH, PG, KC, KB>;
  constexpr int NF = KC + 2 * KB;                  // forms per block
  const int tid = threadIdx.x;
  // "sum_exp": every record holds exp of the factor (the matrix instructions
  // then sum exp(A) exp(B) over the rank, no log2(e) on the h form); padding
  // stays 0
  const bool se = pa.sumexp != 0;
  auto fv = [se](float v) { return se ? expf(v) : v; };
  int g = 0;
  while (g + 1 < pa.ngroups && (int)blockIdx.x >= pa.wg0[g + 1]) ++g;
  const int M = pa.M[g], N = pa.N[g], Bn = pa.B, kr = pa.krank;
  const int nJB = (N + 31) / 32, nIB = (M + 31) / 32;
  const int64_t nsets = (int64_t)Bn * (nJB + nIB) * NF;
  const int64_t set = (int64_t)(blockIdx.x - pa.wg0[g]) * 4 + (tid >> 6);
  if (set >= nsets) return;
  const int lane = tid & 63, l32 = lane & 31, h = lane >> 5;
  const int form = (int)(set % NF);
  const int64_t rest = set / NF;
  const int blk = (int)(rest % (nJB + nIB)), b = (int)(rest / (nJB + nIB));
  float x[8];
  if (blk < nJB) {
    const int jb = blk;
    const float* Bb = pa.Bf[g] + (int64_t)b * kr * N;
    uint16_t* dst = const_cast<uint16_t*>(PK::bside(pa.pk[g], N, b, jb)) + lane * 8;
    if (form < KC) {
      const int j = jb * 32 + l32;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int k = form * 16 + h * 8 + e;
        x[e] = (k < kr && j < N) ? fv(Bb[(int64_t)k * N + j]) : 0.0f;
      }
      split_store_frag<PH>(x, dst + form * PH * kFrag);
    } else {
      const int kb = (form - KC) >> 1, cc = (form - KC) & 1, kk = kb * 32 + l32;
      const int jq = jb * 32 + 16 * cc + h * 4;     // values e of runs jq + (e/4)*8 + e%4
      if ((N & 3) == 0 && kk < kr && jq + 11 < N) {
        const float4 u0 = ld4(Bb + (int64_t)kk * N + jq), u1 = ld4(Bb + (int64_t)kk * N + jq + 8);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[e] = fv(at4(u0, e));
          x[4 + e] = fv(at4(u1, e));
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int j = jq + (e / 4) * 8 + (e % 4);
          x[e] = (kk < kr && j < N) ? fv(Bb[(int64_t)kk * N + j]) : 0.0f;
        }
      }
      split_store_frag<PG>(x, dst + (KC * PH + (kb * 2 + cc) * PG) * kFrag);
    }
  } else {
    const int ib = blk - nJB;
    const float* Ab = pa.A[g] + (int64_t)b * M * kr;
    uint16_t* dst = const_cast<uint16_t*>(PK::aside(pa.pk[g], Bn, M, N, b, ib)) + lane * 8;
    if (form < KC) {
      const int i = ib * 32 + l32, k0 = form * 16 + h * 8;
      if ((kr & 3) == 0 && i < M && k0 + 8 <= kr) {
        const float4 u0 = ld4(Ab + (int64_t)i * kr + k0), u1 = ld4(Ab + (int64_t)i * kr + k0 + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[e] = se ? expf(at4(u0, e)) : at4(u0, e) * kLog2e;
          x[4 + e] = se ? expf(at4(u1, e)) : at4(u1, e) * kLog2e;
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int k = k0 + e;
          x[e] = (k < kr && i < M) ? (se ? expf(Ab[(int64_t)i * kr + k]) : Ab[(int64_t)i * kr + k] * kLog2e) : 0.0f;
        }
      }
      split_store_frag<PH>(x, dst + form * PH * kFrag);
    } else {
      const int kb = (form - KC) >> 1, cc = (form - KC) & 1, kk = kb * 32 + l32;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int i = ib * 32 + 16 * cc + (e / 4) * 8 + h * 4 + (e % 4);
        x[e] = (kk < kr && i < M) ? fv(Ab[(int64_t)i * kr + kk]) : 0.0f;
      }
      split_store_frag<PG>(x, dst + (KC * PH + (kb * 2 + cc) * PG) * kFrag);
    }
  }
}

// Backward coefficients, one (sample, row) per thread over rows padded to 32:
// c1 = f / Sraw, c2 = f / Z (zero where the flow is zero or the node's value
// is -inf, and on the padding rows) and dLL/dA_b[i, k] = c1 U[i, k] - c2 W[i, k]
// ("exp_sum"), exp(A_b[i, k]) (c1 U[i, k] - c2 W[i, k]) ("sum_exp", whose U and
// W sum theta e exp(B) and theta exp(B) over the children).
__global__ __launch_bounds__(256) void k_lr_coef(LRArgs a) {
  // four lanes per (sample, row): lane l takes ranks 4l .. 4l + 3 (+ 16 t), so
  // the four lanes of a row read and write 64 contiguous bytes at a time
  const int ldC = (a.M + 31) / 32 * 32;
  const int64_t xt = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t xc = xt >> 2;
  const int l = (int)(xt & 3);
  if (xc >= (int64_t)a.B * ldC) return;
  const int b = (int)(xc / ldC), i = (int)(xc - (int64_t)b * ldC);
  if (i >= a.M) {
    if (l == 0) {
      a.C1[xc] = 0.0f;
      a.C2[xc] = 0.0f;
    }
    return;
  }
  const int64_t x = (int64_t)b * a.M + i;
  float f;
  if (a.fp_on) {
    // the product node's flow, added to zero as the product backward does,
    // stored for both its children
    f = 0.0f + a.flows[(int64_t)(a.fp_pstart + i) * a.B + b];
    if (l == 0) {
      a.out_flows[(int64_t)(a.out_start + i) * a.B + b] = f;
      a.out_flows[(int64_t)(a.fp_other + i) * a.B + b] = f;
    }
  } else {
    f = a.flows[(int64_t)(a.out_start + i) * a.B + b];
  }
  const float Z = a.Z[x], S = a.S[x];
  const bool ok = f != 0.0f && Z > 0.0f && S > 0.0f;
  const float c1 = ok ? f / S : 0.0f, c2 = ok ? f / Z : 0.0f;
  if (l == 0) {
    a.C1[xc] = c1;
    a.C2[xc] = c2;
  }
  const int kr = a.krank;
  const int64_t o = x * kr;
  if ((kr & 3) == 0) {        // rows of A, U, W, dA 16-byte aligned
    for (int k = 4 * l; k < kr; k += 16) {
      const float4 u = ld4(a.U + o + k), w = ld4(a.W + o + k);
      float4 d = make_float4(c1 * u.x - c2 * w.x, c1 * u.y - c2 * w.y, c1 * u.z - c2 * w.z, c1 * u.w - c2 * w.w);
      if (a.sumexp) {
        const float4 av = ld4(a.A + o + k);
        d = make_float4(expf(av.x) * d.x, expf(av.y) * d.y, expf(av.z) * d.z, expf(av.w) * d.w);
      }
      *(float4*)(a.dA + o + k) = d;
    }
  } else {
    for (int k = l; k < kr; k += 4) {
      const float d = c1 * a.U[o + k] - c2 * a.W[o + k];
      a.dA[o + k] = a.sumexp ? expf(a.A[o + k]) * d : d;
    }
  }
}

// Forward: workgroup = 32 rows x 4 samples (one per wave), all children, in
// chunks of kChunkF children.  Per chunk the weights of the row strip and
// e[j, b] = exp(v[child j, b] - m[b]) of the 4 samples are staged in LDS; a
// wave streams its sample's B records one 32-child block ahead.  SE: the
// "sum_exp" form, whose records hold exp(A), exp(B), so the matrix product is
// the scale g itself (no exp per pair) and U, W sum theta e and theta against
// exp(B) (the coefficient kernel multiplies by exp(A)).
template <int PH, int PG, int KC, int KB, bool SE = false>
__global__ __launch_bounds__(256) void k_lr_fwd(LRArgs a) {
  using PK = LrPack<PH, PG, KC, KB>;
  __shared__ __attribute__((aligned(16))) float slab[kSlabF];   // theta rows [32][C + 4]
  __shared__ __attribute__((aligned(16))) float el[4][kChunkF]; // e of the chunk, per sample
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, h = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int mt = (a.M + 31) / 32;
  const int ib = blockIdx.x % mt, i0 = ib * 32, b0 = (blockIdx.x / mt) * 4, b = b0 + wave;
  const bool act = b < a.B;
  const int M = a.M, N = a.N, kr = a.krank;
  const int bq = act ? b : 0;
  const uint16_t* Bp = PK::bside(a.pk, N, bq, 0);           // block jb at + jb * FB * kFrag
  const uint32_t lb = (uint32_t)lane * 16;
  // this thread's sample for staging e: b0 + (tid & 3), its shift
  const int es = tid & 3;
  const float esh = b0 + es < a.B ? key_to_shift_lr(a.mkeys[(int64_t)a.m_row * a.B + b0 + es]) : 0.0f;

  // second operand of h^T: the h form of A_b for this row strip
  bf16x8_t bA[KC][PH];
  {
    const uint16_t* ap = PK::aside(a.pk, a.B, M, N, bq, ib);
#pragma unroll
    for (int kc = 0; kc < KC; ++kc)
#pragma unroll
      for (int p = 0; p < PH; ++p) bA[kc][p] = ldfrag(ap + (kc * PH + p) * kFrag, lb);
  }
  float Zp = 0.0f, Sp = 0.0f;
  f32x16_t U[KB], W[KB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) U[kb][r] = W[kb][r] = 0.0f;

  struct Ld {
    bf16x8_t bh[KC][PH];   // h form of B_b (first operand of h^T: rows j)
    bf16x8_t bu[KB][2][PG];   // u form of B_b (first operand of U^T, W^T: rows k)
  };
  auto load = [&](int jb, Ld& L) {
    const uint16_t* r = Bp + (int64_t)jb * PK::FB * kFrag;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc)
#pragma unroll
      for (int p = 0; p < PH; ++p) L.bh[kc][p] = ldfrag(r + (kc * PH + p) * kFrag, lb);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int cc = 0; cc < 2; ++cc)
#pragma unroll
        for (int p = 0; p < PG; ++p) L.bu[kb][cc][p] = ldfrag(r + (KC * PH + (kb * 2 + cc) * PG + p) * kFrag, lb);
  };

  for (int c0 = 0; c0 < N; c0 += kChunkF) {
    // weights of the strip, zero outside the block (rows >= M, columns >= N)
    const int cw = (min(kChunkF, N - c0) + 31) / 32 * 32, CP = cw + 4;
    __syncthreads();
    // item = (row r, 4 columns c): 16-byte loads when rows are 16-byte
    // aligned and the 4 columns are inside the block; 4 items in flight
    for (int base = tid; base < 32 * (kChunkF / 4); base += 256 * 4) {
      float4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int idx = base + u * 256, r = idx / (kChunkF / 4), c = (idx % (kChunkF / 4)) * 4;
        const float* src = a.theta + (int64_t)(i0 + r) * N + c0 + c;
        v[u] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        if (c < cw && i0 + r < M) {
          if ((N & 3) == 0 && c0 + c + 3 < N) {
            v[u] = ld4(src);
          } else {
            v[u].x = c0 + c < N ? src[0] : 0.0f;
            v[u].y = c0 + c + 1 < N ? src[1] : 0.0f;
            v[u].z = c0 + c + 2 < N ? src[2] : 0.0f;
            v[u].w = c0 + c + 3 < N ? src[3] : 0.0f;
          }
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int idx = base + u * 256, r = idx / (kChunkF / 4), c = (idx % (kChunkF / 4)) * 4;
        if (c < cw) *(float4*)&slab[r * CP + c] = v[u];
      }
    }
    // e of the chunk: thread t takes child columns c = t/4 + 64 u, sample es
    // (the 4 samples of a child are one 16-byte run of its value row); every
    // index and value load of the chunk in flight before the first exp
    {
      constexpr int U8 = kChunkF / 64;
      int child[U8];
      float v[U8];
#pragma unroll
      for (int u = 0; u < U8; ++u) {
        const int j = c0 + (tid >> 2) + 64 * u;
        child[u] = (j < N) ? a.chblocks[a.blk_off + j / a.cbs] + j % a.cbs : -1;
      }
      const bool bin = b0 + es < a.B;
#pragma unroll
      for (int u = 0; u < U8; ++u)
        v[u] = (child[u] >= 0 && bin) ? a.vals[(int64_t)child[u] * a.B + b0 + es] : -INFINITY;
#pragma unroll
      for (int u = 0; u < U8; ++u) {
        const int c = (tid >> 2) + 64 * u;
        if (c < cw) el[es][c] = (child[u] >= 0 && bin) ? expf(v[u] - esh) : 0.0f;
      }
    }
    __syncthreads();
    if (!act) continue;
    const int nb = cw / 32, jb0 = c0 / 32;
    const float* srow = slab + l32 * CP + h * 4;
    const float* erow = el[wave] + h * 4;
    // one 32-child block from the operands in `cur`, the next block loading
    // into the other buffer meanwhile (ping-pong: no register copies).  The
    // load is unconditional (the last block reloads itself) so that the count
    // of loads in flight is the same on every path and the wait before the
    // next block's matrix instructions leaves this block's loads outstanding.
    // A block past the strip's last one (odd block counts: the second half
    // of the last pair) runs on the reloaded last block with zero weights.
    auto block = [&](int jl, const Ld& cur, Ld& fill) {
      // no instruction moves across a block boundary: the scheduler would
      // otherwise hoist the next block's work next to the loads feeding it
      __builtin_amdgcn_sched_barrier(0);
      load(jb0 + min(jl + 1, nb - 1), fill);
      const float live = jl < nb ? 1.0f : 0.0f;
      const int jc = min(jl, nb - 1);
      // h^T[j, i] = sum_k B_b[k, j] A_b[i, k] log2(e)
      f32x16_t H;
#pragma unroll
      for (int r = 0; r < 16; ++r) H[r] = 0.0f;
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) mfma_planes<PH>(H, cur.bh[kc], bA[kc]);
      // register r: row j = j0 + (r/4)*8 + h*4 + r%4, column i = i0 + l32
      float q[16], qe[16];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 th = *(const float4*)(srow + jc * 32 + g * 8);
        const float4 ev = *(const float4*)(erow + jc * 32 + g * 8);   // e at rows j0 + g*8 + h*4 .. +3
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = g * 4 + e;
          if constexpr (SE) {
            const float tl = at4(th, e) * live;
            const float qq = tl * H[r];
            Zp += qq;
            Sp += qq * at4(ev, e);
            q[r] = tl;                          // U, W operands: theta e and theta
            qe[r] = tl * at4(ev, e);
          } else {
            q[r] = (at4(th, e) * live) * __builtin_amdgcn_exp2f(H[r]);
            qe[r] = q[r] * at4(ev, e);
            Zp += q[r];
            Sp += qe[r];
          }
        }
      }
      // U^T[k, i] += sum_j B_b[k, j] qe[j, i], W^T[k, i] += sum_j B_b[k, j] q[j, i]:
      // the second operand is the accumulator itself (K index 8h + e of chunk
      // cc is register 8cc + e), the u form follows the same order of j
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        float xq[8], xw[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          xq[e] = qe[8 * cc + e];
          xw[e] = q[8 * cc + e];
        }
        bf16x8_t pq[PG], pw[PG];
        split8<PG>(xq, pq);
        split8<PG>(xw, pw);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          mfma_planes<PG>(U[kb], cur.bu[kb][cc], pq);
          mfma_planes<PG>(W[kb], cur.bu[kb][cc], pw);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    Ld L0, L1;
    load(jb0, L0);
    for (int jl = 0; jl < nb; jl += 2) {
      block(jl, L0, L1);
      block(jl + 1, L1, L0);
    }
  }
  const float Z = Zp + __shfl_xor(Zp, 32), S = Sp + __shfl_xor(Sp, 32);
  const int i = i0 + l32;
  const bool live = act && i < M;
  const float v = live ? ((Z > 0.0f && S > 0.0f) ? key_to_shift_lr(a.mkeys[(int64_t)a.m_row * a.B + bq]) + logf(S / Z)
                                                  : -INFINITY)
                       : -INFINITY;
  if (a.ep_on) {
    // the product layer above (its node = children added in child order, as
    // the product kernel does) and the maximum of the wave's 32 rows of
    // sample b for the next sum layer's shift
    float pm = -INFINITY;
    if (live && h == 0) {
      const int q = a.out_start + i - a.ep_base_s;
      if (q >= 0 && q < a.ep_pcount) {
        const float o = a.vals[(int64_t)(a.ep_base_o + q) * a.B + b];
        const float pv = a.ep_qs == 0 ? (0.0f + v) + o : (0.0f + o) + v;
        a.vals[(int64_t)(a.ep_pstart + q) * a.B + b] = pv;
        pm = pv;
      }
    }
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) pm = fmaxf(pm, __shfl_xor(pm, d));
    if (lane == 0 && act) atomicMax(a.mkeys_out + (int64_t)a.ep_mrow * a.B + b, float_to_key_lr(pm));
  }
  if (!live) return;
  if (h == 0) {
    a.Z[(int64_t)b * M + i] = Z;
    a.S[(int64_t)b * M + i] = S;
    a.vals[(int64_t)(a.out_start + i) * a.B + b] = v;
  }
  // accumulator register r of rank block kb: row k = kb*32 + (r/4)*8 + h*4 + r%4, column i
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int k = kb * 32 + (r / 4) * 8 + h * 4 + (r % 4);
      if (k < kr) {
        a.U[((int64_t)b * M + i) * kr + k] = U[kb][r];
        a.W[((int64_t)b * M + i) * kr + k] = W[kb][r];
      }
    }
}

// Backward: workgroup = 32 children x 8 samples (8 waves, one sample each),
// all rows.  The transposed weights of the column strip are staged in LDS; a
// wave streams its sample's A records and coefficients one row block ahead.
// The parameter flows of each 32 x 32 tile are summed over the 8 waves in
// order (through one of two LDS exchange tiles, so one barrier per row block
// suffices) and added to the workgroup's partial matrix, whose tile is read a
// row block ahead so that the read overlaps the block's work.
// With WS (the denominator statistic of the conditional M-step) the same walk
// computes only w[i, j] = c2[i] * exp(h[i, j]) per sample (c2 = f / Z), summed
// over the 8 waves into the partial matrices at a.P like the parameter flows;
// no weights, element flows or dB.
// SE: the "sum_exp" form (records of exp(A), exp(B): the product is g), whose
// dB term is theta (c1 e - c2) against exp(A) and is multiplied by exp(B) at
// the end.
template <int PH, int PG, int KC, int KB, bool WS = false, bool SE = false>
__global__ __launch_bounds__(512) void k_lr_bwd(LRArgs a) {
  using PK = LrPack<PH, PG, KC, KB>;
  __shared__ __attribute__((aligned(16))) float slab[kSlabB];   // theta^T [32][R + 4]
  __shared__ float xch[2][8][1024];                              // per wave: parameter flows of a 32 x 32 tile
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, h = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nt = (a.N + 31) / 32;
  const int jb = blockIdx.x % nt, j0 = jb * 32, sg = blockIdx.x / nt;
  const int M = a.M, N = a.N, kr = a.krank;
  const int b = sg * 8 + wave;
  const bool act = b < a.B;
  const int bq = act ? b : 0;
  const uint32_t lb = (uint32_t)lane * 16;
  // second operand of h: the h form of B_b for this column strip
  bf16x8_t bB[KC][PH];
  {
    const uint16_t* bp = PK::bside(a.pk, N, bq, jb);
#pragma unroll
    for (int kc = 0; kc < KC; ++kc)
#pragma unroll
      for (int p = 0; p < PH; ++p) bB[kc][p] = ldfrag(bp + (kc * PH + p) * kFrag, lb);
  }
  // e[j, b] = exp(v[child j, b] - m[b]) of this lane's child (zero past N)
  float ev = 0.0f;
  if (!WS && act && j0 + l32 < N) {
    const int j = j0 + l32, child = a.chblocks[a.blk_off + j / a.cbs] + j % a.cbs;
    ev = expf(a.vals[(int64_t)child * a.B + b] - key_to_shift_lr(a.mkeys[(int64_t)a.m_row * a.B + b]));
  }
  float fcp = 0.0f;
  f32x16_t dB[KB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) dB[kb][r] = 0.0f;
  float* P = a.P + (int64_t)sg * M * N;
  const int ldC = (M + 31) / 32 * 32;
  const float* C1 = a.C1 + (int64_t)bq * ldC + h * 4;   // rows padded with zeros to ldC
  const float* C2 = a.C2 + (int64_t)bq * ldC + h * 4;
  const uint16_t* Ap = PK::aside(a.pk, a.B, M, N, bq, 0);   // row block ib at + ib * FB * kFrag
  // this thread's two entries of a parameter-flow tile: rows pr[u] of the
  // block, column pj
  int pr[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int x = tid + u * 512, r = x >> 6, ll = x & 63;
    pr[u] = (r / 4) * 8 + (ll >> 5) * 4 + (r % 4);
  }
  const int pj = j0 + (tid & 31);

  struct Fr {
    bf16x8_t ah[KC][PH];   // h form of A_b (first operand of h: rows i)
    bf16x8_t ad[KB][2][PG];   // d form of A_b (first operand of dB: rows k)
  };
  struct Cf {
    float4 c1[4], c2[4];   // rows ib*32 + g*8 + h*4 .. +3
  };
  auto loadF = [&](int ib, Fr& L) {
    const uint16_t* r = Ap + (int64_t)ib * PK::FB * kFrag;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc)
#pragma unroll
      for (int p = 0; p < PH; ++p) L.ah[kc][p] = ldfrag(r + (kc * PH + p) * kFrag, lb);
    if constexpr (!WS)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int cc = 0; cc < 2; ++cc)
#pragma unroll
          for (int p = 0; p < PG; ++p) L.ad[kb][cc][p] = ldfrag(r + (KC * PH + (kb * 2 + cc) * PG + p) * kFrag, lb);
  };
  auto loadC = [&](int ib, Cf& L) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      L.c1[g] = ld4(C1 + ib * 32 + g * 8);
      L.c2[g] = ld4(C2 + ib * 32 + g * 8);
    }
  };
  auto pload = [&](int ib, float (&po)[2]) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {   // clamped address, always loaded
      const int i = min(ib * 32 + pr[u], M - 1);
      po[u] = P[(int64_t)i * N + min(pj, N - 1)];
    }
  };

  for (int r0 = 0; r0 < M; r0 += kChunkB) {
    // transposed weights of the strip, zero outside the block: item = (row
    // ii, 4 columns jq), one 16-byte load when the row is 16-byte aligned
    const int rw = (min(kChunkB, M - r0) + 31) / 32 * 32, RP = rw + 4;
    __syncthreads();
    for (int base = tid; !WS && base < rw * 8; base += 512 * 4) {
      float4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int idx = base + u * 512, ii = idx >> 3, jq = (idx & 7) * 4;
        const float* src = a.theta + (int64_t)(r0 + ii) * N + j0 + jq;
        v[u] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        if (idx < rw * 8 && r0 + ii < M) {
          if ((N & 3) == 0 && j0 + jq + 3 < N) {
            v[u] = ld4(src);
          } else {
            v[u].x = j0 + jq < N ? src[0] : 0.0f;
            v[u].y = j0 + jq + 1 < N ? src[1] : 0.0f;
            v[u].z = j0 + jq + 2 < N ? src[2] : 0.0f;
            v[u].w = j0 + jq + 3 < N ? src[3] : 0.0f;
          }
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int idx = base + u * 512, ii = idx >> 3, jq = (idx & 7) * 4;
        if (idx < rw * 8) {
          slab[(jq + 0) * RP + ii] = v[u].x;
          slab[(jq + 1) * RP + ii] = v[u].y;
          slab[(jq + 2) * RP + ii] = v[u].z;
          slab[(jq + 3) * RP + ii] = v[u].w;
        }
      }
    }
    __syncthreads();
    const int nrb = rw / 32, ib0 = r0 / 32;
    const float* srow = slab + l32 * RP + h * 4;
    auto clampb = [&](int il) { return ib0 + min(il, nrb - 1); };
    // row block il from fragments `fc` (row block il + 3 loading into `ff`)
    // and coefficients `cc_` (row block il + 1 loading into `cn`, its
    // partial tile into `pn`), exchange tile xb.  Loads are unconditional (the
    // last block reloads itself; an idle wave reads sample 0), so the count in
    // flight is the same on every path; blocks past the last one (the end of
    // an unrolled group) only load.  No instruction moves across a block
    // boundary.
    auto blockk = [&](int il, const Fr& fc, Fr& ff, const Cf& cc_, Cf& cn, const float (&po)[2], float (&pn)[2],
                      int xb) {
      __builtin_amdgcn_sched_barrier(0);
      loadF(clampb(il + 3), ff);
      loadC(clampb(il + 1), cn);
      pload(clampb(il + 1), pn);
      if (il < nrb) {
        const int i0 = (ib0 + il) * 32;
        float* xw = &xch[xb][wave][lane];
        if (act) {
          // h[i, j] = sum_k A_b[i, k] log2(e) B_b[k, j]
          f32x16_t H;
#pragma unroll
          for (int r = 0; r < 16; ++r) H[r] = 0.0f;
#pragma unroll
          for (int kc = 0; kc < KC; ++kc) mfma_planes<PH>(H, fc.ah[kc], bB[kc]);
          // register r: row i = i0 + (r/4)*8 + h*4 + r%4, column j = j0 + l32
          if constexpr (WS) {
#pragma unroll
            for (int g = 0; g < 4; ++g)
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const int r = g * 4 + e;
                xw[r * 64] = at4(cc_.c2[g], e) * (SE ? H[r] : __builtin_amdgcn_exp2f(H[r]));
              }
          } else {
          float X[16];
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const float4 th = *(const float4*)(srow + il * 32 + g * 8);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int r = g * 4 + e;
              const float q = at4(th, e) * (SE ? H[r] : __builtin_amdgcn_exp2f(H[r]));
              const float u1 = ev * at4(cc_.c1[g], e);
              const float eps = q * u1;
              X[r] = (SE ? at4(th, e) : q) * (u1 - at4(cc_.c2[g], e));
              fcp += eps;
              xw[r * 64] = eps;
            }
          }
          // dB[k, j] += sum_i A_b[i, k] X[i, j]: K index 8h + e of chunk cc is
          // register 8cc + e (the d form follows the same order of i)
#pragma unroll
          for (int cc = 0; cc < 2; ++cc) {
            float xx[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) xx[e] = X[8 * cc + e];
            bf16x8_t px[PG];
            split8<PG>(xx, px);
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) mfma_planes<PG>(dB[kb], fc.ad[kb][cc], px);
          }
          }
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) xw[r * 64] = 0.0f;
        }
        __syncthreads();
        // parameter flows of the tile, summed over the waves in order
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int x = tid + u * 512;
          float v = xch[xb][0][x];
#pragma unroll
          for (int w = 1; w < 8; ++w) v += xch[xb][w][x];
          const int i = i0 + pr[u];
          if (i < M && pj < N) P[(int64_t)i * N + pj] = po[u] + v;
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    Fr F0, F1, F2, F3;
    Cf Ca, Cb;
    float p0[2], p1[2];
    loadF(clampb(0), F0);
    loadF(clampb(1), F1);
    loadF(clampb(2), F2);
    loadC(clampb(0), Ca);
    pload(clampb(0), p0);
    for (int il = 0; il < nrb; il += 4) {
      blockk(il, F0, F3, Ca, Cb, p0, p1, 0);
      blockk(il + 1, F1, F0, Cb, Ca, p1, p0, 1);
      blockk(il + 2, F2, F1, Ca, Cb, p0, p1, 0);
      blockk(il + 3, F3, F2, Cb, Ca, p1, p0, 1);
    }
  }
  if constexpr (WS) return;
  // child flows, dB
  const float tot = fcp + __shfl_xor(fcp, 32);
  const int j = j0 + l32;
  if (!act || j >= N) return;
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
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int k = kb * 32 + (r / 4) * 8 + h * 4 + (r % 4);
      const int64_t o = ((int64_t)b * kr + k) * N + j;
      if (k < kr) a.dB[o] = SE ? expf(a.Bf[o]) * dB[kb][r] : dB[kb][r];
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

// Precision of the fused kernels: h with PH planes per operand, the gradient
// products with PG (auto: 2 and 1; fp32-level: 3 and 3).  KC K chunks of 16
// cover the rank in h (1, 2 or 4: ranks up to 16, 32, 64) and KB blocks of
// 32 in the gradient products (1 up to rank 32, else 2).
static int lr_kc(int krank) { return krank <= 16 ? 1 : krank <= 32 ? 2 : 4; }
static int lr_kb(int krank) { return krank <= 32 ? 1 : 2; }

template <int PH, int PG, int KC, int KB>
static void lr_fwd_kk(const LRArgs& a, const dim3& grid, hipStream_t s) {
  if (a.sumexp) launch_kernel((k_lr_fwd<PH, PG, KC, KB, true>), grid, dim3(256), 0, s, a);
  else launch_kernel((k_lr_fwd<PH, PG, KC, KB>), grid, dim3(256), 0, s, a);
}
template <int PH, int PG>
static void lr_fwd_k(const LRArgs& a, hipStream_t s) {
  const dim3 grid(((a.M + 31) / 32) * ((a.B + 3) / 4));
  const int kc = lr_kc(a.krank);
  if (kc == 1) lr_fwd_kk<PH, PG, 1, 1>(a, grid, s);
  else if (kc == 2) lr_fwd_kk<PH, PG, 2, 1>(a, grid, s);
  else lr_fwd_kk<PH, PG, 4, 2>(a, grid, s);
}
template <int PH, int PG, int KC, int KB, bool WS>
static void lr_bwd_kk(const LRArgs& a, const dim3& grid, hipStream_t s) {
  if (a.sumexp) launch_kernel((k_lr_bwd<PH, PG, KC, KB, WS, true>), grid, dim3(512), 0, s, a);
  else launch_kernel((k_lr_bwd<PH, PG, KC, KB, WS>), grid, dim3(512), 0, s, a);
}
template <int PH, int PG, bool WS = false>
static void lr_bwd_k(const LRArgs& a, hipStream_t s) {
  const dim3 grid(((a.N + 31) / 32) * ((a.B + 7) / 8));
  const int kc = lr_kc(a.krank);
  if (kc == 1) lr_bwd_kk<PH, PG, 1, 1, WS>(a, grid, s);
  else if (kc == 2) lr_bwd_kk<PH, PG, 2, 1, WS>(a, grid, s);
  else lr_bwd_kk<PH, PG, 4, 2, WS>(a, grid, s);
}

int64_t lr_pack_bytes(int B, int M, int N, int krank, int fp32) {
  const int PH = fp32 ? 3 : 2, PG = fp32 ? 3 : 1, KC = lr_kc(krank), KB = lr_kb(krank);
  return (int64_t)B * ((N + 31) / 32 + (M + 31) / 32) * (KC * PH + 2 * KB * PG) * kFrag * 2;
}
int lr_pack_workgroups(int B, int M, int N, int krank) {
  const int KC = lr_kc(krank), KB = lr_kb(krank);
  const int64_t nsets = (int64_t)B * ((N + 31) / 32 + (M + 31) / 32) * (KC + 2 * KB);
  return (int)((nsets + 3) / 4);
}
template <int PH, int PG>
static void lr_pack_k(const LRPackArgs& pa, const dim3& grid, hipStream_t s) {
  const int kc = lr_kc(pa.krank);
  if (kc == 1) launch_kernel((k_lr_pack<PH, PG, 1, 1>), grid, dim3(256), 0, s, pa);
  else if (kc == 2) launch_kernel((k_lr_pack<PH, PG, 2, 1>), grid, dim3(256), 0, s, pa);
  else launch_kernel((k_lr_pack<PH, PG, 4, 2>), grid, dim3(256), 0, s, pa);
}
void launch_lr_pack(const LRPackArgs& pa, int fp32, hipStream_t s) {
  if (pa.ngroups <= 0) return;
  const dim3 grid(pa.wg0[pa.ngroups]);
  if (fp32) lr_pack_k<3, 3>(pa, grid, s);
  else lr_pack_k<2, 1>(pa, grid, s);
}
void launch_lr_coef(const LRArgs& a, hipStream_t s) {
  const int64_t n = (int64_t)a.B * ((a.M + 31) / 32 * 32) * 4;
  launch_kernel(k_lr_coef, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a);
}
void launch_lr_fwd(const LRArgs& a, int fp32, hipStream_t s) {
  if (fp32) lr_fwd_k<3, 3>(a, s);
  else lr_fwd_k<2, 1>(a, s);
}
void launch_lr_bwd(const LRArgs& a, int fp32, hipStream_t s) {
  if (fp32) lr_bwd_k<3, 3>(a, s);
  else lr_bwd_k<2, 1>(a, s);
}
void launch_lr_zstat(const LRArgs& a, int fp32, hipStream_t s) {
  if (fp32) lr_bwd_k<3, 3, true>(a, s);
  else lr_bwd_k<2, 1, true>(a, s);
}
void launch_lr_fplus(const float* P, int nsg, int64_t elems, float* pflows, hipStream_t s) {
  launch_kernel(k_lr_fplus, dim3(grid_lr(elems)), dim3(256), 0, s, P, nsg, elems, pflows);
}

}  // namespace pc
