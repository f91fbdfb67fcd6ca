// k_gemm.hip -- the sum layer's dense contractions on gfx950 matrix cores.
//
// One kernel template computes C[m, n] = sum_k A[m, k] * B[n, k] for the three
// products of a sum layer (PyJuice pull request #62, Summary items 2 and 3):
//
//   forward        S[i, b]  = sum_j theta[i, j] e[j, b]      A = theta,   B = E (batch-major)
//                  epilogue v[i, b] = m[b] + log S[i, b]
//   element flows  T[j, b]  = sum_i theta[i, j] g[i, b]      A = theta^T, B = G (batch-major)
//                  epilogue f[j, b] (=|+=) e[j, b] * T[j, b],  e recomputed in float32
//   parameter flows P[i, j] = sum_{copies, b} g[i, b] e[j, b] A = G, B = E (node-major)
//                  epilogue F[i, j] += theta[i, j] * P[i, j]
//
// with g = f / S the flow divided by the node's scaled sum (kept by the
// forward).  Both
// operands are bfloat16 with the contraction dimension contiguous, padded to
// tile multiples with zeros.  An operand may be split into planes (x ~ hi +
// lo [+ lo2]); the kernel accumulates every cross product of planes whose
// order is below the larger plane count (3 products for 2x2 planes, 6 for
// 3x3), smallest first, into one float32 accumulator: the fp32-level mode.
//
// Tiling: 128 x 128 output tile per workgroup of 4 waves (2 x 2), each wave
// 64 x 64 = 2 x 2 blocks of v_mfma_f32_32x32x16_bf16; K staged through LDS in
// KT-wide slices, double buffered, one barrier per slice; rows padded by 16
// bytes so the 128-bit LDS reads of a 32-row fragment hit distinct banks.
// Workgroups are renumbered so that each XCD (dispatch is round robin over
// the 8 XCDs) works on a contiguous run of tiles, which share weight rows in
// that XCD's L2.
#include <hip/hip_runtime.h>

#include "pc_kernels.h"

namespace pc {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float key_to_shift(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  float m = __uint_as_float(u);
  return (m == m && fabsf(m) <= 3.0e38f) ? m : 0.0f;   // -inf / unset column -> 0
}

__device__ __forceinline__ int xcd_remap(int bid, int n) {
  const int q = n >> 3, r = n & 7;
  const int x = bid & 7, local = bid >> 3;
  return x * q + (x < r ? x : r) + local;
}

// Last index g in [0, n) with field(g) <= x (fields non-decreasing).
template <typename Rec, typename F>
__device__ __forceinline__ int find_last_le(const Rec* recs, int n, int x, F field) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (field(recs[mid]) <= x) lo = mid; else hi = mid - 1;
  }
  return lo;
}

template <int EPI, int PA, int PB, int KT>
__global__ __launch_bounds__(256) void k_gemm(GemmArgs a) {
  constexpr int MT = 128, NT = 128;
  constexpr int LDK = KT + 8;
  constexpr int ATILE = MT * LDK, BTILE = NT * LDK;
  constexpr int STAGE = PA * ATILE + PB * BTILE;
  constexpr int CPR = KT / 8;                  // 16-byte chunks per row of a slice
  constexpr int CA = MT * CPR / 256, CB = NT * CPR / 256;
  constexpr int PMAX = PA > PB ? PA : PB;
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm0 = (wave >> 1) * 64, wn0 = (wave & 1) * 64;
  const int tile = xcd_remap(blockIdx.x, gridDim.x);

  // ---- locate the problem and the tile -----------------------------------
  const uint16_t* Abase;
  const uint16_t* Bbase;
  int lda, ldb, kst, nseg, m0, n0;
  const GroupRec* gr = nullptr;
  const BlockRec* bl = nullptr;
  if (EPI == EPI_FWD || EPI == EPI_ELEM) {
    const int gt = tile / a.ntiles, nt = tile - gt * a.ntiles;
    int g;
    if (EPI == EPI_FWD)
      g = find_last_le(a.groups, a.ngroups, gt, [](const GroupRec& r) { return r.mt_start; });
    else
      g = find_last_le(a.groups, a.ngroups, gt, [](const GroupRec& r) { return r.ct_start; });
    gr = a.groups + g;
    bl = a.blocks + gr->block;
    n0 = nt * NT;
    if (EPI == EPI_FWD) {
      m0 = (gt - gr->mt_start) * MT;
      lda = (gr->N + K_PAD - 1) / K_PAD * K_PAD;
      Abase = a.opA + bl->th_off + (int64_t)m0 * lda;
      Bbase = a.opB + (int64_t)n0 * a.ldb + gr->e_koff;
    } else {
      m0 = (gt - gr->ct_start) * MT;
      lda = (gr->M + K_PAD - 1) / K_PAD * K_PAD;
      Abase = a.opA + bl->tht_off + (int64_t)m0 * lda;
      Bbase = a.opB + (int64_t)n0 * a.ldb + gr->g_koff;
    }
    ldb = a.ldb;
    kst = lda / KT;
    nseg = 1;
  } else {
    const int b = find_last_le(a.blocks, a.ngroups, tile, [](const BlockRec& r) { return r.pt_start; });
    bl = a.blocks + b;
    const int ntn = (bl->N + ROW_PAD - 1) / ROW_PAD;
    const int lt = tile - bl->pt_start;
    m0 = (lt / ntn) * MT;
    n0 = (lt % ntn) * NT;
    lda = ldb = a.B_padK;
    kst = a.B_padK / KT;
    nseg = bl->ncopies;
    Abase = a.opA + (int64_t)m0 * lda;
    Bbase = a.opB + (int64_t)n0 * ldb;
  }

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  uint4 ra[PA][CA], rb[PB][CB];
  const int total = kst * nseg;

  auto seg_ptrs = [&](int kt, const uint16_t*& Ap, const uint16_t*& Bp) {
    if (EPI == EPI_PARAM) {
      const int s = kt / kst;
      const CopyRec c = a.copies[bl->copy_off + s];
      const int kk = (kt - s * kst) * KT;
      Ap = Abase + c.g_row * (int64_t)a.B_padK + kk;
      Bp = Bbase + c.e_row * (int64_t)a.B_padK + kk;
    } else {
      Ap = Abase + kt * KT;
      Bp = Bbase + kt * KT;
    }
  };
  auto gload = [&](int kt) {
    const uint16_t *Ap, *Bp;
    seg_ptrs(kt, Ap, Bp);
#pragma unroll
    for (int p = 0; p < PA; ++p)
#pragma unroll
      for (int i = 0; i < CA; ++i) {
        const int c = tid + i * 256, row = c / CPR, col = (c % CPR) * 8;
        ra[p][i] = *(const uint4*)(Ap + p * a.planeA + (int64_t)row * lda + col);
      }
#pragma unroll
    for (int p = 0; p < PB; ++p)
#pragma unroll
      for (int i = 0; i < CB; ++i) {
        const int c = tid + i * 256, row = c / CPR, col = (c % CPR) * 8;
        rb[p][i] = *(const uint4*)(Bp + p * a.planeB + (int64_t)row * ldb + col);
      }
  };
  auto lstore = [&](int buf) {
    uint16_t* s = lds + buf * STAGE;
#pragma unroll
    for (int p = 0; p < PA; ++p)
#pragma unroll
      for (int i = 0; i < CA; ++i) {
        const int c = tid + i * 256, row = c / CPR, col = (c % CPR) * 8;
        *(uint4*)(s + p * ATILE + row * LDK + col) = ra[p][i];
      }
#pragma unroll
    for (int p = 0; p < PB; ++p)
#pragma unroll
      for (int i = 0; i < CB; ++i) {
        const int c = tid + i * 256, row = c / CPR, col = (c % CPR) * 8;
        *(uint4*)(s + PA * ATILE + p * BTILE + row * LDK + col) = rb[p][i];
      }
  };

  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < total; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < total) gload(kt + 1);
    const uint16_t* s = lds + cur * STAGE;
#pragma unroll
    for (int ks = 0; ks < KT / 16; ++ks) {
      bf16x8_t fa[PA][2], fb[PB][2];
      const int kof = ks * 16 + (lane >> 5) * 8;
#pragma unroll
      for (int p = 0; p < PA; ++p)
#pragma unroll
        for (int i = 0; i < 2; ++i)
          fa[p][i] = *(const bf16x8_t*)(s + p * ATILE + (wm0 + i * 32 + (lane & 31)) * LDK + kof);
#pragma unroll
      for (int p = 0; p < PB; ++p)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          fb[p][j] = *(const bf16x8_t*)(s + PA * ATILE + p * BTILE + (wn0 + j * 32 + (lane & 31)) * LDK + kof);
      // cross products of planes, highest order (smallest) first
#pragma unroll
      for (int o = PMAX - 1; o >= 0; --o)
#pragma unroll
        for (int pa = 0; pa < PA; ++pa) {
          const int pb = o - pa;
          if (pb < 0 || pb >= PB) continue;
#pragma unroll
          for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[pa][i], fb[pb][j], acc[i][j], 0, 0, 0);
        }
    }
    if (kt + 1 < total) lstore(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue ------------------------------------------------------------
  // accumulator register r of lane l holds row (r/4)*8 + (l/32)*4 + r%4 and
  // column l%32 of the 32 x 32 block.
  const int B = a.B;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm0 + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        const int col = n0 + wn0 + j * 32 + (lane & 31);
        const float v = acc[i][j][r];
        if (EPI == EPI_FWD) {
          if (row < gr->M && col < B) {
            const float sh = key_to_shift(a.mkeys[(int64_t)gr->m_row * B + col]);
            a.vals[(int64_t)(gr->out_start + row) * B + col] = sh + logf(v);
            a.ssum[(gr->s_row + row) * B + col] = v;
          }
        } else if (EPI == EPI_ELEM) {
          if (row < gr->N && col < B) {
            const int child = a.chblocks[gr->blk_off + row / gr->cbs] + row % gr->cbs;
            const float sh = key_to_shift(a.mkeys[(int64_t)gr->m_row * B + col]);
            const float e = expf(a.vals[(int64_t)child * B + col] - sh);
            const float c = (e == 0.0f) ? 0.0f : e * v;
            if (gr->scratch_row >= 0)
              a.scratch[(int64_t)(gr->scratch_row + row) * B + col] = c;
            else if (a.store)
              a.flows[(int64_t)child * B + col] = c;
            else
              a.flows[(int64_t)child * B + col] += c;
          }
        } else {
          if (row < bl->M && col < bl->N) {
            const int64_t idx = bl->param_offset + (int64_t)row * bl->N + col;
            a.pflows[idx] += a.params[idx] * v;
          }
        }
      }
}

template <int EPI, int PA, int PB>
static void launch3(int tiles, const GemmArgs& a, hipStream_t s) {
  constexpr int KT = (PA + PB > 4) ? 32 : 64;
  hipLaunchKernelGGL((k_gemm<EPI, PA, PB, KT>), dim3(tiles), dim3(256), 0, s, a);
}

template <int EPI>
static void launch_planes(int pa, int pb, int tiles, const GemmArgs& a, hipStream_t s) {
  if (pa == 1 && pb == 1) launch3<EPI, 1, 1>(tiles, a, s);
  else if (pa == 2 && pb == 1) launch3<EPI, 2, 1>(tiles, a, s);
  else if (pa == 1 && pb == 2) launch3<EPI, 1, 2>(tiles, a, s);
  else if (pa == 2 && pb == 2) launch3<EPI, 2, 2>(tiles, a, s);
  else launch3<EPI, 3, 3>(tiles, a, s);
}

void launch_gemm(int epi, int pa, int pb, int tiles, const GemmArgs& a, hipStream_t s) {
  if (tiles <= 0) return;
  if (epi == EPI_FWD) launch_planes<EPI_FWD>(pa, pb, tiles, a, s);
  else if (epi == EPI_ELEM) launch_planes<EPI_ELEM>(pa, pb, tiles, a, s);
  else launch_planes<EPI_PARAM>(pa, pb, tiles, a, s);
}

}  // namespace pc
