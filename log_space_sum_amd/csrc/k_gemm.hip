// k_gemm.hip -- the sum layer's dense contractions on gfx950 matrix cores.
//
// One kernel template computes C[m, n] = sum_k A[m, k] * B[n, k] for the three
// products of a sum layer (PyJuice pull request #62, Summary items 2 and 3):
//
//   forward         S[i, b] = sum_j theta[i, j] e[j, b]       A = theta,   B = E (batch-major)
//                   epilogue v[i, b] = m[b] + log S[i, b] (S kept for the backward)
//   element flows   T[j, b] = sum_i theta[i, j] g[i, b]       A = theta^T, B = G (batch-major)
//                   epilogue f[j, b] (=|+=) e[j, b] * T[j, b], e recomputed in float32
//   parameter flows P[i, j] = sum_{copies, b} g[i, b] e[j, b] A = G, B = E (node-major)
//                   epilogue F[i, j] += theta[i, j] * P[i, j]
//
// with g = f / S the flow divided by the node's scaled sum.  Both operands are
// bfloat16 with the contraction dimension contiguous, padded to tile
// multiples with zeros.  An operand may be split into planes (x ~ hi + lo
// [+ lo2]); the kernel accumulates every cross product of planes whose order
// is below the larger plane count (3 products for 2x2 planes, 6 for 3x3),
// smallest first, into one float32 accumulator.
//
// Tiling: MT x NT output tile per workgroup of 4 waves (2 x 2), each wave a
// (MT/2) x (NT/2) grid of v_mfma_f32_32x32x16_bf16 blocks.  K is staged
// through LDS in KT-wide slices, double buffered; the global loads of slice
// k+2 are issued after slice k+1 is stored, so a whole slice of matrix work
// covers their latency (scheduling fences keep the compiler from hoisting the
// LDS stores above the matrix instructions).  LDS rows are padded by 16 bytes
// so the 128-bit fragment reads of 32 consecutive rows hit distinct banks.
//
// Forward and element-flow products at small output sizes split K over
// `splitk` workgroups; each writes its partial tile, and the last to arrive
// (arrival counter per tile) adds the partials in split order and runs the
// epilogue, so results are deterministic.  Workgroups are renumbered so each
// XCD (dispatch is round robin over the 8 XCDs) gets a contiguous run of
// logical tiles: the splits of a tile, and neighbouring tiles sharing weight
// rows, meet in one L2.
#include <hip/hip_runtime.h>

#include "pc_kernels.h"

namespace pc {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

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

// Start of K slice `kt` of an operand: tied copies are consecutive runs of
// `kst` slices at a fixed stride (parameter flows); otherwise one run.
template <int EPI, int KT>
__device__ __forceinline__ const uint16_t* slice_ptr(const uint16_t* base, int64_t stride, int kst, int kt) {
  if (EPI == EPI_PARAM) {
    const int s = kt / kst;
    return base + s * stride + (kt - s * kst) * KT;
  }
  return base + kt * KT;
}

// Global -> register -> LDS staging and the matrix-core loop of one slice.
template <int PA, int PB, int MT, int NT, int KT>
struct Tiles {
  static constexpr int LDK = KT + 8;
  static constexpr int ATILE = MT * LDK, BTILE = NT * LDK;
  static constexpr int CPR = KT / 8;
  static constexpr int CA = MT * CPR / 256, CB = NT * CPR / 256;
  static constexpr int FM = MT / 64, FN = NT / 64;
  static constexpr int PMAX = PA > PB ? PA : PB;

  static __device__ __forceinline__ void gload(u32x4_t (&ra)[PA][CA], u32x4_t (&rb)[PB][CB], const uint16_t* Ap,
                                               const uint16_t* Bp, int64_t pA, int64_t pB, int lda, int ldb,
                                               int tid) {
#pragma unroll
    for (int p = 0; p < PA; ++p)
#pragma unroll
      for (int i = 0; i < CA; ++i) {
        const int c = tid + i * 256, row = c / CPR, col = (c % CPR) * 8;
        ra[p][i] = *(const u32x4_t*)(Ap + p * pA + (int64_t)row * lda + col);
      }
#pragma unroll
    for (int p = 0; p < PB; ++p)
#pragma unroll
      for (int i = 0; i < CB; ++i) {
        const int c = tid + i * 256, row = c / CPR, col = (c % CPR) * 8;
        rb[p][i] = *(const u32x4_t*)(Bp + p * pB + (int64_t)row * ldb + col);
      }
  }

  static __device__ __forceinline__ void lstore(uint16_t* s, const u32x4_t (&ra)[PA][CA], const u32x4_t (&rb)[PB][CB],
                                                int tid) {
#pragma unroll
    for (int p = 0; p < PA; ++p)
#pragma unroll
      for (int i = 0; i < CA; ++i) {
        const int c = tid + i * 256, row = c / CPR, col = (c % CPR) * 8;
        *(u32x4_t*)(s + p * ATILE + row * LDK + col) = ra[p][i];
      }
#pragma unroll
    for (int p = 0; p < PB; ++p)
#pragma unroll
      for (int i = 0; i < CB; ++i) {
        const int c = tid + i * 256, row = c / CPR, col = (c % CPR) * 8;
        *(u32x4_t*)(s + PA * ATILE + p * BTILE + row * LDK + col) = rb[p][i];
      }
  }

  static __device__ __forceinline__ void compute(f32x16_t (&acc)[FM][FN], const uint16_t* s, int wm0, int wn0,
                                                 int lane) {
#pragma unroll
    for (int ks = 0; ks < KT / 16; ++ks) {
      bf16x8_t fa[PA][FM], fb[PB][FN];
      const int kof = ks * 16 + (lane >> 5) * 8;
#pragma unroll
      for (int p = 0; p < PA; ++p)
#pragma unroll
        for (int i = 0; i < FM; ++i)
          fa[p][i] = *(const bf16x8_t*)(s + p * ATILE + (wm0 + i * 32 + (lane & 31)) * LDK + kof);
#pragma unroll
      for (int p = 0; p < PB; ++p)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          fb[p][j] = *(const bf16x8_t*)(s + PA * ATILE + p * BTILE + (wn0 + j * 32 + (lane & 31)) * LDK + kof);
      // cross products of planes, highest order (smallest) first
#pragma unroll
      for (int o = PMAX - 1; o >= 0; --o)
#pragma unroll
        for (int pa = 0; pa < PA; ++pa) {
          const int pb = o - pa;
          if (pb >= 0 && pb < PB) {
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
              for (int j = 0; j < FN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[pa][i], fb[pb][j], acc[i][j], 0, 0, 0);
          }
        }
    }
  }
};

template <int EPI, int PA, int PB, int MT, int NT, int KT>
__global__ __launch_bounds__(256) void k_gemm(GemmArgs a) {
  constexpr int WTM = MT / 2, WTN = NT / 2;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  constexpr int LDK = KT + 8;
  constexpr int ATILE = MT * LDK, BTILE = NT * LDK;
  constexpr int STAGE = PA * ATILE + PB * BTILE;
  constexpr int CPR = KT / 8;                  // 16-byte chunks per row of a slice
  constexpr int CA = MT * CPR / 256, CB = NT * CPR / 256;
  constexpr int PMAX = PA > PB ? PA : PB;
  constexpr int SUB = ROW_PAD / MT;            // tiles per 256-row block
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * STAGE];
  __shared__ int last_flag;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm0 = (wave >> 1) * WTM, wn0 = (wave & 1) * WTN;
  const int logical = xcd_remap(blockIdx.x, gridDim.x);

  // ---- locate the problem, the tile and the K range ------------------------
  int S = 1, split = 0, tile = logical;
  if (EPI != EPI_PARAM) {
    S = a.splitk;
    tile = logical / S;
    split = logical - tile * S;
  }
  const uint16_t* A0;
  const uint16_t* B0;
  int lda, ldb, kst, kbeg, kend, m0, n0;
  int64_t astride = 0, bstride = 0;            // per tied copy (parameter flows)
  const GroupRec* gr = nullptr;
  const BlockRec* bl = nullptr;
  if (EPI == EPI_FWD || EPI == EPI_ELEM) {
    const int gt = tile / a.ntiles, nt = tile - gt * a.ntiles;
    const int unit = gt / SUB;
    int g;
    if (EPI == EPI_FWD)
      g = find_last_le(a.groups, a.ngroups, unit, [](const GroupRec& r) { return r.mt_start; });
    else
      g = find_last_le(a.groups, a.ngroups, unit, [](const GroupRec& r) { return r.ct_start; });
    gr = a.groups + g;
    bl = a.blocks + gr->block;
    n0 = nt * NT;
    if (EPI == EPI_FWD) {
      m0 = (gt - gr->mt_start * SUB) * MT;
      lda = (gr->N + K_PAD - 1) / K_PAD * K_PAD;
      A0 = a.opA + bl->th_off + (int64_t)m0 * lda;
      B0 = a.opB + (int64_t)n0 * a.ldb + gr->e_koff;
    } else {
      m0 = (gt - gr->ct_start * SUB) * MT;
      lda = (gr->M + K_PAD - 1) / K_PAD * K_PAD;
      A0 = a.opA + bl->tht_off + (int64_t)m0 * lda;
      B0 = a.opB + (int64_t)n0 * a.ldb + gr->g_koff;
    }
    ldb = a.ldb;
    kst = lda / KT;
    kbeg = split * kst / S;
    kend = (split + 1) * kst / S;
  } else {
    const int b = (MT == 256)
        ? find_last_le(a.blocks, a.ngroups, tile, [](const BlockRec& r) { return r.pt256; })
        : find_last_le(a.blocks, a.ngroups, tile, [](const BlockRec& r) { return r.pt128; });
    bl = a.blocks + b;
    const int Mp = (bl->M + ROW_PAD - 1) / ROW_PAD * ROW_PAD;
    const int Np = (bl->N + ROW_PAD - 1) / ROW_PAD * ROW_PAD;
    const int ntn = Np / NT;
    const int lt = tile - ((MT == 256) ? bl->pt256 : bl->pt128);
    m0 = (lt / ntn) * MT;
    n0 = (lt % ntn) * NT;
    lda = ldb = a.B_padK;
    kst = a.B_padK / KT;
    kbeg = 0;
    kend = bl->ncopies * kst;
    A0 = a.opA + (bl->g_base + m0) * (int64_t)a.B_padK;
    B0 = a.opB + (bl->e_base + n0) * (int64_t)a.B_padK;
    astride = (int64_t)Mp * a.B_padK;
    bstride = (int64_t)Np * a.B_padK;
  }

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  u32x4_t ra[PA][CA], rb[PB][CB];
  const int64_t pA = a.planeA, pB = a.planeB;
  const int n = kend - kbeg;
  using T = Tiles<PA, PB, MT, NT, KT>;
  if (n > 0) {
    // Branch-free pipeline: slice it+2 is fetched while slice it is multiplied
    // (the fetch index is clamped at the last slice, whose extra copy lands in
    // the idle buffer and is never read).
    T::gload(ra, rb, slice_ptr<EPI, KT>(A0, astride, kst, kbeg), slice_ptr<EPI, KT>(B0, bstride, kst, kbeg),
             pA, pB, lda, ldb, tid);
    T::lstore(lds, ra, rb, tid);
    const int k1 = min(kbeg + 1, kend - 1);
    T::gload(ra, rb, slice_ptr<EPI, KT>(A0, astride, kst, k1), slice_ptr<EPI, KT>(B0, bstride, kst, k1), pA, pB,
             lda, ldb, tid);
    __syncthreads();
    for (int it = 0; it < n; ++it) {
      T::compute(acc, lds + (it & 1) * STAGE, wm0, wn0, lane);
      __builtin_amdgcn_sched_barrier(0);
      T::lstore(lds + ((it + 1) & 1) * STAGE, ra, rb, tid);
      __builtin_amdgcn_sched_barrier(0);
      const int k2 = min(kbeg + it + 2, kend - 1);
      T::gload(ra, rb, slice_ptr<EPI, KT>(A0, astride, kst, k2), slice_ptr<EPI, KT>(B0, bstride, kst, k2), pA,
               pB, lda, ldb, tid);
      __syncthreads();
    }
  }

  // ---- split-K: the last workgroup of a tile adds the partials in order -----
  if (EPI != EPI_PARAM && S > 1) {
    constexpr int NREG = FM * FN * 16;
    float* mine = a.partials + ((int64_t)tile * S + split) * (NREG * 256);
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) mine[((i * FN + j) * 16 + r) * 256 + tid] = acc[i][j][r];
    __threadfence();
    __syncthreads();
    if (tid == 0) last_flag = (atomicAdd(a.counters + tile, 1u) == (unsigned)(S - 1));
    __syncthreads();
    if (!last_flag) return;
    __threadfence();
    const float* base = a.partials + (int64_t)tile * S * (NREG * 256);
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int idx = ((i * FN + j) * 16 + r) * 256 + tid;
          const float own = acc[i][j][r];
          float sum = 0.0f;
          for (int q = 0; q < S; ++q) sum += (q == split) ? own : base[(int64_t)q * (NREG * 256) + idx];
          acc[i][j][r] = sum;
        }
    if (tid == 0) a.counters[tile] = 0u;      // ready for the next launch
  }

  // ---- epilogue ------------------------------------------------------------
  // accumulator register r of lane l holds row (r/4)*8 + (l/32)*4 + r%4 and
  // column l%32 of its 32 x 32 block.
  const int B = a.B;
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
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

// Tile shapes: forward / element flows 128 x 128 (split over K when the
// output has few tiles); parameter flows 256 x 256 when every block is at
// least that large and the planes fit LDS, else 128 x 128.
template <int EPI, int PA, int PB>
static void launch3(int tiles, int big, const GemmArgs& a, hipStream_t s) {
  constexpr bool wide = (PA + PB) <= 3;
  const int grid = tiles * (EPI == EPI_PARAM ? 1 : a.splitk);
  if constexpr (wide) {
    if constexpr (EPI == EPI_PARAM) {
      if (big) {
        hipLaunchKernelGGL((k_gemm<EPI, PA, PB, 256, 256, 32>), dim3(grid), dim3(256), 0, s, a);
        return;
      }
    }
    hipLaunchKernelGGL((k_gemm<EPI, PA, PB, 128, 128, 64>), dim3(grid), dim3(256), 0, s, a);
  } else {
    hipLaunchKernelGGL((k_gemm<EPI, PA, PB, 128, 128, 32>), dim3(grid), dim3(256), 0, s, a);
  }
}

template <int EPI>
static void launch_planes(int pa, int pb, int tiles, int big, const GemmArgs& a, hipStream_t s) {
  if (pa == 1 && pb == 1) launch3<EPI, 1, 1>(tiles, big, a, s);
  else if (pa == 2 && pb == 1) launch3<EPI, 2, 1>(tiles, big, a, s);
  else if (pa == 1 && pb == 2) launch3<EPI, 1, 2>(tiles, big, a, s);
  else if (pa == 2 && pb == 2) launch3<EPI, 2, 2>(tiles, big, a, s);
  else launch3<EPI, 3, 3>(tiles, big, a, s);
}

void launch_gemm(int epi, int pa, int pb, int tiles, int big, const GemmArgs& a, hipStream_t s) {
  if (tiles <= 0) return;
  if (epi == EPI_FWD) launch_planes<EPI_FWD>(pa, pb, tiles, 0, a, s);
  else if (epi == EPI_ELEM) launch_planes<EPI_ELEM>(pa, pb, tiles, 0, a, s);
  else launch_planes<EPI_PARAM>(pa, pb, tiles, big, a, s);
}

}  // namespace pc
