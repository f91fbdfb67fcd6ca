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
// (MT/2) x (NT/2) grid of v_mfma_f32_32x32x16_bf16 blocks.  K streams through
// an LDS ring of NS stages filled by direct global->LDS loads (see Ring):
// while one KT-wide slice is multiplied, the next NS-1 are in flight.
//
// Forward and element-flow products at small output sizes split K over
// `splitk` workgroups; each writes its partial tile, and the last to arrive
// (arrival counter per tile) adds the partials in split order and runs the
// epilogue, so results are deterministic.  Workgroups are renumbered so each
// XCD (dispatch is round robin over the 8 XCDs) gets a contiguous run of
// logical tiles: the splits of a tile, and neighbouring tiles sharing weight
// rows, meet in one L2.
#include <hip/hip_runtime.h>

#include <type_traits>

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

// LDS ring of NS stages, each holding one K slice (KT wide) of every plane of
// both operands, rows unpadded and 16-byte chunks XOR-swizzled by row so the
// 128-bit fragment reads of consecutive rows hit distinct banks.  Slices are
// fetched with gfx950's direct global->LDS 16-byte loads: one wave
// instruction fills 1 KB (64 lanes x 16 B) of a stage, so no registers stage
// the data and NS-1 slices stay in flight while one is multiplied.
// The load is issued from inline assembly: the ring tracks its completion
// with explicit vmcnt waits, and a compiler that cannot tell the stages
// apart would otherwise drain every in-flight load before each LDS read.
// (M0, the LDS base of the instruction, has no other user in these kernels.)
__device__ __forceinline__ void lds_load16(const void* g, const void* lds_dst) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)lds_dst);
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(m0) : "memory", "m0");
}

template <int PA, int PB, int MT, int NT, int KT>
struct Ring {
  static constexpr int RB = KT * 2;                 // bytes per row of a slice
  static constexpr int CPR = RB / 16;               // 16-byte chunks per row (8 or 4)
  static constexpr int RPI = 1024 / RB;             // rows per wave instruction (8 or 16)
  static constexpr int AROWS = MT * RB / 2, BROWS = NT * RB / 2;   // elements per plane
  static constexpr int STAGE = PA * AROWS + PB * BROWS;           // elements per stage
  static constexpr int IA = MT / RPI, IB = NT / RPI;               // instructions per plane
  static constexpr int PER_WAVE = (PA * IA + PB * IB) / 4;         // instructions per wave per slice
  static constexpr int FM = MT / 64, FN = NT / 64;
  static constexpr int PMAX = PA > PB ? PA : PB;

  static __device__ __forceinline__ int slot(int row, int chunk) {
    return CPR == 8 ? (chunk ^ (row & 7)) : (chunk ^ ((row >> 1) & 3));
  }

  // Issue the loads of K slice [k0, k0 + KT) of rows [r0, r0 + MT) of the
  // A panel (R_A rows) and rows [rb0, rb0 + NT) of the B panel into stage
  // `st` (uniform arguments).  A slice spans KT / 32 K blocks of its panel.
  static __device__ __forceinline__ void fetch(uint16_t* st, const uint16_t* Ab, int64_t RA, int64_t ra0, int ka0,
                                               const uint16_t* Bb, int64_t RB, int64_t rb0, int kb0, int64_t pA,
                                               int64_t pB, int wave, int lane) {
    const int rin = lane / CPR, sl = lane % CPR;
    const uint16_t* a0 = Ab + (((int64_t)(ka0 >> 5) * RA + ra0) << 5);
    const uint16_t* b0 = Bb + (((int64_t)(kb0 >> 5) * RB + rb0) << 5);
#pragma unroll
    for (int q0 = 0; q0 < PER_WAVE; ++q0) {
      const int q = q0 * 4 + wave;                  // instruction index within the slice
      const uint16_t* src;
      if (q < PA * IA) {
        const int p = q / IA, qq = q - p * IA, row = qq * RPI + rin;
        const int chunk = slot(row, sl);            // the swizzle is an involution
        src = a0 + p * pA + (chunk >> 2) * (RA << 5) + row * 32 + (chunk & 3) * 8;
      } else {
        const int q2 = q - PA * IA, p = q2 / IB, qq = q2 - p * IB, row = qq * RPI + rin;
        const int chunk = slot(row, sl);
        src = b0 + p * pB + (chunk >> 2) * (RB << 5) + row * 32 + (chunk & 3) * 8;
      }
      lds_load16(src, st + q * 512);
    }
  }

  static __device__ __forceinline__ void compute(f32x16_t (&acc)[FM][FN], const uint16_t* st, int wm0, int wn0,
                                                 int lane) {
#pragma unroll
    for (int ks = 0; ks < KT / 16; ++ks) {
      bf16x8_t fa[PA][FM], fb[PB][FN];
      const int c = ks * 2 + (lane >> 5);
#pragma unroll
      for (int p = 0; p < PA; ++p)
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          const int row = wm0 + i * 32 + (lane & 31);
          fa[p][i] = *(const bf16x8_t*)(st + p * AROWS + row * (RB / 2) + slot(row, c) * 8);
        }
#pragma unroll
      for (int p = 0; p < PB; ++p)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int row = wn0 + j * 32 + (lane & 31);
          fb[p][j] = *(const bf16x8_t*)(st + PA * AROWS + p * BROWS + row * (RB / 2) + slot(row, c) * 8);
        }
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

// s_waitcnt immediate waiting until at most n vector-memory operations are
// outstanding (expcnt and lgkmcnt left at their maxima).
template <int n>
struct VmWait {
  static constexpr int imm = (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8);
};

// Workgroup barrier without a memory fence (the ring's loads stay in flight);
// the signal fences keep the compiler from moving memory operations across it.
__device__ __forceinline__ void ring_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

template <int EPI, int PA, int PB, int MT, int NT, int KT, int NS>
__global__ __launch_bounds__(256) void k_gemm(GemmArgs a) {
  constexpr int WTM = MT / 2, WTN = NT / 2;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  constexpr int SUB = ROW_PAD / MT;            // tiles per 256-row block
  using R = Ring<PA, PB, MT, NT, KT>;
  constexpr int STAGE = R::STAGE;
  // one array per stage: the compiler then tells the loads filling one stage
  // apart from the reads of another and inserts no waits of its own
  __shared__ __attribute__((aligned(1024))) uint16_t st0[STAGE];
  __shared__ __attribute__((aligned(1024))) uint16_t st1[STAGE];
  __shared__ __attribute__((aligned(1024))) uint16_t st2[NS > 2 ? STAGE : 8];
  __shared__ __attribute__((aligned(1024))) uint16_t st3[NS > 3 ? STAGE : 8];
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
  // operand panels: base, rows, first row of the tile, first K of the range
  const uint16_t* Ab;
  const uint16_t* Bb;
  int64_t RA, RB, ra0, rb0;
  int ka0, kb0, kst, kbeg, kend, m0, n0;
  int64_t acopy = 0, bcopy = 0;                // row step per tied copy (parameter flows)
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
    RB = a.B_pad;
    rb0 = n0;
    if (EPI == EPI_FWD) {
      m0 = (gt - gr->mt_start * SUB) * MT;
      kst = (gr->N + K_PAD - 1) / K_PAD * K_PAD / KT;
      Ab = a.opA + bl->th_off;
      RA = (bl->M + ROW_PAD - 1) / ROW_PAD * ROW_PAD;
      kb0 = gr->e_koff;
    } else {
      m0 = (gt - gr->ct_start * SUB) * MT;
      kst = (gr->M + K_PAD - 1) / K_PAD * K_PAD / KT;
      Ab = a.opA + bl->tht_off;
      RA = (bl->N + ROW_PAD - 1) / ROW_PAD * ROW_PAD;
      kb0 = gr->g_koff;
    }
    ra0 = m0;
    ka0 = 0;
    Bb = a.opB;
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
    kst = a.B_padK / KT;
    kbeg = 0;
    kend = bl->ncopies * kst;
    Ab = a.opA;
    Bb = a.opB;
    RA = a.rowsA;
    RB = a.rowsB;
    ra0 = bl->g_base + m0;
    rb0 = bl->e_base + n0;
    acopy = Mp;
    bcopy = Np;
    ka0 = kb0 = 0;
  }

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int64_t pA = a.planeA, pB = a.planeB;
  const int n = kend - kbeg;
  auto stage = [&](int j) -> uint16_t* { return j == 0 ? st0 : j == 1 ? st1 : j == 2 ? st2 : st3; };
  auto fetch = [&](int j, int it) {
    const int kt = min(kbeg + it, kend - 1);   // clamped: a copy past the end is never read
    if (EPI == EPI_PARAM) {
      const int s = kt / kst, kk = (kt - s * kst) * KT;
      R::fetch(stage(j), Ab, RA, ra0 + s * acopy, kk, Bb, RB, rb0 + s * bcopy, kk, pA, pB, wave, lane);
    } else {
      R::fetch(stage(j), Ab, RA, ra0, ka0 + kt * KT, Bb, RB, rb0, kb0 + kt * KT, pA, pB, wave, lane);
    }
  };
  // one pipeline step on slice `it`, held in stage J: wait until it has
  // landed (at most NS-2 newer slices outstanding), barrier (every wave is
  // also done with the stage read in the previous step), refill that stage
  // with slice it+NS-1, multiply slice it.
  auto step = [&](auto J, int it) {
    constexpr int j = decltype(J)::value;
    __builtin_amdgcn_s_waitcnt(VmWait<(NS - 2) * R::PER_WAVE>::imm);
    ring_barrier();
    fetch((j + NS - 1) % NS, it + NS - 1);
    R::compute(acc, stage(j), wm0, wn0, lane);
  };
  if (n > 0) {
#pragma unroll
    for (int j = 0; j < NS - 1; ++j) fetch(j, j);
    for (int it = 0; it < n; it += NS) {
      step(std::integral_constant<int, 0>(), it);
      if (it + 1 < n) step(std::integral_constant<int, 1>(), it + 1);
      if constexpr (NS > 2)
        if (it + 2 < n) step(std::integral_constant<int, 2 % NS>(), it + 2);
      if constexpr (NS > 3)
        if (it + 3 < n) step(std::integral_constant<int, 3 % NS>(), it + 3);
    }
    __builtin_amdgcn_s_waitcnt(0);       // no load may still target LDS when the workgroup ends
  }

  // ---- split-K: the last workgroup of a tile adds the partials in order -----
  // Partials are published with device-scope atomic stores (written through
  // to the device coherence point, so no cache-wide write-back is needed),
  // completed (vmcnt 0) before the arrival counter moves; the last arrival
  // reads them back with device-scope atomic loads.  A __threadfence() here
  // would write back and invalidate the whole L2 of the XCD under every
  // other workgroup still streaming operands through it.
  if (EPI != EPI_PARAM && S > 1) {
    constexpr int NREG = FM * FN * 16;
    float* mine = a.partials + ((int64_t)tile * S + split) * (NREG * 256);
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          __hip_atomic_store(mine + ((i * FN + j) * 16 + r) * 256 + tid, acc[i][j][r], __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0)
      last_flag = (__hip_atomic_fetch_add(a.counters + tile, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                   (unsigned)(S - 1));
    __syncthreads();
    if (!last_flag) return;
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
          for (int q = 0; q < S; ++q)
            sum += (q == split) ? own
                                : __hip_atomic_load(base + (int64_t)q * (NREG * 256) + idx, __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT);
          acc[i][j][r] = sum;
        }
    if (tid == 0) __hip_atomic_store(a.counters + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
// least that large and the planes fit LDS, else 128 x 128.  KT is 64 when a
// stage of that width is at most 48 KB, else 32; NS stages fill up to 160 KB.
template <int PA, int PB, int MT, int NT>
struct Shape {
  static constexpr int KT = ((PA * MT + PB * NT) * 64 * 2 <= 48 * 1024) ? 64 : 32;
  static constexpr int STAGE_BYTES = (PA * MT + PB * NT) * KT * 2;
  static constexpr int NSR = (160 * 1024 - 1024) / STAGE_BYTES;
  static constexpr int NS = NSR > 4 ? 4 : NSR;
};

template <int EPI, int PA, int PB, int MT, int NT>
static void launch_shape(int grid, const GemmArgs& a, hipStream_t s) {
  using Sh = Shape<PA, PB, MT, NT>;
  static_assert(Sh::NS >= 2, "LDS ring needs two stages");
  hipLaunchKernelGGL((k_gemm<EPI, PA, PB, MT, NT, Sh::KT, Sh::NS>), dim3(grid), dim3(256), 0, s, a);
}

template <int EPI, int PA, int PB>
static void launch3(int tiles, int big, const GemmArgs& a, hipStream_t s) {
  constexpr bool wide = (PA + PB) <= 3;
  const int grid = tiles * (EPI == EPI_PARAM ? 1 : a.splitk);
  if constexpr (EPI == EPI_PARAM && wide) {
    if (big) {
      launch_shape<EPI, PA, PB, 256, 256>(grid, a, s);
      return;
    }
  }
  launch_shape<EPI, PA, PB, 128, 128>(grid, a, s);
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
