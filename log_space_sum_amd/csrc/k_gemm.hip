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
// Tiling: MT x NT output tile per workgroup of 4 waves laid out WM x (4/WM),
// each wave a grid of v_mfma_f32_32x32x16_bf16 blocks.  K streams through an
// LDS ring of NS stages filled by direct global->LDS loads: while one KT-wide
// slice is multiplied, the next NS-1 are in flight.  Inside a slice the
// fragments of the next 16-wide K step are read from LDS while the matrix
// instructions of the current one run, and the loads of the slice NS-1 ahead
// are issued between them; the ring barrier sits in the middle of a slice's
// last matrix instructions, so its wait overlaps them.  In the forward,
// element-flow and virtual-batch products the weights (A) skip the ring: they
// are stored in fragment order (frag_major) and each wave loads its own rows
// straight into a register ring of NS slices; the LDS ring carries B only.
//
// Forward and element-flow products of one layer have few output tiles; they
// split K over `splitk` workgroups.  Every split writes its partial tile, and
// the last to arrive (arrival counter per tile) adds all partials in split
// order and runs the epilogue, so results are deterministic.  Workgroups are
// renumbered so each XCD (dispatch is round robin over the 8 XCDs) gets a
// contiguous run of logical tiles: the splits of a tile, and neighbouring
// tiles sharing weight rows, meet in one L2.
#include <hip/hip_runtime.h>

#include <type_traits>
#include <utility>

#include "pc_kernels.h"
#include "pc_ring.h"

namespace pc {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

template <int... I, typename F>
__device__ __forceinline__ void sfor_impl(std::integer_sequence<int, I...>, F&& f) {
  (f(std::integral_constant<int, I>{}), ...);
}
// f(integral_constant<0>), ..., f(integral_constant<N-1>), fully unrolled
template <int N, typename F>
__device__ __forceinline__ void sfor(F&& f) {
  sfor_impl(std::make_integer_sequence<int, N>{}, f);
}

__device__ __forceinline__ float key_to_shift(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  float m = __uint_as_float(u);
  return (m == m && fabsf(m) <= 3.0e38f) ? m : 0.0f;   // -inf / unset column -> 0
}

// Order-preserving 32-bit key of a float (integer atomic max = float max).
__device__ __forceinline__ uint32_t float_to_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// float32 -> bfloat16, round to nearest even (NaN kept quiet), and back.
__device__ __forceinline__ uint32_t bf16_bits(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ float bf16_value(uint32_t h) { return __uint_as_float(h << 16); }
// Split N values into np bfloat16 planes (each the rounding of what the
// previous planes leave) and store each plane's N values as one run.
template <int N>
__device__ __forceinline__ void split_planes(const float* x, int np, uint16_t* dst, int64_t plane) {
  static_assert(N == 4 || N == 8, "4 or 8 values");
  float r[N];
#pragma unroll
  for (int e = 0; e < N; ++e) r[e] = x[e];
  for (int p = 0; p < np; ++p) {
    uint32_t w[N / 2];
#pragma unroll
    for (int e = 0; e < N / 2; ++e) {
      const uint32_t h0 = bf16_bits(r[2 * e]), h1 = bf16_bits(r[2 * e + 1]);
      r[2 * e] -= bf16_value(h0);
      r[2 * e + 1] -= bf16_value(h1);
      w[e] = h0 | (h1 << 16);
    }
    if constexpr (N == 4) *(uint2*)(dst + p * plane) = make_uint2(w[0], w[1]);
    else *(uint4*)(dst + p * plane) = make_uint4(w[0], w[1], w[2], w[3]);
  }
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

// Plane pairs (pa, pb) whose product is accumulated, highest order first.
template <int PA, int PB>
struct Pairs {
  static constexpr int PMAX = PA > PB ? PA : PB;
  static constexpr int count() {
    int n = 0;
    for (int o = PMAX - 1; o >= 0; --o)
      for (int pa = 0; pa < PA; ++pa)
        if (o - pa >= 0 && o - pa < PB) ++n;
    return n;
  }
  static constexpr int N = count();
  static constexpr int at(int t, int which) {
    int n = 0;
    for (int o = PMAX - 1; o >= 0; --o)
      for (int pa = 0; pa < PA; ++pa)
        if (o - pa >= 0 && o - pa < PB) {
          if (n == t) return which == 0 ? pa : o - pa;
          ++n;
        }
    return 0;
  }
};

// Fragment reads of one K step in the order the matrix instructions first
// use them (read u < PA*FM: A plane u/FM, row block u%FM; else B).
template <int PA, int PB, int FM, int FN>
struct ReadOrder {
  using PP = Pairs<PA, PB>;
  static constexpr int NRD = PA * FM + PB * FN;
  static constexpr int at(int o) {
    bool seen[NRD] = {};
    int n = 0;
    for (int t = 0; t < PP::N * FM * FN; ++t) {
      const int pr = t / (FM * FN), i = (t / FN) % FM, j = t % FN;
      const int ua = PP::at(pr, 0) * FM + i, ub = PA * FM + PP::at(pr, 1) * FN + j;
      if (!seen[ua]) {
        seen[ua] = true;
        if (n++ == o) return ua;
      }
      if (!seen[ub]) {
        seen[ub] = true;
        if (n++ == o) return ub;
      }
    }
    return 0;
  }
};

// The same for B alone (the weights in registers): read u < PB*FN is plane
// u/FN, column block u%FN.
template <int PA, int PB, int FM, int FN>
struct ReadOrderB {
  using PP = Pairs<PA, PB>;
  static constexpr int NRD = PB * FN;
  static constexpr int at(int o) {
    bool seen[NRD] = {};
    int n = 0;
    for (int t = 0; t < PP::N * FM * FN; ++t) {
      const int pr = t / (FM * FN), j = t % FN;
      const int ub = PP::at(pr, 1) * FN + j;
      if (!seen[ub]) {
        seen[ub] = true;
        if (n++ == o) return ub;
      }
    }
    return 0;
  }
};

// LDS ring geometry.  A stage holds one K slice (KT wide) of every plane of
// the operands it carries (both, or only B when the weights go straight to
// registers: AD), rows unpadded (KT * 2 bytes), 16-byte chunks XOR-swizzled by
// row so that the 128-bit fragment reads of 16 consecutive rows touch 16
// distinct chunk slots of 64 banks (and those of 8 consecutive rows 8 distinct
// slots of 32 banks).  One wave load instruction fills 1 KB (64 lanes x 16 B)
// of a stage: RPI rows.
template <int PA, int PB, int MT, int NT, int KT, bool AD>
struct Ring {
  static constexpr int RB = KT * 2;                 // bytes per row of a slice
  static constexpr int CPR = RB / 16;               // 16-byte chunks per row (8 or 4)
  static constexpr int RPI = 1024 / RB;             // rows per load instruction (8 or 16)
  static constexpr int AIN = AD ? 0 : PA;           // A planes in the ring
  static constexpr int AEL = MT * KT, BEL = NT * KT;                 // elements per plane
  static constexpr int STAGE = AIN * AEL + PB * BEL;                  // elements per stage
  static constexpr int IA = MT / RPI, IB = NT / RPI;                 // instructions per plane
  static constexpr int PER_WAVE = (AIN * IA + PB * IB) / 4;          // instructions per wave per slice
  static constexpr int QA = AIN * IA / 4;                             // of which A
  static_assert(IA % 4 == 0 && IB % 4 == 0, "each wave loads whole instructions of one plane");

  static __device__ __forceinline__ int swz(int row) {
    return CPR == 8 ? ((row & 7) ^ ((row >> 3) & 1)) : (((row >> 1) ^ (row >> 2)) & 3);
  }
};

template <int EPI, int PA, int PB, int MT, int NT, int WM, int KT, int NS>
__global__ __launch_bounds__(256) void k_gemm(GemmArgs a) {
  constexpr int WN = 4 / WM;
  constexpr int WTM = MT / WM, WTN = NT / WN;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  constexpr int SUB = ROW_PAD / MT;            // tiles per 256-row block
  // forward, element-flow and virtual-batch products: the weights (A) go
  // from global memory straight into registers in fragment order, the ring
  // carries B only
  constexpr bool AD = EPI != EPI_PARAM;
  using R = Ring<PA, PB, MT, NT, KT, AD>;
  using PP = Pairs<PA, PB>;
  constexpr int KS = KT / 16;                  // matrix K steps per slice
  constexpr int NMF = PP::N * FM * FN;         // matrix instructions per K step
  constexpr int NRD = PA * FM + PB * FN;       // fragment reads per K step
  constexpr int PW = R::PER_WAVE;
  constexpr int NREG = FM * FN * 16;
  static_assert(KS % 2 == 0, "fragment buffers alternate per K step");
  static_assert(WM * WN == 4 && FM >= 1 && FN >= 1, "4 waves");
  // the ring: NS stages (the loads filling it are issued from inline
  // assembly, so the compiler tracks no dependence between a stage being
  // filled and the reads of another)
  // (the epilogue reuses it for its pass tile, column shifts, child rows and maxima)
  constexpr int EPI_FLOATS = WM * 32 * (NT + 8) + NT + MT + (256 / (NT / 4)) * NT;
  constexpr int RING_EL = NS * R::STAGE > 2 * EPI_FLOATS ? NS * R::STAGE : 2 * EPI_FLOATS;
  __shared__ __attribute__((aligned(1024))) uint16_t ring[RING_EL];
  __shared__ int last_flag;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave
  const int wm0 = (wave / WN) * WTM, wn0 = (wave % WN) * WTN;
  const int logical = xcd_remap(blockIdx.x, gridDim.x);

  // ---- locate the problem, the tile and the K range ------------------------
  // splitk workgroups share one tile's K range (the parameter-flow product's
  // K is every tied copy's samples; its tiles count from tile0)
  const int S = a.splitk;
  const int ltile = logical / S;               // the launch's tile (split-K partials, arrival counters)
  const int split = logical - ltile * S;
  const int tile = EPI == EPI_PARAM ? ltile + a.tile0 : ltile;
  // the forward's operand layout: weights [M rows, K = N] (forward products,
  // and virtual-batch stores with vs_elem == 0); else the transposed weights
  const bool fwdA = EPI == EPI_FWD || (EPI == EPI_VSTORE && !a.vs_elem);
  const uint16_t* Ab;
  const uint16_t* Bb;
  int64_t RA, RB, ra0, rb0;
  int kst, kbeg, kend, m0, n0;
  int64_t acopy = 0, bcopy = 0;                // row step per tied copy (parameter flows)
  int ka0 = 0, kb0 = 0;
  int ksl_a = 0;                               // AD: K slices of the weight block (its fragment-order row pitch)
  GroupRec gr{};
  BlockRec bl{};
  if (EPI == EPI_FWD || EPI == EPI_ELEM || EPI == EPI_VSTORE) {
    const int gt = tile / a.ntiles, nt = tile - gt * a.ntiles;
    const int unit = gt / SUB;
    int g;
    if (fwdA)
      g = find_last_le(a.groups, a.ngroups, unit, [](const GroupRec& r) { return r.mt_start; });
    else
      g = find_last_le(a.groups, a.ngroups, unit, [](const GroupRec& r) { return r.ct_start; });
    gr = a.groups[g];
    bl = a.blocks[gr.block];
    n0 = nt * NT;
    RB = a.B_pad;
    rb0 = n0;
    if (fwdA) {
      m0 = (gt - gr.mt_start * SUB) * MT;
      kst = (gr.N + K_PAD - 1) / K_PAD * K_PAD / KT;
      Ab = a.opA + bl.th_off;
      RA = (bl.M + ROW_PAD - 1) / ROW_PAD * ROW_PAD;
      kb0 = gr.e_koff;
    } else {
      m0 = (gt - gr.ct_start * SUB) * MT;
      kst = (gr.M + K_PAD - 1) / K_PAD * K_PAD / KT;
      Ab = a.opA + bl.tht_off;
      RA = (bl.N + ROW_PAD - 1) / ROW_PAD * ROW_PAD;
      kb0 = gr.g_koff;
    }
    ra0 = m0;
    ksl_a = ((fwdA ? bl.N : bl.M) + K_PAD - 1) / K_PAD * K_PAD / 32;
    Bb = a.opB;
    kbeg = split * kst / S;
    kend = (split + 1) * kst / S;
    // a tile wholly in the group's row padding has no output (every split of
    // it leaves here, so its arrival counter is never touched)
    if (m0 >= (fwdA ? gr.M : gr.N)) return;
  } else {
    // tile prefix of the block sequence: 256 x 256 tiles, twice as many
    // 128 x 256 tiles (blocks are padded to 256 both ways), or 128 x 128
    const int b = (MT == 256)
        ? find_last_le(a.blocks, a.ngroups, tile, [](const BlockRec& r) { return r.pt256; })
        : (NT == 256)
        ? find_last_le(a.blocks, a.ngroups, tile, [](const BlockRec& r) { return 2 * r.pt256; })
        : find_last_le(a.blocks, a.ngroups, tile, [](const BlockRec& r) { return r.pt128; });
    bl = a.blocks[b];
    const int Mp = (bl.M + ROW_PAD - 1) / ROW_PAD * ROW_PAD;
    const int Np = (bl.N + ROW_PAD - 1) / ROW_PAD * ROW_PAD;
    const int ntn = Np / NT, mtn = Mp / MT;
    const int lt = tile - ((MT == 256) ? bl.pt256 : (NT == 256) ? 2 * bl.pt256 : bl.pt128);
    // tiles in groups of up to 4 tile rows, column-major inside a group, so
    // the 32 workgroups an XCD runs at once cover about 4 x 8 tiles and
    // share both operands' panels in its L2
    constexpr int GM = 4;
    const int grp = lt / (GM * ntn), r0g = grp * GM;
    const int rows = mtn - r0g < GM ? mtn - r0g : GM;
    const int in = lt - grp * GM * ntn;
    m0 = (r0g + in % rows) * MT;
    n0 = (in / rows) * NT;
    if (m0 >= bl.M || n0 >= bl.N) return;      // wholly in the block's padding
    kst = a.B_padK / KT;
    {
      const int c0 = a.copy_lo < bl.ncopies ? a.copy_lo : bl.ncopies;
      const int c1 = a.copy_hi < bl.ncopies ? a.copy_hi : bl.ncopies;
      const int tot = (c1 > c0 ? c1 - c0 : 0) * kst;      // K slices of the copies
      kbeg = c0 * kst + (int)((int64_t)split * tot / S);
      kend = c0 * kst + (int)((int64_t)(split + 1) * tot / S);
    }
    Ab = a.opA;
    Bb = a.opB;
    RA = a.rowsA;
    RB = a.rowsB;
    ra0 = bl.g_base + m0;
    rb0 = bl.e_base + n0;
    acopy = Mp;
    bcopy = Np;
  }

  // ---- per-lane load offsets (bytes within a slice of one plane) -----------
  uint32_t voff[PW];
  sfor<PW>([&](auto Q) {
    constexpr int q0 = decltype(Q)::value;
    const int qq = q0 * 4 + wave;
    constexpr bool isA = q0 < R::QA;
    const int qi = isA ? qq % R::IA : (qq - R::AIN * R::IA) % R::IB;
    const int row = qi * R::RPI + lane / R::CPR;
    const int chunk = (lane % R::CPR) ^ R::swz(row);     // the swizzle is an involution
    const int64_t rows = isA ? RA : RB;
    voff[q0] = (uint32_t)((((chunk >> 2) * rows + row) * 32 + (chunk & 3) * 8) * 2);
  });
  // LDS fragment addresses: rows wm0 + i*32 + lane%32 (A) and wn0 + j*32 +
  // lane%32 (B) share one swizzle key (it depends on the row modulo 32 only),
  // so each K step needs one lane offset per operand; fragments i, j and the
  // stage add constants.
  const int key = (lane >> 5) ^ R::swz(lane & 31);
  int a_off[KS], b_off[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    a_off[ks] = (wm0 + (lane & 31)) * R::RB + (((ks * 2) ^ key) << 4);
    b_off[ks] = (wn0 + (lane & 31)) * R::RB + (((ks * 2) ^ key) << 4);
  }

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int64_t pAb = a.planeA * 2, pBb = a.planeB * 2;   // plane strides in bytes
  const int n = kend - kbeg;
  // slice cursor of the loads (advanced once per issued slice)
  int cur_s = 0, cur_k = 0;                    // parameter flows: copy and K offset within it
  int next_load = 0;
  if (EPI == EPI_PARAM) {
    cur_s = kbeg / kst;
    cur_k = (kbeg - cur_s * kst) * KT;
  }
  const uint32_t ring_lds = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)ring;
  // uniform byte bases of the next slice to load
  const char* sa = nullptr;
  const char* sb = nullptr;
  // AD: this lane's 16 bytes of K step 0 of slice kbeg, row block
  // (m0 + wm0) / 32, plane 0 (fragment order: a slice is 2048 bytes, a K step
  // 1024, the next row block ksl_a slices on, the next plane pAb bytes on)
  const char* a_lane = nullptr;
  if constexpr (AD) a_lane = (const char*)Ab + (((int64_t)((m0 + wm0) >> 5) * ksl_a + kbeg) * 2048 + lane * 16);
  const char* sA = nullptr;
  // (past the last slice the ring keeps re-loading it: the stages it lands in
  // are never read, and every wait stays a constant)
  auto slice_bases = [&]() {
    if (next_load >= n) return;
    int64_t ea, eb;
    if (EPI == EPI_PARAM) {
      ea = ((int64_t)(cur_k >> 5) * RA + ra0 + (int64_t)cur_s * acopy) * 32;
      eb = ((int64_t)(cur_k >> 5) * RB + rb0 + (int64_t)cur_s * bcopy) * 32;
      cur_k += KT;
      if (cur_k == kst * KT) {
        cur_k = 0;
        ++cur_s;
      }
    } else {
      const int k = (kbeg + next_load) * KT;
      ea = ((int64_t)((ka0 + k) >> 5) * RA + ra0) * 32;
      eb = ((int64_t)((kb0 + k) >> 5) * RB + rb0) * 32;
    }
    if constexpr (AD) sA = a_lane + (int64_t)next_load * 2048;
    ++next_load;
    sa = (const char*)Ab + ea * 2;
    sb = (const char*)Bb + eb * 2;
  };
  // load instruction q0 of the slice whose bases are (sa, sb) into stage j
  auto dma = [&](int j, auto Q) {
    constexpr int q0 = decltype(Q)::value;
    constexpr bool isA = q0 < R::QA;
    constexpr int p = isA ? (q0 * 4) / R::IA : (q0 * 4 - R::AIN * R::IA) / R::IB;
    const char* base = isA ? sa + p * pAb : sb + p * pBb;
    lds_load16(base, voff[q0], ring_lds + j * (R::STAGE * 2) + (q0 * 4 + wave) * 1024);
  };

  if constexpr (!AD) {
  bf16x8_t fa[2][PA][FM], fb[2][PB][FN];
  // fragment read u of K step KSI of a stage into buffer BF
  auto frag = [&](auto BF, int sbyte, auto KSI, auto U) {
    constexpr int bf = decltype(BF)::value;
    constexpr int ks = decltype(KSI)::value;
    constexpr int u = decltype(U)::value;
    const char* st = (const char*)ring;
    if constexpr (u < PA * FM) {
      constexpr int p = u / FM, i = u % FM;
      fa[bf][p][i] = *(const bf16x8_t*)(st + (sbyte + a_off[ks]) + (p * R::AEL * 2 + i * 32 * R::RB));
    } else {
      constexpr int p = (u - PA * FM) / FN, jj = (u - PA * FM) % FN;
      fb[bf][p][jj] =
          *(const bf16x8_t*)(st + (sbyte + b_off[ks]) + (R::AIN * R::AEL * 2 + p * R::BEL * 2 + jj * 32 * R::RB));
    }
  };
  auto mfma = [&](auto BF, auto T) {
    constexpr int bf = decltype(BF)::value;
    constexpr int t = decltype(T)::value;
    constexpr int pr = t / (FM * FN), i = (t / FN) % FM, j = t % FN;
    constexpr int pa = PP::at(pr, 0), pb = PP::at(pr, 1);
    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[bf][pa][i], fb[bf][pb][j], acc[i][j], 0, 0, 0);
  };

  // One pipeline step on slice `it` held in stage j (its first fragments are
  // already in buffer 0): refill the stage read in the previous step with
  // slice it+NS-1, multiply slice it, and (unless it is the last) cross the
  // barrier that makes slice it+1 readable at the start of the last K step
  // and read the next slice's first fragments during it.  Fragment reads go
  // into the first half of a K step's matrix instructions, in order of first
  // use, so each has half a K step to land; the slice loads into the second
  // half of the first K step.
  using RO = ReadOrder<PA, PB, FM, FN>;
  constexpr int H = NMF / 2;
  auto step = [&](auto LAST, int j) {
    constexpr bool last = decltype(LAST)::value;
    const int jn = j + 1 == NS ? 0 : j + 1, jl = j == 0 ? NS - 1 : j - 1;
    const int sbyte = j * (R::STAGE * 2), snext = jn * (R::STAGE * 2);
    slice_bases();
    sfor<KS>([&](auto KSI) {
      constexpr int ks = decltype(KSI)::value;
      constexpr int bf = ks & 1;
      using BF = std::integral_constant<int, bf>;
      using BN = std::integral_constant<int, bf ^ 1>;
      constexpr bool lastks = ks + 1 == KS;
      if constexpr (lastks && !last) {
        // slice it+1 has landed once at most the NS-2 slices issued after it are in flight
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(WaitVmLgkm<(NS - 2) * PW>::imm);
        ring_barrier();
      }
      sfor<NMF>([&](auto T) {
        constexpr int t = decltype(T)::value;
        mfma(BF(), T);
        if constexpr (t < H) {
          constexpr int o0 = t * NRD / H, o1 = (t + 1) * NRD / H;
          sfor<o1 - o0>([&](auto O) {
            constexpr int u = RO::at(o0 + decltype(O)::value);
            if constexpr (!lastks) frag(BN(), sbyte, std::integral_constant<int, ks + 1>(), std::integral_constant<int, u>());
            else if constexpr (!last) frag(std::integral_constant<int, 0>(), snext, std::integral_constant<int, 0>(), std::integral_constant<int, u>());
          });
        } else if constexpr (ks == 0) {
          constexpr int o0 = (t - H) * PW / (NMF - H), o1 = (t - H + 1) * PW / (NMF - H);
          sfor<o1 - o0>([&](auto O) { dma(jl, std::integral_constant<int, o0 + decltype(O)::value>()); });
        }
        __builtin_amdgcn_sched_barrier(0);
      });
    });
  };

  if (n > 0) {
    // prologue: slices 0 .. NS-2 in flight, slice 0 readable, its first fragments read
    sfor<NS - 1>([&](auto S0) {
      slice_bases();
      sfor<PW>([&](auto Q) { dma(decltype(S0)::value, Q); });
    });
    __builtin_amdgcn_s_waitcnt(WaitVmLgkm<(NS - 2) * PW>::imm);
    ring_barrier();
    sfor<NRD>([&](auto U) { frag(std::integral_constant<int, 0>(), 0, std::integral_constant<int, 0>(), U); });
    int j = 0;
    for (int it = 0; it < n - 1; ++it) {
      step(std::false_type(), j);
      j = j + 1 == NS ? 0 : j + 1;
    }
    step(std::true_type(), j);
  }
  } else {
  // ---- weights in registers: slice s of A in buffer s % NS -------------------
  // Each wave loads its own FM row blocks of every plane, QD loads of 1 KB per
  // slice (ordinary loads: the compiler waits for them before their first
  // use); B streams through the ring as above.  The main loop is unrolled NS
  // times so that the register buffer and the stage of every step are
  // constants.  Every step issues its loads (past the last slice it re-loads
  // that slice, into a buffer and stage nobody reads), and every step waits
  // for the next slice and reads its first fragments (after the last one the
  // stage read holds an old slice and the values go unused): the waits stay
  // constants.
  constexpr int QD = PA * FM * KS;             // direct weight loads per wave per slice
  constexpr int NRB = PB * FN;                 // fragment reads (B) per K step
  using RB_ = ReadOrderB<PA, PB, FM, FN>;
  bf16x8_t areg[NS][PA][FM][KS];
  bf16x8_t fb[2][PB][FN];
  // direct load q of the slice at sA into buffer BUF
  auto aload = [&](auto BUF, auto Q) {
    constexpr int buf = decltype(BUF)::value, q = decltype(Q)::value;
    constexpr int p = q / (FM * KS), i = (q / KS) % FM, ks = q % KS;
    areg[buf][p][i][ks] = *(const bf16x8_t*)(sA + p * pAb + (int64_t)i * ksl_a * 2048 + ks * 1024);
  };
  // B fragment read u of K step KSI of the stage at byte sbyte into buffer BF
  auto fragb = [&](auto BF, int sbyte, auto KSI, auto U) {
    constexpr int bf = decltype(BF)::value;
    constexpr int ks = decltype(KSI)::value;
    constexpr int u = decltype(U)::value;
    constexpr int p = u / FN, jj = u % FN;
    const char* st = (const char*)ring;
    fb[bf][p][jj] = *(const bf16x8_t*)(st + (sbyte + b_off[ks]) + (p * R::BEL * 2 + jj * 32 * R::RB));
  };
  auto mfmad = [&](auto BUF, auto KSI, auto BF, auto T) {
    constexpr int buf = decltype(BUF)::value, ks = decltype(KSI)::value, bf = decltype(BF)::value;
    constexpr int t = decltype(T)::value;
    constexpr int pr = t / (FM * FN), i = (t / FN) % FM, j = t % FN;
    constexpr int pa = PP::at(pr, 0), pb = PP::at(pr, 1);
    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(areg[buf][pa][i][ks], fb[bf][pb][j], acc[i][j], 0, 0, 0);
  };
  constexpr int H = NMF / 2;
  auto stepd = [&](auto JC) {
    constexpr int J = decltype(JC)::value;
    constexpr int JN = (J + 1) % NS, JL = (J + NS - 1) % NS;
    constexpr int sbyte = J * (R::STAGE * 2), snext = JN * (R::STAGE * 2);
    slice_bases();
    sfor<KS>([&](auto KSI) {
      constexpr int ks = decltype(KSI)::value;
      constexpr int bf = ks & 1;
      using BF = std::integral_constant<int, bf>;
      using BN = std::integral_constant<int, bf ^ 1>;
      constexpr bool lastks = ks + 1 == KS;
      if constexpr (lastks) {
        // the next slice's B has landed in LDS once at most (NS-2)*PW loads
        // are in flight: loads into registers and loads into LDS each
        // complete in issue order, but not in order with each other, and were
        // one of that slice's LDS loads still in flight, so would be the
        // (NS-2)*PW LDS loads issued after it.  (The compiler's own waits for
        // the weight registers count only register loads, so they hold too.)
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(WaitVmLgkm<(NS - 2) * PW>::imm);
        ring_barrier();
      }
      sfor<NMF>([&](auto T) {
        constexpr int t = decltype(T)::value;
        mfmad(std::integral_constant<int, J>(), KSI, BF(), T);
        if constexpr (t < H) {
          constexpr int o0 = t * NRB / H, o1 = (t + 1) * NRB / H;
          sfor<o1 - o0>([&](auto O) {
            constexpr int u = RB_::at(o0 + decltype(O)::value);
            if constexpr (!lastks) fragb(BN(), sbyte, std::integral_constant<int, ks + 1>(), std::integral_constant<int, u>());
            else fragb(std::integral_constant<int, 0>(), snext, std::integral_constant<int, 0>(), std::integral_constant<int, u>());
          });
        } else if constexpr (ks == 0) {
          // the ring's loads in the first K step (all before the step's ring
          // wait, which counts them), the weights' in the second: the
          // requests spread over the slice (3-4 % faster per product than
          // all in the first K step)
          constexpr int o0 = (t - H) * PW / (NMF - H), o1 = (t - H + 1) * PW / (NMF - H);
          sfor<o1 - o0>([&](auto O) { dma(JL, std::integral_constant<int, o0 + decltype(O)::value>()); });
        } else if constexpr (ks == 1) {
          constexpr int o0 = (t - H) * QD / (NMF - H), o1 = (t - H + 1) * QD / (NMF - H);
          sfor<o1 - o0>([&](auto O) {
            aload(std::integral_constant<int, JL>(), std::integral_constant<int, o0 + decltype(O)::value>());
          });
        }
        __builtin_amdgcn_sched_barrier(0);
      });
    });
  };
  if (n > 0) {
    // prologue: slices 0 .. NS-2 in flight, slice 0 readable, its first fragments read
    sfor<NS - 1>([&](auto S0) {
      slice_bases();
      sfor<QD>([&](auto Q) { aload(S0, Q); });
      sfor<PW>([&](auto Q) { dma(decltype(S0)::value, Q); });
    });
    __builtin_amdgcn_s_waitcnt(WaitVmLgkm<(NS - 2) * PW>::imm);
    ring_barrier();
    sfor<NRB>([&](auto U) { fragb(std::integral_constant<int, 0>(), 0, std::integral_constant<int, 0>(), U); });
    // whole rounds of NS steps with no branch between the steps (so the
    // compiler's waits for the weight registers count every load issued
    // since), then the last n % NS steps
    int it0 = 0;
    for (; it0 + NS <= n; it0 += NS) sfor<NS>([&](auto JC) { stepd(JC); });
    if (it0 < n)
      sfor<NS - 1>([&](auto JC) {
        if (it0 + decltype(JC)::value < n) stepd(JC);
      });
  }
  }
  // 32 wait states between the last matrix instructions and the branches to
  // the code that reads the accumulators (split-K partials, epilogue).
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0);       // no load may still target LDS past this point

  // ---- split-K: the last workgroup of a tile adds the partials in order -----
  // Partials are written and read with device-scope atomics (no data race).
  // Ordering: the workgroup barrier orders every lane's partial stores before
  // the arrival increment of lane 0, a device-scope release; the last arriving
  // workgroup's increment is an acquire that reads it, and its barrier orders
  // that acquire before its lanes' partial loads.  Happens-before is
  // transitive across the two scopes, so the last arrival reads every split's
  // finished partials; it adds them in split order (deterministic).
  if (S > 1) {
    float* mine = a.partials + ((int64_t)ltile * S + split) * (NREG * 256);
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
      last_flag = (__hip_atomic_fetch_add(a.counters + ltile, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT) ==
                   (unsigned)(S - 1));
    __syncthreads();
    if (!last_flag) return;
    const float* base = a.partials + (int64_t)ltile * S * (NREG * 256);
    // in chunks of CH registers over all SM >= S splits (about 128 values
    // per lane): every load of a chunk in flight at once, then the splits
    // added in order
    auto reduce = [&](auto ch_c, auto sm_c) {
      constexpr int CH = decltype(ch_c)::value < NREG ? decltype(ch_c)::value : NREG;
      constexpr int SM = decltype(sm_c)::value;
#pragma unroll
      for (int c0 = 0; c0 < NREG; c0 += CH) {
        float t[SM][CH];
#pragma unroll
        for (int q = 0; q < SM; ++q)
          if (q < S)
#pragma unroll
            for (int x = 0; x < CH; ++x)
              t[q][x] = __hip_atomic_load(base + (int64_t)q * (NREG * 256) + (c0 + x) * 256 + tid,
                                          __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
        for (int q = 1; q < SM; ++q)
          if (q < S)
#pragma unroll
            for (int x = 0; x < CH; ++x) t[0][x] += t[q][x];
#pragma unroll
        for (int x = 0; x < CH; ++x) {
          const int reg = c0 + x, blk = reg / 16;
          acc[blk / FN][blk % FN][reg % 16] = t[0][x];
        }
      }
    };
    if (S <= 2) reduce(std::integral_constant<int, 64>(), std::integral_constant<int, 2>());
    else if (S <= 4) reduce(std::integral_constant<int, 32>(), std::integral_constant<int, 4>());
    else reduce(std::integral_constant<int, 16>(), std::integral_constant<int, 8>());
    if (tid == 0) __hip_atomic_store(a.counters + ltile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  if constexpr (EPI == EPI_VSTORE) {
    // straight from the accumulators: register r of lane l holds row
    // (r/4)*8 + (l/32)*4 + r%4 and column l%32 of its 32 x 32 block; output
    // (row, q') to [b][row][r] of the q' < Q or the q' >= Q half
    const int rows = fwdA ? gr.M : gr.N;
    const int kr = a.vs_rank, Q = a.vs_half;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = m0 + wm0 + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
          const int q2 = n0 + wn0 + j * 32 + (lane & 31);
          if (row >= rows || q2 >= 2 * Q) continue;
          const int q = q2 < Q ? q2 : q2 - Q;
          const int b = q / kr, rr = q - b * kr;
          (q2 < Q ? a.vs_lo : a.vs_hi)[((int64_t)b * rows + row) * kr + rr] = acc[i][j][r];
        }
    return;
  }

  // ---- epilogue ------------------------------------------------------------
  // accumulator register r of lane l holds row (r/4)*8 + (l/32)*4 + r%4 and
  // column l%32 of its 32 x 32 block.  The tile goes through LDS (free once
  // every load has landed and every wave is past its last fragment read) in
  // passes of WM*32 rows, one row block of every wave row at a time, so that
  // the loads and stores of node values, flows and parameters are 16-byte
  // runs along a row; per-column shifts and per-row child nodes are staged
  // beside it.
  constexpr int LDT = NT + 8;                  // row pitch: the two half-waves' rows 4 apart hit other banks
  constexpr int PR = WM * 32;                  // rows per pass
  constexpr int NCH = PR * NT / 4 / 256;       // 4-column chunks per thread per pass
  constexpr int TPC = 256 / (NT / 4);          // threads sharing a 4-column chunk (product-epilogue maxima)
  static_assert(PR * NT % 1024 == 0, "whole chunks per thread");
  static_assert((PR * LDT + NT + MT + TPC * NT) * 4 <= RING_EL * 2, "epilogue tile fits the ring");
  const int B = a.B;
  float* tl = (float*)ring;                    // [PR][LDT]
  float* sh_col = tl + PR * LDT;               // [NT]
  int* ch_row = (int*)(sh_col + NT);           // [MT]
  float* red = (float*)(ch_row + MT);          // [TPC][NT]
  // product epilogue: this thread's running column maxima (its 4 columns are
  // the same in every chunk: (tid % (NT/4)) * 4)
  const bool ep = EPI == EPI_FWD && a.ep_on;
  // element-flow product epilogue packing the next layer's G (needs a whole
  // tile of samples: the batch is a multiple of 256)
  const bool gp = EPI == EPI_ELEM && a.gp_on;
  float pm[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
  __syncthreads();
  if (EPI == EPI_FWD || EPI == EPI_ELEM) {
    for (int t = tid; t < NT; t += 256) {
      const int col = n0 + t;
      sh_col[t] = col < B ? key_to_shift(a.mkeys[(int64_t)gr.m_row * B + col]) : 0.0f;
    }
    if (EPI == EPI_ELEM)
      for (int t = tid; t < MT; t += 256) {
        const int row = m0 + t;
        ch_row[t] = row < gr.N ? a.chblocks[gr.blk_off + row / gr.cbs] + row % gr.cbs : -1;
      }
  }
  const int wr = wave / WN;
  const bool to_scratch = EPI == EPI_ELEM && gr.scratch_row >= 0;
  const bool add = EPI == EPI_ELEM && !to_scratch && !a.store;
  float* dst_base = to_scratch ? a.scratch + (int64_t)gr.scratch_row * B : a.flows;
  const int ncol = EPI == EPI_PARAM ? bl.N : B;
  const bool vec = EPI == EPI_PARAM ? ((bl.param_offset | (int64_t)bl.N) & 3) == 0 : (B & 3) == 0;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    // write row block i of every wave into the pass tile
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int lr = wr * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        tl[lr * LDT + wn0 + j * 32 + (lane & 31)] = acc[i][j][r];
      }
    __syncthreads();
    // chunk q = tid + 256 c: pass row q / (NT/4), columns 4 (q % (NT/4)) + 0..3
    int trow[NCH], c4[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int q = tid + 256 * c, lr = q / (NT / 4);
      trow[c] = (lr >> 5) * WTM + i * 32 + (lr & 31);
      c4[c] = (q % (NT / 4)) * 4;
    }
    // every load of the pass in flight before the first store
    float x[NCH][4], old[NCH][4], sv[NCH][4];
    int64_t at[NCH];
    int32_t pi[NCH];                           // product node of the row (product epilogue), -1 if none
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int row = m0 + trow[c], col = n0 + c4[c];
      bool ok;
      if (EPI == EPI_FWD) {
        ok = row < gr.M;
        at[c] = (int64_t)row * B + col;
        pi[c] = -1;
        if (ep && ok) {
          const int i = gr.out_start + row - a.ep_base_s;
          if (i >= 0 && i < a.ep_pcount) {
            pi[c] = i;
            // the product node's other child
            const float* src = a.vals + (int64_t)(a.ep_base_o + i) * B + col;
            if (vec && col + 3 < B) {
              const float4 t = *(const float4*)src;
              x[c][0] = t.x; x[c][1] = t.y; x[c][2] = t.z; x[c][3] = t.w;
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e) x[c][e] = col + e < B ? src[e] : 0.0f;
            }
          }
        }
      } else if (EPI == EPI_ELEM) {
        const int child = ch_row[trow[c]];
        ok = child >= 0;
        at[c] = to_scratch ? (int64_t)row * B + col : (int64_t)child * B + col;
        const float* src = a.vals + (int64_t)(ok ? child : 0) * B + col;
        if (ok && vec && col + 3 < B) {
          const float4 t = *(const float4*)src;
          x[c][0] = t.x; x[c][1] = t.y; x[c][2] = t.z; x[c][3] = t.w;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) x[c][e] = (ok && col + e < B) ? src[e] : 0.0f;
        }
        if (gp && ok) {
          // scaled sums of the packed layer's node `row` (the batch is a
          // multiple of 64: a 4-column chunk is all samples or all padding)
          if (col < B) {
            const float4 t = *(const float4*)(a.ssum + (a.gp_s_row + row) * B + col);
            sv[c][0] = t.x; sv[c][1] = t.y; sv[c][2] = t.z; sv[c][3] = t.w;
          } else {
            sv[c][0] = sv[c][1] = sv[c][2] = sv[c][3] = 0.0f;
          }
        }
      } else if (!a.params) {
        // no weights: F += P (the LowRank denominator statistic W)
        ok = row < bl.M;
        at[c] = (int64_t)row * bl.N + col;
#pragma unroll
        for (int e = 0; e < 4; ++e) x[c][e] = 1.0f;
      } else {
        ok = row < bl.M;
        at[c] = (int64_t)row * bl.N + col;
        const float* src = a.params + bl.param_offset + (ok ? at[c] : 0);
        if (ok && vec && col + 3 < bl.N) {
          const float4 t = *(const float4*)src;
          x[c][0] = t.x; x[c][1] = t.y; x[c][2] = t.z; x[c][3] = t.w;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) x[c][e] = (ok && col + e < bl.N) ? src[e] : 0.0f;
        }
      }
      if (!ok) at[c] = -1;
      const bool rd_old = EPI == EPI_PARAM || add;
      if (rd_old) {
        const float* src = (EPI == EPI_PARAM ? a.pflows + bl.param_offset : dst_base) + (ok ? at[c] : 0);
        if (ok && vec && col + 3 < ncol) {
          const float4 t = *(const float4*)src;
          old[c][0] = t.x; old[c][1] = t.y; old[c][2] = t.z; old[c][3] = t.w;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) old[c][e] = (ok && col + e < ncol) ? src[e] : 0.0f;
        }
      }
    }
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      if (at[c] < 0) continue;
      const int col = n0 + c4[c];
      float* pv = tl + (trow[c] - (trow[c] / WTM) * WTM - i * 32 + (trow[c] / WTM) * 32) * LDT + c4[c];
      const float4 pt = *(const float4*)pv;
      const float acc4[4] = {pt.x, pt.y, pt.z, pt.w};
      float o[4], o2[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (EPI == EPI_FWD) {
          o[e] = sh_col[c4[c] + e] + logf(acc4[e]);
          o2[e] = acc4[e];
        } else if (EPI == EPI_ELEM) {
          const float ex = expf(x[c][e] - sh_col[c4[c] + e]);
          const float cc = (ex == 0.0f) ? 0.0f : ex * acc4[e];
          o[e] = add ? old[c][e] + cc : cc;
        } else {
          o[e] = old[c][e] + x[c][e] * acc4[e];
        }
      }
      float* d0 = EPI == EPI_FWD ? a.vals + (int64_t)gr.out_start * B + at[c]
                : EPI == EPI_ELEM ? dst_base + at[c] : a.pflows + bl.param_offset + at[c];
      if (vec && col + 3 < ncol) {
        *(float4*)d0 = make_float4(o[0], o[1], o[2], o[3]);
        if (EPI == EPI_FWD && a.ssum) *(float4*)(a.ssum + gr.s_row * B + at[c]) = make_float4(o2[0], o2[1], o2[2], o2[3]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (col + e < ncol) {
            d0[e] = o[e];
            if (EPI == EPI_FWD && a.ssum) a.ssum[gr.s_row * B + at[c] + e] = o2[e];
          }
      }
      if (EPI == EPI_ELEM && gp) {
        // the product node's flow (this output) to both its children, and
        // g = f / S of the packed layer's node into its node-major G rows;
        // g goes back into this chunk's tile slot for the batch-major G
        const int row = m0 + trow[c];
        float f[4], gq[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          f[e] = 0.0f + o[e];
          gq[e] = (f[e] == 0.0f || !(sv[c][e] > 0.0f)) ? 0.0f : f[e] / sv[c][e];
        }
        if (col < B) {                         // padded samples: zeros in the batch-major G only
          const float4 f4 = make_float4(f[0], f[1], f[2], f[3]);
          *(float4*)(a.flows + (int64_t)(a.gp_out_start + row) * B + col) = f4;
          *(float4*)(a.flows + (int64_t)(a.gp_other + row) * B + col) = f4;
          split_planes<4>(gq, a.gp_np_direct, a.gp_direct + panel(a.gp_g_row + row, col, a.gp_direct_rows),
                          a.gp_direct_plane);
        }
        *(float4*)pv = make_float4(gq[0], gq[1], gq[2], gq[3]);
      }
      if (EPI == EPI_FWD && ep && pi[c] >= 0) {
        // product node = its children added in child order, as the product kernel does
        float pv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pv[e] = a.ep_qs == 0 ? (0.0f + o[e]) + x[c][e] : (0.0f + x[c][e]) + o[e];
          if (col + e < B) pm[e] = fmaxf(pm[e], pv[e]);
        }
        float* dp = a.vals + (int64_t)(a.ep_pstart + pi[c]) * B + col;
        if (vec && col + 3 < B) {
          *(float4*)dp = make_float4(pv[0], pv[1], pv[2], pv[3]);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (col + e < B) dp[e] = pv[e];
        }
      }
    }
    if (EPI == EPI_ELEM && gp) {
      // batch-major G: item = (sample, 8 consecutive rows of one 32-row run)
      __syncthreads();
      for (int it = tid; it < PR * NT / 8; it += 256) {
        const int bl = it % NT, lr0 = (it / NT) * 8;
        const int row = m0 + (lr0 >> 5) * WTM + i * 32 + (lr0 & 31);
        if (row >= gr.N) continue;
        float y[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = tl[(lr0 + e) * LDT + bl];
        split_planes<8>(y, a.gp_np_trans, a.gp_trans + panel(n0 + bl, a.gp_g_koff + row, a.B_pad), a.gp_trans_plane);
      }
    }
    if (i + 1 < FM) __syncthreads();           // the pass tile is rewritten next
  }
  if (EPI == EPI_FWD && ep) {
    // column maxima of the tile's product nodes: the TPC threads of each
    // 4-column chunk through LDS, then one integer atomic max per column
    const int c4 = (tid % (NT / 4)) * 4;
#pragma unroll
    for (int e = 0; e < 4; ++e) red[(tid / (NT / 4)) * NT + c4 + e] = pm[e];
    __syncthreads();
    for (int t = tid; t < NT; t += 256) {
      float m = red[t];
#pragma unroll
      for (int k = 1; k < TPC; ++k) m = fmaxf(m, red[k * NT + t]);
      if (n0 + t < B) atomicMax(a.mkeys_out + (int64_t)a.ep_mrow * B + n0 + t, float_to_key(m));
    }
  }
}

template <int EPI, int PA, int PB, int MT, int NT, int WM>
static void launch_shape(int grid, const GemmArgs& a, hipStream_t s) {
  constexpr int KT = gemm_kt(PA, PB, MT, NT);
  constexpr int NS = EPI == EPI_PARAM ? gemm_stages(PA, PB, MT, NT) : gemm_stages_direct(PA, PB, MT, NT, MT / WM / 32);
  static_assert(NS >= (EPI == EPI_PARAM ? 2 : 3), "LDS ring stages");
  launch_kernel((k_gemm<EPI, PA, PB, MT, NT, WM, KT, NS>), dim3(grid), dim3(256), 0, s, a);
}

template <int EPI, int PA, int PB>
static void launch_tile(int tile, int grid, const GemmArgs& a, hipStream_t s) {
  if constexpr (EPI == EPI_PARAM) {
    if constexpr (PA + PB <= 3) {
      if (tile == TILE_256x256) {
        launch_shape<EPI, PA, PB, 256, 256, 2>(grid, a, s);
        return;
      }
    }
    if (tile == TILE_128x256) launch_shape<EPI, PA, PB, 128, 256, 2>(grid, a, s);
    else launch_shape<EPI, PA, PB, 128, 128, 2>(grid, a, s);
  } else {
    // the weights go to registers: 128 x 64 and 256 x 128 with the waves
    // stacked along M, each loading only its own rows; 64 x 128, 128 x 128
    // and 128 x 256 with 2 x 2 waves, two waves loading each row block (four
    // 32 x 128 waves on 128 x 128 tiles gave wrong sums in three accumulator
    // registers with fewer than three planes per operand, cause not found)
    if (tile == TILE_256x128) launch_shape<EPI, PA, PB, 256, 128, 4>(grid, a, s);
    else if (tile == TILE_128x256) launch_shape<EPI, PA, PB, 128, 256, 2>(grid, a, s);
    else if (tile == TILE_128x64) launch_shape<EPI, PA, PB, 128, 64, 4>(grid, a, s);
    else if (tile == TILE_64x128) launch_shape<EPI, PA, PB, 64, 128, 2>(grid, a, s);
    else launch_shape<EPI, PA, PB, 128, 128, 2>(grid, a, s);
  }
}

// virtual-batch stores: the automatic per-layer tiles only
template <int PA, int PB>
static void launch_vstore(int tile, int grid, const GemmArgs& a, hipStream_t s) {
  if (tile == TILE_64x128) launch_shape<EPI_VSTORE, PA, PB, 64, 128, 2>(grid, a, s);
  else launch_shape<EPI_VSTORE, PA, PB, 128, 64, 4>(grid, a, s);
}

template <int EPI>
static void launch_planes(int pa, int pb, int tile, int grid, const GemmArgs& a, hipStream_t s) {
  if constexpr (EPI == EPI_VSTORE) {
    if (pa == 1 && pb == 1) launch_vstore<1, 1>(tile, grid, a, s);
    else if (pa == 2 && pb == 1) launch_vstore<2, 1>(tile, grid, a, s);
    else if (pa == 1 && pb == 2) launch_vstore<1, 2>(tile, grid, a, s);
    else if (pa == 2 && pb == 2) launch_vstore<2, 2>(tile, grid, a, s);
    else launch_vstore<3, 3>(tile, grid, a, s);
    return;
  }
  if (pa == 1 && pb == 1) launch_tile<EPI, 1, 1>(tile, grid, a, s);
  else if (pa == 2 && pb == 1) launch_tile<EPI, 2, 1>(tile, grid, a, s);
  else if (pa == 1 && pb == 2) launch_tile<EPI, 1, 2>(tile, grid, a, s);
  else if (pa == 2 && pb == 2) launch_tile<EPI, 2, 2>(tile, grid, a, s);
  else launch_tile<EPI, 3, 3>(tile, grid, a, s);
}

void launch_gemm(int epi, int pa, int pb, const GemmShape& sh, const GemmArgs& a, hipStream_t s) {
  if (sh.tiles <= 0) return;
  const int grid = sh.tiles * sh.splitk;
  if (epi == EPI_FWD) launch_planes<EPI_FWD>(pa, pb, sh.tile, grid, a, s);
  else if (epi == EPI_ELEM) launch_planes<EPI_ELEM>(pa, pb, sh.tile, grid, a, s);
  else if (epi == EPI_VSTORE) launch_planes<EPI_VSTORE>(pa, pb, sh.tile, grid, a, s);
  else launch_planes<EPI_PARAM>(pa, pb, sh.tile, grid, a, s);
}

}  // namespace pc
