// k_f8gemm.hip -- the LowRank "sum_exp" parameter flows from e4m3 operands
// (pyjuice.parameterizations.LowRank, Parameters: flow_precision "fp8", the
// opt-in for the two products at the end of the pass, the parameter flows
// theta * (Y1 X^T) and the denominator statistic Y2 C^T over every (copy,
// sample, rank), with a power-of-two scale per row and fp32 accumulation).
//
// Operands (written by the virtual-batch pack kernels): node-major rows
// (nodes or children of each tied copy), K = the copy's virtual columns q,
// e4m3 bytes in K-blocked panels -- byte (r, k) of an operand with R rows at
// ((k / 64) * R + r) * 64 + k % 64, so a 64-wide K step of 128 consecutive
// rows is one contiguous 8 KB run -- and one E8M0 scale byte per row and 32
// consecutive k at (k / 32) * R + r (the value is byte * 2^(scale - 127)).
// The scale is finer than one per row: gfx950's scaled matrix instruction
// takes one per lane, i.e. per row and 32-wide K half of each instruction.
//
// Workgroup: a 128 x 128 output tile, 4 waves of 64 x 64 (2 x 2 blocks of
// v_mfma_scale_f32_32x32x64_f8f6f4), the K steps of its split of the
// contraction streamed through a ring of LDS stages filled by direct
// global->LDS loads several steps ahead.  Lane l of an instruction holds row l % 32 and, with h = l / 32,
// the 16-byte chunks h and 2 + h of the 64-byte step (A and B alike); the
// scale that lane l passes applies to its row's K half h, i.e. bytes
// [32 h, 32 h + 32) = chunks 2h and 2h + 1, which the two lanes of the row
// hold between them (measured on gfx950: bytes 0..15 of both lanes take the
// first lane's scale, bytes 16..31 the second's).  Split-K partials are added
// by the last arriving workgroup in split order (deterministic), as in the
// bf16 product kernel.
#include <hip/hip_runtime.h>

#include "pc_kernels.h"
#include "pc_ring.h"

namespace pc {

namespace {

typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int F8T = 128;            // tile rows and columns
constexpr int F8_STAGE = 2 * F8T * 64 + 4 * F8T;   // A, B bytes + 4 scale runs of 128
constexpr int F8_NS = 4;            // ring stages
constexpr int F8_PW = 5;            // loads per wave per stage

__device__ __forceinline__ int f8_remap(int bid, int n) {   // consecutive tiles on one XCD
  const int q = n >> 3, r = n & 7;
  const int x = bid & 7, local = bid >> 3;
  return x * q + (x < r ? x : r) + local;
}

// 16-byte chunk slot of chunk c in a 64-byte LDS row: 8 consecutive rows'
// reads of one chunk land on 8 distinct 4-bank groups
__device__ __forceinline__ int f8_swz(int row) { return ((row >> 1) ^ (row >> 2)) & 3; }

}  // namespace

__global__ __launch_bounds__(256, 2) void k_f8param(F8Args a) {
  __shared__ __attribute__((aligned(1024))) uint8_t ring[F8_NS * F8_STAGE];
  __shared__ int last_flag;
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, h = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
  const int S = a.splitk;
  const int logical = f8_remap(blockIdx.x, gridDim.x);
  // the splits of the launch's tiles in split-major order: the workgroups an
  // XCD runs at once take neighbouring tiles over the same K range, sharing
  // the operand rows of that range in its L2
  const int ntiles = gridDim.x / S;
  const int split = logical / ntiles, tile = logical - split * ntiles;

  // block and tile position
  int bi = 0;
  {
    int lo = 0, hi = a.nblocks - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (a.blocks[mid].pt128 <= tile) lo = mid; else hi = mid - 1;
    }
    bi = lo;
  }
  const BlockRec bl = a.blocks[bi];
  const int64_t Mp = (bl.M + ROW_PAD - 1) / ROW_PAD * ROW_PAD, Np = (bl.N + ROW_PAD - 1) / ROW_PAD * ROW_PAD;
  const int ntn = (int)(Np / F8T);
  const int lt = tile - bl.pt128;
  const int m0 = (lt / ntn) * F8T, n0 = (lt % ntn) * F8T;
  if (m0 >= bl.M || n0 >= bl.N) return;       // wholly in the block's padding (every split leaves)
  const int kpc = a.QK / 64;                  // K steps per copy
  const int tot = bl.ncopies * kpc;
  const int kbeg = (int)((int64_t)split * tot / S), kend = (int)((int64_t)(split + 1) * tot / S);
  const int n = kend - kbeg;

  // Ring of F8_NS stages, one 64-wide K step each: A rows [0, 128) x 64 bytes,
  // B rows likewise, then the four scale runs (A half 0, A half 1, B half 0,
  // B half 1; 128 bytes each).  Wave w fills, per stage, A load instructions
  // 2w and 2w + 1, B ones likewise (1 KB each: 16 rows) and scale run w
  // (lanes 0..31, 4 bytes each): F8_PW loads per wave per stage.  LDS slot s
  // of an operand's 8 KB holds the global 16-byte chunk of row s / 4 whose
  // index is (s % 4) ^ swz(row) (the swizzle is an involution).
  uint32_t voff[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int slot = (2 * wave + u) * 64 + lane, row = slot >> 2;
    voff[u] = (uint32_t)((row * 4 + ((slot & 3) ^ f8_swz(row))) * 16);
  }
  const uint32_t ring_lds = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)ring;
  const bool sc_op_a = wave < 2;
  const int sc_half = wave & 1;
  const int64_t sc_rows = sc_op_a ? a.rowsA : a.rowsB;
  const uint8_t* sc_base = sc_op_a ? a.sA : a.sB;
  int next = 0;                               // next step (relative to kbeg) whose loads are issued
  auto issue = [&](int slot) {
    // past the last step the ring re-loads it into stages never read, so
    // every wait stays a constant
    const int t = kbeg + (next < n ? next : n - 1);
    ++next;
    const int s = t / kpc, kb = t - s * kpc;
    const int64_t ra = bl.g_base + (int64_t)s * Mp + m0, rb = bl.e_base + (int64_t)s * Np + n0;
    const uint8_t* A = a.A + ((int64_t)kb * a.rowsA + ra) * 64;
    const uint8_t* B = a.B + ((int64_t)kb * a.rowsB + rb) * 64;
    const uint32_t st = ring_lds + slot * F8_STAGE;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      lds_load16(A, voff[u], st + (2 * wave + u) * 1024);
      lds_load16(B, voff[u], st + F8T * 64 + (2 * wave + u) * 1024);
    }
    const uint8_t* sc = sc_base + ((int64_t)(2 * kb + sc_half) * sc_rows + (sc_op_a ? ra : rb));
    if (lane < 32) lds_load4(sc, (uint32_t)lane * 4, st + 2 * F8T * 64 + wave * F8T);
  };

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  if (n > 0) {
    // prologue: steps 0 .. NS-2 in flight; step 0 readable
#pragma unroll
    for (int q = 0; q < F8_NS - 1; ++q) issue(q);
    __builtin_amdgcn_s_waitcnt(WaitVmLgkm<(F8_NS - 2) * F8_PW>::imm);
    ring_barrier();
    int j = 0;
    for (int it = 0; it < n; ++it) {
      // refill the stage read in the previous step with step it + NS - 1
      issue(j == 0 ? F8_NS - 1 : j - 1);
      const uint8_t* st = ring + j * F8_STAGE;
      i32x8_t fa[2], fb[2];
      int sa[2], sb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int row = wm + i * 32 + l32;
        const uint4 x0 = *(const uint4*)(st + row * 64 + ((h ^ f8_swz(row)) << 4));
        const uint4 x1 = *(const uint4*)(st + row * 64 + (((2 + h) ^ f8_swz(row)) << 4));
        fa[i] = i32x8_t{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
        sa[i] = st[2 * F8T * 64 + h * F8T + row];
      }
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const int row = wn + jj * 32 + l32;
        const uint4 x0 = *(const uint4*)(st + F8T * 64 + row * 64 + ((h ^ f8_swz(row)) << 4));
        const uint4 x1 = *(const uint4*)(st + F8T * 64 + row * 64 + (((2 + h) ^ f8_swz(row)) << 4));
        fb[jj] = i32x8_t{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
        sb[jj] = st[2 * F8T * 64 + (2 + h) * F8T + row];
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
          acc[i][jj] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[i], fb[jj], acc[i][jj], 0, 0, 0, sa[i], 0,
                                                                       sb[jj]);
      // step it + 1 has landed once at most the NS-2 steps issued after it
      // are in flight; the barrier also ends every wave's reads of stage j
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(WaitVmLgkm<(F8_NS - 2) * F8_PW>::imm);
      ring_barrier();
      j = j + 1 == F8_NS ? 0 : j + 1;
    }
  }
  __builtin_amdgcn_s_waitcnt(0);       // no load may still target LDS past this point

  // ---- split-K: the last arriving workgroup adds the partials in order ------
  // (atomic stores and loads at device scope; the arrival increment is a
  // device-scope acquire-release, the barriers order every lane's partials
  // before it and the last arrival's loads after it)
  if (S > 1) {
    float* mine = a.partials + ((int64_t)tile * S + split) * (64 * 256);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          __hip_atomic_store(mine + ((i * 2 + j) * 16 + r) * 256 + tid, acc[i][j][r], __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0)
      last_flag = (__hip_atomic_fetch_add(a.counters + tile, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT) ==
                   (unsigned)(S - 1));
    __syncthreads();
    if (!last_flag) return;
    const float* base = a.partials + (int64_t)tile * S * (64 * 256);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int reg = (i * 2 + j) * 16 + r;
          float v = __hip_atomic_load(base + reg * 256 + tid, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          for (int q = 1; q < S; ++q)
            v += __hip_atomic_load(base + ((int64_t)q * 64 + reg) * 256 + tid, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
          acc[i][j][r] = v;
        }
    if (tid == 0) __hip_atomic_store(a.counters + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  // ---- epilogue: out[i, j] += (theta[i, j] or 1) * product -------------------
  // accumulator register r of block (i, j): row 8 (r / 4) + 4 h + r % 4,
  // column l32 of the 32 x 32 block
  float* out = a.out + bl.param_offset;
  const float* th = a.params ? a.params + bl.param_offset : nullptr;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = n0 + wn + j * 32 + l32;
      if (col >= bl.N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm + i * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
        if (row < bl.M) {
          const int64_t o = (int64_t)row * bl.N + col;
          out[o] += (th ? th[o] : 1.0f) * acc[i][j][r];
        }
      }
    }
}

void launch_f8param(const F8Args& a, int tiles, hipStream_t s) {
  if (tiles <= 0) return;
  launch_kernel(k_f8param, dim3(tiles * a.splitk), dim3(256), 0, s, a);
}

}  // namespace pc
