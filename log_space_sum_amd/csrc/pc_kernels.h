// pc_kernels.h -- launchers of the gfx950 kernels (host side).
#pragma once
#include <hip/hip_runtime.h>

#include "pc_device.h"

namespace pc {

enum Epi { EPI_FWD = 0, EPI_ELEM = 1, EPI_PARAM = 2 };

// Arguments of the MFMA product kernel (see k_gemm.hip).
struct GemmArgs {
  int32_t B, B_pad, B_padK;
  int64_t rowsA, rowsB;        // panel rows of the kept operands (parameter flows)
  int32_t ntiles;               // tiles along the batch (forward / element flows)
  int32_t splitk;               // workgroups sharing one tile's K range (forward / element flows)
  int32_t ngroups;              // groups of the layer, or blocks (parameter flows)
  const GroupRec* groups;
  const BlockRec* blocks;
  const int32_t* chblocks;      // the layer's child-block starts
  const uint16_t* opA;
  int64_t planeA;
  const uint16_t* opB;
  int64_t planeB;
  int32_t ldb;                  // row stride of the batch-major operand (forward / element flows)
  float* vals;                  // node values (written by forward, read by element flows)
  float* flows;                 // node flows
  float* scratch;               // element-flow scratch of overlapping layers
  const uint32_t* mkeys;        // column-max keys
  float* ssum;                  // scaled sums kept by the forward
  int32_t store;                // element flows: store instead of add
  const float* params;
  float* pflows;
  float* partials;              // split-K partial tiles
  uint32_t* counters;           // split-K arrival counters, zero between launches
};

// Launch the product kernel for `tiles` tiles with the given operand split.
// `big`: parameter flows may use 256 x 256 tiles (every block at least that large).
void launch_gemm(int epi, int pa, int pb, int tiles, int big, const GemmArgs& a, hipStream_t s);

// K splits for a forward / element-flow launch of `tiles` 128 x 128 tiles
// with `ksteps` K slices: enough workgroups for the 256 CUs, >= 4 slices each.
inline int choose_split(int tiles, int ksteps) {
  int S = 1;
  while (tiles * S < 256 && S < 8 && ksteps / (S * 2) >= 4) S *= 2;
  return S;
}
// K slice width of a forward / element-flow launch for the given planes.
inline int gemm_kt(int pa, int pb) { return (pa + pb) <= 3 ? 64 : 32; }

}  // namespace pc
