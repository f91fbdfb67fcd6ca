// pc_kernels.h -- launchers of the gfx950 kernels (host side).
#pragma once
#include <hip/hip_runtime.h>

#include "pc_device.h"

namespace pc {

enum Epi { EPI_FWD = 0, EPI_ELEM = 1, EPI_PARAM = 2 };

// Arguments of the MFMA product kernel (see k_gemm.hip).
struct GemmArgs {
  int32_t B, B_pad, B_padK;
  int32_t ntiles;               // tiles along the batch (forward / element flows)
  int32_t ngroups;              // groups of the layer, or blocks (parameter flows)
  const GroupRec* groups;
  const BlockRec* blocks;
  const CopyRec* copies;
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
};

// Launch the product kernel for `tiles` tiles with the given operand split.
void launch_gemm(int epi, int pa, int pb, int tiles, const GemmArgs& a, hipStream_t s);

}  // namespace pc
