// launch.hpp -- internal interface between the C ABI (abi.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>

#include "device_common.hpp"

namespace attn {

// STAGE_STATS_DQ: row statistics and dQ in one pass (bf16 only).
enum { STAGE_ROW_STATS = 0, STAGE_KV = 1, STAGE_DQ = 2, STAGE_STATS_DQ = 3 };

// Launches one dense stage over `nblocks` workgroups of 256 threads.
hipError_t launch_dense_stage(int stage, bool bf16_in, int D, int mode, const DenseParams &p,
                              int nblocks, hipStream_t stream);

}  // namespace attn
