// launch.hpp -- internal interface between the C ABI (abi.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>

#include "attn_bwd.h"
#include "device_common.hpp"

namespace attn {

// STAGE_STATS_DQ: row statistics and dQ in one pass (bf16 only).
enum { STAGE_ROW_STATS = 0, STAGE_KV = 1, STAGE_DQ = 2, STAGE_STATS_DQ = 3 };

// Launches one dense stage over `nblocks` workgroups of 256 threads.
hipError_t launch_dense_stage(int stage, bool bf16_in, int D, int mode, const DenseParams &p,
                              int nblocks, hipStream_t stream);

// The whole dense backward of attn_bwd (validation included), on the
// workspace the arguments name (abi.cpp).
int run_dense_all(const attn_bwd_args *a, void *stream);

// Records a message for attn_bwd_last_error() (abi.cpp).
void set_last_error(const char *msg);

}  // namespace attn
