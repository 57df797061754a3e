// Host launchers of the liblcsa kernels.  Each returns the HIP status of the
// launch; arguments were validated by the entry points in entry.hip.
#pragma once

#include <hip/hip_runtime.h>

#include "kernel_params.h"

namespace lcsa {

hipError_t launch_pool(const PoolParams& p, int batch, int block_tokens, hipStream_t stream);
hipError_t launch_select(const SelectParams& p, int batch, int max_window, hipStream_t stream);
hipError_t launch_attend(const AttendParams& p, int block_tokens, hipStream_t stream);

// Bytes of one split piece's partial result (O in float32, then m and l).
inline int64_t attend_piece_bytes(int block_tokens) {
  return static_cast<int64_t>(block_tokens) * (128 + 2) * 4;
}
// Workgroups of the attention kernel resident on one CU (eight waves).
inline int attend_groups_per_cu(int block_tokens) { return 8 / (block_tokens / 32); }

}  // namespace lcsa
