// Host launchers of the liblcsa kernels.  Each returns the HIP status of the
// launch; arguments were validated by the entry points in entry.hip.
#pragma once

#include <hip/hip_runtime.h>

#include "kernel_params.h"

namespace lcsa {

hipError_t launch_pool(const PoolParams& p, int batch, int block_tokens, hipStream_t stream);
hipError_t launch_select(const SelectParams& p, int batch, int max_window, hipStream_t stream);
hipError_t launch_attend(const AttendParams& p, int block_tokens, hipStream_t stream);

}  // namespace lcsa
