// Host launchers of the liblcsa kernels.  Each returns the HIP status of the
// launch; arguments were validated by the entry points in entry.hip.
#pragma once

#include <hip/hip_runtime.h>

#include <cmath>

#include "kernel_params.h"

namespace lcsa {

hipError_t launch_pool(const PoolParams& p, int batch, int block_tokens, bool rope,
                       hipStream_t stream);
hipError_t launch_select(const SelectParams& p, int batch, int max_window, hipStream_t stream);
hipError_t launch_attend(const AttendParams& p, int block_tokens, hipStream_t stream);
// Longest-first order of the CSR rows of p (p.row_ptr, p.col_idx, p.nnz,
// p.rows, p.g, p.tile) into order[rows], with len[rows] as scratch.
hipError_t launch_row_order(const AttendParams& p, int32_t* len, int32_t* order,
                            hipStream_t stream);

// Bytes of one split piece's partial result (O in float32, then m and l).
inline int64_t attend_piece_bytes(int block_tokens) {
  return static_cast<int64_t>(block_tokens) * (128 + 2) * 4;
}
// Workgroups of the attention kernel resident on one CU (eight waves).
inline int attend_groups_per_cu(int block_tokens) { return 8 / (block_tokens / 32); }
// Side of the square position tiles of the attention visiting order: one
// tile with all its query frames is about one XCD's resident workgroups
// (slots / 8).  A side covering the frame gives plain row order.
inline int attend_tile(int64_t slots, int q_frames, int nbh, int nbw) {
  const double per_xcd = static_cast<double>(slots / 8);
  int t = static_cast<int>(std::sqrt(per_xcd / (q_frames > 0 ? q_frames : 1)) + 0.5);
  const int side = nbh > nbw ? nbh : nbw;
  t = t < 1 ? 1 : t;
  return t > side ? side : t;
}

}  // namespace lcsa
