// Private declarations shared by the host plan and the HIP entry points of
// liblcsa.  Not installed; the public interface is include/lcsa.h.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "lcsa.h"

struct lcsa_plan_s {
  lcsa_desc desc;
  lcsa_plan_info info;
  std::vector<int32_t> row_ptr;      // rows + 1
  std::vector<int32_t> frame_count;  // per spatial block position: min(k, |window|)
};

namespace lcsa {

// Largest window (eligible key blocks of one query block) the select kernel
// holds in LDS.
constexpr int kMaxWindow = 1024;
constexpr int kHeadDim = 128;
// Compute units of the largest gfx950 device (MI355X, MI350X); sizes the
// attention workspace for split rows.
constexpr uint64_t kMaxCus = 256;
// Memory-side cache (Infinity Cache) of an MI355X: data a pass streams once
// that is larger than this cannot stay there for the next kernel anyway.
constexpr uint64_t kMemorySideCacheBytes = 256ull << 20;
// Bytes of the attention workspace's split-piece area: one device-wide round
// of pieces (8 waves per CU) of BT x (128 + 2) float32 each.  The row lengths
// and row order of lcsa_attend_varlen follow it.
inline uint64_t attend_pieces_bytes(int block_tokens) {
  const uint64_t bt = static_cast<uint64_t>(block_tokens);
  return kMaxCus * (8 / (bt / 32)) * bt * (128 + 2) * 4;
}

// Record a formatted error for lcsa_last_error() and return the status.
lcsa_status fail(lcsa_status st, const char* fmt, ...);
void clear_error();

// Spatial window bounds of block position (by, bx): inclusive ranges.
inline void window_bounds(const lcsa_plan_info& in, int by, int bx, int* y0, int* y1, int* x0,
                          int* x1) {
  const int r = in.half_window;
  *y0 = by - r < 0 ? 0 : by - r;
  *y1 = by + r > in.nbh - 1 ? in.nbh - 1 : by + r;
  *x0 = bx - r < 0 ? 0 : bx - r;
  *x1 = bx + r > in.nbw - 1 ? in.nbw - 1 : bx + r;
}

}  // namespace lcsa
