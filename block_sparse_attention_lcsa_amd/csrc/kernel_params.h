// Kernel argument blocks of liblcsa (host and device).
#pragma once

#include <cstdint>

namespace lcsa {

constexpr int kMaxKvFrames = 64;

// Geometry of the token grid and its blocks, shared by every kernel.
struct GridGeom {
  int32_t heads;
  int32_t grid_h, grid_w;
  int32_t block_h, block_w, log2_bw;  // block_w is a power of two
  int32_t nbh, nbw, nbf;              // block rows / columns / blocks per frame
  int32_t nqb, nkb;                   // query / key blocks
  int32_t q_frames, kv_frames;
  int32_t half;                       // window half-width in blocks
  int32_t k;                          // kept-block budget
  int64_t q_tokens;
  // Division by nbf and nbw as a multiply and shift (exact for n < 2^31):
  // n / d == (n * m) >> s with a 64-bit product.
  uint32_t nbf_m, nbf_s, nbw_m, nbw_s;
  // Frame of the K/V storage holding KV-window frame t (the identity for a
  // contiguous window, ring slots otherwise).
  int32_t kv_slot[kMaxKvFrames];
};

struct View {
  const uint16_t* data;  // bf16 bits
  int64_t sb, ss, sh;    // strides in elements
};

struct OutView {
  uint16_t* data;        // bf16 bits
  int64_t sb, ss, sh;    // strides in elements
};

// Factored 3D rotary embedding: channel pair j < pt turns by table_t of the
// token's KV-window frame, pt <= j < pt + ph by table_h of its token row, the
// rest by table_w of its column; tables hold (cos, sin) float pairs.
struct RopeParams {
  const float* table_t;  // [kv_frames][pt][2]
  const float* table_h;  // [grid_h][ph][2]
  const float* table_w;  // [grid_w][64 - pt - ph][2]
  int32_t pt, ph;
  OutView q_rot, k_rot;  // rotated Q and K (bf16), written by the pool kernel
};

// Pooled K lives per storage frame, in groups of 8 positions:
// kcache[slot][B*H][NBF / 8 rounded up][64][8][2] holds channel 2c + e of
// position p at [p / 8][c][p % 8][e].
struct PoolParams {
  GridGeom g;
  View q, k;
  double* qbar;          // [B][H][NQB][128]
  double* kcache;        // [slots][B*H][ceil(NBF / 8)][64][8][2]
  int32_t k_first;       // first KV-window frame whose K blocks are pooled
  RopeParams rope;       // used by the rotary variant of the pool kernel only
};

struct SelectParams {
  GridGeom g;
  const double* qbar;    // [B][H][NQB][128]
  const double* kcache;  // [slots][B*H][ceil(NBF / 8)][64][8][2]
  int32_t batch;
  int32_t* row_ptr;
  int32_t* col_idx;
  double* scores;        // optional [B][H][NQB][NKB]
  // Top-k selection (tau == nullptr): optional [rows] output, each row's
  // keep-th largest window score.  Threshold selection (tau set): row r
  // keeps the window blocks scored >= tau[r], written to col_idx entries
  // [r * pad, (r + 1) * pad) in ascending order, then -1 to the row's end.
  double* kth;
  const double* tau;
  int32_t pad;
};

struct AttendParams {
  GridGeom g;
  View q, k, v;
  uint16_t* o;
  int64_t o_sb, o_ss, o_sh;
  float* lse;            // optional [B][H][q_tokens]
  const int32_t* row_ptr;
  const int32_t* col_idx;
  int64_t nnz;
  int64_t rows;          // CSR rows
  // Rows [0, full_rows) run as one workgroup each; every later row is split
  // into `pieces` parts of its CSR range, each a workgroup that writes its
  // unnormalised partial result to `part` for the merge kernel.
  int64_t full_rows;
  int32_t pieces;
  // Visiting order of the rows: enumeration index e runs over (batch*head,
  // tile of tile x tile block positions, query frame, position in the tile);
  // work items above are enumeration indices.
  int32_t tile;
  // Rows per XCD chunk of the whole-row workgroups (>= 1): one XCD's
  // resident workgroups.
  int32_t xcd_chunk;
  float* part;           // [items][BT][128] partial O, then [items][BT][2] (m, l)
  float scale_log2;      // softmax scale * log2(e)
  // Optional order of the rows (a permutation of [0, rows)): workgroup i
  // takes row order[i] instead of the visiting order above (the split rows
  // are order[full_rows ..]).  NULL: the visiting order.
  const int32_t* order;
};

}  // namespace lcsa
