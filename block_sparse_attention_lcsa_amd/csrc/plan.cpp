// Host-side plan of an LCSA layer call: validation, block geometry, KV window
// length, kept-block budget, window sizes and the CSR row pointer.  Touches no
// GPU.
//
// Geometry follows the streaming layout of the NxDI FlashVSR contrib page
// ("Description": first chunk of 6 latent frames, stream chunks of 2) and the
// controls of the FlashVSR Inference skill page ("Non-Negotiable Streaming
// Contract": kv_ratio, topk_ratio = sparse_ratio * 768 * 1280 / (H * W),
// local_range).  The budget k is topk_ratio times the blocks of one frame,
// rounded half up, which keeps the kept-block count per query block equal to
// sparse_ratio * 30 at every resolution.

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>

#include "lcsa_internal.h"

namespace lcsa {

static thread_local std::string g_last_error;

lcsa_status fail(lcsa_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

void clear_error() { g_last_error.clear(); }

const char* last_error() { return g_last_error.c_str(); }

// Integer nearest to x when within 1e-9 of it; otherwise ceil / round-half-up.
static int64_t snap_or(double x, bool ceil_mode) {
  const double n = std::nearbyint(x);
  if (std::fabs(x - n) < 1e-9) return static_cast<int64_t>(n);
  return static_cast<int64_t>(ceil_mode ? std::ceil(x) : std::floor(x + 0.5));
}

}  // namespace lcsa

using lcsa::fail;

extern "C" {

int32_t lcsa_abi_version(void) { return LCSA_ABI_VERSION; }

const char* lcsa_last_error(void) { return lcsa::last_error(); }

const char* lcsa_status_string(lcsa_status st) {
  switch (st) {
    case LCSA_OK: return "ok";
    case LCSA_ERR_NULL: return "null pointer";
    case LCSA_ERR_INVALID: return "invalid value";
    case LCSA_ERR_SHAPE: return "unsupported shape";
    case LCSA_ERR_ALIGN: return "misaligned data or stride";
    case LCSA_ERR_WORKSPACE: return "workspace or buffer too small";
    case LCSA_ERR_DEVICE: return "no gfx950 device";
    case LCSA_ERR_LAUNCH: return "kernel launch failed";
    case LCSA_ERR_INTERNAL: return "internal error";
    default: return "unknown status";
  }
}

lcsa_status lcsa_plan_create(const lcsa_desc* d, lcsa_plan_t* out) {
  lcsa::clear_error();
  if (!d || !out) return fail(LCSA_ERR_NULL, "lcsa_plan_create: desc and out must be non-NULL");
  *out = nullptr;
  if (d->batch <= 0 || d->heads <= 0)
    return fail(LCSA_ERR_INVALID, "batch (%d) and heads (%d) must be positive", d->batch, d->heads);
  if (d->head_dim != lcsa::kHeadDim)
    return fail(LCSA_ERR_INVALID, "head_dim must be 128 (got %d)", d->head_dim);
  if (d->grid_h <= 0 || d->grid_w <= 0)
    return fail(LCSA_ERR_INVALID, "grid %dx%d must be positive", d->grid_h, d->grid_w);
  if (d->q_frames <= 0 || d->cached_frames < 0)
    return fail(LCSA_ERR_INVALID, "q_frames (%d) must be > 0, cached_frames (%d) >= 0",
                d->q_frames, d->cached_frames);
  if (!(d->kv_ratio <= 0.0f || d->kv_ratio >= 1.0f) || std::isnan(d->kv_ratio))
    return fail(LCSA_ERR_INVALID, "kv_ratio %g: must be <= 0 (unbounded) or >= 1", d->kv_ratio);
  if (d->local_range < 1 || d->local_range % 2 == 0)
    return fail(LCSA_ERR_INVALID, "local_range %d must be odd and >= 1", d->local_range);
  if (d->topk < 0) return fail(LCSA_ERR_INVALID, "topk %d must be >= 0", d->topk);
  if (d->topk == 0 && !(d->topk_ratio > 0.0 && std::isfinite(d->topk_ratio)))
    return fail(LCSA_ERR_INVALID, "topk_ratio %g must be positive when topk is 0", d->topk_ratio);
  if (!(d->scale >= 0.0f) || std::isinf(d->scale))
    return fail(LCSA_ERR_INVALID, "scale %g must be finite and >= 0", d->scale);
  if (d->block_t != 0 && d->block_t != 1)
    return fail(LCSA_ERR_INVALID, "block_t %d: blocks span exactly one latent frame", d->block_t);
  if (d->block_h < 0 || d->block_w < 0)
    return fail(LCSA_ERR_INVALID, "block_h/block_w must be >= 0");

  int bh = d->block_h, bw = d->block_w;
  if (bh == 0 && bw == 0) {
    if (d->grid_w % 16 == 0 && d->grid_h % 8 == 0) {
      bh = 8; bw = 16;
    } else if (d->grid_h % 16 == 0 && d->grid_w % 8 == 0) {
      bh = 16; bw = 8;
    } else {
      return fail(LCSA_ERR_SHAPE, "grid %dx%d is tiled by neither 8x16 nor 16x8 blocks",
                  d->grid_h, d->grid_w);
    }
  }
  if (bh <= 0 || bw <= 0)
    return fail(LCSA_ERR_INVALID, "block_h and block_w must both be set or both be 0");
  if ((bw & (bw - 1)) != 0 || (bh & (bh - 1)) != 0)
    return fail(LCSA_ERR_SHAPE, "block %dx%d: sides must be powers of two", bh, bw);
  if (bh * bw != 64 && bh * bw != 128)
    return fail(LCSA_ERR_SHAPE, "block %dx%d holds %d tokens; 64 or 128 are supported", bh, bw,
                bh * bw);
  if (d->grid_h % bh || d->grid_w % bw)
    return fail(LCSA_ERR_SHAPE, "block %dx%d does not tile grid %dx%d", bh, bw, d->grid_h,
                d->grid_w);

  int64_t kvf = static_cast<int64_t>(d->q_frames) + d->cached_frames;
  if (d->kv_ratio > 0.0f) {
    const int64_t cap = lcsa::snap_or(static_cast<double>(d->kv_ratio) * d->q_frames, true);
    if (cap < kvf) kvf = cap;
  }
  const int64_t nbh = d->grid_h / bh, nbw = d->grid_w / bw, nbf = nbh * nbw;
  const int64_t nqb = nbf * d->q_frames, nkb = nbf * kvf;
  const int64_t fs = static_cast<int64_t>(d->grid_h) * d->grid_w;
  const int64_t rows = static_cast<int64_t>(d->batch) * d->heads * nqb;
  if (nkb > INT32_MAX / 2 || rows >= INT32_MAX || fs * kvf > INT32_MAX)
    return fail(LCSA_ERR_SHAPE, "problem too large for 32-bit block and token indices");

  if (kvf > LCSA_MAX_KV_FRAMES)
    return fail(LCSA_ERR_SHAPE, "KV window of %lld frames exceeds %d", (long long)kvf,
                LCSA_MAX_KV_FRAMES);

  int64_t k;
  if (d->topk > 0) {
    k = d->topk;
  } else {
    k = lcsa::snap_or(d->topk_ratio * static_cast<double>(nbf), false);
  }
  if (k < 1) k = 1;
  if (k > nkb) k = nkb;

  lcsa_plan_s* p = new (std::nothrow) lcsa_plan_s();
  if (!p) return fail(LCSA_ERR_INTERNAL, "out of host memory");
  p->desc = *d;
  lcsa_plan_info& in = p->info;
  std::memset(&in, 0, sizeof(in));
  in.kv_frames = static_cast<int32_t>(kvf);
  in.blocks_per_frame = static_cast<int32_t>(nbf);
  in.nbh = static_cast<int32_t>(nbh);
  in.nbw = static_cast<int32_t>(nbw);
  in.nqb = static_cast<int32_t>(nqb);
  in.nkb = static_cast<int32_t>(nkb);
  in.k = static_cast<int32_t>(k);
  in.block_h = bh;
  in.block_w = bw;
  in.block_tokens = bh * bw;
  in.half_window = d->local_range / 2;
  in.rows = rows;
  in.q_tokens = fs * d->q_frames;
  in.kv_tokens = fs * kvf;
  in.scale = d->scale > 0.0f ? static_cast<double>(d->scale) : 1.0 / std::sqrt(128.0);

  // Kept blocks per spatial position (the same for every frame, head, batch).
  try {
    p->frame_count.resize(static_cast<size_t>(nbf));
  } catch (...) {
    delete p;
    return fail(LCSA_ERR_INTERNAL, "out of host memory");
  }
  int64_t per_frame = 0;
  int32_t mx = 0, mn = INT32_MAX, mxw = 0;
  for (int by = 0; by < nbh; ++by) {
    for (int bx = 0; bx < nbw; ++bx) {
      int y0, y1, x0, x1;
      lcsa::window_bounds(in, by, bx, &y0, &y1, &x0, &x1);
      const int64_t w = kvf * (y1 - y0 + 1) * (x1 - x0 + 1);
      const int32_t c = static_cast<int32_t>(w < k ? w : k);
      p->frame_count[by * nbw + bx] = c;
      per_frame += c;
      if (c > mx) mx = c;
      if (w < mn) mn = static_cast<int32_t>(w);
      if (w > mxw) mxw = static_cast<int32_t>(w);
    }
  }
  const int64_t nnz = per_frame * d->q_frames * d->heads * d->batch;
  if (nnz >= INT32_MAX) {
    delete p;
    return fail(LCSA_ERR_SHAPE, "selected block count %lld exceeds int32 CSR", (long long)nnz);
  }
  in.max_row_nnz = mx;
  in.min_window = mn;
  in.max_window = mxw;
  in.nnz = nnz;
  in.useful_flops = 4.0 * 128.0 * in.block_tokens * in.block_tokens * static_cast<double>(nnz);
  // Pooled K per frame slot: [B*H][ceil(NBF / 8)][64 channel pairs][8][2]
  // float64.  Select workspace: pooled Q [B][H][NQB][128] float64, then
  // one such slot per KV-window frame.
  in.kcache_slot_bytes = static_cast<uint64_t>(d->batch) * d->heads * 128ull *
                         static_cast<uint64_t>((nbf + 7) / 8 * 8) * 8ull;
  in.select_workspace_bytes = static_cast<uint64_t>(d->batch) * d->heads * 128ull *
                                  static_cast<uint64_t>(nqb) * 8ull +
                              static_cast<uint64_t>(in.kv_frames) * in.kcache_slot_bytes;
  // Attend: at most one partly filled round of split pieces, i.e. as many
  // pieces as workgroups fit on the largest gfx950 device at once; then, for
  // lcsa_attend_varlen, the row lengths and row order (int32 [rows] each).
  const uint64_t bt = static_cast<uint64_t>(in.block_tokens);
  in.attend_workspace_bytes = lcsa::attend_pieces_bytes(static_cast<int>(bt)) +
                              (static_cast<uint64_t>(rows) * 8 + 255) / 256 * 256;

  try {
    p->row_ptr.resize(static_cast<size_t>(rows) + 1);
  } catch (...) {
    delete p;
    return fail(LCSA_ERR_INTERNAL, "out of host memory");
  }
  int64_t acc = 0;
  size_t r = 0;
  p->row_ptr[r++] = 0;
  for (int64_t bhq = 0; bhq < static_cast<int64_t>(d->batch) * d->heads * d->q_frames; ++bhq) {
    for (int64_t pos = 0; pos < nbf; ++pos) {
      acc += p->frame_count[pos];
      p->row_ptr[r++] = static_cast<int32_t>(acc);
    }
  }
  *out = p;
  return LCSA_OK;
}

void lcsa_plan_destroy(lcsa_plan_t plan) { delete plan; }

lcsa_status lcsa_plan_get_info(lcsa_plan_t plan, lcsa_plan_info* info) {
  lcsa::clear_error();
  if (!plan || !info) return fail(LCSA_ERR_NULL, "lcsa_plan_get_info: NULL argument");
  *info = plan->info;
  return LCSA_OK;
}

lcsa_status lcsa_plan_row_ptr(lcsa_plan_t plan, int32_t* host_out, int64_t capacity) {
  lcsa::clear_error();
  if (!plan || !host_out) return fail(LCSA_ERR_NULL, "lcsa_plan_row_ptr: NULL argument");
  const int64_t n = static_cast<int64_t>(plan->row_ptr.size());
  if (capacity < n)
    return fail(LCSA_ERR_WORKSPACE, "row_ptr needs %lld entries, capacity %lld", (long long)n,
                (long long)capacity);
  std::memcpy(host_out, plan->row_ptr.data(), static_cast<size_t>(n) * sizeof(int32_t));
  return LCSA_OK;
}

lcsa_status lcsa_plan_window(lcsa_plan_t plan, int32_t qb, int32_t* host_out, int32_t capacity,
                             int32_t* count) {
  lcsa::clear_error();
  if (!plan || !host_out || !count) return fail(LCSA_ERR_NULL, "lcsa_plan_window: NULL argument");
  const lcsa_plan_info& in = plan->info;
  if (qb < 0 || qb >= in.nqb)
    return fail(LCSA_ERR_INVALID, "query block %d outside [0, %d)", qb, in.nqb);
  const int pos = qb % in.blocks_per_frame;
  const int by = pos / in.nbw, bx = pos % in.nbw;
  int y0, y1, x0, x1;
  lcsa::window_bounds(in, by, bx, &y0, &y1, &x0, &x1);
  const int n = in.kv_frames * (y1 - y0 + 1) * (x1 - x0 + 1);
  *count = n;
  if (capacity < n) return fail(LCSA_ERR_WORKSPACE, "window has %d blocks, capacity %d", n, capacity);
  int i = 0;
  for (int t = 0; t < in.kv_frames; ++t)
    for (int y = y0; y <= y1; ++y)
      for (int x = x0; x <= x1; ++x) host_out[i++] = t * in.blocks_per_frame + y * in.nbw + x;
  return LCSA_OK;
}

}  // extern "C"
