// C-ABI entry points lcsa_select and lcsa_attend: validate on the host, then
// enqueue the kernels on the caller's stream.  Nothing is enqueued when a
// check fails, and there is no alternative code path (the FlashVSR+ README,
// "Install an attention backend", and the FlashVSR Inference skill page,
// "Backend Gate", both make an unavailable sparse kernel an error rather than
// a silent dense fallback).

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>
#include <mutex>

#include "kernel_params.h"
#include "launch.h"
#include "lcsa_internal.h"

namespace lcsa {
namespace {

lcsa_status check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0)
    return fail(LCSA_ERR_DEVICE, "no current HIP device");
  static std::mutex mu;
  static signed char known[256] = {0};  // 0 unknown, 1 gfx950, -1 other
  if (dev >= 256) return fail(LCSA_ERR_DEVICE, "device ordinal %d out of range", dev);
  std::lock_guard<std::mutex> lock(mu);
  if (known[dev] == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
      return fail(LCSA_ERR_DEVICE, "cannot query device %d", dev);
    known[dev] = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
    if (known[dev] < 0)
      return fail(LCSA_ERR_DEVICE, "device %d is %s; liblcsa is built for gfx950 only", dev,
                  prop.gcnArchName);
  }
  return known[dev] > 0 ? LCSA_OK : fail(LCSA_ERR_DEVICE, "device %d is not gfx950", dev);
}

// Compute units of the current device (cached per device).
lcsa_status device_cus(int* out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 256)
    return fail(LCSA_ERR_DEVICE, "no current HIP device");
  static std::mutex mu;
  static int cached[256] = {0};
  std::lock_guard<std::mutex> lock(mu);
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      return fail(LCSA_ERR_DEVICE, "cannot query the compute-unit count of device %d", dev);
    cached[dev] = n;
  }
  *out = cached[dev];
  return LCSA_OK;
}

// A view's pointer, dtype, alignment and strides, and its extents against
// [batch, tokens, heads, 128] of the plan and call.
lcsa_status check_view(const char* name, const lcsa_tensor* t, int batch, int64_t tokens,
                       int heads, bool allow_null_data = false) {
  if (!t) return fail(LCSA_ERR_NULL, "%s: tensor descriptor is NULL", name);
  if (!t->data && !allow_null_data) return fail(LCSA_ERR_NULL, "%s: data is NULL", name);
  if (t->dtype != LCSA_DTYPE_BF16) return fail(LCSA_ERR_INVALID, "%s: dtype must be bf16", name);
  if (reinterpret_cast<uintptr_t>(t->data) % 16)
    return fail(LCSA_ERR_ALIGN, "%s: data pointer not 16-byte aligned", name);
  if (t->stride_b < 0 || t->stride_s <= 0 || t->stride_h <= 0)
    return fail(LCSA_ERR_INVALID, "%s: strides must be positive (batch stride >= 0)", name);
  if (t->stride_b % 8 || t->stride_s % 8 || t->stride_h % 8)
    return fail(LCSA_ERR_ALIGN, "%s: strides must be multiples of 8 elements", name);
  if (t->batch != batch || t->tokens != tokens || t->heads != heads || t->head_dim != kHeadDim)
    return fail(LCSA_ERR_SHAPE, "%s: extents [%lld, %lld, %lld, %lld], the plan needs [%d, %lld, %d, %d]",
                name, (long long)t->batch, (long long)t->tokens, (long long)t->heads,
                (long long)t->head_dim, batch, (long long)tokens, heads, kHeadDim);
  return LCSA_OK;
}

// Tokens of a K/V view: the contiguous window, or every slot of a ring.
int64_t kv_view_tokens(const lcsa_plan_s* p, const lcsa_kv_ring* ring) {
  return ring ? static_cast<int64_t>(ring->slots) * p->desc.grid_h * p->desc.grid_w
              : p->info.kv_tokens;
}

// Magic multiplier for n / d with 0 <= n < 2^31 and d >= 1 (round-up
// method): l = ceil(log2 d), m = floor(2^(31+l) / d) + 1 < 2^32, and
// n / d == (n * m) >> (31 + l) because m * d - 2^(31+l) <= d <= 2^l.
void magic_div(uint32_t d, uint32_t* m, uint32_t* shift) {
  uint32_t l = 0;
  while ((1ull << l) < d) ++l;
  *m = static_cast<uint32_t>(((1ull << (31 + l)) / d) + 1);
  *shift = 31 + l;
}

GridGeom make_geom(const lcsa_plan_s* p, const lcsa_kv_ring* ring) {
  const lcsa_plan_info& in = p->info;
  GridGeom g;
  g.heads = p->desc.heads;
  g.grid_h = p->desc.grid_h;
  g.grid_w = p->desc.grid_w;
  g.block_h = in.block_h;
  g.block_w = in.block_w;
  g.log2_bw = 0;
  while ((1 << g.log2_bw) < in.block_w) ++g.log2_bw;
  g.nbh = in.nbh;
  g.nbw = in.nbw;
  g.nbf = in.blocks_per_frame;
  g.nqb = in.nqb;
  g.nkb = in.nkb;
  g.q_frames = p->desc.q_frames;
  g.kv_frames = in.kv_frames;
  g.half = in.half_window;
  g.k = in.k;
  g.q_tokens = in.q_tokens;
  magic_div(static_cast<uint32_t>(g.nbf), &g.nbf_m, &g.nbf_s);
  magic_div(static_cast<uint32_t>(g.nbw), &g.nbw_m, &g.nbw_s);
  for (int t = 0; t < kMaxKvFrames; ++t)
    g.kv_slot[t] = t < g.kv_frames ? (ring ? ring->frame_slot[t] : t) : 0;
  return g;
}

lcsa_status check_ring(const char* fn, const lcsa_plan_s* p, const lcsa_kv_ring* ring) {
  if (!ring) return fail(LCSA_ERR_NULL, "%s: ring is NULL", fn);
  if (ring->slots < 1) return fail(LCSA_ERR_INVALID, "%s: ring has %d slots", fn, ring->slots);
  for (int t = 0; t < p->info.kv_frames; ++t)
    if (ring->frame_slot[t] < 0 || ring->frame_slot[t] >= ring->slots)
      return fail(LCSA_ERR_INVALID, "%s: frame %d is in slot %d, outside [0, %d)", fn, t,
                  ring->frame_slot[t], ring->slots);
  return LCSA_OK;
}

View make_view(const lcsa_tensor* t) {
  View v;
  v.data = static_cast<const uint16_t*>(t->data);
  v.sb = t->stride_b;
  v.ss = t->stride_s;
  v.sh = t->stride_h;
  return v;
}

}  // namespace

// Shared body of lcsa_select (ring == NULL: K is the contiguous window, the
// pooled K of every window frame goes to the workspace) and lcsa_select_ring
// (the newest new_frames frames are pooled into the caller's cache).
// Rotary tables and the rotated Q / K outputs of lcsa_select_rope and
// lcsa_select_ring_rope.
lcsa_status check_rope(const char* fn, const lcsa_plan_s* plan, const lcsa_kv_ring* ring,
                       const lcsa_rope* rope, const lcsa_tensor* q_rot, const lcsa_tensor* k_rot) {
  if (!rope) return fail(LCSA_ERR_NULL, "%s: rope is NULL", fn);
  const int pt = rope->pairs_t, ph = rope->pairs_h, pw = rope->pairs_w;
  if (pt < 0 || ph < 0 || pw < 0 || pt + ph + pw != kHeadDim / 2 || rope->reserved != 0)
    return fail(LCSA_ERR_INVALID, "%s: rotary pairs %d + %d + %d must be %d (reserved 0)", fn,
                pt, ph, pw, kHeadDim / 2);
  if ((pt > 0 && !rope->table_t) || (ph > 0 && !rope->table_h) || (pw > 0 && !rope->table_w))
    return fail(LCSA_ERR_NULL, "%s: a rotary table with pairs is NULL", fn);
  const float* tabs[3] = {rope->table_t, rope->table_h, rope->table_w};
  for (const float* tb : tabs)
    if (reinterpret_cast<uintptr_t>(tb) % 8)
      return fail(LCSA_ERR_ALIGN, "%s: rotary tables must be 8-byte aligned", fn);
  lcsa_status st;
  const int batch = plan->desc.batch, heads = plan->desc.heads;
  if ((st = check_view("q_rot", q_rot, batch, plan->info.q_tokens, heads))) return st;
  if ((st = check_view("k_rot", k_rot, batch, kv_view_tokens(plan, ring), heads))) return st;
  return LCSA_OK;
}

lcsa_status select_impl(const char* fn, const lcsa_plan_s* plan, const lcsa_tensor* q,
                        const lcsa_tensor* k, const lcsa_kv_ring* ring, int new_frames,
                        double* d_kcache, int32_t* d_row_ptr, int32_t* d_col_idx,
                        double* d_scores, void* d_workspace, size_t workspace_bytes,
                        void* stream, const lcsa_rope* rope = nullptr,
                        const lcsa_tensor* q_rot = nullptr, const lcsa_tensor* k_rot = nullptr,
                        double* d_kth = nullptr, const double* d_tau = nullptr) {
  if (!plan) return fail(LCSA_ERR_NULL, "%s: plan is NULL", fn);
  const lcsa_plan_info& in = plan->info;
  lcsa_status st;
  const int batch = plan->desc.batch, heads = plan->desc.heads;
  if (ring && (st = check_ring(fn, plan, ring))) return st;
  if ((st = check_view("q", q, batch, in.q_tokens, heads))) return st;
  if ((st = check_view("k", k, batch, kv_view_tokens(plan, ring), heads))) return st;
  if (rope && (st = check_rope(fn, plan, ring, rope, q_rot, k_rot))) return st;
  if (!d_row_ptr || !d_col_idx) return fail(LCSA_ERR_NULL, "%s: CSR buffers are NULL", fn);
  if (d_tau && in.rows * static_cast<int64_t>(in.max_window) >= INT32_MAX)
    return fail(LCSA_ERR_SHAPE, "%s: %lld rows of %d entries exceed int32 CSR", fn,
                (long long)in.rows, in.max_window);
  if ((reinterpret_cast<uintptr_t>(d_kth) | reinterpret_cast<uintptr_t>(d_tau)) % 8)
    return fail(LCSA_ERR_ALIGN, "%s: threshold arrays must be 8-byte aligned", fn);
  if (in.max_window > kMaxWindow)
    return fail(LCSA_ERR_SHAPE, "window of %d key blocks exceeds the select limit of %d",
                in.max_window, kMaxWindow);
  const size_t qbar_bytes = static_cast<size_t>(in.rows) * 128 * sizeof(double);
  const uint64_t ws_need = ring ? qbar_bytes : in.select_workspace_bytes;
  if (!d_workspace || workspace_bytes < ws_need)
    return fail(LCSA_ERR_WORKSPACE, "%s needs %llu workspace bytes, got %llu", fn,
                (unsigned long long)ws_need, (unsigned long long)workspace_bytes);
  if (reinterpret_cast<uintptr_t>(d_workspace) % 256)
    return fail(LCSA_ERR_ALIGN, "workspace must be 256-byte aligned");
  if ((st = check_device())) return st;

  const hipStream_t s = static_cast<hipStream_t>(stream);
  PoolParams pp;
  pp.g = make_geom(plan, ring);
  pp.q = make_view(q);
  pp.k = make_view(k);
  pp.qbar = static_cast<double*>(d_workspace);
  pp.kcache = ring ? d_kcache
                   : reinterpret_cast<double*>(static_cast<char*>(d_workspace) + qbar_bytes);
  pp.k_first = ring ? in.kv_frames - new_frames : 0;
  pp.rope = RopeParams{};
  if (rope) {
    pp.rope.table_t = rope->table_t;
    pp.rope.table_h = rope->table_h;
    pp.rope.table_w = rope->table_w;
    pp.rope.pt = rope->pairs_t;
    pp.rope.ph = rope->pairs_h;
    pp.rope.q_rot = OutView{static_cast<uint16_t*>(q_rot->data), q_rot->stride_b, q_rot->stride_s,
                            q_rot->stride_h};
    pp.rope.k_rot = OutView{static_cast<uint16_t*>(k_rot->data), k_rot->stride_b, k_rot->stride_s,
                            k_rot->stride_h};
  }
  hipError_t e = launch_pool(pp, plan->desc.batch, in.block_tokens, rope != nullptr, s);
  if (e != hipSuccess) return fail(LCSA_ERR_LAUNCH, "pool launch: %s", hipGetErrorString(e));

  SelectParams sp;
  sp.g = pp.g;
  sp.qbar = pp.qbar;
  sp.kcache = pp.kcache;
  sp.batch = plan->desc.batch;
  sp.row_ptr = d_row_ptr;
  sp.col_idx = d_col_idx;
  sp.scores = d_scores;
  sp.kth = d_kth;
  sp.tau = d_tau;
  sp.pad = in.max_window;
  e = launch_select(sp, plan->desc.batch, in.max_window, s);
  if (e != hipSuccess) return fail(LCSA_ERR_LAUNCH, "select launch: %s", hipGetErrorString(e));
  return LCSA_OK;
}

// Shared body of lcsa_attend (ring == NULL), lcsa_attend_ring and, with
// varlen, lcsa_attend_varlen (rows longest first).
lcsa_status attend_impl(const char* fn, const lcsa_plan_s* plan, const lcsa_tensor* q,
                        const lcsa_tensor* k, const lcsa_tensor* v, const lcsa_kv_ring* ring,
                        const int32_t* d_row_ptr, const int32_t* d_col_idx, int64_t nnz,
                        const lcsa_tensor* o, float* d_lse, void* d_workspace,
                        size_t workspace_bytes, void* stream, bool varlen = false) {
  if (!plan) return fail(LCSA_ERR_NULL, "%s: plan is NULL", fn);
  const lcsa_plan_info& in = plan->info;
  lcsa_status st;
  const int batch = plan->desc.batch, heads = plan->desc.heads;
  if (ring && (st = check_ring(fn, plan, ring))) return st;
  const int64_t kv_tokens = kv_view_tokens(plan, ring);
  if ((st = check_view("q", q, batch, in.q_tokens, heads))) return st;
  if ((st = check_view("k", k, batch, kv_tokens, heads))) return st;
  if ((st = check_view("v", v, batch, kv_tokens, heads))) return st;
  if ((st = check_view("o", o, batch, in.q_tokens, heads))) return st;
  if (!d_row_ptr) return fail(LCSA_ERR_NULL, "%s: row_ptr is NULL", fn);
  if (nnz < 0) return fail(LCSA_ERR_INVALID, "%s: nnz %lld < 0", fn, (long long)nnz);
  if (nnz > 0 && !d_col_idx) return fail(LCSA_ERR_NULL, "%s: col_idx is NULL", fn);
  if (nnz >= INT32_MAX)
    return fail(LCSA_ERR_SHAPE, "%s: nnz %lld exceeds int32 CSR", fn, (long long)nnz);
  // The kernel addresses K/V rows inside one block with 32-bit byte offsets.
  const int64_t in_block = (static_cast<int64_t>(in.block_h - 1) * plan->desc.grid_w + in.block_w) * 2;
  if (in_block * k->stride_s >= INT32_MAX || in_block * v->stride_s >= INT32_MAX)
    return fail(LCSA_ERR_SHAPE, "%s: token stride too large for one key block", fn);
  if (d_workspace && reinterpret_cast<uintptr_t>(d_workspace) % 256)
    return fail(LCSA_ERR_ALIGN, "%s: workspace not 256-byte aligned", fn);
  if (varlen && (!d_workspace || workspace_bytes < in.attend_workspace_bytes))
    return fail(LCSA_ERR_WORKSPACE, "%s needs a workspace of %llu bytes, got %llu", fn,
                (unsigned long long)in.attend_workspace_bytes,
                (unsigned long long)(d_workspace ? workspace_bytes : 0));
  if ((st = check_device())) return st;

  // Split the rows of a last, partly filled round of workgroups: with S
  // workgroups resident at once, rows % S rows would otherwise run alone on
  // a mostly idle device.  Each of them becomes `pieces` workgroups over
  // consecutive parts of its CSR range (at most S pieces in all), merged by
  // a second kernel.
  int64_t full_rows = in.rows;
  int pieces = 1;
  int cus = 0;
  if ((st = device_cus(&cus))) return st;
  const int64_t slots = static_cast<int64_t>(cus) * attend_groups_per_cu(in.block_tokens);
  if (d_workspace) {
    const int64_t tail = in.rows % slots;
    if (tail > 0) {
      int64_t want = slots / tail;
      const int64_t cap = in.max_row_nnz < 16 ? in.max_row_nnz : 16;
      if (want > cap) want = cap;
      if (want >= 2) {
        const uint64_t need =
            static_cast<uint64_t>(tail * want) * attend_piece_bytes(in.block_tokens);
        if (workspace_bytes < need)
          return fail(LCSA_ERR_WORKSPACE, "%s: workspace %zu bytes < %llu needed", fn,
                      workspace_bytes, (unsigned long long)need);
        full_rows = in.rows - tail;
        pieces = static_cast<int>(want);
      }
    }
  }

  AttendParams ap;
  ap.g = make_geom(plan, ring);
  ap.q = make_view(q);
  ap.k = make_view(k);
  ap.v = make_view(v);
  ap.o = static_cast<uint16_t*>(o->data);
  ap.o_sb = o->stride_b;
  ap.o_ss = o->stride_s;
  ap.o_sh = o->stride_h;
  ap.lse = d_lse;
  ap.row_ptr = d_row_ptr;
  ap.col_idx = d_col_idx;
  ap.nnz = nnz;
  ap.rows = in.rows;
  ap.full_rows = full_rows;
  ap.pieces = pieces;
  ap.tile = attend_tile(slots, plan->desc.q_frames, in.nbh, in.nbw);
  ap.xcd_chunk = static_cast<int32_t>(slots / 8 > 0 ? slots / 8 : 1);
  ap.part = static_cast<float*>(d_workspace);
  ap.scale_log2 = static_cast<float>(in.scale * 1.4426950408889634);
  ap.order = nullptr;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (varlen) {
    int32_t* len = reinterpret_cast<int32_t*>(static_cast<char*>(d_workspace) +
                                              attend_pieces_bytes(in.block_tokens));
    int32_t* order = len + in.rows;
    const hipError_t e = launch_row_order(ap, len, order, s);
    if (e != hipSuccess) return fail(LCSA_ERR_LAUNCH, "row order launch: %s", hipGetErrorString(e));
    ap.order = order;
  }
  const hipError_t e = launch_attend(ap, in.block_tokens, s);
  if (e != hipSuccess) return fail(LCSA_ERR_LAUNCH, "attend launch: %s", hipGetErrorString(e));
  return LCSA_OK;
}

// Shared body of lcsa_select_steady and lcsa_select_reuse: the ring and the
// rotary tables are each optional.
lcsa_status threshold_select_impl(const char* fn, lcsa_plan_t plan, const lcsa_tensor* q,
                                  const lcsa_tensor* k, const lcsa_kv_ring* ring,
                                  int32_t new_frames, double* d_kcache, const lcsa_rope* rope,
                                  const lcsa_tensor* q_rot, const lcsa_tensor* k_rot,
                                  int32_t* d_row_ptr, int32_t* d_col_idx, double* d_kth,
                                  const double* d_tau, double* d_scores, void* d_workspace,
                                  size_t workspace_bytes, void* stream) {
  if (!plan) return fail(LCSA_ERR_NULL, "%s: plan is NULL", fn);
  if (ring) {
    lcsa_status st;
    if ((st = check_ring(fn, plan, ring))) return st;
    if (new_frames < 0 || new_frames > plan->info.kv_frames)
      return fail(LCSA_ERR_INVALID, "%s: new_frames %d outside [0, %d]", fn, new_frames,
                  plan->info.kv_frames);
    if (!d_kcache) return fail(LCSA_ERR_NULL, "%s: pooled-K cache is NULL", fn);
    if (reinterpret_cast<uintptr_t>(d_kcache) % 256)
      return fail(LCSA_ERR_ALIGN, "%s: pooled-K cache not 256-byte aligned", fn);
  }
  return select_impl(fn, plan, q, k, ring, ring ? new_frames : 0, ring ? d_kcache : nullptr,
                     d_row_ptr, d_col_idx, d_scores, d_workspace, workspace_bytes, stream, rope,
                     q_rot, k_rot, d_kth, d_tau);
}

// Workspace of lcsa_select_noalloc: one array per device, in the library's
// device code object, held until the process ends.  In host code the name
// `scratch` is a host-side stand-in, not a device address; the device
// address is looked up per device (scratch_address) and only that address
// is handed to kernels.
static __device__ __align__(256) double scratch[LCSA_SELECT_NOALLOC_MAX_BYTES / sizeof(double)];

namespace {

// Device address of the current device's scratch array, looked up once per
// device with that device current.
lcsa_status scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 256)
    return fail(LCSA_ERR_DEVICE, "no current HIP device");
  static std::mutex mu;
  static void* addr[256] = {nullptr};
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(LCSA_ERR_DEVICE, "scratch array of device %d: %s", dev, hipGetErrorString(e));
    addr[dev] = ptr;
  }
  *out = addr[dev];
  return LCSA_OK;
}

}  // namespace
}  // namespace lcsa

using lcsa::fail;

extern "C" {

lcsa_status lcsa_select(lcsa_plan_t plan, const lcsa_tensor* q, const lcsa_tensor* k,
                        int32_t* d_row_ptr, int32_t* d_col_idx, double* d_scores,
                        void* d_workspace, size_t workspace_bytes, void* stream) {
  lcsa::clear_error();
  return lcsa::select_impl("lcsa_select", plan, q, k, nullptr, 0, nullptr, d_row_ptr, d_col_idx,
                           d_scores, d_workspace, workspace_bytes, stream);
}

lcsa_status lcsa_select_noalloc(lcsa_plan_t plan, const lcsa_tensor* q, const lcsa_tensor* k,
                                int32_t* d_row_ptr, int32_t* d_col_idx, double* d_scores,
                                void* stream) {
  lcsa::clear_error();
  if (!plan) return fail(LCSA_ERR_NULL, "lcsa_select_noalloc: plan is NULL");
  if (plan->info.select_workspace_bytes > LCSA_SELECT_NOALLOC_MAX_BYTES)
    return fail(LCSA_ERR_WORKSPACE,
                "lcsa_select_noalloc: the plan needs %llu workspace bytes, above the %llu of the "
                "library's scratch array; use lcsa_select with a caller workspace",
                (unsigned long long)plan->info.select_workspace_bytes,
                (unsigned long long)LCSA_SELECT_NOALLOC_MAX_BYTES);
  lcsa_status st;
  if ((st = lcsa::check_device())) return st;
  void* ws = nullptr;
  if ((st = lcsa::scratch_address(&ws))) return st;
  // Every entry of the workspace that select reads, pool writes first in
  // the same call, so the array needs no clearing between calls.
  return lcsa::select_impl("lcsa_select_noalloc", plan, q, k, nullptr, 0, nullptr, d_row_ptr,
                           d_col_idx, d_scores, ws, LCSA_SELECT_NOALLOC_MAX_BYTES, stream);
}

lcsa_status lcsa_select_ring(lcsa_plan_t plan, const lcsa_tensor* q, const lcsa_tensor* k_ring,
                             const lcsa_kv_ring* ring, int32_t new_frames, double* d_kcache,
                             int32_t* d_row_ptr, int32_t* d_col_idx, double* d_scores,
                             void* d_workspace, size_t workspace_bytes, void* stream) {
  lcsa::clear_error();
  if (!plan) return fail(LCSA_ERR_NULL, "lcsa_select_ring: plan is NULL");
  lcsa_status st;
  if ((st = lcsa::check_ring("lcsa_select_ring", plan, ring))) return st;
  if (new_frames < 0 || new_frames > plan->info.kv_frames)
    return fail(LCSA_ERR_INVALID, "lcsa_select_ring: new_frames %d outside [0, %d]", new_frames,
                plan->info.kv_frames);
  if (!d_kcache) return fail(LCSA_ERR_NULL, "lcsa_select_ring: pooled-K cache is NULL");
  if (reinterpret_cast<uintptr_t>(d_kcache) % 256)
    return fail(LCSA_ERR_ALIGN, "lcsa_select_ring: pooled-K cache not 256-byte aligned");
  return lcsa::select_impl("lcsa_select_ring", plan, q, k_ring, ring, new_frames, d_kcache,
                           d_row_ptr, d_col_idx, d_scores, d_workspace, workspace_bytes, stream);
}

lcsa_status lcsa_select_rope(lcsa_plan_t plan, const lcsa_tensor* q, const lcsa_tensor* k,
                             const lcsa_rope* rope, const lcsa_tensor* q_rot,
                             const lcsa_tensor* k_rot, int32_t* d_row_ptr, int32_t* d_col_idx,
                             double* d_scores, void* d_workspace, size_t workspace_bytes,
                             void* stream) {
  lcsa::clear_error();
  if (!rope) return fail(LCSA_ERR_NULL, "lcsa_select_rope: rope is NULL");
  return lcsa::select_impl("lcsa_select_rope", plan, q, k, nullptr, 0, nullptr, d_row_ptr,
                           d_col_idx, d_scores, d_workspace, workspace_bytes, stream, rope, q_rot,
                           k_rot);
}

lcsa_status lcsa_select_ring_rope(lcsa_plan_t plan, const lcsa_tensor* q,
                                  const lcsa_tensor* k_ring, const lcsa_kv_ring* ring,
                                  int32_t new_frames, double* d_kcache, const lcsa_rope* rope,
                                  const lcsa_tensor* q_rot, const lcsa_tensor* k_rot_ring,
                                  int32_t* d_row_ptr, int32_t* d_col_idx, double* d_scores,
                                  void* d_workspace, size_t workspace_bytes, void* stream) {
  lcsa::clear_error();
  if (!plan) return fail(LCSA_ERR_NULL, "lcsa_select_ring_rope: plan is NULL");
  if (!rope) return fail(LCSA_ERR_NULL, "lcsa_select_ring_rope: rope is NULL");
  lcsa_status st;
  if ((st = lcsa::check_ring("lcsa_select_ring_rope", plan, ring))) return st;
  if (new_frames < 0 || new_frames > plan->info.kv_frames)
    return fail(LCSA_ERR_INVALID, "lcsa_select_ring_rope: new_frames %d outside [0, %d]",
                new_frames, plan->info.kv_frames);
  if (!d_kcache) return fail(LCSA_ERR_NULL, "lcsa_select_ring_rope: pooled-K cache is NULL");
  if (reinterpret_cast<uintptr_t>(d_kcache) % 256)
    return fail(LCSA_ERR_ALIGN, "lcsa_select_ring_rope: pooled-K cache not 256-byte aligned");
  return lcsa::select_impl("lcsa_select_ring_rope", plan, q, k_ring, ring, new_frames, d_kcache,
                           d_row_ptr, d_col_idx, d_scores, d_workspace, workspace_bytes, stream,
                           rope, q_rot, k_rot_ring);
}

lcsa_status lcsa_select_steady(lcsa_plan_t plan, const lcsa_tensor* q, const lcsa_tensor* k,
                               const lcsa_kv_ring* ring, int32_t new_frames, double* d_kcache,
                               const lcsa_rope* rope, const lcsa_tensor* q_rot,
                               const lcsa_tensor* k_rot, int32_t* d_row_ptr, int32_t* d_col_idx,
                               double* d_kth, double* d_scores, void* d_workspace,
                               size_t workspace_bytes, void* stream) {
  lcsa::clear_error();
  if (!d_kth) return fail(LCSA_ERR_NULL, "lcsa_select_steady: kth is NULL");
  return lcsa::threshold_select_impl("lcsa_select_steady", plan, q, k, ring, new_frames,
                                     d_kcache, rope, q_rot, k_rot, d_row_ptr, d_col_idx, d_kth,
                                     nullptr, d_scores, d_workspace, workspace_bytes, stream);
}

lcsa_status lcsa_select_reuse(lcsa_plan_t plan, const lcsa_tensor* q, const lcsa_tensor* k,
                              const lcsa_kv_ring* ring, int32_t new_frames, double* d_kcache,
                              const lcsa_rope* rope, const lcsa_tensor* q_rot,
                              const lcsa_tensor* k_rot, const double* d_tau, int32_t* d_row_ptr,
                              int32_t* d_col_idx, double* d_scores, void* d_workspace,
                              size_t workspace_bytes, void* stream) {
  lcsa::clear_error();
  if (!d_tau) return fail(LCSA_ERR_NULL, "lcsa_select_reuse: tau is NULL");
  return lcsa::threshold_select_impl("lcsa_select_reuse", plan, q, k, ring, new_frames, d_kcache,
                                     rope, q_rot, k_rot, d_row_ptr, d_col_idx, nullptr, d_tau,
                                     d_scores, d_workspace, workspace_bytes, stream);
}

lcsa_status lcsa_attend(lcsa_plan_t plan, const lcsa_tensor* q, const lcsa_tensor* k,
                        const lcsa_tensor* v, const int32_t* d_row_ptr,
                        const int32_t* d_col_idx, int64_t nnz, const lcsa_tensor* o,
                        float* d_lse, void* d_workspace, size_t workspace_bytes,
                        void* stream) {
  lcsa::clear_error();
  return lcsa::attend_impl("lcsa_attend", plan, q, k, v, nullptr, d_row_ptr, d_col_idx, nnz, o,
                           d_lse, d_workspace, workspace_bytes, stream);
}

lcsa_status lcsa_attend_varlen(lcsa_plan_t plan, const lcsa_tensor* q, const lcsa_tensor* k,
                               const lcsa_tensor* v, const lcsa_kv_ring* ring,
                               const int32_t* d_row_ptr, const int32_t* d_col_idx, int64_t nnz,
                               const lcsa_tensor* o, float* d_lse, void* d_workspace,
                               size_t workspace_bytes, void* stream) {
  lcsa::clear_error();
  return lcsa::attend_impl("lcsa_attend_varlen", plan, q, k, v, ring, d_row_ptr, d_col_idx, nnz,
                           o, d_lse, d_workspace, workspace_bytes, stream, true);
}

lcsa_status lcsa_attend_ring(lcsa_plan_t plan, const lcsa_tensor* q, const lcsa_tensor* k_ring,
                             const lcsa_tensor* v_ring, const lcsa_kv_ring* ring,
                             const int32_t* d_row_ptr, const int32_t* d_col_idx, int64_t nnz,
                             const lcsa_tensor* o, float* d_lse, void* d_workspace,
                             size_t workspace_bytes, void* stream) {
  lcsa::clear_error();
  if (!plan) return fail(LCSA_ERR_NULL, "lcsa_attend_ring: plan is NULL");
  lcsa_status st;
  if ((st = lcsa::check_ring("lcsa_attend_ring", plan, ring))) return st;
  return lcsa::attend_impl("lcsa_attend_ring", plan, q, k_ring, v_ring, ring, d_row_ptr,
                           d_col_idx, nnz, o, d_lse, d_workspace, workspace_bytes, stream);
}

}  // extern "C"
