// Block selection kernels for gfx950.
//
//  pool_kernel    mean of every query block of Q and key block of K, per head
//                 (float64 sums of the bf16 values).
//  select_kernel  one workgroup per (batch, head, spatial position, group of
//                 query frames): its waves score the pooled queries against
//                 every pooled key block of their shared spatial window into
//                 an LDS table, then one wave per CSR row finds the k-th best
//                 score and emits the kept blocks in ascending order.
//
// Pooling and mask selection are the "attention glue" of the FlashVSR Hopper
// PR page ("What Was Actually Slow"), with the mask emitted as CSR ("Rebuild
// sparse attention for Hopper": fused CSR construction).  Locality: only key
// blocks in a spatial window around the query block compete (agentlens
// FlashVSR summary, "How it works", item 2; local_range on the FlashVSR
// Inference skill page, "Non-Negotiable Streaming Contract").
//
// Arithmetic: a bf16 value has 8 significant bits, so the float64 sum of a
// block's 64 or 128 values is exact for any practical value range; pooled
// vectors are order-independent and scores are float64 dot products, so the
// ranking differs from an exact one only at score gaps of ~1e-16 relative.
//
// Top-k: scores map to order-preserving 64-bit keys; the k-th largest key is
// found by deciding its bits from the top, each bit by one wave-wide count
// (ballot + popcount) of the keys at or above the trial value.  Keys above
// it are kept; keys equal to it are kept in ascending block order until k
// are kept (ties go to the lower block index).  The bits that all keys of a
// row share (found from a wave-wide OR and AND) need no count.
//
// Steady threshold reuse (FlashVSR Hopper PR page, "Remove the remaining
// control-plane tax" and "Recommended GH200 Controls": each DiT block holds
// on to the mask threshold of a steady chunk for the chunks after it): the
// top-k run can also
// write each row's keep-th largest window score, and a threshold run keeps,
// instead of the top-k, every window block scored at or above its row's
// given threshold.  Threshold rows vary in length, so they are written at a
// fixed width (the largest window) with -1 after the kept blocks; attention
// skips -1 entries and trims them from a row's end.

#include <hip/hip_runtime.h>

#include "kernel_params.h"
#include "launch.h"
#include "lcsa_internal.h"
#include "topk_wave.h"

namespace lcsa {
namespace {

constexpr int kPoolThreads = 256;
constexpr int kSelectWaves = 4;
constexpr int kMaxPerLane = kMaxWindow / 64;   // window candidates per lane

__device__ inline double bf16_lo(uint32_t w) { return (double)__uint_as_float(w << 16); }
__device__ inline double bf16_hi(uint32_t w) { return (double)__uint_as_float(w & 0xffff0000u); }

// 16-byte load of Q or K in the pooling pass.  STREAM marks it non-temporal:
// when Q and K are far larger than the caches, the stream then no longer
// evicts the pass's own dirty output lines from L2 while it runs.  When they
// fit in the memory-side cache, plain loads leave them there for the
// attention that follows.
template <bool STREAM>
__device__ inline uint4 load16_qk(const uint16_t* ptr) {
  if constexpr (STREAM) {
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(ptr));
    return make_uint4(v[0], v[1], v[2], v[3]);
  } else {
    return *reinterpret_cast<const uint4*>(ptr);
  }
}

// Raster token index of element j (0 .. block_tokens-1) of block (t, by, bx).
__device__ inline int64_t block_token(const GridGeom& g, int t, int by, int bx, int j) {
  const int y = by * g.block_h + (j >> g.log2_bw);
  const int x = bx * g.block_w + (j & (g.block_w - 1));
  return ((int64_t)t * g.grid_h + y) * g.grid_w + x;
}

// bf16 bits of a double rounded to the nearest bf16 value, ties to even, in
// one step (bf16 keeps 7 of the 52 fraction bits of a double).
__device__ inline uint32_t bf16_rne_bits(double v) {
  uint64_t u = (uint64_t)__double_as_longlong(v);
  u = (u + 0xFFFFFFFFFFFull + ((u >> 45) & 1ull)) & ~((1ull << 45) - 1ull);
  return __float_as_uint((float)__longlong_as_double((long long)u)) >> 16;   // exact
}

// One channel pair (x0, x1) turned by the angle with cosine cs.x and sine
// cs.y, rounded to bf16: both products are exact in double (8 by 24
// significant bits), so each component is rounded once, to double, then to
// bf16.  Returns the two bf16 bit patterns packed (x0' low).
__device__ inline uint32_t rope_pair(uint32_t w, float2 cs) {
  const double x0 = bf16_lo(w), x1 = bf16_hi(w);
  const double r0 = fma(x0, (double)cs.x, -(x1 * (double)cs.y));
  const double r1 = fma(x0, (double)cs.y, x1 * (double)cs.x);
  return bf16_rne_bits(r0) | (bf16_rne_bits(r1) << 16);
}

// grid ((NQB + pooled key blocks) x heads, 1, batch): block index x / heads
// (head x % heads) < NQB pools that query block, otherwise key block
// x / heads - NQB of the KV-window frames k_first onwards, read
// from (and stored for) their storage frame kv_slot[t].  Thread (c, tg) sums
// channels 8c..8c+7 of tokens tg, tg+16, ...  With ROPE each 16-byte slice
// (channel pairs 4c..4c+3) is first turned by the rotary tables, written to
// the rotated Q / K output, and the rotated bf16 values are what is pooled.
// STREAM: non-temporal Q/K loads (see load16_qk).
template <int BT, bool ROPE, bool STREAM>
__global__ void __launch_bounds__(kPoolThreads) pool_kernel(PoolParams p) {
  __shared__ double red[16 * 128];
  const GridGeom& g = p.g;
  // heads vary fastest along the grid, so the workgroups of one block's
  // heads, which read neighbouring 256-byte slices of the same token rows,
  // are dispatched together
  const int h = (int)(blockIdx.x % (unsigned)g.heads), b = blockIdx.z;
  const int xb = (int)(blockIdx.x / (unsigned)g.heads);
  const bool is_q = xb < g.nqb;
  const int blk = is_q ? xb : xb - g.nqb + p.k_first * g.nbf;
  const View& x = is_q ? p.q : p.k;
  const int t = blk / g.nbf, pos = blk - t * g.nbf;
  const int by = pos / g.nbw, bx = pos - by * g.nbw;
  const int tf = is_q ? t : g.kv_slot[t];   // frame of the storage
  const uint16_t* base = x.data + (int64_t)b * x.sb + (int64_t)h * x.sh;
  const int tid = threadIdx.x, c = tid & 15, tg = tid >> 4;
  double acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0;
  // Rotary tables of this thread's four channel pairs: each pair reads the
  // row of its axis (0 frame, 1 token row, 2 token column) at stride rs.
  const float2* rtab[4];
  int raxis[4], rs[4];
  uint16_t* rot = nullptr;
  int64_t rot_ss = 0;
  if constexpr (ROPE) {
    const RopeParams& rp = p.rope;
    const int tw = is_q ? g.kv_frames - g.q_frames + t : t;   // KV-window frame
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int pr = 4 * c + u;
      if (pr < rp.pt) {
        raxis[u] = 0;
        rs[u] = 0;
        rtab[u] = reinterpret_cast<const float2*>(rp.table_t) + (int64_t)tw * rp.pt + pr;
      } else if (pr < rp.pt + rp.ph) {
        raxis[u] = 1;
        rs[u] = rp.ph;
        rtab[u] = reinterpret_cast<const float2*>(rp.table_h) + (pr - rp.pt);
      } else {
        raxis[u] = 2;
        rs[u] = 64 - rp.pt - rp.ph;
        rtab[u] = reinterpret_cast<const float2*>(rp.table_w) + (pr - rp.pt - rp.ph);
      }
    }
    const OutView& ov = is_q ? rp.q_rot : rp.k_rot;
    rot = ov.data + (int64_t)b * ov.sb + (int64_t)h * ov.sh + c * 8;
    rot_ss = ov.ss;
  }
  // All loads of the thread first: with the rotary outputs allowed to be the
  // inputs themselves, the compiler could not move a load above an earlier
  // token's store.
  uint4 wv[BT / 16];
#pragma unroll
  for (int i = 0; i < BT / 16; ++i)
    wv[i] = load16_qk<STREAM>(base + block_token(g, tf, by, bx, tg + 16 * i) * x.ss + c * 8);
  // (cos, sin) of every pair of every token, also loaded up front
  float2 cs[ROPE ? BT / 16 : 1][4];
  if constexpr (ROPE) {
#pragma unroll
    for (int i = 0; i < BT / 16; ++i) {
      const int j = tg + 16 * i;
      const int y = by * g.block_h + (j >> g.log2_bw), xx = bx * g.block_w + (j & (g.block_w - 1));
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int pos_a = raxis[u] == 0 ? 0 : raxis[u] == 1 ? y : xx;
        cs[i][u] = rtab[u][pos_a * rs[u]];
      }
    }
  }
#pragma unroll
  for (int i = 0; i < BT / 16; ++i) {
    const int j = tg + 16 * i;
    uint4 w = wv[i];
    if constexpr (ROPE) {
      uint32_t* wp = reinterpret_cast<uint32_t*>(&w);
#pragma unroll
      for (int u = 0; u < 4; ++u) wp[u] = rope_pair(wp[u], cs[i][u]);
      *reinterpret_cast<uint4*>(rot + block_token(g, tf, by, bx, j) * rot_ss) = w;
    }
    acc[0] += bf16_lo(w.x); acc[1] += bf16_hi(w.x);
    acc[2] += bf16_lo(w.y); acc[3] += bf16_hi(w.y);
    acc[4] += bf16_lo(w.z); acc[5] += bf16_hi(w.z);
    acc[6] += bf16_lo(w.w); acc[7] += bf16_hi(w.w);
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[tg * 128 + c * 8 + e] = acc[e];
  __syncthreads();
  if (tid < 128) {
    double s = 0.0;
#pragma unroll
    for (int q = 0; q < 16; ++q) s += red[q * 128 + tid];
    s *= (1.0 / BT);
    const int64_t bh = (int64_t)b * g.heads + h;
    if (is_q)
      p.qbar[(bh * g.nqb + blk) * 128 + tid] = s;
    else
      p.kcache[((((int64_t)tf * gridDim.z * g.heads + bh) * ((g.nbf + 7) >> 3) + (pos >> 3)) * 64 +
                (tid >> 1)) * 16 + (pos & 7) * 2 + (tid & 1)] = s;
  }
}

struct WindowBox {
  int y0, y1, x0, x1, nr, nc, n;
};

__device__ inline WindowBox window_box(const GridGeom& g, int by, int bx) {
  WindowBox w;
  w.y0 = max(by - g.half, 0);
  w.y1 = min(by + g.half, g.nbh - 1);
  w.x0 = max(bx - g.half, 0);
  w.x1 = min(bx + g.half, g.nbw - 1);
  w.nr = w.y1 - w.y0 + 1;
  w.nc = w.x1 - w.x0 + 1;
  w.n = g.kv_frames * w.nr * w.nc;
  return w;
}

// Key block of the e-th window candidate; candidates run frame-major, then
// block row, then block column, i.e. in ascending key-block order.
__device__ inline int window_kb(const GridGeom& g, const WindowBox& w, int e) {
  const int per_frame = w.nr * w.nc;
  const int t = e / per_frame;
  const int rem = e - t * per_frame;
  const int yy = rem / w.nc;
  const int xx = rem - yy * w.nc;
  return t * g.nbf + (w.y0 + yy) * g.nbw + (w.x0 + xx);
}

// The wave's cross-lane operations for the top-k of topk_wave.h.
struct DeviceWave {
  __device__ uint64_t ballot(bool pred) const { return __builtin_amdgcn_ballot_w64(pred); }
  // Wave-wide OR and AND of a 64-bit value, returned in scalar registers:
  // DPP moves combine each 16-lane row (swap within pairs, within quads,
  // then rotate the row by 4 and by 8), and the four rows' results are read
  // from lanes 0, 16, 32 and 48.  Needs every lane active.
  template <int CTRL>
  __device__ static uint32_t dpp(uint32_t x) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xF, 0xF, false);
  }
  __device__ static uint32_t row_or(uint32_t x) {
    x |= dpp<0xB1>(x);    // quad_perm [1,0,3,2]
    x |= dpp<0x4E>(x);    // quad_perm [2,3,0,1]
    x |= dpp<0x124>(x);   // row_ror:4
    x |= dpp<0x128>(x);   // row_ror:8
    return x;
  }
  __device__ static uint32_t row_and(uint32_t x) {
    x &= dpp<0xB1>(x);
    x &= dpp<0x4E>(x);
    x &= dpp<0x124>(x);
    x &= dpp<0x128>(x);
    return x;
  }
  __device__ static uint32_t rows_or(uint32_t x) {
    return __builtin_amdgcn_readlane(x, 0) | __builtin_amdgcn_readlane(x, 16) |
           __builtin_amdgcn_readlane(x, 32) | __builtin_amdgcn_readlane(x, 48);
  }
  __device__ static uint32_t rows_and(uint32_t x) {
    return __builtin_amdgcn_readlane(x, 0) & __builtin_amdgcn_readlane(x, 16) &
           __builtin_amdgcn_readlane(x, 32) & __builtin_amdgcn_readlane(x, 48);
  }
  // wave-wide sum of a 32-bit integer, in a scalar register
  __device__ static int sum(int x) {
    uint32_t v = (uint32_t)x;
    v += dpp<0xB1>(v);
    v += dpp<0x4E>(v);
    v += dpp<0x124>(v);
    v += dpp<0x128>(v);
    return (int)(__builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16) +
                 __builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48));
  }
  __device__ void or_and(uint64_t& o, uint64_t& a) const {
    const uint32_t olo = rows_or(row_or((uint32_t)o)), ohi = rows_or(row_or((uint32_t)(o >> 32)));
    const uint32_t alo = rows_and(row_and((uint32_t)a)), ahi = rows_and(row_and((uint32_t)(a >> 32)));
    o = ((uint64_t)ohi << 32) | olo;
    a = ((uint64_t)ahi << 32) | alo;
  }
};

// Workgroup barrier that completes this wave's own LDS operations but leaves
// its in-flight global loads running (a plain __syncthreads would wait for
// them too).
__device__ inline void barrier_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// g.kv_slot[t] for a per-lane t that does not decrease from lane to lane.
// When the wave's frames span at most 4 (a window's candidates run through
// a few frames), four scalar loads cover them; a per-lane load of the table
// would be a vector-memory round trip ahead of the first pooled-K load.
__device__ inline int frame_slot(const GridGeom& g, int t) {
  const int t_lo = __builtin_amdgcn_readfirstlane(t);
  const int t_hi = __builtin_amdgcn_readlane(t, 63);
  if (t_hi - t_lo < 4) {
    int slot = g.kv_slot[t_lo];
#pragma unroll
    for (int c = 1; c < 4; ++c) {
      const int sc = g.kv_slot[min(t_lo + c, kMaxKvFrames - 1)];
      slot = t == t_lo + c ? sc : slot;
    }
    return slot;
  }
  return g.kv_slot[t];
}

// Scoring waves of a workgroup whose rows have up to 64 M window candidates,
// and candidates per scoring lane.
template <int M>
struct ScoreShape {
  static constexpr int waves = kSelectWaves;
  static constexpr int slots = (M + waves - 1) / waves;
};

// One workgroup takes the rows of up to R query frames at one spatial
// position; they share the window.  Scores: scoring wave w < SW computes
// window candidates e = lane + 64 (SW j + w) of every row into an LDS table,
// so each pooled-key load feeds R dot products.  Top-k: wave w then takes
// rows w, w + 4, ... and reads candidate e = lane + 64 j (j < M) of its row.
template <int M, int R>
__global__ void __launch_bounds__(kSelectWaves * 64, (M <= 4 && R <= 3 ? 4 : 1)) select_kernel(SelectParams p) {
  constexpr int SW = ScoreShape<M>::waves;
  constexpr int MW = ScoreShape<M>::slots;   // scoring slots per lane
  __shared__ double qs[R][128];
  __shared__ double sc[R][64 * M];
  __shared__ int kbs[64 * M];
  const GridGeom& g = p.g;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int pos = (int)(blockIdx.x % (unsigned)g.nbf);
  const int tq0 = (int)(blockIdx.x / (unsigned)g.nbf) * R;
  const int h = blockIdx.y % g.heads, b = blockIdx.y / g.heads;
  const int nr = min(R, g.q_frames - tq0);
  const int by = pos / g.nbw, bx = pos - by * g.nbw;
  const WindowBox w = window_box(g, by, bx);
  const int64_t bh = (int64_t)b * g.heads + h;
  const bool scoring = wave < SW && 64 * wave < w.n;

  // Float64 scores.  The pooled K of key block (t, pos') sits in its frame
  // slot's group of 8 positions, pos' / 8, as 64 channel pairs of 8
  // positions: pair dp of the block is 128 bytes after pair dp - 1, so a
  // lane addresses every pair of its candidate from one pointer with a
  // constant offset, and the 8 lanes of neighbouring positions read one
  // 128-byte line per pair.
  //
  // Two levels of prefetch, so that loads are in flight while FMAs run:
  //  - pooled-K pairs in batches of kD, double-buffered: batch i + 1 is
  //    loaded before the FMAs of batch i (batch 0 before the pooled queries
  //    reach LDS, so that both loads overlap);
  //  - the pooled queries of pair dp + QL are read from LDS before the FMAs
  //    of pair dp.
  // The compiler sees all of these loads as free to move, and hoisting them
  // together exhausts the registers (it spills), so their addresses are made
  // to depend on the scores: batch i + 1 on every score after batch i - 1,
  // the queries of pair dp + QL on every score after pair dp - 1.  The FMA
  // order is dp ascending for every score.
  constexpr int kD = MW == 1 ? 8 : MW == 2 ? 4 : 2;
  constexpr int kNB = 64 / kD;
  constexpr int QL = MW == 1 ? 3 : 1;   // QL + 1 divides 2 kD: buffer indices stay constant
  // Candidates of the lane's scoring slots (lanes past the window take the
  // window's last candidate: in-bounds loads, scores never used), then the
  // loads: pooled queries first, so that waiting for them does not wait for
  // the pooled K, then pooled-K batch 0.  Every wave issues them, so that no
  // branch joins before the waits (which would make them wait for all).
  const double2* kp[MW];
  double2 buf0[kD][MW], buf1[kD][MW];
  double acc[MW][R];
  {
    const int64_t bh_all = (int64_t)p.batch * g.heads;
    const int64_t groups = (g.nbf + 7) >> 3;
    const double2* kd = reinterpret_cast<const double2*>(p.kcache);
#pragma unroll
    for (int j = 0; j < MW; ++j) {
      const int e = min(lane + 64 * (SW * j + wave), w.n - 1);
      const int kb = window_kb(g, w, e);
      const int t = kb / g.nbf, kpos = kb - t * g.nbf;
      const int slot = frame_slot(g, t);
      kp[j] = kd + (((int64_t)slot * bh_all + bh) * groups + (kpos >> 3)) * 512 + (kpos & 7);
#pragma unroll
      for (int r = 0; r < R; ++r) acc[j][r] = 0.0;
    }
  }
  // (rows past the last query frame load the last frame's row, unused)
  double qreg[(R * 128 + kSelectWaves * 64 - 1) / (kSelectWaves * 64)];
#pragma unroll
  for (int u = 0; u < (int)(sizeof(qreg) / sizeof(double)); ++u) {
    const int i = min(tid + u * kSelectWaves * 64, R * 128 - 1);
    const int tq = min(tq0 + (i >> 7), g.q_frames - 1);
    qreg[u] = p.qbar[(bh * g.nqb + (int64_t)tq * g.nbf + pos) * 128 + (i & 127)];
  }
#pragma unroll
  for (int u = 0; u < kD; ++u)
#pragma unroll
    for (int j = 0; j < MW; ++j) buf0[u][j] = kp[j][u * 8];
  // Key block of every window candidate, for the top-k after the scoring:
  // worked out once per workgroup while the loads above are in flight.
  for (int e = tid; e < 64 * M; e += kSelectWaves * 64) kbs[e] = e < w.n ? window_kb(g, w, e) : 0;
  // CSR offset of these rows (worked out while the loads above are in
  // flight): rows run (b, h, frame, position); every frame
  // holds the same per-position counts min(k, |window(position)|).
  int lt = 0, all = 0;
  for (int q = p.tau ? g.nbf : lane; q < g.nbf; q += 64) {
    const int qy = q / g.nbw, qx = q - qy * g.nbw;
    const int c = min(g.k, window_box(g, qy, qx).n);
    all += c;
    lt += q < pos ? c : 0;
  }
  lt = DeviceWave::sum(lt);
  all = DeviceWave::sum(all);
#pragma unroll
  for (int u = 0; u < (int)(sizeof(qreg) / sizeof(double)); ++u) {
    const int i = tid + u * kSelectWaves * 64;
    // only a last, partial round needs the test
    if ((u + 1) * kSelectWaves * 64 <= R * 128 || i < R * 128) qs[i >> 7][i & 127] = qreg[u];
  }
  barrier_lds();

  if (scoring) {
    double2 qv[QL + 1][R];
    const double2* q2 = reinterpret_cast<const double2*>(&qs[0][0]);   // [R][64]
    // always 0; they carry the dependencies of the pooled-K loads and the
    // query reads (an integer, so that the pointers keep their address space)
    int ko = 0, qo = 0;
#pragma unroll
    for (int l = 0; l < QL; ++l)
#pragma unroll
      for (int r = 0; r < R; ++r) qv[l][r] = q2[r * 64 + l];
    // one batch: load batch bi + 1 into nxt, then the FMAs of batch bi
    auto batch = [&](int bi, const double2 (&cur)[kD][MW], double2 (&nxt)[kD][MW]) {
      if (bi + 1 < kNB) {
        if (bi > 0) {
#pragma unroll
          for (int j = 0; j < MW; ++j)
#pragma unroll
            for (int r = 0; r < R; ++r) asm volatile("" : "+v"(ko) : "v"(acc[j][r]));
        }
#pragma unroll
        for (int u = 0; u < kD; ++u)
#pragma unroll
          for (int j = 0; j < MW; ++j) nxt[u][j] = kp[j][ko + ((bi + 1) * kD + u) * 8];
      }
#pragma unroll
      for (int u = 0; u < kD; ++u) {
        const int dp = bi * kD + u;
        if (dp + QL < 64) {
          if (dp > 0) {
#pragma unroll
            for (int j = 0; j < MW; ++j)
#pragma unroll
              for (int r = 0; r < R; ++r) asm volatile("" : "+v"(qo) : "v"(acc[j][r]));
          }
#pragma unroll
          for (int r = 0; r < R; ++r) qv[(u + QL) % (QL + 1)][r] = q2[qo + r * 64 + dp + QL];
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const double2 qq = qv[u % (QL + 1)][r];
#pragma unroll
          for (int j = 0; j < MW; ++j)
            acc[j][r] = fma(qq.y, cur[u][j].y, fma(qq.x, cur[u][j].x, acc[j][r]));
        }
      }
    };
#pragma unroll
    for (int bi = 0; bi < kNB; bi += 2) {
      batch(bi, buf0, buf1);
      batch(bi + 1, buf1, buf0);
    }
#pragma unroll
    for (int j = 0; j < MW; ++j) {
      const int e = lane + 64 * (SW * j + wave);
      if (e < w.n) {
#pragma unroll
        for (int r = 0; r < R; ++r) sc[r][e] = acc[j][r];
      }
    }
  }
  __syncthreads();
  if (wave >= nr) return;

  const int keep = __builtin_amdgcn_readfirstlane(min(g.k, w.n));
  const uint64_t below = (1ull << lane) - 1ull;
  DeviceWave dw;
  int kb[M];
  bool valid[M];
#pragma unroll
  for (int j = 0; j < M; ++j) {
    const int e = lane + 64 * j;
    valid[j] = e < w.n;
    kb[j] = kbs[e];
  }

  for (int r = wave; r < nr; r += kSelectWaves) {
    const int tq = tq0 + r;
    const int64_t row = bh * g.nqb + tq * g.nbf + pos;
    double s[M];
#pragma unroll
    for (int j = 0; j < M; ++j) s[j] = valid[j] ? sc[r][lane + 64 * j] : 0.0;
    if (p.scores) {  // every key block written once: -inf outside the window
      double* srow = p.scores + row * g.nkb;
      for (int x = lane; x < g.nkb; x += 64) {
        const int xt = x / g.nbf, xp = x - xt * g.nbf;
        const int xy = xp / g.nbw, xx = xp - xy * g.nbw;
        if (xy < w.y0 || xy > w.y1 || xx < w.x0 || xx > w.x1) srow[x] = -__builtin_huge_val();
      }
#pragma unroll
      for (int j = 0; j < M; ++j)
        if (valid[j]) srow[kb[j]] = s[j];
    }
    if (p.tau) {
      // Threshold selection: the window blocks at or above the row's
      // threshold, ascending, then -1 up to the row's fixed width.
      const double th = p.tau[row];
      const int64_t off = row * (int64_t)p.pad;
      if (lane == 0) {
        p.row_ptr[row + 1] = (int32_t)(off + p.pad);
        if (row == 0) p.row_ptr[0] = 0;
      }
      int base = 0;
#pragma unroll
      for (int j = 0; j < M; ++j) {
        const bool keep_j = valid[j] && s[j] >= th;
        const uint64_t m = __builtin_amdgcn_ballot_w64(keep_j);
        if (keep_j) p.col_idx[off + base + __popcll(m & below)] = kb[j];
        base += __popcll(m);
      }
      for (int x = base + lane; x < p.pad; x += 64) p.col_idx[off + x] = -1;
      continue;
    }
    const int64_t off = (bh * g.q_frames + tq) * (int64_t)all + lt;
    if (lane == 0) {
      p.row_ptr[row + 1] = (int32_t)(off + keep);
      if (row == 0) p.row_ptr[0] = 0;
    }

    bool sel[M];
    if (keep >= w.n) {
#pragma unroll
      for (int j = 0; j < M; ++j) sel[j] = valid[j];
    } else {
      uint64_t key[M];
#pragma unroll
      for (int j = 0; j < M; ++j) key[j] = valid[j] ? order_key(s[j]) : 0ull;
      topk_select<M>(dw, lane, key, valid, keep, sel);
    }

    if (p.kth) {  // the smallest kept score is the keep-th largest
      double mn = __builtin_huge_val();
#pragma unroll
      for (int j = 0; j < M; ++j) mn = sel[j] ? fmin(mn, s[j]) : mn;
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) mn = fmin(mn, __shfl_xor(mn, m));
      if (lane == 0) p.kth[row] = mn;
    }

    // Emit kept blocks in ascending candidate (= key block) order; a row
    // writes at most its own keep entries.
    int at[M];
    kept_positions<M>(dw, lane, sel, keep, at);
#pragma unroll
    for (int j = 0; j < M; ++j)
      if (at[j] >= 0) p.col_idx[off + at[j]] = kb[j];
  }
}

template <int BT, bool ROPE>
void launch_pool_bt(const PoolParams& p, const dim3 grid, bool stream_loads, hipStream_t stream) {
  if (stream_loads)
    hipLaunchKernelGGL((pool_kernel<BT, ROPE, true>), grid, dim3(kPoolThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((pool_kernel<BT, ROPE, false>), grid, dim3(kPoolThreads), 0, stream, p);
}

}  // namespace

hipError_t launch_pool(const PoolParams& p, int batch, int block_tokens, bool rope,
                       hipStream_t stream) {
  const int64_t blocks = p.g.nqb + (int64_t)(p.g.kv_frames - p.k_first) * p.g.nbf;
  const dim3 grid((unsigned)(blocks * p.g.heads), 1, batch);
  // Q and K bytes this pass reads against the 256 MiB memory-side cache.
  const bool stream_loads =
      (uint64_t)blocks * p.g.heads * batch * block_tokens * 256 > kMemorySideCacheBytes;
  if (block_tokens == 128) {
    if (rope)
      launch_pool_bt<128, true>(p, grid, stream_loads, stream);
    else
      launch_pool_bt<128, false>(p, grid, stream_loads, stream);
  } else {
    if (rope)
      launch_pool_bt<64, true>(p, grid, stream_loads, stream);
    else
      launch_pool_bt<64, false>(p, grid, stream_loads, stream);
  }
  return hipGetLastError();
}

template <int M, int R>
void launch_select_mr(const SelectParams& p, int batch, hipStream_t stream) {
  const int fgroups = (p.g.q_frames + R - 1) / R;
  const dim3 grid(p.g.nbf * fgroups, p.g.heads * batch);
  hipLaunchKernelGGL((select_kernel<M, R>), grid, dim3(kSelectWaves * 64), 0, stream, p);
}

template <int M, int RMAX>
void launch_select_m(const SelectParams& p, int batch, hipStream_t stream) {
  // rows per workgroup: the query frames there are, up to RMAX
  const int qf = p.g.q_frames;
  if (qf <= 1)
    launch_select_mr<M, 1>(p, batch, stream);
  else if (qf <= 2 || RMAX <= 2)
    launch_select_mr<M, (RMAX < 2 ? RMAX : 2)>(p, batch, stream);
  else if (qf <= 4 || RMAX <= 4)
    launch_select_mr<M, (RMAX < 4 ? RMAX : 4)>(p, batch, stream);
  else if (M <= 4 && qf <= 6)
    // narrow windows: two workgroups of 3 rows instead of one of 6, so twice
    // the waves hide the latency of the scoring loop and every row's top-k
    // runs in one round (14.6 against 15.4 us at the first 768x1280 chunk)
    launch_select_mr<M, 3>(p, batch, stream);
  else if (qf <= 6 || RMAX <= 6)
    launch_select_mr<M, (RMAX < 6 ? RMAX : 6)>(p, batch, stream);
  else
    launch_select_mr<M, RMAX>(p, batch, stream);
}

hipError_t launch_select(const SelectParams& p, int batch, int max_window, hipStream_t stream) {
  // Candidates per lane in the top-k, rounded up to a compiled width; up to
  // 8 rows per workgroup (the LDS score table is R x 64 M float64, at most
  // 64 KiB), since every row shares the workgroup's pooled-K loads.
  const int m = (max_window + 63) / 64;
  if (m <= 1)
    launch_select_m<1, 8>(p, batch, stream);
  else if (m <= 2)
    launch_select_m<2, 8>(p, batch, stream);
  else if (m <= 3)
    launch_select_m<3, 8>(p, batch, stream);
  else if (m <= 4)
    launch_select_m<4, 8>(p, batch, stream);
  else if (m <= 6)
    launch_select_m<6, 8>(p, batch, stream);
  else if (m <= 8)
    launch_select_m<8, 8>(p, batch, stream);
  else if (m <= 12)
    launch_select_m<12, 8>(p, batch, stream);
  else
    launch_select_m<kMaxPerLane, 8>(p, batch, stream);
  return hipGetLastError();
}

}  // namespace lcsa
