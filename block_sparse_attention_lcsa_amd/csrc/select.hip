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

namespace lcsa {
namespace {

constexpr int kPoolThreads = 256;
constexpr int kSelectWaves = 4;
constexpr int kMaxPerLane = kMaxWindow / 64;   // window candidates per lane

__device__ inline double bf16_lo(uint32_t w) { return (double)__uint_as_float(w << 16); }
__device__ inline double bf16_hi(uint32_t w) { return (double)__uint_as_float(w & 0xffff0000u); }

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

// grid (NQB + pooled key blocks, heads, batch): x < NQB pools query block x,
// otherwise key block x - NQB of the KV-window frames k_first onwards, read
// from (and stored for) their storage frame kv_slot[t].  Thread (c, tg) sums
// channels 8c..8c+7 of tokens tg, tg+16, ...  With ROPE each 16-byte slice
// (channel pairs 4c..4c+3) is first turned by the rotary tables, written to
// the rotated Q / K output, and the rotated bf16 values are what is pooled.
template <int BT, bool ROPE>
__global__ void __launch_bounds__(kPoolThreads) pool_kernel(PoolParams p) {
  __shared__ double red[16 * 128];
  const GridGeom& g = p.g;
  const int h = blockIdx.y, b = blockIdx.z;
  const bool is_q = (int)blockIdx.x < g.nqb;
  const int blk = is_q ? (int)blockIdx.x : (int)blockIdx.x - g.nqb + p.k_first * g.nbf;
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
    wv[i] = *reinterpret_cast<const uint4*>(base + block_token(g, tf, by, bx, tg + 16 * i) * x.ss + c * 8);
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
      p.kcache[((((int64_t)tf * gridDim.z * g.heads + bh) * 64 + (tid >> 1)) * g.nbf + pos) * 2 + (tid & 1)] = s;
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

// Order-preserving key of a double (larger score -> larger key; -0 == +0).
__device__ inline uint64_t order_key(double s) {
  const uint64_t u = (uint64_t)__double_as_longlong(s + 0.0);
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

__device__ inline int wave_count(bool pred) {
  return __popcll(__builtin_amdgcn_ballot_w64(pred));
}

// Wave-wide OR and AND of a 64-bit value.
__device__ inline void wave_or_and(uint64_t& o, uint64_t& a) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    o |= (uint64_t)__shfl_xor((unsigned long long)o, m);
    a &= (uint64_t)__shfl_xor((unsigned long long)a, m);
  }
}

// One workgroup takes the rows of up to R query frames at one spatial
// position; they share the window.  Scores: wave w computes window
// candidates e = lane + 64 (4 j + w) of every row into an LDS table, so each
// pooled-key load feeds R dot products.  Top-k: wave w then takes rows w,
// w + 4, ... and reads candidate e = lane + 64 j (j < M) of its row.
template <int M, int R>
__global__ void __launch_bounds__(kSelectWaves * 64) select_kernel(SelectParams p) {
  constexpr int MW = (M + kSelectWaves - 1) / kSelectWaves;   // scoring slots per lane
  __shared__ double qs[R][128];
  __shared__ double sc[R][64 * M];
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

  // Pooled queries of the rows -> LDS (read back as broadcasts).
  for (int i = tid; i < nr * 128; i += kSelectWaves * 64)
    qs[i >> 7][i & 127] = p.qbar[(bh * g.nqb + (int64_t)(tq0 + (i >> 7)) * g.nbf + pos) * 128 + (i & 127)];
  __syncthreads();

  // Float64 scores.  Channels d, d + 1 (d even) of the pooled K of key block
  // (t, pos') sit together at kcache[kv_slot[t]][bh][d / 2][pos'][0..1], so
  // a lane reads two channels per 16-byte load and neighbouring lanes
  // (neighbouring positions) read neighbouring 16 bytes.
  if (64 * wave < w.n) {
    int64_t koff[MW];
    bool valid[MW];
    double acc[MW][R];
    const int64_t bh_all = (int64_t)p.batch * g.heads;
#pragma unroll
    for (int j = 0; j < MW; ++j) {
      const int e = lane + 64 * (kSelectWaves * j + wave);
      valid[j] = e < w.n;
      const int kb = valid[j] ? window_kb(g, w, e) : 0;
      const int t = kb / g.nbf;
      koff[j] = ((int64_t)g.kv_slot[t] * bh_all + bh) * 64 * g.nbf + (kb - t * g.nbf);   // in pairs
#pragma unroll
      for (int r = 0; r < R; ++r) acc[j][r] = 0.0;
    }
    const double2* kd = reinterpret_cast<const double2*>(p.kcache);
    if constexpr (MW == 1) {
      // One candidate per lane: latency-bound.  Channel pairs go in steps of
      // kU, and the loads of step i + 1 are issued before the FMAs of step i,
      // so a load latency overlaps a step of arithmetic (same FMA order).
      constexpr int kU = 4;
      double2 cur[kU], nxt[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) cur[u] = kd[(int64_t)u * g.nbf + koff[0]];
#pragma unroll
      for (int dp0 = 0; dp0 < 64; dp0 += kU) {
        if (dp0 + kU < 64) {
#pragma unroll
          for (int u = 0; u < kU; ++u) nxt[u] = kd[(int64_t)(dp0 + kU + u) * g.nbf + koff[0]];
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          const int dp = dp0 + u;
#pragma unroll
          for (int r = 0; r < R; ++r) {
            const double q0 = qs[r][2 * dp], q1 = qs[r][2 * dp + 1];
            acc[0][r] = fma(q1, cur[u].y, fma(q0, cur[u].x, acc[0][r]));
          }
        }
        if (dp0 + kU < 64) {
#pragma unroll
          for (int u = 0; u < kU; ++u) cur[u] = nxt[u];
        }
      }
    } else {
#pragma unroll 2
      for (int dp = 0; dp < 64; ++dp) {
        double2 kv[MW];
#pragma unroll
        for (int j = 0; j < MW; ++j) kv[j] = kd[(int64_t)dp * g.nbf + koff[j]];
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const double q0 = qs[r][2 * dp], q1 = qs[r][2 * dp + 1];
#pragma unroll
          for (int j = 0; j < MW; ++j) acc[j][r] = fma(q1, kv[j].y, fma(q0, kv[j].x, acc[j][r]));
        }
      }
    }
#pragma unroll
    for (int j = 0; j < MW; ++j) {
      if (valid[j]) {
        const int e = lane + 64 * (kSelectWaves * j + wave);
#pragma unroll
        for (int r = 0; r < R; ++r) sc[r][e] = acc[j][r];
      }
    }
  }
  __syncthreads();
  if (wave >= nr) return;

  // CSR offset of these rows: rows run (b, h, frame, position); every frame
  // holds the same per-position counts min(k, |window(position)|).
  int lt = 0, all = 0;
  for (int q = p.tau ? g.nbf : lane; q < g.nbf; q += 64) {
    const int qy = q / g.nbw, qx = q - qy * g.nbw;
    const int c = min(g.k, window_box(g, qy, qx).n);
    all += c;
    lt += q < pos ? c : 0;
  }
  for (int m = 32; m >= 1; m >>= 1) {
    lt += __shfl_xor(lt, m);
    all += __shfl_xor(all, m);
  }
  const int keep = min(g.k, w.n);
  const uint64_t below = (1ull << lane) - 1ull;
  int kb[M];
  bool valid[M];
#pragma unroll
  for (int j = 0; j < M; ++j) {
    const int e = lane + 64 * j;
    valid[j] = e < w.n;
    kb[j] = valid[j] ? window_kb(g, w, e) : 0;
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
      uint64_t kor = 0ull, kand = ~0ull;
#pragma unroll
      for (int j = 0; j < M; ++j) {
        key[j] = valid[j] ? order_key(s[j]) : 0ull;
        kor |= valid[j] ? key[j] : 0ull;
        kand &= valid[j] ? key[j] : ~0ull;
      }
      wave_or_and(kor, kand);
      // Every valid key shares the bits above the highest bit where two of
      // them differ, so the bisection starts there.  Largest T with
      // #{key >= T} >= keep, decided bit by bit from the top.  Invalid lanes
      // hold key 0, which never reaches a trial value > 0.
      const uint64_t diff = kor ^ kand;
      const int hb = diff ? 63 - __clzll(diff) : -1;
      uint64_t t = hb >= 63 ? 0ull : kand & ~((2ull << hb) - 1ull);
      bool exact = false;
      for (int bit = hb; bit >= 0; --bit) {
        const uint64_t trial = t | (1ull << bit);
        int cnt = 0;
#pragma unroll
        for (int j = 0; j < M; ++j) cnt += wave_count(key[j] >= trial);
        if (cnt >= keep) t = trial;
        if (cnt == keep) {  // the set {key >= trial} is exactly the top keep
          exact = true;
          break;
        }
      }
      if (exact) {
#pragma unroll
        for (int j = 0; j < M; ++j) sel[j] = valid[j] && key[j] >= t;
      } else {
        // t is the keep-th largest key; keys == t are admitted by index.
        int need = keep;
#pragma unroll
        for (int j = 0; j < M; ++j) need -= wave_count(valid[j] && key[j] > t);
#pragma unroll
        for (int j = 0; j < M; ++j) {
          const bool tie = valid[j] && key[j] == t;
          const uint64_t tm = __builtin_amdgcn_ballot_w64(tie);
          const int rank = __popcll(tm & below);
          sel[j] = (valid[j] && key[j] > t) || (tie && rank < need);
          need -= __popcll(tm);
          need = need < 0 ? 0 : need;
        }
      }
    }

    if (p.kth) {  // the smallest kept score is the keep-th largest
      double mn = __builtin_huge_val();
#pragma unroll
      for (int j = 0; j < M; ++j) mn = sel[j] ? fmin(mn, s[j]) : mn;
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) mn = fmin(mn, __shfl_xor(mn, m));
      if (lane == 0) p.kth[row] = mn;
    }

    // Emit kept blocks in ascending candidate (= key block) order.
    int base = 0;
#pragma unroll
    for (int j = 0; j < M; ++j) {
      const uint64_t m = __builtin_amdgcn_ballot_w64(sel[j]);
      if (sel[j]) p.col_idx[off + base + __popcll(m & below)] = kb[j];
      base += __popcll(m);
    }
  }
}

}  // namespace

hipError_t launch_pool(const PoolParams& p, int batch, int block_tokens, bool rope,
                       hipStream_t stream) {
  const dim3 grid(p.g.nqb + (p.g.kv_frames - p.k_first) * p.g.nbf, p.g.heads, batch);
  if (block_tokens == 128) {
    if (rope)
      hipLaunchKernelGGL((pool_kernel<128, true>), grid, dim3(kPoolThreads), 0, stream, p);
    else
      hipLaunchKernelGGL((pool_kernel<128, false>), grid, dim3(kPoolThreads), 0, stream, p);
  } else {
    if (rope)
      hipLaunchKernelGGL((pool_kernel<64, true>), grid, dim3(kPoolThreads), 0, stream, p);
    else
      hipLaunchKernelGGL((pool_kernel<64, false>), grid, dim3(kPoolThreads), 0, stream, p);
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
