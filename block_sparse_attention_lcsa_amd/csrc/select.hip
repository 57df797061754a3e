// Block selection kernels for gfx950: mean-pool K per key block, then per
// (batch, head, spatial block position) mean-pool Q for every query frame,
// score the window's pooled keys, keep the top k and emit the CSR block mask.
//
// Pooling and mask selection are the "attention glue" of the FlashVSR Hopper
// PR page ("What Was Actually Slow"), with the mask emitted as CSR ("Rebuild
// sparse attention for Hopper": fused CSR construction).  Locality: only key
// blocks in a spatial window around the query block compete (agentlens
// FlashVSR summary, "How it works", item 2; local_range on the FlashVSR
// Inference skill page, "Non-Negotiable Streaming Contract").
//
// Arithmetic: block sums and scores are float64.  A bf16 value has 8
// significant bits, so a sum of 128 of them is exact in float64 for any
// practical value range; pooled vectors are therefore order-independent and
// the ranking differs from an exact one only at score gaps of ~1e-16.

#include <hip/hip_runtime.h>

#include "kernel_params.h"
#include "launch.h"
#include "lcsa_internal.h"

namespace lcsa {
namespace {

constexpr int kThreads = 256;

__device__ inline double bf16_lo(uint32_t w) { return (double)__uint_as_float(w << 16); }
__device__ inline double bf16_hi(uint32_t w) { return (double)__uint_as_float(w & 0xffff0000u); }

// Raster token index of element j (0 .. block_tokens-1) of block (t, by, bx).
__device__ inline int64_t block_token(const GridGeom& g, int t, int by, int bx, int j) {
  const int y = by * g.block_h + (j >> g.log2_bw);
  const int x = bx * g.block_w + (j & (g.block_w - 1));
  return ((int64_t)t * g.grid_h + y) * g.grid_w + x;
}

// Sum of one block's rows of one head into red[16][128]: thread (c, tg) adds
// 8 channels 8c..8c+7 of tokens tg, tg+16, ...
template <int BT>
__device__ inline void block_sum_partial(const GridGeom& g, const uint16_t* base, int64_t ss,
                                         int t, int by, int bx, double* red) {
  const int tid = threadIdx.x;
  const int c = tid & 15, tg = tid >> 4;
  double acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0;
#pragma unroll
  for (int j = tg; j < BT; j += 16) {
    const uint4 w = *reinterpret_cast<const uint4*>(base + block_token(g, t, by, bx, j) * ss + c * 8);
    acc[0] += bf16_lo(w.x); acc[1] += bf16_hi(w.x);
    acc[2] += bf16_lo(w.y); acc[3] += bf16_hi(w.y);
    acc[4] += bf16_lo(w.z); acc[5] += bf16_hi(w.z);
    acc[6] += bf16_lo(w.w); acc[7] += bf16_hi(w.w);
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[tg * 128 + c * 8 + e] = acc[e];
}

template <int BT>
__global__ void __launch_bounds__(kThreads) pool_k_kernel(PoolKParams p) {
  __shared__ double red[16 * 128];
  const GridGeom& g = p.g;
  const int kb = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int t = kb / g.nbf, pos = kb - t * g.nbf;
  const int by = pos / g.nbw, bx = pos - by * g.nbw;
  const uint16_t* base = p.k.data + (int64_t)b * p.k.sb + (int64_t)h * p.k.sh;
  block_sum_partial<BT>(g, base, p.k.ss, t, by, bx, red);
  __syncthreads();
  const int d = threadIdx.x;
  if (d < 128) {
    double s = 0.0;
#pragma unroll
    for (int q = 0; q < 16; ++q) s += red[q * 128 + d];
    p.kbar_t[(((int64_t)b * g.heads + h) * 128 + d) * g.nkb + kb] = s * (1.0 / BT);
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

// Candidate x ranks before y: higher score, then lower index; padding last.
__device__ inline bool ranks_before(const double* sc, int n, int x, int y) {
  if (x >= n) return false;
  if (y >= n) return true;
  const double sx = sc[x], sy = sc[y];
  return sx > sy || (sx == sy && x < y);
}

template <int BT>
__global__ void __launch_bounds__(kThreads) select_kernel(SelectParams p) {
  // Region A is the pooling reduction buffer first, then the score table.
  __shared__ double region_a[kSelectFrames * kMaxWindow];
  __shared__ double qbar[kSelectFrames * 128];
  __shared__ uint16_t order[kMaxWindow];
  __shared__ uint8_t flag[kMaxWindow];
  __shared__ int s_sum[2];

  const GridGeom& g = p.g;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int pos = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int by = pos / g.nbw, bx = pos - by * g.nbw;
  const WindowBox w = window_box(g, by, bx);
  const int keep = min(g.k, w.n);

  // Offset of this position inside one frame's CSR rows, and the per-frame
  // total: sums of min(k, |window|) over spatial positions.
  if (tid < 2) s_sum[tid] = 0;
  __syncthreads();
  {
    int lt = 0, all = 0;
    for (int q = tid; q < g.nbf; q += kThreads) {
      const int qy = q / g.nbw, qx = q - qy * g.nbw;
      const WindowBox wq = window_box(g, qy, qx);
      const int c = min(g.k, wq.n);
      all += c;
      if (q < pos) lt += c;
    }
    atomicAdd(&s_sum[0], lt);
    atomicAdd(&s_sum[1], all);
  }

  const uint16_t* qbase = p.q.data + (int64_t)b * p.q.sb + (int64_t)h * p.q.sh;
  const double* kcol = p.kbar_t + ((int64_t)b * g.heads + h) * 128 * g.nkb;

  for (int tq0 = 0; tq0 < g.q_frames; tq0 += kSelectFrames) {
    const int ntq = min(kSelectFrames, g.q_frames - tq0);
    // ---- pool the query block of each frame
    for (int u = 0; u < ntq; ++u) {
      __syncthreads();
      block_sum_partial<BT>(g, qbase, p.q.ss, tq0 + u, by, bx, region_a);
      __syncthreads();
      if (tid < 128) {
        double s = 0.0;
#pragma unroll
        for (int q = 0; q < 16; ++q) s += region_a[q * 128 + tid];
        qbar[u * 128 + tid] = s * (1.0 / BT);
      }
    }
    __syncthreads();
    // ---- score every window candidate against every pooled query
    for (int e = tid; e < w.n; e += kThreads) {
      const int kb = window_kb(g, w, e);
      double acc[kSelectFrames];
#pragma unroll
      for (int u = 0; u < kSelectFrames; ++u) acc[u] = 0.0;
      for (int d = 0; d < 128; ++d) {
        const double kv = kcol[(int64_t)d * g.nkb + kb];
#pragma unroll
        for (int u = 0; u < kSelectFrames; ++u)
          if (u < ntq) acc[u] = fma(qbar[u * 128 + d], kv, acc[u]);
      }
#pragma unroll
      for (int u = 0; u < kSelectFrames; ++u)
        if (u < ntq) region_a[u * kMaxWindow + e] = acc[u];
    }
    __syncthreads();
    if (p.scores) {
      for (int u = 0; u < ntq; ++u) {
        const int qb = (tq0 + u) * g.nbf + pos;
        double* srow = p.scores + (((int64_t)b * g.heads + h) * g.nqb + qb) * g.nkb;
        for (int kb = tid; kb < g.nkb; kb += kThreads) {
          const int kt = kb / g.nbf, kp = kb - kt * g.nbf;
          const int ky = kp / g.nbw, kx = kp - ky * g.nbw;
          double v = -__builtin_huge_val();
          if (ky >= w.y0 && ky <= w.y1 && kx >= w.x0 && kx <= w.x1)
            v = region_a[u * kMaxWindow + (kt * w.nr + (ky - w.y0)) * w.nc + (kx - w.x0)];
          srow[kb] = v;
        }
      }
    }
    // ---- top-k per query frame, emitted ascending
    const int prefix = s_sum[0], frame_total = s_sum[1];
    for (int u = 0; u < ntq; ++u) {
      const int tq = tq0 + u;
      const int64_t row = ((int64_t)b * g.heads + h) * g.nqb + (int64_t)tq * g.nbf + pos;
      const int64_t off =
          (((int64_t)b * g.heads + h) * g.q_frames + tq) * (int64_t)frame_total + prefix;
      if (tid == 0) {
        p.row_ptr[row + 1] = (int32_t)(off + keep);
        if (row == 0) p.row_ptr[0] = 0;
      }
      const double* sc = region_a + u * kMaxWindow;
      if (keep < w.n) {
        int n2 = 1;
        while (n2 < w.n) n2 <<= 1;
        for (int i = tid; i < n2; i += kThreads) order[i] = (uint16_t)i;
        __syncthreads();
        for (int size = 2; size <= n2; size <<= 1) {
          for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = tid; i < n2; i += kThreads) {
              const int j = i ^ stride;
              if (j > i) {
                const int a = order[i], c = order[j];
                const bool first_half_best = (i & size) == 0;
                const bool swap = first_half_best ? ranks_before(sc, w.n, c, a)
                                                  : ranks_before(sc, w.n, a, c);
                if (swap) {
                  order[i] = (uint16_t)c;
                  order[j] = (uint16_t)a;
                }
              }
            }
            __syncthreads();
          }
        }
        for (int i = tid; i < w.n; i += kThreads) flag[i] = 0;
        __syncthreads();
        for (int i = tid; i < keep; i += kThreads) flag[order[i]] = 1;
      } else {
        for (int i = tid; i < w.n; i += kThreads) flag[i] = 1;
      }
      __syncthreads();
      if (wave == 0) {
        int base = 0;
        for (int c0 = 0; c0 < w.n; c0 += 64) {
          const int e = c0 + lane;
          const bool f = e < w.n && flag[e];
          const uint64_t m = __ballot(f);
          if (f) {
            const int before = __popcll(m & ((1ull << lane) - 1ull));
            p.col_idx[off + base + before] = window_kb(g, w, e);
          }
          base += __popcll(m);
        }
      }
      __syncthreads();
    }
  }
}

}  // namespace

hipError_t launch_pool_k(const PoolKParams& p, int batch, int block_tokens, hipStream_t stream) {
  const dim3 grid(p.g.nkb, p.g.heads, batch);
  if (block_tokens == 128)
    hipLaunchKernelGGL(pool_k_kernel<128>, grid, dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL(pool_k_kernel<64>, grid, dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_select(const SelectParams& p, int batch, int block_tokens, hipStream_t stream) {
  const dim3 grid(p.g.nbf, p.g.heads, batch);
  if (block_tokens == 128)
    hipLaunchKernelGGL(select_kernel<128>, grid, dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL(select_kernel<64>, grid, dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace lcsa
