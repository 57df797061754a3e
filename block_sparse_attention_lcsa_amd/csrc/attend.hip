// Block-sparse attention forward for gfx950 (CDNA4): one workgroup per CSR
// row (batch, head, query block), online softmax over the tokens of the row's
// key blocks, bf16 MFMA for both contractions.
//
// The pages' kernels (an HMMA block-sparse kernel and a warp-specialised
// WGMMA/TMA rewrite on the FlashVSR Hopper PR page, "How I Fixed It") are
// prior art for other hardware.  What carries over: the softmax argument as
// one FMA with scale*log2(e) followed by exp2 ("FFMA-form softmax math"),
// reading Q/K/V through strides in raster token order ("strided IO",
// "zero-copy raster V handling") and a CSR block list per query block.
//
// Layout of the work (wave64, 32x32x16 bf16 MFMA):
//  * Each wave owns 32 query rows.  It computes S^T = K Q^T so that every lane
//    holds the scores of ONE query (lane & 31) against 16 keys per 32-key
//    tile; row max and row sum are per-lane plus one exchange with lane ^ 32.
//  * K rows feed MFMA operand A in a permuted order pi(m) chosen so that the
//    S^T accumulator register r of lane half g holds key 16g + r.  Those 8-key
//    runs are exactly MFMA operand B of O^T = V^T P^T, so P never leaves the
//    registers.  The O^T accumulator is again one query per lane, so the
//    online-softmax rescale is a per-lane scalar.
//  * K is staged row-major and V transposed (V^T: [d][key]) in LDS, both with
//    an XOR swizzle on 16-byte chunks so the MFMA operand reads and the tile
//    writes spread over the banks.  The next block's K/V are loaded from HBM
//    into registers while the current block is computed.

#include <hip/hip_runtime.h>

#include "kernel_params.h"
#include "launch.h"

namespace lcsa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

__device__ inline uint4 load16(const uint16_t* ptr) { return *reinterpret_cast<const uint4*>(ptr); }

__device__ inline bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// Chunk swizzles (16-byte chunks).  K tile: row j (key), 16 chunks of 8
// channels.  V^T tile: row d (channel), BT/8 chunks of 8 keys.
__device__ inline int swz_k(int j) { return (j & 7) | (((j >> 4) & 1) << 3); }
__device__ inline int swz_v(int d) { return (d & 15) ^ ((d >> 4) & 7); }

// A-operand row m of a 32-key S^T tile reads key pi(m): with the 32x32 MFMA
// accumulator layout (row 8*(r/4) + 4*g + r%4 in register r of lane half g)
// this puts key 16*g + r into register r.
__device__ inline int key_perm(int m) { return (((m >> 2) & 1) << 4) | ((m >> 3) << 2) | (m & 3); }

// 16-bit lane `sel` of word pair (lo word a, hi word b).
__device__ inline uint32_t pick_lo(uint32_t a, uint32_t b) { return (a & 0xffffu) | (b << 16); }
__device__ inline uint32_t pick_hi(uint32_t a, uint32_t b) { return (a >> 16) | (b & 0xffff0000u); }

__device__ inline uint32_t word(const uint4& v, int i) {
  return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

__device__ inline float xor32(float x) { return __shfl_xor(x, 32); }

__device__ inline int64_t block_token(const GridGeom& g, int t, int by, int bx, int j) {
  const int y = by * g.block_h + (j >> g.log2_bw);
  const int x = bx * g.block_w + (j & (g.block_w - 1));
  return ((int64_t)t * g.grid_h + y) * g.grid_w + x;
}

template <int BT>
struct Tile {
  static constexpr int kWaves = BT / 32;
  static constexpr int kThreads = kWaves * 64;
  static constexpr int kKeyTiles = BT / 32;
  static constexpr int kVChunks = BT / 8;        // 16-byte chunks per V^T row
  static constexpr int kKBytes = BT * 256;       // K tile: BT x 128 bf16
  static constexpr int kVBytes = 128 * BT * 2;   // V^T tile: 128 x BT bf16
  static constexpr int kRowStep = BT / 8;        // K rows between a thread's loads
};

template <int BT>
__global__ void __launch_bounds__(BT * 2) attend_fwd_kernel(AttendParams p) {
  using T = Tile<BT>;
  __shared__ __attribute__((aligned(16))) unsigned char smem[T::kKBytes + T::kVBytes];
  unsigned char* const ks = smem;
  unsigned char* const vt = smem + T::kKBytes;

  const GridGeom& g = p.g;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;

  const int64_t row = blockIdx.x;
  const int qb = (int)(row % g.nqb);
  const int64_t bh = row / g.nqb;
  const int h = (int)(bh % g.heads);
  const int b = (int)(bh / g.heads);
  const int tq = qb / g.nbf, qpos = qb - tq * g.nbf;
  const int qby = qpos / g.nbw, qbx = qpos - qby * g.nbw;

  // Q fragments: this lane's query row, channels 16s + 8*half .. +7.
  const int qi = wave * 32 + l32;
  const int64_t qtok = block_token(g, tq, qby, qbx, qi);
  bf16x8_t qf[8];
  {
    const uint16_t* qrow = p.q.data + (int64_t)b * p.q.sb + qtok * p.q.ss + (int64_t)h * p.q.sh;
#pragma unroll
    for (int s = 0; s < 8; ++s) qf[s] = as_bf16x8(load16(qrow + 16 * s + 8 * half));
  }

  int64_t start = p.row_ptr[row], end = p.row_ptr[row + 1];
  start = start < 0 ? 0 : (start > p.nnz ? p.nnz : start);
  end = end < start ? start : (end > p.nnz ? p.nnz : end);

  const uint16_t* kbase = p.k.data + (int64_t)b * p.k.sb + (int64_t)h * p.k.sh;
  const uint16_t* vbase = p.v.data + (int64_t)b * p.v.sb + (int64_t)h * p.v.sh;
  const int c = tid & 15;            // channel chunk this thread loads
  const int jk0 = tid >> 4;          // first K row this thread loads
  const int jv0 = (tid >> 4) * 8;    // first of the 8 V rows this thread loads

  uint4 kr[8], vr[8];
  auto load_block = [&](int kb) {
    const int t = kb / g.nbf, ps = kb - t * g.nbf;
    const int kby = ps / g.nbw, kbx = ps - kby * g.nbw;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t tk = block_token(g, t, kby, kbx, jk0 + T::kRowStep * i);
      kr[i] = load16(kbase + tk * p.k.ss + c * 8);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t tv = block_token(g, t, kby, kbx, jv0 + i);
      vr[i] = load16(vbase + tv * p.v.ss + c * 8);
    }
  };
  auto next_valid = [&](int64_t i) {
    while (i < end) {
      const int kb = __builtin_amdgcn_readfirstlane(p.col_idx[i]);
      if (kb >= 0 && kb < g.nkb) break;
      ++i;
    }
    return i;
  };

  f32x16_t o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dt][r] = 0.0f;
  float m_run = -__builtin_huge_valf(), l_run = 0.0f;
  const float sl2 = p.scale_log2;

  int64_t it = next_valid(start);
  if (it < end) load_block(__builtin_amdgcn_readfirstlane(p.col_idx[it]));

  while (it < end) {
    __syncthreads();  // every wave is done with the previous tiles
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int j = jk0 + T::kRowStep * i;
      *reinterpret_cast<uint4*>(ks + j * 256 + ((c ^ swz_k(j)) & 15) * 16) = kr[i];
    }
#pragma unroll
    for (int dd = 0; dd < 8; ++dd) {
      const int wi = dd >> 1;
      uint4 w;
      if (dd & 1) {
        w.x = pick_hi(word(vr[0], wi), word(vr[1], wi));
        w.y = pick_hi(word(vr[2], wi), word(vr[3], wi));
        w.z = pick_hi(word(vr[4], wi), word(vr[5], wi));
        w.w = pick_hi(word(vr[6], wi), word(vr[7], wi));
      } else {
        w.x = pick_lo(word(vr[0], wi), word(vr[1], wi));
        w.y = pick_lo(word(vr[2], wi), word(vr[3], wi));
        w.z = pick_lo(word(vr[4], wi), word(vr[5], wi));
        w.w = pick_lo(word(vr[6], wi), word(vr[7], wi));
      }
      const int d = 8 * c + dd;
      const int x = tid >> 4;
      *reinterpret_cast<uint4*>(vt + d * (BT * 2) + ((x ^ swz_v(d)) & (T::kVChunks - 1)) * 16) = w;
    }
    __syncthreads();  // tiles visible

    const int64_t nx = next_valid(it + 1);
    if (nx < end) load_block(__builtin_amdgcn_readfirstlane(p.col_idx[nx]));

    // ---- S^T = K Q^T, one 32x32 tile per 32 keys
    f32x16_t s[T::kKeyTiles];
#pragma unroll
    for (int kt = 0; kt < T::kKeyTiles; ++kt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kt][r] = 0.0f;
      const int j = 32 * kt + key_perm(l32);
      const unsigned char* krow = ks + j * 256;
      const int sw = swz_k(j);
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(krow + (((2 * st + half) ^ sw) & 15) * 16);
        s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[st], s[kt], 0, 0, 0);
      }
    }

    // ---- online softmax (one query per lane; keys split over lane ^ 32)
    float mx = s[0][0];
#pragma unroll
    for (int kt = 0; kt < T::kKeyTiles; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kt][r]);
    mx = fmaxf(mx, xor32(mx));
    const float m_new = fmaxf(m_run, mx * sl2);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    const float neg_m = -m_new;
    float rs = 0.0f;
    bf16x8_t pb[T::kKeyTiles][2];
#pragma unroll
    for (int kt = 0; kt < T::kKeyTiles; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = __builtin_amdgcn_exp2f(fmaf(s[kt][r], sl2, neg_m));
        rs += e;
        pb[kt][r >> 3][r & 7] = (__bf16)e;
      }
    l_run = l_run * alpha + rs;
    m_run = m_new;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;

    // ---- O^T += V^T P^T
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const int d = 32 * dt + l32;
      const unsigned char* vrow = vt + d * (BT * 2);
      const int sw = swz_v(d);
#pragma unroll
      for (int kt = 0; kt < T::kKeyTiles; ++kt)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          const int x = 4 * kt + 2 * half + s2;
          const bf16x8_t a =
              *reinterpret_cast<const bf16x8_t*>(vrow + ((x ^ sw) & (T::kVChunks - 1)) * 16);
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[kt][s2], o[dt], 0, 0, 0);
        }
    }
    it = nx;
  }

  // ---- epilogue: normalise, round to bf16, store; LSE
  const float l_tot = l_run + xor32(l_run);
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  uint16_t* orow = p.o + (int64_t)b * p.o_sb + qtok * p.o_ss + (int64_t)h * p.o_sh;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) {
      uint2 w;
      const __bf16 v0 = (__bf16)(o[dt][4 * a4 + 0] * inv);
      const __bf16 v1 = (__bf16)(o[dt][4 * a4 + 1] * inv);
      const __bf16 v2 = (__bf16)(o[dt][4 * a4 + 2] * inv);
      const __bf16 v3 = (__bf16)(o[dt][4 * a4 + 3] * inv);
      w.x = (uint32_t)__builtin_bit_cast(uint16_t, v0) | ((uint32_t)__builtin_bit_cast(uint16_t, v1) << 16);
      w.y = (uint32_t)__builtin_bit_cast(uint16_t, v2) | ((uint32_t)__builtin_bit_cast(uint16_t, v3) << 16);
      *reinterpret_cast<uint2*>(orow + 32 * dt + 8 * a4 + 4 * half) = w;
    }
  if (p.lse && half == 0) {
    const float lse = l_tot > 0.0f ? (m_run + __builtin_log2f(l_tot)) * 0.69314718055994531f
                                   : -__builtin_huge_valf();
    p.lse[((int64_t)b * g.heads + h) * g.q_tokens + qtok] = lse;
  }
}

}  // namespace

hipError_t launch_attend(const AttendParams& p, int block_tokens, hipStream_t stream) {
  if (p.rows <= 0) return hipSuccess;
  const dim3 grid((unsigned)p.rows);
  if (block_tokens == 128)
    hipLaunchKernelGGL(attend_fwd_kernel<128>, grid, dim3(Tile<128>::kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL(attend_fwd_kernel<64>, grid, dim3(Tile<64>::kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace lcsa
