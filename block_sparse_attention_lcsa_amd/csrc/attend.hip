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
// Work layout (wave64, 32x32x16 bf16 MFMA, BT = tokens per block):
//  * Each wave owns 32 query rows and computes S^T = K Q^T, so every lane
//    holds the scores of ONE query (lane & 31) against 16 keys per 32-key
//    tile: row max / row sum are per lane plus one permlane32 swap.
//  * K rows feed MFMA operand A in a permuted order chosen so that S^T
//    accumulator register r of lane half g holds key 16g + r.  Those 8-key
//    runs are exactly MFMA operand B of O^T = V^T P^T: P never leaves the
//    registers, and the O^T accumulator is again one query per lane, so the
//    online-softmax rescale is a per-lane scalar.
//  * K and V tiles stream HBM -> LDS with direct-to-LDS 16-byte loads (no
//    register staging), both row-major [key][128] with a 16-byte-chunk XOR
//    swizzle.  Operand A of V^T P^T is read with the LDS transpose read
//    (ds_read_b64_tr_b16), which returns 4 keys of one channel per lane.
//  * K and V buffers have separate lifetimes: V(i) streams in while S(i) and
//    the softmax run, K(i+1) while PV(i) runs; the loads of a tile are
//    spread over the MFMA loop (one per step) instead of issued in a burst.
//    Barriers are raw s_barrier with explicit vmcnt waits, so in-flight
//    tile loads are not drained at every barrier.
//  * Max-free softmax: P is computed against the running reference first;
//    only when some lane's partial row sum leaves [0, 2^16] (a row's first
//    block, or scores far above the reference) is the block max taken, O and
//    the row sum rescaled and P recomputed.  O and the row sum share the
//    reference, so the result is unchanged; P <= 2^16 keeps sums finite.
//  * Rows are visited head by head, in square tiles of block positions with
//    all query frames of a tile together.  The order is dealt to the XCDs
//    (workgroup id mod 8) in chunks of one XCD's resident workgroups, round
//    robin: the rows in flight on an XCD have overlapping windows and select
//    largely the same key blocks, which stay in that XCD's L2, and the eight
//    XCDs work on neighbouring chunks of one head, whose K/V then stay in the
//    memory-side cache.

#include <hip/hip_runtime.h>

#include "kernel_params.h"
#include "launch.h"

namespace lcsa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4_t;

// Largest partial row sum (64 values of P per lane) accepted without moving
// the softmax reference.
constexpr float kSumBound = 65536.0f;
constexpr int kXcds = 8;

__device__ inline uint4 load16(const uint16_t* ptr) { return *reinterpret_cast<const uint4*>(ptr); }

// CSR row at enumeration index e of the visiting order (batch*head, tile row,
// tile, query frame, position in the tile); tiles are tile x tile block
// positions, clipped at the right and bottom edges of the frame.
__device__ inline int64_t visit_row(const GridGeom& g, int tile, int64_t e) {
  const int64_t bh = e / g.nqb;
  int r = (int)(e - bh * g.nqb);
  const int qf = g.q_frames;
  const int band = tile * g.nbw * qf;            // indices per full tile row
  const int ty = r / band;
  r -= ty * band;
  const int th = min(tile, g.nbh - ty * tile);
  const int tx = r / (th * tile * qf);
  r -= tx * th * tile * qf;
  const int tw = min(tile, g.nbw - tx * tile);
  const int tq = r / (th * tw);
  const int pp = r - tq * th * tw;
  const int py = pp / tw, px = pp - py * tw;
  return bh * g.nqb + (int64_t)tq * g.nbf + (ty * tile + py) * g.nbw + tx * tile + px;
}
__device__ inline bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// 16-byte chunk swizzles of the row-major [key][128] tiles (16 chunks per
// 256-byte row).  K: conflict-free ds_read_b128 for the permuted key rows of
// an S^T operand.  V: conflict-free transpose reads (4 rows x 4 chunks per
// half wave).
__device__ inline int swz_k(int j) { return (j & 7) | (((j >> 4) & 1) << 3); }
__device__ inline int swz_v(int j) { return (j & 3) << 2; }

// A-operand row m of a 32-key S^T tile reads key key_perm(m): with the 32x32
// MFMA accumulator layout (row 8*(r/4) + 4*g + r%4 in register r of lane
// half g) this puts key 16*g + r into register r.
__device__ inline int key_perm(int m) { return (((m >> 2) & 1) << 4) | ((m >> 3) << 2) | (m & 3); }

__device__ inline int64_t block_token(const GridGeom& g, int t, int by, int bx, int j) {
  const int y = by * g.block_h + (j >> g.log2_bw);
  const int x = bx * g.block_w + (j & (g.block_w - 1));
  return ((int64_t)t * g.grid_h + y) * g.grid_w + x;
}

// n / d for 0 <= n < 2^31 with a host-computed magic multiplier.
__device__ inline int fast_div(int n, uint32_t m, uint32_t shift) {
  return (int)(((uint64_t)(uint32_t)n * m) >> shift);
}

// Workgroup barrier that completes this wave's own LDS reads (lgkmcnt) but
// leaves its in-flight HBM -> LDS tile loads (vmcnt) running.
__device__ inline void barrier_raw() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Wait until at most N vector-memory operations of this wave are pending.
template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  // gfx9 s_waitcnt: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt_hi[15:14]
  constexpr int imm = (N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(imm);
  asm volatile("" ::: "memory");
}

// One 16-byte-per-lane direct load HBM -> LDS: lane L's 16 bytes from
// sbase + voff land at LDS address lds_addr + 16 * L.  Issued as inline asm
// so that the compiler's conservative LDS-DMA tracking (which would drain all
// in-flight tile loads before any LDS read) does not apply; ordering is
// enforced with wait_vmcnt and barrier_raw instead.  The instruction writes
// only LDS and has no register result.  M0 holds the LDS destination and is
// listed as clobbered; the compiler keeps no value of its own in M0 in these
// kernels (none of the LDS instructions they use reads it; the generated code
// touches M0 only in these statements), so the clobber is sound even though
// clang warns that it cannot save a reserved register.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ inline void dma16(const void* sbase, int voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(lds_addr)
               : "memory", "m0");
}
#pragma clang diagnostic pop

__device__ inline uint32_t lds_address(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

__device__ inline float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int BT>
struct Tile {
  static constexpr int kWaves = BT / 32;
  static constexpr int kThreads = kWaves * 64;
  static constexpr int kKeyTiles = BT / 32;
  static constexpr int kTileBytes = BT * 256;               // BT x 128 bf16
  static constexpr int kLoads = kTileBytes / (kThreads * 16); // 16-byte loads per lane per tile
};

template <int BT>
__global__ void __launch_bounds__(BT * 2, 2) attend_fwd_kernel(AttendParams p) {
  using T = Tile<BT>;
  static_assert(T::kLoads == 8, "8 direct loads per lane per tile");
  __shared__ __attribute__((aligned(1024))) unsigned char k_lds[T::kTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char v_lds[T::kTileBytes];

  const GridGeom& g = p.g;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, l32 = lane & 31;

  // Work item: workgroups [0, full_rows) take whole rows, in an XCD-aware
  // order (workgroup ids go round-robin over the XCDs; XCD x takes chunks
  // x, x + 8, x + 16, ... of xcd_chunk rows of the visiting order, and the
  // rows past the last whole round of 8 chunks in plain order); later
  // workgroups take piece `piece` of a split row.
  // With a row order, workgroup i takes row order[i]: the order is meant to
  // be dispatched as it stands (longest rows first), round-robin over the
  // XCDs.
  int64_t row, item = -1;
  int piece = -1;
  {
    const int64_t pid = blockIdx.x, n = p.full_rows;
    if (pid < n) {
      if (p.order) {
        row = pid;
      } else {
        const int64_t c = p.xcd_chunk, whole = n / (kXcds * c) * (kXcds * c);
        if (pid < whole) {
          const int64_t xcd = pid % kXcds, idx = pid / kXcds;
          row = ((idx / c) * kXcds + xcd) * c + idx % c;
        } else {
          row = pid;
        }
      }
    } else {
      item = pid - n;
      row = n + item / p.pieces;
      piece = (int)(item % p.pieces);
    }
    row = p.order ? (int64_t)((const __attribute__((address_space(4))) int32_t*)p.order)[row]
                  : visit_row(g, p.tile, row);
  }
  const int qb = (int)(row % g.nqb);
  const int64_t bh = row / g.nqb;
  const int h = (int)(bh % g.heads);
  const int b = (int)(bh / g.heads);
  const int tq = qb / g.nbf, qpos = qb - tq * g.nbf;
  const int qby = qpos / g.nbw, qbx = qpos - qby * g.nbw;

  // The CSR is read-only here: read it through the constant address space so
  // the (uniform) reads become scalar loads, which do not wait on the vector
  // memory counter that tracks the in-flight tile loads.
  const __attribute__((address_space(4))) int32_t* row_ptr =
      (const __attribute__((address_space(4))) int32_t*)p.row_ptr;
  const __attribute__((address_space(4))) int32_t* col_idx =
      (const __attribute__((address_space(4))) int32_t*)p.col_idx;
  // Row bounds clamped to [0, nnz] (nnz < 2^31 is checked on the host).
  const int nnz = (int)p.nnz;
  int start = row_ptr[row], end = row_ptr[row + 1];
  start = start < 0 ? 0 : (start > nnz ? nnz : start);
  end = end < start ? start : (end > nnz ? nnz : end);
  // Entries outside [0, nkb) at the row's end (the -1 padding of a
  // threshold selection) are cut off before the row is split or walked, so
  // that a split row's pieces share its blocks evenly and a whole row does
  // not step through them one by one: one scalar load when the row ends in
  // a valid block, else one wave-wide look per 64 entries from the end.
  if (end > start) {
    const int last = col_idx[end - 1];
    if (last < 0 || last >= g.nkb) {
      int e = end, cut = start;
      while (e > start) {
        const int i = e - 64 + lane;
        const int kb = i >= start ? p.col_idx[i] : -1;
        const uint64_t m = __builtin_amdgcn_ballot_w64(kb >= 0 && kb < g.nkb);
        if (m) {
          cut = e - 64 + (64 - __clzll(m));
          break;
        }
        e -= 64;
      }
      end = cut;
    }
  }
  if (piece >= 0) {
    // consecutive parts of the row's CSR range
    const int64_t len = end - start;
    const int s0 = start + (int)(len * piece / p.pieces);
    end = start + (int)(len * (piece + 1) / p.pieces);
    start = s0;
  }
  start = __builtin_amdgcn_readfirstlane(start);
  end = __builtin_amdgcn_readfirstlane(end);

  // Q fragments (MFMA operand B of S^T): query lane&31, channels 16s+8*half..+7.
  const int qi = wave * 32 + l32;
  const int64_t qtok = block_token(g, tq, qby, qbx, qi);
  bf16x8_t qf[8];
  {
    const uint16_t* qrow = p.q.data + (int64_t)b * p.q.sb + qtok * p.q.ss + (int64_t)h * p.q.sh;
#pragma unroll
    for (int s = 0; s < 8; ++s) qf[s] = as_bf16x8(load16(qrow + 16 * s + 8 * half));
  }

  // Per-lane byte offsets (inside one key block) of the 8 direct loads of a
  // tile: load i of wave w fills LDS slots [(i*waves + w)*64, +64); slot s
  // holds row s>>4, logical chunk (s&15) ^ swizzle(row).
  const int row_stride_k = (int)(p.k.ss * 2), row_stride_v = (int)(p.v.ss * 2);
  int koff[8], voff[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int s = (i * T::kWaves + wave) * 64 + lane;
    const int j = s >> 4;
    const int tj = (j >> g.log2_bw) * g.grid_w + (j & (g.block_w - 1));  // token offset in block
    koff[i] = tj * row_stride_k + (((s & 15) ^ swz_k(j)) << 4);
    voff[i] = tj * row_stride_v + (((s & 15) ^ swz_v(j)) << 4);
  }
  const char* kbase = reinterpret_cast<const char*>(p.k.data + (int64_t)b * p.k.sb + (int64_t)h * p.k.sh);
  const char* vbase = reinterpret_cast<const char*>(p.v.data + (int64_t)b * p.v.sb + (int64_t)h * p.v.sh);
  auto block_tok0 = [&](int kb) {
    const int t = fast_div(kb, g.nbf_m, g.nbf_s), ps = kb - t * g.nbf;
    const int kby = fast_div(ps, g.nbw_m, g.nbw_s), kbx = ps - kby * g.nbw;
    return ((int64_t)g.kv_slot[t] * g.grid_h + (int64_t)kby * g.block_h) * g.grid_w +
           (int64_t)kbx * g.block_w;
  };
  const uint32_t k_lds_addr = lds_address(k_lds) + wave * 1024;
  const uint32_t v_lds_addr = lds_address(v_lds) + wave * 1024;
  // Next CSR position >= i holding a valid key block (uniform; scalar loads).
  auto next_valid = [&](int i, int& kbv) {
    i = __builtin_amdgcn_readfirstlane(i);
    kbv = 0;
    while (i < end) {
      const int kb = col_idx[i];
      if (kb >= 0 && kb < g.nkb) {
        kbv = kb;
        break;
      }
      i = __builtin_amdgcn_readfirstlane(i + 1);
    }
    return i;
  };

  // LDS read addresses of this lane.
  // S^T operand A: row 32*kt + key_perm(l32), chunk (2*st + half) ^ swz_k.
  const int kp = key_perm(l32);
  const int ksw = swz_k(kp);
  const unsigned char* krow = k_lds + kp * 256;
  // V^T operand A via transpose reads: 16-lane group G = lane >> 4 covers
  // channels 32*dt + 16*(G&1) .. +15 and keys 32*kt + 16*half + 8*s2 + 4*r
  // + 0..3; lane s of the group points at row (s >> 2) of that 4-key run,
  // channels 4*(s & 3) .. +3 of the group's 16.
  const int gs = lane & 15, grp = lane >> 4;
  const unsigned char* vrow = v_lds + (16 * half + (gs >> 2)) * 256 + (gs & 1) * 8;
  const int vchunk_lo = 2 * (grp & 1) + ((gs & 3) >> 1);
  const int vsw = swz_v(gs >> 2);

  f32x16_t o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dt][r] = 0.0f;
  float m_run = -__builtin_huge_valf(), l_run = 0.0f;
  const float sl2 = p.scale_log2;

  int kb_cur;
  int it = next_valid(start, kb_cur);
  const int first = it;
  int64_t tok_cur = 0;
  if (it < end) {   // K of the first block
    tok_cur = block_tok0(kb_cur);
    const char* src = kbase + tok_cur * row_stride_k;
#pragma unroll
    for (int i = 0; i < 8; ++i) dma16(src, koff[i], k_lds_addr + i * T::kWaves * 1024);
  }

  while (it < end) {
    // V(it) is issued one load per S step below, so the loads do not queue
    // up in front of the MFMAs.  The next valid block and its first token
    // (two scalar round trips: the CSR entry, then the frame slot) are
    // settled here, before the waits, where the wave waits for K(it) anyway;
    // left to the compiler they land in front of the softmax.
    const char* vsrc = vbase + tok_cur * row_stride_v;
    int kb_nx;
    const int nx = next_valid(it + 1, kb_nx);
    const int64_t tok_nx = nx < end ? block_tok0(kb_nx) : tok_cur;
    // K(nx) is issued one load per PV step below (after the V barrier, when
    // every wave is done with K(it)); on the last block the current block is
    // re-read instead, which keeps the loop body branch-free.
    const char* ksrc = kbase + tok_nx * row_stride_k;
    asm volatile("" : "+s"(vsrc), "+s"(ksrc));
    wait_vmcnt<0>();          // K(it) landed (this wave's share)
    barrier_raw();            // ... everyone's; V buffer free (PV of it-1 done)

    // ---- S^T = K Q^T (the first step starts from a zero accumulator)
    f32x16_t s[T::kKeyTiles];
    // K operands of step st + 1 are read while the MFMAs of step st run;
    // scheduling barriers keep the compiler from sinking the reads back next
    // to their MFMAs.
    bf16x8_t ka[2][T::kKeyTiles];
#pragma unroll
    for (int kt = 0; kt < T::kKeyTiles; ++kt)
      ka[0][kt] = *reinterpret_cast<const bf16x8_t*>(krow + kt * 32 * 256 + ((half ^ ksw) & 15) * 16);
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      if (st < 7) {
        const int offn = (((2 * (st + 1) + half) ^ ksw) & 15) * 16;
#pragma unroll
        for (int kt = 0; kt < T::kKeyTiles; ++kt)
          ka[(st + 1) & 1][kt] = *reinterpret_cast<const bf16x8_t*>(krow + kt * 32 * 256 + offn);
      }
      dma16(vsrc, voff[st], v_lds_addr + st * T::kWaves * 1024);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kt = 0; kt < T::kKeyTiles; ++kt) {
        const bf16x8_t a = ka[st & 1][kt];
        if (st == 0) {
          const f32x16_t zero = {};
          s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[0], zero, 0, 0, 0);
        } else {
          s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[st], s[kt], 0, 0, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }

    // Wave priorities: softmax 2, PV 1, S 0.  The two waves sharing a SIMD
    // come from different workgroups and tend to fall into step (the one
    // behind gets the MFMA pipe to itself while the other runs its softmax,
    // and catches up), after which their VALU and MFMA phases coincide.
    // Favouring the softmax and then PV keeps them apart.
    __builtin_amdgcn_s_setprio(2);
    // ---- online softmax (one query per lane, keys split over lane ^ 32)
    // P = exp2(S * scale*log2(e) - m_run) rounded to bf16 pairs; the row sum
    // adds exactly these rounded values (dot with (1, 1)), one chain per key
    // tile.  The reference m_run moves only when some lane's partial row sum
    // leaves [0, kSumBound]: on a row's first block (m_run = -inf gives
    // infinite sums) and when a block's scores rise far above m_run.  Then
    // the block max is taken, O and the row sum are rescaled, and P is
    // recomputed.  Otherwise no max is needed: P <= kSumBound keeps every
    // accumulation finite, and O and the row sum share the reference.
    const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};
    bf16x8_t pb[T::kKeyTiles][2];
    auto make_p = [&](const float neg_m) __attribute__((always_inline)) {
      float rs[T::kKeyTiles];
#pragma unroll
      for (int kt = 0; kt < T::kKeyTiles; ++kt) {
        rs[kt] = 0.0f;
        bf16x2_t pp[8];
#pragma unroll
        for (int r2 = 0; r2 < 8; ++r2) {
          f32x2_t e;
          e[0] = __builtin_amdgcn_exp2f(fmaf(s[kt][2 * r2], sl2, neg_m));
          e[1] = __builtin_amdgcn_exp2f(fmaf(s[kt][2 * r2 + 1], sl2, neg_m));
          pp[r2] = __builtin_convertvector(e, bf16x2_t);
          rs[kt] = __builtin_amdgcn_fdot2_f32_bf16(pp[r2], ones, rs[kt], false);
        }
        pb[kt][0] = __builtin_shufflevector(__builtin_shufflevector(pp[0], pp[1], 0, 1, 2, 3),
                                            __builtin_shufflevector(pp[2], pp[3], 0, 1, 2, 3),
                                            0, 1, 2, 3, 4, 5, 6, 7);
        pb[kt][1] = __builtin_shufflevector(__builtin_shufflevector(pp[4], pp[5], 0, 1, 2, 3),
                                            __builtin_shufflevector(pp[6], pp[7], 0, 1, 2, 3),
                                            0, 1, 2, 3, 4, 5, 6, 7);
      }
      float sum = rs[0];
#pragma unroll
      for (int kt = 1; kt < T::kKeyTiles; ++kt) sum += rs[kt];
      return sum;
    };
    // On a row's first block the reference is -inf and P against it would
    // only be thrown away: go straight to the max.
    float rsum = it == first ? __builtin_huge_valf() : make_p(-m_run);
    if (__builtin_amdgcn_ballot_w64(!(rsum <= kSumBound)) != 0) {
      // Independent max chains per key tile keep the reduction short.
      float mt[T::kKeyTiles];
#pragma unroll
      for (int kt = 0; kt < T::kKeyTiles; ++kt) {
        mt[kt] = fmaxf(s[kt][0], s[kt][1]);
#pragma unroll
        for (int r = 2; r < 16; ++r) mt[kt] = fmaxf(mt[kt], s[kt][r]);
      }
      float mx = mt[0];
#pragma unroll
      for (int kt = 1; kt < T::kKeyTiles; ++kt) mx = fmaxf(mx, mt[kt]);
      const float m_new = fmaxf(m_run, pair_max(mx) * sl2);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
      rsum = make_p(-m_run);
    }
    l_run += rsum;

    wait_vmcnt<0>();          // V(it) landed (the only loads in flight)
    barrier_raw();            // ... everyone's; every wave is past S, so K(it) is free

    __builtin_amdgcn_s_setprio(1);
    // ---- O^T += V^T P^T
    // V^T operands of PV step j + 1 are read while the MFMAs of step j run
    // (scheduling barriers keep the order).
    constexpr int kPvSteps = 2 * T::kKeyTiles, kPerStep = 8 / kPvSteps;
    static_assert(kPerStep * kPvSteps == 8, "K loads spread evenly over PV steps");
    auto vfrag = [&](int j, int dt) __attribute__((always_inline)) {
      const int off = (((4 * dt + vchunk_lo) ^ vsw) & 15) * 16;
      const unsigned char* base = vrow + (32 * (j >> 1) + 8 * (j & 1)) * 256 + off;
      const bf16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(base));
      const bf16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(base + 4 * 256));
      return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    };
    bf16x8_t va[2][4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) va[0][dt] = vfrag(0, dt);
#pragma unroll
    for (int j = 0; j < kPvSteps; ++j) {
      if (j + 1 < kPvSteps) {
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) va[(j + 1) & 1][dt] = vfrag(j + 1, dt);
      }
      // loads [j*L, j*L + L) of K(nx) at PV step j, L = 8 / steps
#pragma unroll
      for (int i = j * kPerStep; i < (j + 1) * kPerStep; ++i)
        dma16(ksrc, koff[i], k_lds_addr + i * T::kWaves * 1024);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[j & 1][dt], pb[j >> 1][j & 1], o[dt], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
    it = nx;
    tok_cur = tok_nx;
  }
  wait_vmcnt<0>();            // no load may still target LDS when the workgroup retires

  const float l_tot = pair_sum(l_run);
  if (piece >= 0) {
    // ---- split row: unnormalised O and (m, l) of this piece, in float32
    float* op = p.part + (item * BT + qi) * 128;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const float4 w = {o[dt][4 * a4 + 0], o[dt][4 * a4 + 1], o[dt][4 * a4 + 2], o[dt][4 * a4 + 3]};
        *reinterpret_cast<float4*>(op + 32 * dt + 8 * a4 + 4 * half) = w;
      }
    if (half == 0) {
      const int64_t items = (p.rows - p.full_rows) * p.pieces;
      const float2 ml = {m_run, l_tot};
      *reinterpret_cast<float2*>(p.part + items * BT * 128 + (item * BT + qi) * 2) = ml;
    }
    return;
  }

  // ---- epilogue: normalise, round to bf16, store; LSE
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

// Merge of split rows: workgroup (x, y) takes split row x, queries 16 y ..
// 16 y + 15; thread t handles query 16 y + t / 16 and channels 8 (t % 16) ..
// +7, so 16 lanes read one query's 512-byte partial row.  Pieces hold O and
// the row sum against their own reference m (log2 units); the merge rescales
// them to a running maximum, four pieces at a time.  A row whose pieces hold
// no valid block gives O = 0, LSE = -inf.
constexpr int kMergeThreads = 256;
template <int BT>
__global__ void __launch_bounds__(kMergeThreads) attend_merge_kernel(AttendParams p) {
  const GridGeom& g = p.g;
  const int64_t tr = blockIdx.x;
  const int64_t row = p.order ? (int64_t)p.order[p.full_rows + tr] : visit_row(g, p.tile, p.full_rows + tr);
  const int t = threadIdx.x, qi = (int)blockIdx.y * 16 + (t >> 4), c0 = (t & 15) * 8;
  const int qb = (int)(row % g.nqb);
  const int64_t bh = row / g.nqb;
  const int h = (int)(bh % g.heads);
  const int b = (int)(bh / g.heads);
  const int tq = qb / g.nbf, qpos = qb - tq * g.nbf;
  const int qby = qpos / g.nbw, qbx = qpos - qby * g.nbw;
  const int64_t qtok = block_token(g, tq, qby, qbx, qi);
  const int64_t items = (p.rows - p.full_rows) * p.pieces;
  const float* ml = p.part + items * BT * 128;

  // Pieces in groups of four: all loads of a group are issued before any
  // use, and groups fold into a running (m, l, acc) with one rescale each.
  constexpr int kG = 4;
  float m = -__builtin_huge_valf(), l = 0.0f;
  float acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) acc[c] = 0.0f;
  for (int pc0 = 0; pc0 < p.pieces; pc0 += kG) {
    const int np = min(kG, p.pieces - pc0);
    float2 mlp[kG];
    float4 x[kG][2];
#pragma unroll
    for (int u = 0; u < kG; ++u) {
      if (u < np) {
        const int64_t it = tr * p.pieces + pc0 + u;
        mlp[u] = *reinterpret_cast<const float2*>(ml + (it * BT + qi) * 2);
        const float4* src = reinterpret_cast<const float4*>(p.part + (it * BT + qi) * 128 + c0);
        x[u][0] = src[0];
        x[u][1] = src[1];
      }
    }
    float mc = m;
#pragma unroll
    for (int u = 0; u < kG; ++u)
      if (u < np) mc = fmaxf(mc, mlp[u].x);
    if (mc > -__builtin_huge_valf()) {
      const float sc = __builtin_amdgcn_exp2f(m - mc);   // 0 while nothing was held
      l *= sc;
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[c] *= sc;
#pragma unroll
      for (int u = 0; u < kG; ++u) {
        if (u < np) {
          const float w = __builtin_amdgcn_exp2f(mlp[u].x - mc);   // 0 for an empty piece
          l = fmaf(w, mlp[u].y, l);
#pragma unroll
          for (int c4 = 0; c4 < 2; ++c4) {
            acc[4 * c4 + 0] = fmaf(w, x[u][c4].x, acc[4 * c4 + 0]);
            acc[4 * c4 + 1] = fmaf(w, x[u][c4].y, acc[4 * c4 + 1]);
            acc[4 * c4 + 2] = fmaf(w, x[u][c4].z, acc[4 * c4 + 2]);
            acc[4 * c4 + 3] = fmaf(w, x[u][c4].w, acc[4 * c4 + 3]);
          }
        }
      }
      m = mc;
    }
  }
  const float inv = l > 0.0f ? 1.0f / l : 0.0f;
  uint16_t* orow = p.o + (int64_t)b * p.o_sb + qtok * p.o_ss + (int64_t)h * p.o_sh + c0;
  uint4 w;
  uint32_t* wp = reinterpret_cast<uint32_t*>(&w);
#pragma unroll
  for (int k2 = 0; k2 < 4; ++k2) {
    f32x2_t x;
    x[0] = acc[2 * k2] * inv;
    x[1] = acc[2 * k2 + 1] * inv;
    wp[k2] = __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2_t));
  }
  *reinterpret_cast<uint4*>(orow) = w;
  if (p.lse && c0 == 0) {
    const float lse = l > 0.0f ? (m + __builtin_log2f(l)) * 0.69314718055994531f : -__builtin_huge_valf();
    p.lse[((int64_t)b * g.heads + h) * g.q_tokens + qtok] = lse;
  }
}

// Longest-first row order for CSRs whose rows differ in length (threshold
// selections, caller masks).  Workgroups take rows in dispatch order, so with
// rows in the visiting order a long row started late sets the finish time;
// longest first, the short rows fill in at the end and the rows of the last,
// partly filled round, which are split, are the shortest.

// len[r]: row r's CSR range after the entries outside [0, nkb) at its end are
// cut off, as the attention kernel cuts them (one wave per row).
__global__ void __launch_bounds__(256) row_len_kernel(const int32_t* row_ptr, const int32_t* col_idx,
                                                      int64_t nnz, int64_t rows, int nkb,
                                                      int32_t* len) {
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= rows) return;
  const int n = (int)nnz;
  int start = row_ptr[r], end = row_ptr[r + 1];
  start = start < 0 ? 0 : (start > n ? n : start);
  end = end < start ? start : (end > n ? n : end);
  int e = end, cut = start;
  while (e > start) {
    const int i = e - 64 + lane;
    const int kb = i >= start ? col_idx[i] : -1;
    const uint64_t m = __builtin_amdgcn_ballot_w64(kb >= 0 && kb < nkb);
    if (m) {
      cut = e - 64 + (64 - __clzll(m));
      break;
    }
    e -= 64;
  }
  if (lane == 0) len[r] = cut - start;
}

// order: the rows by descending length (lengths of kOrderBuckets - 1 and up
// share the first bucket), rows of equal length in the visiting order (which
// keeps neighbouring positions together for the L2 caches).  One workgroup:
// each wave counts the lengths of its contiguous share of the visiting order,
// the counts give every (bucket, wave) its first position, and each wave
// then places its rows, 64 at a time, ranking lanes of equal length by lane.
// Stable, so the order is the same on every run.
constexpr int kOrderBuckets = 512;
constexpr int kOrderWaves = 16;
__global__ void __launch_bounds__(kOrderWaves * 64) row_order_kernel(GridGeom g, int tile,
                                                                     int64_t rows,
                                                                     const int32_t* len,
                                                                     int32_t* order) {
  __shared__ int32_t base[kOrderWaves][kOrderBuckets];
  __shared__ int32_t total[2][kOrderBuckets];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < kOrderWaves * kOrderBuckets; i += kOrderWaves * 64) (&base[0][0])[i] = 0;
  __syncthreads();
  const int64_t per = (rows + kOrderWaves - 1) / kOrderWaves;
  const int64_t e0 = min(rows, wave * per), e1 = min(rows, e0 + per);
  auto bucket = [&](int64_t row) {
    const int l = len[row];
    return kOrderBuckets - 1 - (l < 0 ? 0 : (l > kOrderBuckets - 1 ? kOrderBuckets - 1 : l));
  };
  for (int64_t e = e0 + lane; e < e1; e += 64) atomicAdd(&base[wave][bucket(visit_row(g, tile, e))], 1);
  __syncthreads();
  // exclusive prefix of the bucket totals (bucket 0 = longest; a scan in
  // log2(buckets) steps), then of the waves within each bucket
  static_assert(kOrderBuckets <= kOrderWaves * 64, "one thread per bucket");
  int own = 0;
  if (tid < kOrderBuckets) {
    for (int w = 0; w < kOrderWaves; ++w) own += base[w][tid];
    total[0][tid] = own;
  }
  __syncthreads();
  int src = 0;
  for (int d = 1; d < kOrderBuckets; d <<= 1) {
    if (tid < kOrderBuckets)
      total[src ^ 1][tid] = total[src][tid] + (tid >= d ? total[src][tid - d] : 0);
    src ^= 1;
    __syncthreads();
  }
  if (tid < kOrderBuckets) {
    int s = total[src][tid] - own;
    for (int w = 0; w < kOrderWaves; ++w) {
      const int c = base[w][tid];
      base[w][tid] = s;
      s += c;
    }
  }
  __syncthreads();
  const uint64_t below = (1ull << lane) - 1ull;
  for (int64_t c0 = e0; c0 < e1; c0 += 64) {
    const int64_t e = c0 + lane;
    const bool ok = e < e1;
    const int64_t row = ok ? visit_row(g, tile, e) : 0;
    const int b = ok ? bucket(row) : -1;
    int rank = 0, cnt = 0;
    uint64_t todo = __builtin_amdgcn_ballot_w64(ok);
    while (todo) {
      const int bl = __builtin_amdgcn_readlane(b, __builtin_ctzll(todo));
      const uint64_t m = __builtin_amdgcn_ballot_w64(ok && b == bl);
      if (ok && b == bl) {
        rank = __popcll(m & below);
        cnt = __popcll(m);
      }
      todo &= ~m;
    }
    if (ok) order[base[wave][b] + rank] = (int32_t)row;
    // every lane has read its base above (a wave's LDS operations complete
    // in order); the first lane of each length moves it on
    if (ok && rank == 0) base[wave][b] += cnt;
  }
}

template <int BT>
hipError_t launch_bt(const AttendParams& p, hipStream_t stream) {
  const int64_t split = p.rows - p.full_rows;
  const int64_t groups = p.full_rows + split * p.pieces;
  hipLaunchKernelGGL(attend_fwd_kernel<BT>, dim3((unsigned)groups), dim3(Tile<BT>::kThreads), 0,
                     stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || split == 0) return e;
  hipLaunchKernelGGL(attend_merge_kernel<BT>, dim3((unsigned)split, BT / 16), dim3(kMergeThreads), 0,
                     stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attend(const AttendParams& p, int block_tokens, hipStream_t stream) {
  if (p.rows <= 0) return hipSuccess;
  return block_tokens == 128 ? launch_bt<128>(p, stream) : launch_bt<64>(p, stream);
}

hipError_t launch_row_order(const AttendParams& p, int32_t* len, int32_t* order,
                            hipStream_t stream) {
  if (p.rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(row_len_kernel, dim3((unsigned)((p.rows + 3) / 4)), dim3(256), 0, stream,
                     p.row_ptr, p.col_idx, p.nnz, p.rows, p.g.nkb, len);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(row_order_kernel, dim3(1), dim3(kOrderWaves * 64), 0, stream, p.g, p.tile,
                     p.rows, static_cast<const int32_t*>(len), order);
  return hipGetLastError();
}

}  // namespace lcsa
