// Pyramid summaries and their incremental update ("Attention clairsemée PISA :
// noyaux Triton sans matrice de scores", section "Le pooling comme première
// réduction": a node summarises its keys, so appending keys changes only the
// nodes that hold them).
//
// Shared by the pooling kernels and by the decode step that appends its tokens
// in the same launch as its selection.
#pragma once

#include <type_traits>

#include "pisa_internal.h"

namespace pisa {

// Rows a lane slot adds per round in a leaf sum (the build's and the append's).
constexpr int kPoolUnroll = 8;

// Summary arithmetic: the mean (fp64 sums, one rounding) or the element-wise
// maximum (exact).
template <bool MX>
struct Pool {
  using Acc = typename std::conditional<MX, float, double>::type;
  __device__ __forceinline__ static Acc init() { return MX ? (Acc)-__builtin_inff() : (Acc)0; }
  __device__ __forceinline__ static Acc add(Acc a, float x) {
    if constexpr (MX) return fmaxf(a, x);
    else return a + (double)x;
  }
  // a row read from a clamped address (past the block) repeats the last row:
  // harmless for the maximum, left out of the sum
  __device__ __forceinline__ static Acc add_row(Acc a, float x, bool real) {
    if constexpr (MX) return fmaxf(a, x);
    else return a + (real ? (double)x : 0.0);
  }
  __device__ __forceinline__ static Acc join(Acc a, Acc b) {
    if constexpr (MX) return fmaxf(a, b);
    else return a + b;
  }
  // summary of `count` folded values; for a power-of-two count the multiply by
  // its reciprocal is the exact quotient
  __device__ __forceinline__ static float fin(Acc a, int count) {
    if constexpr (MX) return a;
    else return (float)((count & (count - 1)) == 0 ? a * (1.0 / (double)count) : a / (double)count);
  }
};

// 16-byte units of LDS an append stages CH key rows in.
template <typename T, int D, int CH>
constexpr int kAppendRowUnits = CH * D / Wide<T>::kVec;

// The append for one (batch, kv head) slab, by a workgroup of NT threads: the
// nodes holding tokens [len0, len1) are recomputed over their tokens before
// len1, so that each equals what the build gives for a cache of len1 tokens.
// Nothing is written when len0 < 0, len1 > N or len0 >= len1 (uniform). `rows`
// is LDS of kAppendRowUnits<T, D, CH> units; a leaf's rows are staged there CH
// at a time. Ends with a workgroup barrier after its last write.
template <typename T, int D, bool MX, int NT, int CH>
__device__ void append_slab(const Geo& g, const T* __restrict__ k, float* __restrict__ pyr, int slab, int len0,
                            int len1, uint4* rows) {
  using PO = Pool<MX>;
  constexpr int VEC = Wide<T>::kVec;
  constexpr int LPR = D / VEC;
  constexpr int RPI = 64 / LPR;
  if (len0 < 0 || len1 > g.N || len0 >= len1) return;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = (lane % LPR) * VEC;
  const int rsub = lane / LPR;
  const T* kb = k + (int64_t)slab * g.N * D;
  float* pb = pyr + (int64_t)slab * g.off[g.L] * D;
  int a = len0 / g.bs, z = (len1 - 1) / g.bs;  // affected nodes of the level being built
  // Each affected leaf, its rows staged in LDS CH at a time by all
  // waves: the first wave sums them exactly as pool_leaf_kernel sums a block --
  // lane slot rsub adds rows r0 + rsub, r0 + rsub + RPI, ... in ascending order,
  // in rounds of kPoolUnroll rows, the rows of a last partial round past r1
  // adding +0.0; then the slots fold by xor over the lane bits -- so the summary
  // equals the build's bit for bit. A chunk holds whole rounds.
  constexpr int ROUND = RPI * kPoolUnroll;
  static_assert(CH % ROUND == 0, "a chunk of whole rounds");
  for (int j = a; j <= z; ++j) {
    const int r0 = j * g.bs;
    const int nrows = min(len1, r0 + g.bs) - r0;  // rows of the leaf present
    const int nfull = nrows / ROUND;               // full rounds
    const T* src = kb + (int64_t)r0 * D;
    typename PO::Acc acc[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] = PO::init();
    int it = 0;     // rounds added
    int rr = rsub;  // this lane slot's next row within the leaf
    for (int c0 = 0; c0 < nrows; c0 += CH) {
      const int units = min(CH, nrows - c0) * LPR;
      for (int e = threadIdx.x; e < units; e += NT)
        rows[e] = Wide<T>::raw(src + (int64_t)(c0 + e / LPR) * D + (e % LPR) * VEC);
      __syncthreads();
      if (wave == 0) {
        const int rend = min(nfull, (c0 + CH) / ROUND);
        for (; it < rend; ++it) {
#pragma unroll
          for (int u = 0; u < kPoolUnroll; ++u, rr += RPI) {
            float x[VEC];
            Wide<T>::widen(rows[(rr - c0) * LPR + col / VEC], x);
#pragma unroll
            for (int e = 0; e < VEC; ++e) acc[e] = PO::add(acc[e], x[e]);
          }
        }
        if (c0 + CH >= nrows && nfull * ROUND < nrows) {  // the last chunk holds the partial round
#pragma unroll
          for (int u = 0; u < kPoolUnroll; ++u, rr += RPI) {
            // rows past the leaf add +0.0 to the sum (the maximum ignores them)
            uint4 raw = rr < nrows ? rows[(rr - c0) * LPR + col / VEC] : make_uint4(0u, 0u, 0u, 0u);
            if constexpr (MX)
              if (rr >= nrows) raw = rows[(nrows - 1 - c0) * LPR + col / VEC];
            float x[VEC];
            Wide<T>::widen(raw, x);
#pragma unroll
            for (int e = 0; e < VEC; ++e) acc[e] = PO::add(acc[e], x[e]);
          }
        }
      }
      __syncthreads();
    }
    if (wave == 0) {
#pragma unroll
      for (int sh = LPR; sh < 64; sh <<= 1)
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[e] = PO::join(acc[e], __shfl_xor(acc[e], sh));
      if (rsub == 0) {
        float outv[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) outv[e] = PO::fin(acc[e], nrows);
        float* dst = pb + (int64_t)j * D + col;
#pragma unroll
        for (int e = 0; e < VEC; e += 4)
          *reinterpret_cast<float4*>(dst + e) = make_float4(outv[e], outv[e + 1], outv[e + 2], outv[e + 3]);
      }
    }
    __syncthreads();
  }
  int present = z + 1;  // nodes of the level below that hold tokens before len1
  for (int l = 1; l < g.L; ++l) {
    const int na = a / g.f, nz = z / g.f;
    for (int e = threadIdx.x; e < (nz - na + 1) * D; e += NT) {
      const int n = na + e / D, c = e % D;
      const int c0 = n * g.f;
      const int c1 = min(c0 + g.f, present);
      typename PO::Acc sum = PO::init();
      for (int ch = c0; ch < c1; ++ch) sum = PO::add(sum, pb[(int64_t)(g.off[l - 1] + ch) * D + c]);
      pb[(int64_t)(g.off[l] + n) * D + c] = PO::fin(sum, c1 - c0);
    }
    __syncthreads();
    a = na;
    z = nz;
    present = (present + g.f - 1) / g.f;
  }
}

}  // namespace pisa
