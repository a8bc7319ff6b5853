// Key pyramid by pooling -- the mean, or the element-wise maximum as a variant ("Attention clairsemée PISA : noyaux Triton sans
// matrice de scores", sections "Une pyramide de clés plutôt qu'un tapis
// uniforme" and "Le pooling comme première réduction").
//
// Level 0 (one summary per key block) and level 1 come from one streaming pass
// over K: a workgroup owns one level-1 node (fanout consecutive blocks), each
// wave reduces whole blocks with 16-byte loads and fp64 accumulators, and the
// workgroup folds its blocks' stored fp32 summaries into the level-1 node.
// Coarser levels are tiny: one more launch folds them all, a workgroup per
// top-level node.
#include <type_traits>

#include "pisa_internal.h"

namespace pisa {
namespace {

constexpr int kPoolThreads = 256;
constexpr int kUnroll = 8;
constexpr int kMaxChunk = 16;  // blocks per workgroup (fanout <= 16)

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

template <typename T, int D, bool MX>
__global__ __launch_bounds__(kPoolThreads) __attribute__((amdgpu_waves_per_eu(4))) void pool_leaf_kernel(Geo g, const T* __restrict__ k,
                                                                  float* __restrict__ pyr, int chunk_blocks) {
  using PO = Pool<MX>;
  constexpr int VEC = Wide<T>::kVec;
  constexpr int LPR = D / VEC;   // lanes covering one key row
  constexpr int RPI = 64 / LPR;  // rows one wave instruction covers
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = (lane % LPR) * VEC;
  const int rsub = lane / LPR;
  const int slab = blockIdx.y;
  const T* kb = k + (int64_t)slab * g.N * D;
  float* pb = pyr + (int64_t)slab * g.off[g.L] * D;

  __shared__ float leaf[kMaxChunk][D];
  const int j_first = blockIdx.x * chunk_blocks;
  const int nblk = min(chunk_blocks, g.nb - j_first);

  for (int jj = wave; jj < nblk; jj += kPoolThreads / 64) {
    const int j = j_first + jj;
    const int r0 = j * g.bs;
    const int r1 = min(g.N, r0 + g.bs);
    typename PO::Acc acc[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] = PO::init();
    // rounds of kUnroll loads covering whole row groups run unmasked; one masked
    // round (clamped rows) takes the rest
    const int nfull = (r1 - r0) / (RPI * kUnroll);  // uniform
    const T* ptr = kb + (int64_t)(r0 + rsub) * D + col;
#pragma unroll 1
    for (int it = 0; it < nfull; ++it, ptr += RPI * kUnroll * D) {
      uint4 raw[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) raw[u] = Wide<T>::stream(ptr + u * RPI * D);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        float x[VEC];
        Wide<T>::widen(raw[u], x);
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[e] = PO::add(acc[e], x[e]);
      }
    }
    const int r = r0 + nfull * RPI * kUnroll + rsub;
    if (r0 + nfull * RPI * kUnroll < r1) {
      uint4 raw[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)  // unconditional loads from clamped rows, all in flight
        raw[u] = Wide<T>::stream(kb + (int64_t)min(r + u * RPI, r1 - 1) * D + col);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        // a clamped row repeats the block's last row: harmless for the maximum;
        // for the sum its bits are cleared (+0.0) before widening
        if constexpr (!MX)
          if (r + u * RPI >= r1) raw[u] = make_uint4(0u, 0u, 0u, 0u);
        float x[VEC];
        Wide<T>::widen(raw[u], x);
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[e] = PO::add(acc[e], x[e]);
      }
    }
    // fold the row slots that share these columns
#pragma unroll
    for (int s = LPR; s < 64; s <<= 1)
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[e] = PO::join(acc[e], __shfl_xor(acc[e], s));
    if (rsub == 0) {
      float outv[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        // the mean divides by the row count (a power of two for full blocks, exact)
        outv[e] = PO::fin(acc[e], r1 - r0);
        leaf[jj][col + e] = outv[e];
      }
      float* dst = pb + (int64_t)j * D + col;
#pragma unroll
      for (int e = 0; e < VEC; e += 4) *reinterpret_cast<float4*>(dst + e) = make_float4(outv[e], outv[e + 1], outv[e + 2], outv[e + 3]);
    }
  }
  if (g.L < 2) return;
  __syncthreads();
  for (int c = threadIdx.x; c < D; c += kPoolThreads) {
    typename PO::Acc s = PO::init();
    for (int jj = 0; jj < nblk; ++jj) s = PO::add(s, leaf[jj][c]);
    pb[(int64_t)(g.off[1] + blockIdx.x) * D + c] = PO::fin(s, nblk);
  }
}

// Update after an append: tokens [len0, len1) of sequence b were written to the
// key cache. Every node whose tokens meet [len0, len1) is recomputed over its
// tokens before len1 -- leaves from the key rows, coarser nodes from the
// children present at len1 -- which leaves the pyramid equal, node for node, to
// one built over the first len1 tokens. Nodes before len0 are untouched. One
// workgroup per (batch, kv head); a decode step's append touches one leaf and
// one node per coarser level.
template <typename T, int D, bool MX>
__global__ __launch_bounds__(kPoolThreads) void pool_append_kernel(Geo g, const T* __restrict__ k,
                                                                   float* __restrict__ pyr,
                                                                   const int32_t* __restrict__ old_lens,
                                                                   const int32_t* __restrict__ new_lens) {
  using PO = Pool<MX>;
  constexpr int VEC = Wide<T>::kVec;
  constexpr int LPR = D / VEC;
  constexpr int RPI = 64 / LPR;
  const int slab = blockIdx.x;
  const int b = slab / g.Hkv;
  const int len0 = old_lens[b];
  const int len1 = new_lens[b];
  if (len0 < 0 || len1 > g.N || len0 >= len1) return;  // nothing appended (uniform across the workgroup)
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = (lane % LPR) * VEC;
  const int rsub = lane / LPR;
  const T* kb = k + (int64_t)slab * g.N * D;
  float* pb = pyr + (int64_t)slab * g.off[g.L] * D;
  int a = len0 / g.bs, z = (len1 - 1) / g.bs;  // affected nodes of the level being built
  // each affected leaf with all waves: wave w reads rows r0 + RPI (w + NWV i) + rsub,
  // and the waves' column sums are joined in LDS. The fp64 sum of at most 128
  // rows is exact, whatever the order of the additions, when a column's values
  // span at most 38 binades (bf16 keys) or 22 (fp32 keys); only beyond that can
  // the order move the summary by one unit in its last place.
  constexpr int NWV = kPoolThreads / 64;
  __shared__ typename PO::Acc part[NWV][D];
  for (int j = a; j <= z; ++j) {
    const int r0 = j * g.bs;
    const int r1 = min(len1, r0 + g.bs);
    typename PO::Acc acc[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] = PO::init();
    for (int r = r0 + wave * RPI + rsub; r < r1; r += RPI * NWV * kUnroll) {
      uint4 raw[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
        raw[u] = Wide<T>::raw(kb + (int64_t)min(r + u * RPI * NWV, r1 - 1) * D + col);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        float x[VEC];
        Wide<T>::widen(raw[u], x);
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[e] = PO::add_row(acc[e], x[e], r + u * RPI * NWV < r1);
      }
    }
#pragma unroll
    for (int sh = LPR; sh < 64; sh <<= 1)
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[e] = PO::join(acc[e], __shfl_xor(acc[e], sh));
    if (rsub == 0) {
#pragma unroll
      for (int e = 0; e < VEC; ++e) part[wave][col + e] = acc[e];
    }
    __syncthreads();
    for (int c = threadIdx.x; c < D; c += kPoolThreads) {
      typename PO::Acc sum = part[0][c];
#pragma unroll
      for (int w = 1; w < NWV; ++w) sum = PO::join(sum, part[w][c]);
      pb[(int64_t)j * D + c] = PO::fin(sum, r1 - r0);
    }
    __syncthreads();
  }
  int present = z + 1;  // nodes of the level below that hold tokens before len1
  for (int l = 1; l < g.L; ++l) {
    const int na = a / g.f, nz = z / g.f;
    for (int e = threadIdx.x; e < (nz - na + 1) * D; e += kPoolThreads) {
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

// All levels from 2 up in one launch: a workgroup owns one top-level node and
// builds its subtree level by level from the level-1 summaries. Within a level
// each thread folds NM nodes of one column, and all F x NM child loads of a
// round are issued before any is used.
constexpr int kUpperThreads = 256;

template <int D, bool MX, int F>
__global__ __launch_bounds__(kUpperThreads) void pool_upper_kernel(Geo g, float* __restrict__ pyr) {
  using PO = Pool<MX>;
  constexpr int CPT = kUpperThreads / D;  // node groups per column
  constexpr int NM = 64 / F;              // nodes a thread folds per round
  const int top = blockIdx.x;
  const int slab = blockIdx.y;
  float* pb = pyr + (int64_t)slab * g.off[g.L] * D;
  const int c = threadIdx.x % D;
  const int grp = threadIdx.x / D;
  for (int l = 2; l < g.L; ++l) {
    const int sub = g.span[g.L - 1] / g.span[l];  // level-l nodes under one top node
    const int n0 = top * sub;
    const int n1 = min(n0 + sub, g.nodes[l]);
    const int below = g.nodes[l - 1];
    for (int nb0 = n0 + grp * NM; nb0 < n1; nb0 += CPT * NM) {
      float x[NM][F];
#pragma unroll
      for (int u = 0; u < NM; ++u)
#pragma unroll
        for (int ch = 0; ch < F; ++ch)  // clamped, unconditional loads
          x[u][ch] = pb[(int64_t)(g.off[l - 1] + min((nb0 + u) * F + ch, below - 1)) * D + c];
#pragma unroll
      for (int u = 0; u < NM; ++u) {
        const int n = nb0 + u;
        const int cnt = min(F, below - n * F);  // children present (the last node may have fewer)
        typename PO::Acc acc = PO::init();
#pragma unroll
        for (int ch = 0; ch < F; ++ch) acc = PO::add_row(acc, x[u][ch], ch < cnt);
        if (n < n1) pb[(int64_t)(g.off[l] + n) * D + c] = PO::fin(acc, cnt);
      }
    }
    __syncthreads();  // this level's summaries are read by the next
  }
}

template <int D, bool MX>
hipError_t launch_upper(const Geo& g, float* pyr, hipStream_t s) {
  const dim3 grid(g.nodes[g.L - 1], g.B * g.Hkv);
  switch (g.f) {
    case 2: hipLaunchKernelGGL((pool_upper_kernel<D, MX, 2>), grid, dim3(kUpperThreads), 0, s, g, pyr); break;
    case 4: hipLaunchKernelGGL((pool_upper_kernel<D, MX, 4>), grid, dim3(kUpperThreads), 0, s, g, pyr); break;
    case 8: hipLaunchKernelGGL((pool_upper_kernel<D, MX, 8>), grid, dim3(kUpperThreads), 0, s, g, pyr); break;
    default: hipLaunchKernelGGL((pool_upper_kernel<D, MX, 16>), grid, dim3(kUpperThreads), 0, s, g, pyr); break;
  }
  return hipGetLastError();
}

template <typename T, int D, bool MX>
hipError_t launch_append_m(const Geo& g, const void* k, float* pyr, const int32_t* old_lens, const int32_t* new_lens,
                           hipStream_t s) {
  hipLaunchKernelGGL((pool_append_kernel<T, D, MX>), dim3(g.B * g.Hkv), dim3(kPoolThreads), 0, s, g, (const T*)k, pyr,
                     old_lens, new_lens);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_append_t(const Geo& g, const void* k, float* pyr, const int32_t* old_lens, const int32_t* new_lens,
                           hipStream_t s) {
  return g.pool == PISA_POOL_MAX ? launch_append_m<T, D, true>(g, k, pyr, old_lens, new_lens, s)
                                 : launch_append_m<T, D, false>(g, k, pyr, old_lens, new_lens, s);
}

template <typename T, int D, bool MX>
hipError_t launch_pool_m(const Geo& g, const void* k, float* pyr, hipStream_t s) {
  const int slabs = g.B * g.Hkv;
  const int chunk = g.L >= 2 ? g.f : 8;
  dim3 grid((g.nb + chunk - 1) / chunk, slabs);
  hipLaunchKernelGGL((pool_leaf_kernel<T, D, MX>), grid, dim3(kPoolThreads), 0, s, g, (const T*)k, pyr, chunk);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (g.L < 3) return hipSuccess;
  return launch_upper<D, MX>(g, pyr, s);
}

template <typename T, int D>
hipError_t launch_pool_t(const Geo& g, const void* k, float* pyr, hipStream_t s) {
  return g.pool == PISA_POOL_MAX ? launch_pool_m<T, D, true>(g, k, pyr, s) : launch_pool_m<T, D, false>(g, k, pyr, s);
}

}  // namespace

hipError_t launch_pyramid_append(const Geo& g, const void* k, float* pyr, const int32_t* old_lens,
                                 const int32_t* new_lens, hipStream_t s) {
  if (g.dtype == PISA_BF16)
    return g.D == 128 ? launch_append_t<uint16_t, 128>(g, k, pyr, old_lens, new_lens, s)
                      : launch_append_t<uint16_t, 64>(g, k, pyr, old_lens, new_lens, s);
  return g.D == 128 ? launch_append_t<float, 128>(g, k, pyr, old_lens, new_lens, s)
                    : launch_append_t<float, 64>(g, k, pyr, old_lens, new_lens, s);
}

hipError_t launch_build_pyramid(const Geo& g, const void* k, float* pyr, hipStream_t s) {
  if (g.dtype == PISA_BF16) {
    return g.D == 128 ? launch_pool_t<uint16_t, 128>(g, k, pyr, s) : launch_pool_t<uint16_t, 64>(g, k, pyr, s);
  }
  return g.D == 128 ? launch_pool_t<float, 128>(g, k, pyr, s) : launch_pool_t<float, 64>(g, k, pyr, s);
}

}  // namespace pisa
