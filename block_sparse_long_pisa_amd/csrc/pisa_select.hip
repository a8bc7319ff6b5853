// Pyramid-guided top-K selection ("Attention clairsemée PISA : noyaux Triton
// sans matrice de scores", section "La sélection top-K guidée par la
// pyramide"): prune hard at the top level, refine one level at a time.
//
// One workgroup per (batch, kv head, query block). It first streams the query
// block's rows of all heads in the KV group (the HBM-heavy part) into an fp64
// mean, then descends the pyramid: each level scores its candidate pool with
// fp64 dot products (16 lanes per node, one 512-byte summary row per lane
// group), keeps the K best with a bitonic sort in LDS ordered by (score
// descending, index ascending), and expands the kept nodes' children plus the
// complete children of the query block's own ancestor.
//
// The same descent serves decode, where the "block" is one query token.
#include "pisa_internal.h"
#include "pisa_select_common.h"

namespace pisa {
namespace {

// Mean of the query block's rows over the group's heads, into qbar (LDS, fp64).
template <typename T, int D>
__device__ void block_query_mean(const Geo& g, const T* __restrict__ q, int b, int kvh, int qb, double* qbar,
                                 double (*red)[D]) {
  constexpr int VEC = Wide<T>::kVec;
  constexpr int LPR = D / VEC;
  constexpr int RPI = 64 / LPR;
  constexpr int kUnroll = 8;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = (lane % LPR) * VEC;
  const int rsub = lane / LPR;
  const int r0 = qb * g.bs;
  const int rows = min(g.bs, g.N - r0);
  const int total = rows * g.G;  // (head, row) pairs
  double acc[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) acc[e] = 0.0;
  for (int t = wave * RPI + rsub; t < total; t += kSelectThreads / 64 * RPI * kUnroll) {
    float x[kUnroll][VEC];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int tt = t + u * (kSelectThreads / 64) * RPI;
      if (tt < total) {
        const int h = kvh * g.G + tt / rows;
        const int r = r0 + tt % rows;
        Wide<T>::load(q + (((int64_t)b * g.Hq + h) * g.N + r) * D + col, x[u]);
      } else {
#pragma unroll
        for (int e = 0; e < VEC; ++e) x[u][e] = 0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[e] += (double)x[u][e];
  }
#pragma unroll
  for (int s = LPR; s < 64; s <<= 1)
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] += __shfl_xor(acc[e], s);
  if (rsub == 0) {
#pragma unroll
    for (int e = 0; e < VEC; ++e) red[wave][col + e] = acc[e];
  }
  __syncthreads();
  for (int c = threadIdx.x; c < D; c += kSelectThreads) {
    double s = 0.0;
#pragma unroll
    for (int w = 0; w < kSelectThreads / 64; ++w) s += red[w][c];
    qbar[c] = s / (double)total;
  }
  __syncthreads();
}

template <typename T, int D>
__global__ __launch_bounds__(kSelectThreads) void select_kernel(Geo g, const T* __restrict__ q,
                                                                const float* __restrict__ pyr,
                                                                int32_t* __restrict__ idx, int32_t* __restrict__ cnt) {
  __shared__ double qbar[D];
  __shared__ double red[kSelectThreads / 64][D];
  __shared__ DescentSmem sm;
  const int qb = blockIdx.x;
  const int slab = blockIdx.y;
  const int b = slab / g.Hkv;
  const int kvh = slab % g.Hkv;
  block_query_mean<T, D>(g, q, b, kvh, qb, qbar, red);
  const float* ps = pyr + (int64_t)slab * g.off[g.L] * D;
  const int64_t unit = (int64_t)slab * g.nb + qb;
  descend<D>(g, ps, qbar, qb, idx + unit * g.K, cnt + unit, sm);
}

template <typename T, int D>
hipError_t launch_select_t(const Geo& g, const void* q, const float* pyr, int32_t* idx, int32_t* cnt, hipStream_t s) {
  dim3 grid(g.nb, g.B * g.Hkv);
  hipLaunchKernelGGL((select_kernel<T, D>), grid, dim3(kSelectThreads), 0, s, g, (const T*)q, pyr, idx, cnt);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_select(const Geo& g, const void* q, const float* pyr, int32_t* idx, int32_t* cnt, hipStream_t s) {
  if (g.dtype == PISA_BF16)
    return g.D == 128 ? launch_select_t<uint16_t, 128>(g, q, pyr, idx, cnt, s)
                      : launch_select_t<uint16_t, 64>(g, q, pyr, idx, cnt, s);
  return g.D == 128 ? launch_select_t<float, 128>(g, q, pyr, idx, cnt, s)
                    : launch_select_t<float, 64>(g, q, pyr, idx, cnt, s);
}

}  // namespace pisa
