// Pyramid descent shared by prefill selection and decode selection
// ("La sélection top-K guidée par la pyramide").
#pragma once

#include <limits.h>

#include "pisa_internal.h"

namespace pisa {

constexpr int kSelectThreads = 256;

struct DescentSmem {
  double score[kPoolMax];
  int id[kPoolMax];
  int kept[kMaxTopK];
  int n_pool;
};

// Scores of pool nodes sm.id[0, M) against the fp64 query mean: 16 lanes per
// node, each lane reading D/16 contiguous floats of the node's summary row.
template <int D>
__device__ __forceinline__ void score_pool(const float* __restrict__ lvl, const double* qbar, int M, DescentSmem& sm) {
  constexpr int DPL = D / 16;
  const int grp = threadIdx.x >> 4;
  const int sub = threadIdx.x & 15;
  double qv[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) qv[e] = qbar[sub * DPL + e];
  for (int base = 0; base < M; base += kSelectThreads / 16) {
    const int i = base + grp;
    double s = 0.0;
    if (i < M) {
      const float4* row = reinterpret_cast<const float4*>(lvl + (int64_t)sm.id[i] * D + sub * DPL);
#pragma unroll
      for (int e4 = 0; e4 < DPL / 4; ++e4) {
        const float4 x = row[e4];
        s += qv[e4 * 4 + 0] * (double)x.x;
        s += qv[e4 * 4 + 1] * (double)x.y;
        s += qv[e4 * 4 + 2] * (double)x.z;
        s += qv[e4 * 4 + 3] * (double)x.w;
      }
    }
    s += __shfl_xor(s, 1);
    s += __shfl_xor(s, 2);
    s += __shfl_xor(s, 4);
    s += __shfl_xor(s, 8);
    if (sub == 0 && i < M) sm.score[i] = s;
  }
}

__device__ __forceinline__ bool ranks_before(double sa, int ia, double sb, int ib) {
  return sa > sb || (sa == sb && ia < ib);
}

// Bitonic sort of (score, id) pairs [0, M) in LDS, best first; pads to a power of two.
__device__ __forceinline__ void bitonic_best_first(DescentSmem& sm, int M) {
  int P = 1;
  while (P < M) P <<= 1;
  for (int i = M + threadIdx.x; i < P; i += kSelectThreads) {
    sm.score[i] = -__builtin_inf();
    sm.id[i] = INT_MAX;
  }
  __syncthreads();
  for (int k = 2; k <= P; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < P; i += kSelectThreads) {
        const int ixj = i ^ j;
        if (ixj > i) {
          const double si = sm.score[i], sj = sm.score[ixj];
          const int ii = sm.id[i], ij = sm.id[ixj];
          const bool asc = (i & k) == 0;
          const bool sw = asc ? ranks_before(sj, ij, si, ii) : ranks_before(si, ii, sj, ij);
          if (sw) {
            sm.score[i] = sj;
            sm.score[ixj] = si;
            sm.id[i] = ij;
            sm.id[ixj] = ii;
          }
        }
      }
      __syncthreads();
    }
  }
}

// Descent for query block (or decode token) qb of one (batch, kv head) slab.
// ps: the slab's pyramid; qbar: fp64 query mean in LDS (already synchronised).
// Writes out_idx[0, K) (ascending, -1 padded) and *out_cnt.
template <int D>
__device__ void descend(const Geo& g, const float* __restrict__ ps, const double* qbar, int qb,
                        int32_t* __restrict__ out_idx, int32_t* __restrict__ out_cnt, DescentSmem& sm) {
  const int tid = threadIdx.x;
  const int L = g.L;
  if (g.K == 0) {
    if (tid == 0) *out_cnt = 0;
    return;
  }
  {
    const int lo = g.j0 / g.span[L - 1];
    const int hi = qb / g.span[L - 1];
    const int n = max(0, hi - lo);
    for (int i = tid; i < n; i += kSelectThreads) sm.id[i] = lo + i;
    if (tid == 0) sm.n_pool = n;
  }
  __syncthreads();
  for (int l = L - 1; l >= 0; --l) {
    const int M = sm.n_pool;
    score_pool<D>(ps + (int64_t)g.off[l] * D, qbar, M, sm);
    __syncthreads();
    int nk = M;
    if (M > g.K) {
      bitonic_best_first(sm, M);
      nk = g.K;
    }
    if (l == 0) {
      for (int t = tid; t < nk; t += kSelectThreads) {
        const int v = sm.id[t];
        int r = 0;
        for (int u = 0; u < nk; ++u) r += (sm.id[u] < v);
        out_idx[r] = v;
      }
      for (int t = nk + tid; t < g.K; t += kSelectThreads) out_idx[t] = -1;
      if (tid == 0) *out_cnt = nk;
      return;
    }
    for (int t = tid; t < nk; t += kSelectThreads) sm.kept[t] = sm.id[t];
    __syncthreads();
    if (tid == 0) sm.n_pool = 0;
    __syncthreads();
    const int lo = g.j0 / g.span[l - 1];
    const int a_l = qb / g.span[l];
    const int a_below = qb / g.span[l - 1];
    const int nchild = nk * g.f;
    const int nanc = a_below - a_l * g.f;  // complete children of qb's own ancestor
    for (int t = tid; t < nchild + nanc; t += kSelectThreads) {
      const int c = t < nchild ? sm.kept[t / g.f] * g.f + t % g.f : a_l * g.f + (t - nchild);
      if (c >= lo) sm.id[atomicAdd(&sm.n_pool, 1)] = c;
    }
    __syncthreads();
  }
}

}  // namespace pisa
