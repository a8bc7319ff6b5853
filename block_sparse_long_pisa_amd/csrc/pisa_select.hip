// Pyramid-guided top-K selection ("Attention clairsemée PISA : noyaux Triton
// sans matrice de scores", section "La sélection top-K guidée par la
// pyramide"): prune hard at the top level, refine one level at a time.
//
// One wave per (batch, kv head, query block). It first streams the query
// block's rows of all heads in the KV group (the HBM-heavy part) into an fp64
// mean, then descends the pyramid: each level scores its candidate pool with
// fp64 dot products, keeps the K best (score descending, index ascending), and
// expands the kept nodes' children plus the complete children of the query
// block's own ancestor.
//
// The same descent serves decode, where the "block" is one query token.
#include "pisa_internal.h"
#include "pisa_select_common.h"

namespace pisa {
namespace {

// Mean of the query block's rows over the group's heads (fp64), by one wave.
// The unit's rows are G runs of `rows` consecutive rows, one run per head. A
// lane covers VEC columns of every RPI-th row. Rounds of U loads are issued
// before any is summed; full rounds run unmasked and one masked round takes the
// rest. Since whole blocks hold a multiple of RPI rows, every lane leaves a
// head's run at the same load, so the stepping from one run to the next is
// uniform (scalar) and the loads need no per-lane index arithmetic beyond one
// pointer add. A short last block takes a plain per-load (head, row) split.
template <typename T, int D>
__device__ __forceinline__ void wave_query_mean(const Geo& g, const T* __restrict__ q, int b, int kvh, int qb,
                                                double* qbar, int lane) {
  constexpr int VEC = Wide<T>::kVec;
  constexpr int LPR = D / VEC;   // lanes covering one row
  constexpr int RPI = 64 / LPR;  // rows per wave load
  constexpr int U = 8;           // loads in flight per lane (six waves per SIMD keep enough in flight)
  const int col = (lane % LPR) * VEC;
  const int rsub = lane / LPR;
  const int r0 = qb * g.bs;
  const int rows = min(g.bs, g.N - r0);
  const int total = rows * g.G;  // (head, row) pairs
  const T* base = q + (((int64_t)b * g.Hq + (int64_t)kvh * g.G) * g.N + r0) * D + col;
  double acc[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) acc[e] = 0.0;
  auto add = [&](const uint4& raw) {
    float x[VEC];
    Wide<T>::widen(raw, x);
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] += (double)x[e];
  };
  if (rows % RPI == 0) {
    const int groups = rows / RPI;      // wave loads per head's run
    const int nsteps = groups * g.G;    // wave loads in all
    const int64_t step = (int64_t)RPI * D;
    const int64_t step_next = step + ((int64_t)g.N - rows) * D;  // last group of a run -> first of the next
    const T* ptr = base + (int64_t)rsub * D;
    int kr = 0;  // row group within the current run (uniform)
    auto advance = [&]() {
      const bool wrap = ++kr == groups;
      kr = wrap ? 0 : kr;
      ptr += wrap ? step_next : step;
    };
    int s = 0;
    for (; s + U <= nsteps; s += U) {
      uint4 raw[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        raw[u] = Wide<T>::stream(ptr);
        advance();
      }
#pragma unroll
      for (int u = 0; u < U; ++u) add(raw[u]);
    }
    if (s < nsteps) {
      uint4 raw[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const bool live = s + u < nsteps;  // uniform
        raw[u] = Wide<T>::stream(live ? ptr : base);
        if (live) advance();
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (s + u < nsteps) add(raw[u]);
    }
  } else {
    for (int t = rsub; t < total; t += RPI * U) {
      uint4 raw[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        // unconditional loads from a clamped (head, row) keep all of them in flight
        const int tt = min(t + u * RPI, total - 1);
        raw[u] = Wide<T>::stream(base + ((int64_t)(tt / rows) * g.N + tt % rows) * D);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float x[VEC];
        Wide<T>::widen(raw[u], x);
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[e] += t + u * RPI < total ? (double)x[e] : 0.0;
      }
    }
  }
#pragma unroll
  for (int s = LPR; s < 64; s <<= 1)
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] += __shfl_xor(acc[e], s);
  if (rsub == 0) {
#pragma unroll
    for (int e = 0; e < VEC; ++e) qbar[col + e] = acc[e] / (double)total;
  }
  __builtin_amdgcn_wave_barrier();
}

// One wave per (batch, kv head, query block); four query blocks of one slab per workgroup.
template <typename T, int D, int E>
__global__ __launch_bounds__(kSelectThreads) __attribute__((amdgpu_waves_per_eu(E <= 5 ? 6 : 4))) void select_kernel(Geo g, const T* __restrict__ q,
                                                                const float* __restrict__ pyr,
                                                                int32_t* __restrict__ idx, int32_t* __restrict__ cnt) {
  __shared__ WaveSmem<E, D> smem[kSelectWaves];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: keep the descent scalar
  // consecutive workgroups take consecutive slabs, so that workgroups placed
  // round-robin on the XCDs keep one slab's pyramid per XCD's L2
  const int slabs = g.B * g.Hkv;
  const int slab = blockIdx.x % slabs;
  const int qb = (blockIdx.x / slabs) * kSelectWaves + wave;
  if (qb >= g.nb) return;
  const int u = slab * g.nb + qb;
  if (g.K == 0) {
    if (lane == 0) cnt[u] = 0;
    return;
  }
  wave_query_mean<T, D>(g, q, slab / g.Hkv, slab % g.Hkv, qb, smem[wave].qbar, lane);
  wave_descend<E, D>(g, pyr + (int64_t)slab * g.off[g.L] * D, qb, idx + (int64_t)u * g.K, cnt + u, smem[wave], lane);
}

template <typename T, int D, int E>
hipError_t launch_select_e(const Geo& g, const void* q, const float* pyr, int32_t* idx, int32_t* cnt, hipStream_t s) {
  const int blocks = g.B * g.Hkv * ((g.nb + kSelectWaves - 1) / kSelectWaves);
  PISA_LAUNCH(g, (select_kernel<T, D, E>), dim3(blocks), dim3(kSelectThreads), 0, s, g, (const T*)q, pyr, idx, cnt);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_select_t(const Geo& g, const void* q, const float* pyr, int32_t* idx, int32_t* cnt, hipStream_t s) {
  // the ranking's cost grows with the slots, so the pool gets the fewest that hold it
  const int e = pool_slots_per_lane(g);
  if (e <= 1) return launch_select_e<T, D, 1>(g, q, pyr, idx, cnt, s);
  if (e <= 2) return launch_select_e<T, D, 2>(g, q, pyr, idx, cnt, s);
  if (e <= 3) return launch_select_e<T, D, 3>(g, q, pyr, idx, cnt, s);
  if (e <= 4) return launch_select_e<T, D, 4>(g, q, pyr, idx, cnt, s);
  if (e <= 5) return launch_select_e<T, D, 5>(g, q, pyr, idx, cnt, s);
  if (e <= 6) return launch_select_e<T, D, 6>(g, q, pyr, idx, cnt, s);
  if (e <= 8) return launch_select_e<T, D, 8>(g, q, pyr, idx, cnt, s);
  if (e <= 10) return launch_select_e<T, D, 10>(g, q, pyr, idx, cnt, s);
  if (e <= 12) return launch_select_e<T, D, 12>(g, q, pyr, idx, cnt, s);
  return launch_select_e<T, D, 16>(g, q, pyr, idx, cnt, s);
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
