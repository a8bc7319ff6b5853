// Fused selection and attention in one launch ("Attention clairsemée PISA :
// noyaux Triton sans matrice de scores", sections "La sélection top-K guidée par
// la pyramide" and "Des noyaux Triton qui ne matérialisent rien": similarity,
// selection and aggregation in a single pass, no intermediate in HBM but the
// pyramid).
//
// The grid is the sparse attention's: one workgroup per (unit, part), where a
// unit is (batch, kv head, query block). Each workgroup
//   1. streams the unit's query rows of all heads in the GQA group into an fp64
//      mean (every thread of the workgroup, 16-byte non-temporal loads),
//   2. descends the pyramid with the whole workgroup (the decode's descent:
//      scoring rounds of loads, then the first wave's threshold top-K), the
//      descent's scratch living in the LDS that later holds the K/V tiles,
//   3. attends its query rows over the selected blocks exactly as the sparse
//      attention kernel does.
// The parts of a unit each select (the same blocks; part 0 writes them out), so
// a unit's query rows are read once per part for the mean.
#include "pisa_attn_fwd.h"
#include "pisa_select_common.h"

namespace pisa {
namespace {

// fp64 mean of the unit's query rows over the group's heads, by all NT threads.
// red: NT/64 x D doubles of scratch; the mean lands in qbar (D doubles).
template <int D, int NT>
__device__ __forceinline__ void block_query_mean(const Geo& g, const uint16_t* __restrict__ q, int b, int kvh, int qb,
                                                 double* red, double* qbar) {
  constexpr int VEC = 8;          // bf16 per 16-byte load
  constexpr int LPR = D / VEC;    // lanes per row
  constexpr int RPP = NT / LPR;   // rows per pass of the workgroup
  constexpr int U = 8;            // loads in flight per thread
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = (tid % LPR) * VEC;
  const int rsub = tid / LPR;
  const int r0 = qb * g.bs;
  const int rows = min(g.bs, g.N - r0);
  const int total = rows * g.G;  // (head, row) pairs
  const uint16_t* base = q + (((int64_t)b * g.Hq + (int64_t)kvh * g.G) * g.N + r0) * D + col;
  double acc[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) acc[e] = 0.0;
  for (int t = rsub; t < total; t += RPP * U) {
    uint4 raw[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {  // unconditional loads of clamped pairs, all in flight
      const int tt = min(t + u * RPP, total - 1);
      raw[u] = Wide<uint16_t>::stream(base + ((int64_t)(tt / rows) * g.N + tt % rows) * D);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (t + u * RPP >= total) raw[u] = make_uint4(0u, 0u, 0u, 0u);  // +0.0 for a clamped pair
      float x[VEC];
      Wide<uint16_t>::widen(raw[u], x);
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[e] += (double)x[e];
    }
  }
  // fold the lanes of a wave that hold the same columns, then the waves
#pragma unroll
  for (int s = LPR; s < 64; s <<= 1)
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] += __shfl_xor(acc[e], s);
  if (lane < LPR) {
#pragma unroll
    for (int e = 0; e < VEC; ++e) red[wave * D + col + e] = acc[e];
  }
  __syncthreads();
  for (int c = tid; c < D; c += NT) {
    double s = 0.0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) s += red[w * D + c];
    qbar[c] = s / (double)total;
  }
  __syncthreads();
}

template <int D, int BS, int NW>
__global__ __launch_bounds__(NW * 64) void select_attn_bf16_kernel(Geo g, const uint16_t* __restrict__ q,
                                                                   const uint16_t* __restrict__ k,
                                                                   const uint16_t* __restrict__ v,
                                                                   const float* __restrict__ pyr,
                                                                   int32_t* __restrict__ idx,
                                                                   int32_t* __restrict__ cnt,
                                                                   uint16_t* __restrict__ out,
                                                                   float* __restrict__ lse, int parts) {
  constexpr int NT = NW * 64;
  using TP = TilePitch<D, BS, kSwizzled<D, NW>>;
  // two stages of K and V tiles; before the first tile they hold the mean's and
  // the descent's scratch
  __shared__ __attribute__((aligned(16))) uint16_t stage[2 * (TP::KSIZE + TP::VSIZE)];
  __shared__ int sel[kMaxTopK];
  __shared__ int nsel_s;
  constexpr int kSmemBytes = (sizeof(BlockSmem) + 15) / 16 * 16;
  static_assert(kSmemBytes + (NW + 1) * D * sizeof(double) <= sizeof(stage), "descent scratch fits the stages");
  BlockSmem& bsm = *reinterpret_cast<BlockSmem*>(stage);
  double* qbar = reinterpret_cast<double*>(reinterpret_cast<char*>(stage) + kSmemBytes);
  double* red = qbar + D;

  // the sparse attention's grid order: heaviest units first, slabs fastest
  const int slabs = g.B * g.Hkv;
  const int wg = blockIdx.x;
  const int slab = wg % slabs;
  const int part = (wg / slabs) % parts;
  const int qb = g.nb - 1 - wg / (slabs * parts);
  const int64_t unit = (int64_t)slab * g.nb + qb;

  block_query_mean<D, NT>(g, q, slab / g.Hkv, slab % g.Hkv, qb, red, qbar);
  block_descend<D, NT, 8, kPoolMax / 64>(g, pyr + (int64_t)slab * g.off[g.L] * D, qb, qbar, sel, &nsel_s, bsm);
  __syncthreads();  // the selection is complete and the scratch is dead before tiles land
  const int nsel = min(max(nsel_s, 0), g.K);
  if (part == 0) {
    if (idx != nullptr)
      for (int t = threadIdx.x; t < g.K; t += NT) idx[unit * g.K + t] = sel[t];
    if (cnt != nullptr && threadIdx.x == 0) cnt[unit] = nsel;
  }
  attend_unit<D, BS, NW>(g, q, k, v, out, lse, slab, part, qb, sel, nsel, stage, stage + TP::KSIZE,
                         stage + TP::KSIZE + TP::VSIZE, stage + 2 * TP::KSIZE + TP::VSIZE);
}

template <int D, int BS, int NW>
hipError_t launch_fused(const Geo& g, const void* q, const void* k, const void* v, const float* pyr, int32_t* idx,
                        int32_t* cnt, void* out, float* lse, hipStream_t s) {
  const int parts = g.G * BS / 32 / NW;
  const int64_t grid = (int64_t)g.nb * g.B * g.Hkv * parts;
  PISA_LAUNCH(g, (select_attn_bf16_kernel<D, BS, NW>), dim3((unsigned)grid), dim3(NW * 64), 0, s, g,
                     (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, pyr, idx, cnt, (uint16_t*)out, lse,
                     parts);
  return hipGetLastError();
}

template <int D, int BS>
hipError_t launch_fused_nw(const Geo& g, const void* q, const void* k, const void* v, const float* pyr, int32_t* idx,
                           int32_t* cnt, void* out, float* lse, hipStream_t s) {
  // (head, 32-query chunk) pairs per unit: a multiple of BS / 32, so blocks of
  // 128 take 4 or 8 waves and blocks of 64 at least 2 (the others are not built)
  const int pairs = g.G * BS / 32;
  if (pairs % 8 == 0) return launch_fused<D, BS, 8>(g, q, k, v, pyr, idx, cnt, out, lse, s);
  if (pairs % 4 == 0) return launch_fused<D, BS, 4>(g, q, k, v, pyr, idx, cnt, out, lse, s);
  if constexpr (BS <= 64) {
    if (pairs % 2 == 0) return launch_fused<D, BS, 2>(g, q, k, v, pyr, idx, cnt, out, lse, s);
    if constexpr (BS <= 32) return launch_fused<D, BS, 1>(g, q, k, v, pyr, idx, cnt, out, lse, s);
  }
  return hipErrorInvalidValue;  // not reached: see above
}

template <int D>
hipError_t launch_fused_bs(const Geo& g, const void* q, const void* k, const void* v, const float* pyr, int32_t* idx,
                           int32_t* cnt, void* out, float* lse, hipStream_t s) {
  switch (g.bs) {
    case 32: return launch_fused_nw<D, 32>(g, q, k, v, pyr, idx, cnt, out, lse, s);
    case 64: return launch_fused_nw<D, 64>(g, q, k, v, pyr, idx, cnt, out, lse, s);
    default: return launch_fused_nw<D, 128>(g, q, k, v, pyr, idx, cnt, out, lse, s);
  }
}

}  // namespace

hipError_t launch_select_attn(const Geo& g, const void* q, const void* k, const void* v, const float* pyr,
                              int32_t* idx, int32_t* cnt, void* out, float* lse, hipStream_t s) {
  return g.D == 128 ? launch_fused_bs<128>(g, q, k, v, pyr, idx, cnt, out, lse, s)
                    : launch_fused_bs<64>(g, q, k, v, pyr, idx, cnt, out, lse, s);
}

}  // namespace pisa
