// Exact softmax attention over the selected blocks ("Attention clairsemée PISA :
// noyaux Triton sans matrice de scores", section "Des noyaux Triton qui ne
// matérialisent rien"), with the attention-sink prefix of the Pulsar Attention
// page ("Phase 1 : Encodage statistique du contexte").
//
// The attended set of query i in block qb is
//   ([0, sink) U selected blocks U [qb*bs, i]) intersected with [0, i],
// walked as a list of key tiles of one block each: the blocks wholly inside the
// sink, the partial sink block (unless it was selected), the selected blocks in
// ascending order, and the local block under the causal mask. No score ever
// leaves the registers.
//
// bf16 path: one workgroup serves up to 8 waves x 32 query rows of one
// (batch, kv head, query block) unit -- rows of all heads in the GQA group --
// so every K/V tile staged in LDS feeds up to 256 rows. Tiles arrive by
// asynchronous global->LDS copies into two stages, the next tile in flight while
// the current one is computed. Units of at most 64 rows take one stage of
// unpadded (swizzled, at d = 128) tiles, split by phase: the next tile's keys
// load during this tile's softmax and value product, its values during its own
// scores; four such workgroups share a compute unit. Per tile each wave computes
// S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (a lane then owns one query
// column), runs the online softmax in registers, and accumulates O^T += V^T P^T
// on the same matrix cores, reading V^T fragments with gfx950's transposing LDS
// reads.
// fp32 path: plain VALU, one thread per query row.
#include <algorithm>

#include "pisa_attn_fwd.h"

namespace pisa {
namespace {

// Workgroups of at most two waves (units of at most 64 query rows): one stage of
// K/V tiles and at most 256 registers per wave, so that four workgroups -- two
// waves per SIMD -- share a compute unit.
template <int NW>
constexpr int kStages = NW <= 2 ? 1 : 2;

template <int D, int BS, int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(NW <= 2 ? 2 : 1))) void attn_bf16_kernel(Geo g, const uint16_t* __restrict__ q,
                                                            const uint16_t* __restrict__ k,
                                                            const uint16_t* __restrict__ v,
                                                            const int32_t* __restrict__ idx,
                                                            const int32_t* __restrict__ cnt, uint16_t* __restrict__ out,
                                                            float* __restrict__ lse, int parts, int order) {
  constexpr int NT = NW * 64;
  // kStages<NW> stages of K and V tiles, filled by asynchronous copies
  using TL = TilePitch<D, BS, kSwizzled<D, NW>>;
  __shared__ __attribute__((aligned(16))) uint16_t K0[TL::KSIZE];
  __shared__ __attribute__((aligned(16))) uint16_t V0[TL::VSIZE];
  __shared__ __attribute__((aligned(16))) uint16_t K1[kStages<NW> == 2 ? TL::KSIZE : 8];
  __shared__ __attribute__((aligned(16))) uint16_t V1[kStages<NW> == 2 ? TL::VSIZE : 8];
  __shared__ int sel[kMaxTopK];

  // Persistent: each workgroup takes every gridDim.x-th (unit, part) item of its
  // list, heaviest units (latest query blocks) first. order 2: workgroup i runs
  // on XCD i % 8 (round-robin placement) and takes only the slabs x, x + 8, ...
  // of its XCD x, one slab after another, so that an XCD's L2 holds the keys and
  // values of one slab at a time. order 1: all of one slab's items before the
  // next slab's, over the whole GPU. order 0: consecutive items walk the slabs.
  // order 3: as order 0, but the parts of a unit go to workgroups of one XCD
  // (i, i + 8, ...), so that the parts after the first find its tiles in that
  // XCD's L2 (the grid is a multiple of 8 * parts).
  const int slabs = g.B * g.Hkv;
  const int64_t items = (int64_t)g.nb * slabs * parts;
  const int64_t per_slab = (int64_t)g.nb * parts;
  const int64_t first = order == 2   ? blockIdx.x / 8
                        : order == 3 ? ((int64_t)(blockIdx.x / 8) / parts * 8 + blockIdx.x % 8) * parts +
                                           (blockIdx.x / 8) % parts
                                     : blockIdx.x;
  const int64_t stride = order == 2 ? gridDim.x / 8 : gridDim.x;
  const int64_t count = order == 2 ? items / 8 : items;
  for (int64_t wg = first; wg < count; wg += stride) {
    int slab, part, qb;
    if (order == 2) {
      slab = (int)(blockIdx.x % 8) + 8 * (int)(wg / per_slab);
      part = (int)(wg % parts);
      qb = g.nb - 1 - (int)((wg % per_slab) / parts);
    } else if (order == 1) {
      slab = (int)(wg / per_slab);
      part = (int)(wg % parts);
      qb = g.nb - 1 - (int)((wg % per_slab) / parts);
    } else if (order == 3) {
      const int64_t unit_i = wg / parts;
      part = (int)(wg % parts);
      slab = (int)(unit_i % slabs);
      qb = g.nb - 1 - (int)(unit_i / slabs);
    } else {
      slab = (int)(wg % slabs);
      part = (int)((wg / slabs) % parts);
      qb = g.nb - 1 - (int)(wg / ((int64_t)slabs * parts));
    }
    const int64_t unit = (int64_t)slab * g.nb + qb;
    const int nsel = min(max(cnt[unit], 0), g.K);
    for (int t = threadIdx.x; t < nsel; t += NT) sel[t] = idx[unit * g.K + t];
    __syncthreads();
    attend_unit<D, BS, NW, kStages<NW>>(g, q, k, v, out, lse, slab, part, qb, sel, nsel, K0, V0, K1, V1);
    __syncthreads();  // every wave is done with sel and the stages before the next item
  }
}

// fp32: one thread per query row, keys streamed through LDS 32 at a time.
template <int D>
__global__ __launch_bounds__(128) void attn_f32_kernel(Geo g, const float* __restrict__ q, const float* __restrict__ k,
                                                       const float* __restrict__ v, const int32_t* __restrict__ idx,
                                                       const int32_t* __restrict__ cnt, float* __restrict__ out,
                                                       float* __restrict__ lse) {
  constexpr int TK = 32;
  __shared__ float Ks[TK][D];
  __shared__ float Vs[TK][D];
  __shared__ int sel[kMaxTopK];
  const int qb = blockIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int kvh = h / g.G;
  const int slab = b * g.Hkv + kvh;
  const int qpos = qb * g.bs + threadIdx.x;
  const bool qvalid = qpos < g.N;
  const int local_rows = min(g.bs, g.N - qb * g.bs);
  const int64_t unit = (int64_t)slab * g.nb + qb;
  const int nsel = min(max(cnt[unit], 0), g.K);
  for (int t = threadIdx.x; t < nsel; t += blockDim.x) sel[t] = idx[unit * g.K + t];

  float qr[D], o[D];
  const float* qrow = q + (((int64_t)b * g.Hq + h) * g.N + (qvalid ? qpos : 0)) * D;
#pragma unroll
  for (int d = 0; d < D; ++d) {
    qr[d] = qvalid ? qrow[d] : 0.f;
    o[d] = 0.f;
  }
  float m = -__builtin_inff(), l = 0.f;
  const float* kbase = k + (int64_t)slab * g.N * D;
  const float* vbase = v + (int64_t)slab * g.N * D;
  __syncthreads();
  const TileWalk walk = make_walk(g, qb, sel, nsel);
  for (int t = 0; t < walk.ntiles; ++t) {
    int j, nvalid;
    bool local;
    walk.at(t, sel, g, qb, local_rows, j, nvalid, local);
    for (int sub = 0; sub < g.bs; sub += TK) {
      for (int e = threadIdx.x; e < TK * D; e += blockDim.x) {
        const int row = e / D, col = e % D;
        const int key = sub + row;
        const bool in = key < nvalid;
        Ks[row][col] = in ? kbase[((int64_t)j * g.bs + key) * D + col] : 0.f;
        Vs[row][col] = in ? vbase[((int64_t)j * g.bs + key) * D + col] : 0.f;
      }
      __syncthreads();
      for (int r = 0; r < TK; ++r) {
        const int key = sub + r;
        if (key >= nvalid || (local && j * g.bs + key > qpos)) continue;
        float s = 0.f;
#pragma unroll
        for (int d = 0; d < D; ++d) s = fmaf(qr[d], Ks[r][d], s);
        s *= g.scale;
        const float m_new = fmaxf(m, s);
        const float corr = expf(m - m_new);
        const float p = expf(s - m_new);
        l = l * corr + p;
#pragma unroll
        for (int d = 0; d < D; ++d) o[d] = fmaf(p, Vs[r][d], o[d] * corr);
        m = m_new;
      }
      __syncthreads();
    }
  }
  if (qvalid) {
    float* orow = out + (((int64_t)b * g.Hq + h) * g.N + qpos) * D;
    const float inv = 1.f / l;
#pragma unroll
    for (int d = 0; d < D; ++d) orow[d] = o[d] * inv;
    if (lse != nullptr) lse[((int64_t)b * g.Hq + h) * g.N + qpos] = m + logf(l);
  }
}

// persistent workgroups per compute unit: units of at most two waves take as
// many as fit at once (four, one stage of LDS each), so that an XCD visits each
// of its slabs once; the eight-wave units take eight (one resident at a time)
template <int NW>
constexpr int kAttnWgPerCu = NW <= 2 ? 4 : 8;

template <int D, int BS, int NW>
hipError_t launch_bf16(const Geo& g, const void* q, const void* k, const void* v, const int32_t* idx,
                       const int32_t* cnt, void* out, float* lse, hipStream_t s) {
  const int parts = g.G * BS / 32 / NW;
  const int64_t items = (int64_t)g.nb * g.B * g.Hkv * parts;
  // a few items per workgroup: fewer workgroup launches and a short tail
  int cus = 0;
  hipError_t e = device_cus(&cus);
  if (e != hipSuccess) return e;
  const int64_t grid = std::min<int64_t>(items, (int64_t)kAttnWgPerCu<NW> * cus);
  // item order: slabs divisible among the 8 XCDs -- each XCD walks its own
  // slabs, one after another (2); otherwise many slabs -- one slab after another
  // over the whole GPU (1); few -- slab-fastest, with a unit's parts on one XCD
  // when the grid allows it (3), else as they come (0)
  const int slabs = g.B * g.Hkv;
  const int order = slabs % 8 == 0 && grid % 8 == 0 ? 2
                    : slabs > 8                       ? 1
                    : parts > 1 && grid % (8 * parts) == 0 ? 3
                                                           : 0;
  PISA_LAUNCH(g, (attn_bf16_kernel<D, BS, NW>), dim3((unsigned)grid), dim3(NW * 64), 0, s, g,
                     (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, idx, cnt, (uint16_t*)out, lse, parts,
                     order);
  return hipGetLastError();
}

template <int D, int BS>
hipError_t launch_bf16_nw(const Geo& g, const void* q, const void* k, const void* v, const int32_t* idx,
                          const int32_t* cnt, void* out, float* lse, hipStream_t s) {
  // (head, 32-query chunk) pairs per unit: a multiple of BS / 32, so blocks of
  // 128 take 4 or 8 waves and blocks of 64 at least 2
  const int pairs = g.G * BS / 32;
  if (pairs % 8 == 0) return launch_bf16<D, BS, 8>(g, q, k, v, idx, cnt, out, lse, s);
  if (pairs % 4 == 0) return launch_bf16<D, BS, 4>(g, q, k, v, idx, cnt, out, lse, s);
  if constexpr (BS <= 64) {
    if (pairs % 2 == 0) return launch_bf16<D, BS, 2>(g, q, k, v, idx, cnt, out, lse, s);
    if constexpr (BS <= 32) return launch_bf16<D, BS, 1>(g, q, k, v, idx, cnt, out, lse, s);
  }
  return hipErrorInvalidValue;  // not reached: see above
}

template <int D>
hipError_t launch_bf16_bs(const Geo& g, const void* q, const void* k, const void* v, const int32_t* idx,
                          const int32_t* cnt, void* out, float* lse, hipStream_t s) {
  switch (g.bs) {
    case 32: return launch_bf16_nw<D, 32>(g, q, k, v, idx, cnt, out, lse, s);
    case 64: return launch_bf16_nw<D, 64>(g, q, k, v, idx, cnt, out, lse, s);
    default: return launch_bf16_nw<D, 128>(g, q, k, v, idx, cnt, out, lse, s);
  }
}

}  // namespace

hipError_t launch_attn(const Geo& g, const void* q, const void* k, const void* v, const int32_t* idx,
                       const int32_t* cnt, void* out, float* lse, hipStream_t s) {
  if (g.dtype == PISA_BF16)
    return g.D == 128 ? launch_bf16_bs<128>(g, q, k, v, idx, cnt, out, lse, s)
                      : launch_bf16_bs<64>(g, q, k, v, idx, cnt, out, lse, s);
  dim3 grid(g.nb, g.Hq, g.B);
  if (g.D == 128)
    PISA_LAUNCH(g, (attn_f32_kernel<128>), grid, dim3(g.bs), 0, s, g, (const float*)q, (const float*)k,
                       (const float*)v, idx, cnt, (float*)out, lse);
  else
    PISA_LAUNCH(g, (attn_f32_kernel<64>), grid, dim3(g.bs), 0, s, g, (const float*)q, (const float*)k,
                       (const float*)v, idx, cnt, (float*)out, lse);
  return hipGetLastError();
}

}  // namespace pisa
