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
// the current one is computed. Per tile each wave computes S^T = K Q^T with
// v_mfma_f32_32x32x16_bf16 (a lane then owns one query column), runs the
// online softmax in registers, and accumulates O^T += V^T P^T on the same
// matrix cores, reading V^T fragments with gfx950's transposing LDS reads.
// fp32 path: plain VALU, one thread per query row.
#include "pisa_attn_common.h"

namespace pisa {
namespace {

template <int D, int BS>
struct AttnState {
  static constexpr int NKB = BS / 32;
  static constexpr int NDS = D / 16;
  static constexpr int NDB = D / 32;
  bf16x8_t qf[NDS];
  f32x16_t oacc[NDB];
  float m_run, l_run;
  int offk;      // byte offset of this lane's first K-fragment chunk in a K tile
  int offv;      // byte offset of this lane's first V^T transposing read in a V tile
};

// One key tile: S^T = K Q^T, mask, online softmax, O^T += V^T P^T, in chunks of
// at most 64 keys (32 live accumulator registers for S per chunk).
template <int D, int BS>
__device__ __forceinline__ void compute_tile(AttnState<D, BS>& st, const uint16_t* ks, const uint16_t* vs, int nvalid,
                                             bool local, int key0, int qpos, int hi, float c, int wg_qmax) {
  constexpr int CPR = D / 8;
  constexpr int NDS = D / 16, NDB = D / 32;
  constexpr int KC = BS < 64 ? BS : 64;  // keys per chunk
  constexpr int NKB = KC / 32;
  const char* kb_base = reinterpret_cast<const char*>(ks);
  const char* vb_base = reinterpret_cast<const char*>(vs);
#pragma unroll
  for (int ch = 0; ch < BS / KC; ++ch) {
    // a chunk past the valid keys, or wholly after the workgroup's last query on
    // the causal diagonal, contributes nothing to any row (uniform test)
    if (ch > 0 && (ch * KC >= nvalid || (local && key0 + ch * KC > wg_qmax))) break;
    f32x16_t sacc[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[kb][i] = 0.f;
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds) {
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(kb_base + st.offk + ds * 32 +
                                                              (ch * KC + kb * 32) * TilePitch<D>::K * 2);
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, st.qf[ds], sacc[kb], 0, 0, 0);
      }
    }
    if (__builtin_expect(local || nvalid < BS, 0)) {  // uniform across the workgroup
      // keys of this tile beyond `lim` are masked (partial block, causal diagonal)
      const int lim = min(nvalid - 1, local ? qpos - key0 : BS - 1) - (ch * KC + hi * 4);
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (kb * 32 + (i >> 2) * 8 + (i & 3) > lim) sacc[kb][i] = -__builtin_inff();
    }
    // online softmax in the log2 domain; the reference max only moves when the
    // chunk max exceeds it by more than 8 (a factor 2^8), then O and l rescale
    float mx = -__builtin_inff();
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kb][i]);
    mx = max_halves(mx);
    const float mt = mx * c;
    const bool move = mt > st.m_run + 8.f;
    const float m_ref = move ? mt : st.m_run;
    const float m_use = m_ref == -__builtin_inff() ? 0.f : m_ref;
    if (__any(move)) {
      const float alpha = fast_exp2(st.m_run - m_use);
      st.l_run *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) st.oacc[db][i] *= alpha;
    }
    st.m_run = m_ref;
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = fast_exp2(fmaf(sacc[kb][i], c, -m_use));
        sacc[kb][i] = p;
        rs += p;
      }
    // O^T[d][query] += V^T P^T over 16-key steps; slot (hi, e) of step (kb, hh)
    // holds key kb*32 + hh*16 + (e/4)*8 + hi*4 + e%4
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        bf16x8_t pb;
#pragma unroll
        for (int e = 0; e < 8; ++e) pb[e] = (__bf16)sacc[kb][hh * 8 + e];
        const int step = (ch * KC + kb * 32 + hh * 16) * TilePitch<D>::V * 2;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_v4i16_ptr)(vb_base + st.offv + step + db * 64));
          const v4i16_t up = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_v4i16_ptr)(vb_base + st.offv + step + db * 64 + 8 * TilePitch<D>::V * 2));
          const v4i16_t a8[2] = {lo, up};
          const bf16x8_t a = __builtin_bit_cast(bf16x8_t, a8);
          st.oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, st.oacc[db], 0, 0, 0);
        }
      }
    }
    st.l_run += sum_halves(rs);
  }
}

template <int D, int BS, int NW>
__global__ __launch_bounds__(NW * 64) void attn_bf16_kernel(Geo g, const uint16_t* __restrict__ q,
                                                            const uint16_t* __restrict__ k,
                                                            const uint16_t* __restrict__ v,
                                                            const int32_t* __restrict__ idx,
                                                            const int32_t* __restrict__ cnt, uint16_t* __restrict__ out,
                                                            float* __restrict__ lse, int parts) {
  constexpr int NT = NW * 64;
  constexpr int CPR = D / 8;
  constexpr int NDS = D / 16;
  constexpr int NDB = D / 32;
  // two stages of K and V tiles, filled by asynchronous copies
  __shared__ __attribute__((aligned(16))) uint16_t K0[TilePitch<D, BS>::KSIZE];
  __shared__ __attribute__((aligned(16))) uint16_t V0[TilePitch<D, BS>::VSIZE];
  __shared__ __attribute__((aligned(16))) uint16_t K1[TilePitch<D, BS>::KSIZE];
  __shared__ __attribute__((aligned(16))) uint16_t V1[TilePitch<D, BS>::VSIZE];
  __shared__ int sel[kMaxTopK];

  // heaviest units first; consecutive workgroups walk the (batch, kv head) slabs
  // so that one slab's workgroups land on one XCD
  const int slabs = g.B * g.Hkv;
  const int wg = blockIdx.x;
  const int slab = wg % slabs;
  const int part = (wg / slabs) % parts;
  const int qb = g.nb - 1 - wg / (slabs * parts);
  const int b = slab / g.Hkv;
  const int kvh = slab % g.Hkv;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: keep it scalar
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int pair = part * NW + wave;
  const int h = kvh * g.G + pair % g.G;
  const int qpos = qb * BS + (pair / g.G) * 32 + l32;
  const bool qvalid = qpos < g.N;
  const int local_rows = min(BS, g.N - qb * BS);

  const int64_t unit = (int64_t)slab * g.nb + qb;
  const int nsel = min(max(cnt[unit], 0), g.K);
  for (int t = threadIdx.x; t < nsel; t += NT) sel[t] = idx[unit * g.K + t];

  AttnState<D, BS> st;
  {
    const uint16_t* qrow = q + (((int64_t)b * g.Hq + h) * g.N + (qvalid ? qpos : 0)) * D;
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
      uint4 u = qvalid ? *reinterpret_cast<const uint4*>(qrow + ds * 16 + hi * 8) : make_uint4(0, 0, 0, 0);
      st.qf[ds] = __builtin_bit_cast(bf16x8_t, u);
    }
  }
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) st.oacc[db][i] = 0.f;
  st.m_run = -__builtin_inff();
  st.l_run = 0.f;
  // K fragment: row l32, d = ds*16 + hi*8. V^T transposing read: lanes 4j..4j+3 of
  // each 16-lane block supply row j's four 8-byte pieces of a 16-column slice.
  st.offk = (l32 * TilePitch<D>::K + hi * 8) * 2;
  st.offv = ((hi * 4 + ((lane & 15) >> 2)) * TilePitch<D>::V + 16 * ((lane >> 4) & 1) + 4 * (lane & 3)) * 2;
  const float c = g.scale * kLog2e;
  // last query position any wave of this workgroup holds (chunks of keys beyond
  // it are masked for every row and are skipped)
  const int wg_qmax = qb * BS + (((part + 1) * NW - 1) / g.G) * 32 + 31;

  const uint16_t* kbase = k + ((int64_t)b * g.Hkv + kvh) * g.N * D;
  const uint16_t* vbase = v + ((int64_t)b * g.Hkv + kvh) * g.N * D;
  __syncthreads();
  const TileWalk walk = make_walk(g, qb, sel, nsel);
  DmaPlan<D, BS, NW> plan;
  plan.init(wave, lane);

  int j, nvalid;
  bool local;
  walk.at(0, sel, g, qb, local_rows, j, nvalid, local);
  issue_tile<D, BS, NW>(kbase + (int64_t)j * BS * D, vbase + (int64_t)j * BS * D, min(BS, g.N - j * BS), K0, V0,
                        wave, lane, plan);
  for (int t = 0; t < walk.ntiles; t += 2) {
    // even tile: compute from stage 0 while stage 1 fills
    wait_loads_and_sync();
    int j1 = 0, nv1 = 0;
    bool loc1 = false;
    if (t + 1 < walk.ntiles) {
      walk.at(t + 1, sel, g, qb, local_rows, j1, nv1, loc1);
      issue_tile<D, BS, NW>(kbase + (int64_t)j1 * BS * D, vbase + (int64_t)j1 * BS * D, min(BS, g.N - j1 * BS), K1,
                            V1, wave, lane, plan);
    }
    compute_tile<D, BS>(st, K0, V0, nvalid, local, j * BS, qpos, hi, c, wg_qmax);
    if (t + 1 >= walk.ntiles) break;
    // odd tile: compute from stage 1 while stage 0 fills
    wait_loads_and_sync();
    if (t + 2 < walk.ntiles) {
      walk.at(t + 2, sel, g, qb, local_rows, j, nvalid, local);
      issue_tile<D, BS, NW>(kbase + (int64_t)j * BS * D, vbase + (int64_t)j * BS * D, min(BS, g.N - j * BS), K0, V0,
                            wave, lane, plan);
    }
    compute_tile<D, BS>(st, K1, V1, nv1, loc1, j1 * BS, qpos, hi, c, wg_qmax);
  }

  if (qvalid) {
    const float inv = 1.f / st.l_run;
    uint16_t* orow = out + (((int64_t)b * g.Hq + h) * g.N + qpos) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 16; i += 4) {
        const int d = db * 32 + (i >> 2) * 8 + hi * 4;
        uint2 w;
        w.x = pack_bf16x2(st.oacc[db][i] * inv, st.oacc[db][i + 1] * inv);
        w.y = pack_bf16x2(st.oacc[db][i + 2] * inv, st.oacc[db][i + 3] * inv);
        *reinterpret_cast<uint2*>(orow + d) = w;
      }
    if (lse != nullptr && hi == 0) lse[((int64_t)b * g.Hq + h) * g.N + qpos] = (st.m_run + log2f(st.l_run)) * kLn2;
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

template <int D, int BS, int NW>
hipError_t launch_bf16(const Geo& g, const void* q, const void* k, const void* v, const int32_t* idx,
                       const int32_t* cnt, void* out, float* lse, hipStream_t s) {
  const int parts = g.G * BS / 32 / NW;
  const int64_t grid = (int64_t)g.nb * g.B * g.Hkv * parts;
  hipLaunchKernelGGL((attn_bf16_kernel<D, BS, NW>), dim3((unsigned)grid), dim3(NW * 64), 0, s, g,
                     (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, idx, cnt, (uint16_t*)out, lse, parts);
  return hipGetLastError();
}

template <int D, int BS>
hipError_t launch_bf16_nw(const Geo& g, const void* q, const void* k, const void* v, const int32_t* idx,
                          const int32_t* cnt, void* out, float* lse, hipStream_t s) {
  const int pairs = g.G * BS / 32;  // (head, 32-query chunk) pairs per unit
  if (pairs % 8 == 0) return launch_bf16<D, BS, 8>(g, q, k, v, idx, cnt, out, lse, s);
  if (pairs % 4 == 0) return launch_bf16<D, BS, 4>(g, q, k, v, idx, cnt, out, lse, s);
  if (pairs % 2 == 0) return launch_bf16<D, BS, 2>(g, q, k, v, idx, cnt, out, lse, s);
  return launch_bf16<D, BS, 1>(g, q, k, v, idx, cnt, out, lse, s);
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
    hipLaunchKernelGGL((attn_f32_kernel<128>), grid, dim3(g.bs), 0, s, g, (const float*)q, (const float*)k,
                       (const float*)v, idx, cnt, (float*)out, lse);
  else
    hipLaunchKernelGGL((attn_f32_kernel<64>), grid, dim3(g.bs), 0, s, g, (const float*)q, (const float*)k,
                       (const float*)v, idx, cnt, (float*)out, lse);
  return hipGetLastError();
}

}  // namespace pisa
