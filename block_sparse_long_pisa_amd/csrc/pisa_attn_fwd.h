// Forward attention of one (unit, part) on the matrix cores: the per-wave state,
// one key tile's online-softmax step, and the tile walk over a unit's attended
// blocks ("Attention clairsemée PISA : noyaux Triton sans matrice de scores",
// section "Des noyaux Triton qui ne matérialisent rien"). Used by the sparse
// attention kernel and by the fused selection + attention kernel.
#pragma once

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

// One (unit, part) of the bf16 attention: the tile walk over the selected
// blocks sel[0, nsel) (in LDS, visible to every wave), through two stages of K/V
// tiles in LDS (K0/V0 and K1/V1).
template <int D, int BS, int NW>
__device__ __forceinline__ void attend_unit(const Geo& g, const uint16_t* __restrict__ q,
                                            const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                                            uint16_t* __restrict__ out, float* __restrict__ lse, int slab, int part,
                                            int qb, const int* sel, int nsel, uint16_t* K0, uint16_t* V0,
                                            uint16_t* K1, uint16_t* V1) {
  constexpr int NDS = D / 16;
  constexpr int NDB = D / 32;
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

}  // namespace
}  // namespace pisa
