// Forward attention of one (unit, part) on the matrix cores: the per-wave state,
// one key tile's online-softmax step, and the tile walk over a unit's attended
// blocks ("Attention clairsemée PISA : noyaux Triton sans matrice de scores",
// section "Des noyaux Triton qui ne matérialisent rien"). Used by the sparse
// attention kernel and by the fused selection + attention kernel.
#pragma once

#include "pisa_attn_common.h"

namespace pisa {
namespace {

// Units of at most two waves take swizzled (unpadded) tiles at d = 128: their
// kernel is bound by the copies' traffic, and the per-lane offset tables fit in
// their registers.
template <int D, int NW>
constexpr bool kSwizzled = D == 128 && NW <= 2;

template <int D, int BS, bool SW>
struct AttnState {
  using TP = TilePitch<D, BS, SW>;
  static constexpr int NDS = D / 16;
  static constexpr int NDB = D / 32;
  bf16x8_t qf[NDS];
  f32x16_t oacc[NDB];
  float m_run, l_run;
  // byte offsets in a tile of this lane's K-fragment reads (one per step ds when
  // swizzled, else the first) and of its V^T transposing reads (one per slice db
  // and half of the 16-row step when swizzled, else the first)
  int offk[SW ? NDS : 1];
  int offv[SW ? NDB : 1];
  int offu[SW ? NDB : 1];
  __device__ __forceinline__ int k_at(int ds) const { return SW ? offk[ds] : offk[0] + ds * 32; }
  __device__ __forceinline__ int v_lo(int db) const { return SW ? offv[db] : offv[0] + db * 64; }
  __device__ __forceinline__ int v_up(int db) const { return SW ? offu[db] : offv[0] + db * 64 + 8 * TP::V * 2; }
  __device__ __forceinline__ void init_offsets(int lane) {
    const int l32 = lane & 31, hi = lane >> 5;
    // K fragment: row l32, d = ds*16 + hi*8. V^T transposing read: lanes 4j..4j+3
    // of each 16-lane block supply row j's four 8-byte pieces of a 16-column slice.
    const int rr = hi * 4 + ((lane & 15) >> 2);
    if constexpr (SW) {
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds) offk[ds] = (l32 * D + (((2 * ds + hi) ^ tile_swz(l32)) * 8)) * 2;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int col = 32 * db + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
        offv[db] = (rr * D + (((col >> 3) ^ tile_swz(rr)) * 8) + (col & 7)) * 2;
        offu[db] = ((rr + 8) * D + (((col >> 3) ^ tile_swz(rr + 8)) * 8) + (col & 7)) * 2;
      }
    } else {
      offk[0] = (l32 * TP::K + hi * 8) * 2;
      offv[0] = (rr * TP::V + 16 * ((lane >> 4) & 1) + 4 * (lane & 3)) * 2;
    }
  }
};

// Keys per chunk of a tile: the scores of at most 64 keys (32 live accumulator
// registers) are held at a time.
template <int BS>
constexpr int kChunk = BS < 64 ? BS : 64;

// S^T = K Q^T for the keys [ch * KC, ch * KC + KC) of the tile in `ks`, with the
// keys beyond `nvalid` (partial block) and after the query (causal diagonal)
// masked.
template <int D, int BS, bool SW>
__device__ __forceinline__ void tile_scores(const AttnState<D, BS, SW>& st, const uint16_t* ks, int ch, int nvalid,
                                            bool local, int key0, int qpos, int hi,
                                            f32x16_t (&sacc)[kChunk<BS> / 32]) {
  constexpr int NDS = D / 16;
  constexpr int KC = kChunk<BS>;
  constexpr int NKB = KC / 32;
  // the chunk's K fragments in product order (32-key block kb, step ds); PD
  // reads are kept in flight ahead of the product that takes them
  constexpr int NF = NKB * NDS;
  constexpr int PD = NF < 4 ? NF : 4;
  const char* kb_base = reinterpret_cast<const char*>(ks);
  auto frag = [&](int f) {
    return *reinterpret_cast<const bf16x8_t*>(kb_base + st.k_at(f % NDS) +
                                              (ch * KC + (f / NDS) * 32) * TilePitch<D, BS, SW>::K * 2);
  };
  bf16x8_t a[PD];
#pragma unroll
  for (int f = 0; f < PD; ++f) a[f] = frag(f);
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    const int kb = f / NDS;
    if (f % NDS == 0)
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[kb][i] = 0.f;
    sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[f % PD], st.qf[f % NDS], sacc[kb], 0, 0, 0);
    if (f + PD < NF) a[f % PD] = frag(f + PD);
  }
  // hold the schedule to that order (the compiler would otherwise keep fewer
  // reads in flight): PD reads, then one product per further read
  __builtin_amdgcn_sched_group_barrier(0x100, PD, 0);
#pragma unroll
  for (int f = PD; f < NF; ++f) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, PD, 0);
  if (__builtin_expect(local || nvalid < BS, 0)) {  // uniform across the workgroup
    // keys of this tile beyond `lim` are masked (partial block, causal diagonal)
    const int lim = min(nvalid - 1, local ? qpos - key0 : BS - 1) - (ch * KC + hi * 4);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (kb * 32 + (i >> 2) * 8 + (i & 3) > lim) sacc[kb][i] = -__builtin_inff();
  }
}

// Online softmax of one chunk's scores and O^T += V^T P^T with the chunk's
// values from the tile in `vs`.
template <int D, int BS, bool SW>
__device__ __forceinline__ void tile_update(AttnState<D, BS, SW>& st, f32x16_t (&sacc)[kChunk<BS> / 32],
                                            const uint16_t* vs, int ch, float c) {
  constexpr int NDB = D / 32;
  constexpr int KC = kChunk<BS>;
  constexpr int NKB = KC / 32;
  const char* vb_base = reinterpret_cast<const char*>(vs);
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
  // the chunk's V^T fragments in product order (32-key block kb, 16-key half
  // hh, 32-column slice db); PV reads are kept in flight ahead of the product
  // that takes them, and the first PV load while the exponentials are computed
  constexpr int NV = NKB * 2 * NDB;
  constexpr int PV = NV < 4 ? NV : 4;
  auto vfrag = [&](int f) {
    const int kb = f / (2 * NDB), hh = (f / NDB) % 2, db = f % NDB;
    const int step = (ch * KC + kb * 32 + hh * 16) * TilePitch<D, BS, SW>::V * 2;
    const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_ptr)(vb_base + st.v_lo(db) + step));
    const v4i16_t up = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_ptr)(vb_base + st.v_up(db) + step));
    const v4i16_t a8[2] = {lo, up};
    return __builtin_bit_cast(bf16x8_t, a8);
  };
  bf16x8_t va[PV];
#pragma unroll
  for (int f = 0; f < PV; ++f) va[f] = vfrag(f);
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
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int f = (kb * 2 + hh) * NDB + db;
        st.oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[f % PV], pb, st.oacc[db], 0, 0, 0);
        if (f + PV < NV) va[f % PV] = vfrag(f + PV);
      }
    }
  }
  st.l_run += sum_halves(rs);
}

// One key tile: S^T = K Q^T, mask, online softmax, O^T += V^T P^T, chunk by chunk.
template <int D, int BS, bool SW>
__device__ __forceinline__ void compute_tile(AttnState<D, BS, SW>& st, const uint16_t* ks, const uint16_t* vs, int nvalid,
                                             bool local, int key0, int qpos, int hi, float c, int wg_qmax) {
  constexpr int KC = kChunk<BS>;
#pragma unroll
  for (int ch = 0; ch < BS / KC; ++ch) {
    // a chunk past the valid keys, or wholly after the workgroup's last query on
    // the causal diagonal, contributes nothing to any row (uniform test)
    if (ch > 0 && (ch * KC >= nvalid || (local && key0 + ch * KC > wg_qmax))) break;
    f32x16_t sacc[KC / 32];
    tile_scores(st, ks, ch, nvalid, local, key0, qpos, hi, sacc);
    tile_update(st, sacc, vs, ch, c);
  }
}

// One (unit, part) of the bf16 attention: the tile walk over the selected
// blocks sel[0, nsel) (in LDS, visible to every wave), through two stages of K/V
// tiles in LDS (K0/V0 and K1/V1), or with ST = 1 through one stage (K0/V0; K1
// and V1 unused): each tile's copy then waits for the previous tile's products,
// and the other workgroups that the smaller LDS footprint lets share the compute
// unit cover that wait.
template <int D, int BS, int NW, int ST = 2>
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

  constexpr bool SW = kSwizzled<D, NW>;
  AttnState<D, BS, SW> st;
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
  st.init_offsets(lane);
  const float c = g.scale * kLog2e;
  // last query position any wave of this workgroup holds (chunks of keys beyond
  // it are masked for every row and are skipped)
  const int wg_qmax = qb * BS + (((part + 1) * NW - 1) / g.G) * 32 + 31;

  const uint16_t* kbase = k + ((int64_t)b * g.Hkv + kvh) * g.N * D;
  const uint16_t* vbase = v + ((int64_t)b * g.Hkv + kvh) * g.N * D;
  const TileWalk walk = make_walk(g, qb, sel, nsel);
  DmaPlan<D, BS, NW, SW> plan;
  plan.init(wave, lane);

  int j, nvalid;
  bool local;
  walk.at(0, sel, g, qb, local_rows, j, nvalid, local);
  issue_tile(kbase + (int64_t)j * BS * D, vbase + (int64_t)j * BS * D, min(BS, g.N - j * BS), K0, V0, wave, plan);
  if constexpr (ST == 1) {
    // One stage, split by phase: the keys of tile t + 1 load while tile t's
    // softmax and value product run, its values while tile t + 1's scores run.
    // Each wave's copies complete in the order issued (K before V), so waiting
    // until at most VMIN of its copies are outstanding -- no more than the V
    // copies it issued after them -- means its K copies have landed.
    static_assert(BS <= 64, "a one-stage tile is one chunk of keys");
    constexpr int VMIN = TilePitch<D, BS, SW>::VI / NW;
    // the query fragments, loaded before the first tile's copies, have landed
    wait_loads<TilePitch<D, BS, SW>::KI / NW + VMIN>();
    for (int t = 0; t < walk.ntiles; ++t) {
      wait_loads<VMIN>();
      lds_read_barrier();  // K(t) has landed for every wave (no fence: V(t) keeps loading)
      f32x16_t sacc[BS / 32];
      tile_scores(st, K0, 0, nvalid, local, j * BS, qpos, hi, sacc);
      wait_loads<0>();
      lds_read_barrier();  // V(t) has landed; every wave is done with K(t)
      // The copies are issued on every tile, past the last one with an empty
      // range (the hardware then writes zeros and reads nothing): with copies
      // into LDS issued on some paths only, the compiler waits for all of them
      // before any LDS read of the next tile, which would leave V(t + 1) no
      // scores to hide behind.
      const bool more = t + 1 < walk.ntiles;
      int j1 = j, nv1 = 0;
      bool loc1 = false;
      if (more) walk.at(t + 1, sel, g, qb, local_rows, j1, nv1, loc1);
      const int rows1 = more ? min(BS, g.N - j1 * BS) : 0;
      issue_half<true>(kbase + (int64_t)j1 * BS * D, rows1, K0, wave, plan);
      tile_update(st, sacc, V0, 0, c);
      lds_read_barrier();  // every wave is done with V(t); K(t + 1) keeps loading
      issue_half<false>(vbase + (int64_t)j1 * BS * D, rows1, V0, wave, plan);
      j = j1;
      nvalid = nv1;
      local = loc1;
    }
  } else
  for (int t = 0; t < walk.ntiles; t += 2) {
    // even tile: compute from stage 0 while stage 1 fills
    wait_loads_and_sync();
    int j1 = 0, nv1 = 0;
    bool loc1 = false;
    if (t + 1 < walk.ntiles) {
      walk.at(t + 1, sel, g, qb, local_rows, j1, nv1, loc1);
      issue_tile(kbase + (int64_t)j1 * BS * D, vbase + (int64_t)j1 * BS * D, min(BS, g.N - j1 * BS), K1, V1,
                 wave, plan);
    }
    compute_tile(st, K0, V0, nvalid, local, j * BS, qpos, hi, c, wg_qmax);
    if (t + 1 >= walk.ntiles) break;
    // odd tile: compute from stage 1 while stage 0 fills
    wait_loads_and_sync();
    if (t + 2 < walk.ntiles) {
      walk.at(t + 2, sel, g, qb, local_rows, j, nvalid, local);
      issue_tile(kbase + (int64_t)j * BS * D, vbase + (int64_t)j * BS * D, min(BS, g.N - j * BS), K0, V0,
                 wave, plan);
    }
    compute_tile(st, K1, V1, nv1, loc1, j1 * BS, qpos, hi, c, wg_qmax);
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
