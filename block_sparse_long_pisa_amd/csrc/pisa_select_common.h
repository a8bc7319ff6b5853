// Pyramid descent shared by prefill selection and decode selection
// ("Attention clairsemée PISA : noyaux Triton sans matrice de scores", section
// "La sélection top-K guidée par la pyramide").
//
// One wave descends for one query block (or decode token). The candidate pool
// of a level lives in registers, E slots per lane (pool capacity 64*E); nodes
// are scored by 16-lane groups with fp64 dot products against the query mean,
// and the best K -- score descending, node index ascending -- are found by a
// bitwise search for the K-th largest score with wave-wide counts, no sort. No
// workgroup barrier is involved, so waves of one workgroup never wait on each
// other.
#pragma once

#include <limits.h>

#include "pisa_internal.h"

namespace pisa {

constexpr int kSelectThreads = 256;
constexpr int kSelectWaves = kSelectThreads / 64;

// Pool slots per lane, ceil(pool / 64), covering the largest pool of any level:
// the top level's nodes, or K kept nodes' children plus the ancestor's.
inline int pool_slots_per_lane(const Geo& g) {
  const int mmax = max(g.nodes[g.L - 1], g.K * g.f + g.f - 1);
  return max(1, (mmax + 63) / 64);
}

// Per-wave LDS: scores staged from the scoring layout to the sort layout, the
// level's pool as node ids, the nodes kept at the previous level, and the query
// mean.
template <int E, int D>
struct WaveSmem {
  double sc[64 * E];
  int node[64 * E];  // node held by each pool slot of the level, -1 if none
  int kept[kMaxTopK];
  double qbar[D];
};

// Order-preserving map of an fp64 score to an unsigned key (larger score,
// larger key); -0.0 counts as +0.0, as equal scores must tie.
__device__ __forceinline__ uint64_t score_key(double s) {
  const uint64_t u = (uint64_t)__double_as_longlong(s + 0.0);
  return (u >> 63) ? ~u : (u | (1ull << 63));
}

// Keep the nk best of the wave's pool slots -- score descending, node index
// ascending -- without sorting. key[e] is 0 for an empty slot, so only valid
// slots (nk <= their count) are ever kept, and empty slots need no test of
// their own (a guard per slot group costs more than the count it would skip). A threshold is found bit by bit, most significant first, with
// wave-wide counts of the keys at or above it. As soon as exactly nk keys lie at
// or above the prefix found so far, those are the nk best and the search stops
// (with distinct scores near the boundary this takes about as many bits as
// separate the nk-th key from the next). Otherwise the search ends at T, the
// nk-th largest key: every slot above T is kept, and of the slots at T the
// lowest node indices fill the rest. Writes the kept node ids to kept[] in slot
// order. Counts are scalar and branch-free within a step.
template <int E>
__device__ __forceinline__ void wave_keep_best(const uint64_t (&key)[E], const int (&id)[E], int nk, int* kept,
                                               int lane) {
  uint64_t T = 0;
  bool exact = false;  // exactly nk keys are >= T
  for (int b = 63; b >= 0; --b) {
    const uint64_t cand = T | (1ull << b);
    int c = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) c += __popcll(__ballot(key[e] >= cand));
    if (c >= nk) {
      T = cand;
      if (c == nk) {
        exact = true;
        break;
      }
    }
  }
  int I = INT_MAX;  // keys at T are kept when their node index is <= I
  if (!exact) {
    int above = 0, at = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      above += __popcll(__ballot(key[e] > T));
      at += __popcll(__ballot(key[e] == T));
    }
    const int need = nk - above;  // >= 1 slots at T to keep
    // when more slots tie at T than are needed, keep those with index <= I, the
    // need-th smallest index among them (indices of valid slots are distinct)
    if (at > need) {
      int lo = 0, hi = INT_MAX;  // smallest I with #{tied, id <= I} >= need
      while (lo < hi) {
        const int mid = lo + (hi - lo) / 2;
        int c = 0;
#pragma unroll
        for (int e = 0; e < E; ++e) c += __popcll(__ballot(key[e] == T && id[e] <= mid));
        if (c >= need) hi = mid; else lo = mid + 1;
      }
      I = lo;
    }
  }
  int base = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const bool keep = key[e] > T || (key[e] == T && id[e] <= I);
    const unsigned long long m = __ballot(keep);
    if (keep) kept[base + __popcll(m & ((1ull << lane) - 1))] = id[e];
    base += __popcll(m);
  }
}

// fp64 value of the lane a DPP row control names (both halves moved as dwords).
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double x) {
  const int lo = __builtin_amdgcn_mov_dpp(__double2loint(x), CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_mov_dpp(__double2hiint(x), CTRL, 0xF, 0xF, false);
  return __hiloint2double(hi, lo);
}

// Sum over each row of 16 lanes, left in every lane of the row. After the two
// quad swaps every lane of a quad holds the quad's sum; the half-row mirror then
// pairs each quad with the other quad of its half-row, and the row mirror each
// half-row with the other -- the same pairing as exchanges across lane bits
// 0, 1, 2 and 3, done on the vector ALU instead of through LDS.
__device__ __forceinline__ double row16_sum(double v) {
  v += dpp_f64<0xB1>(v);   // quad_perm [1, 0, 3, 2]
  v += dpp_f64<0x4E>(v);   // quad_perm [2, 3, 0, 1]
  v += dpp_f64<0x141>(v);  // row_half_mirror
  v += dpp_f64<0x140>(v);  // row_mirror
  return v;
}

// Is node n of level l a candidate node for query block qb? Causal: it holds a
// block outside the sink (pools only ever hold complete nodes before the query
// block's ancestor); bidirectional: it exists and holds a block outside the sink
// other than qb itself.
__device__ __forceinline__ bool node_ok(const Geo& g, int l, int n, int qb, int lo) {
  if (g.causal) return n >= lo;
  if (n >= g.nodes[l]) return false;
  const int a = max(n * g.span[l], g.j0);
  const int b = min((n + 1) * g.span[l], g.nb);
  return b - a - ((a <= qb && qb < b) ? 1 : 0) > 0;
}

// Node id held by pool slot p at level l (kept children first, then the
// complete children of the query block's own ancestor).
__device__ __forceinline__ int slot_node(int p, int nchild, int f, const int* kept, int anc_first) {
  return p < nchild ? kept[p / f] * f + p % f : anc_first + (p - nchild);
}

// Node rows are scored by 16-lane groups: lane s of a group holds the 16-byte
// units s, s + 16, ... of the row (four floats each), so that each load
// instruction reads whole 128-byte lines of its four rows. qcol(s, e) is the
// column of the e-th value lane s holds.
__device__ __forceinline__ int qcol(int s, int e) { return ((e >> 2) * 16 + s) * 4 + (e & 3); }

// Score pool slots [0, M) into sm.sc (fp64 dot products with the query mean);
// the slots' nodes come from sm.node (-1: no node; its score is meaningless).
// 16 lanes per node, four nodes per wave load, U loads in flight.
template <int E, int D>
__device__ __forceinline__ void score_slots(const float* __restrict__ lvl, int M, WaveSmem<E, D>& sm,
                                            const double (&qv)[D / 16], int lane) {
  constexpr int DPL = D / 16;
  constexpr int U = 4;  // few registers: more waves per SIMD hide the latency instead
  const int grp = lane >> 4;
  const int sub = lane & 15;
  for (int base = 0; base < M; base += 4 * U) {  // base + 4U <= 64E, so every slot read is in the table
    float4 x[U][DPL / 4];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      // slots without a node read node 0 (always present) so that no load is
      // conditional; their scores are never ranked
      const int n = max(sm.node[base + u * 4 + grp], 0);
      const float4* row = reinterpret_cast<const float4*>(lvl + (int64_t)n * D);
#pragma unroll
      for (int e4 = 0; e4 < DPL / 4; ++e4) x[u][e4] = row[e4 * 16 + sub];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      double acc = 0.0;
#pragma unroll
      for (int e4 = 0; e4 < DPL / 4; ++e4) {
        acc += qv[e4 * 4 + 0] * (double)x[u][e4].x;
        acc += qv[e4 * 4 + 1] * (double)x[u][e4].y;
        acc += qv[e4 * 4 + 2] * (double)x[u][e4].z;
        acc += qv[e4 * 4 + 3] * (double)x[u][e4].w;
      }
      acc = row16_sum(acc);
      if (sub == 0) sm.sc[base + u * 4 + grp] = acc;
    }
  }
}

// Descent of one wave for query block (or decode token) qb of one slab.
// ps: the slab's pyramid; sm.qbar: the fp64 query mean (written by this wave).
// Writes out_idx[0, K) ascending, -1 padded, and *out_cnt. A level whose valid
// pool holds at most K nodes keeps them all, so it is not scored.
template <int E, int D>
__device__ void wave_descend(const Geo& g, const float* __restrict__ ps, int qb, int32_t* __restrict__ out_idx,
                             int32_t* __restrict__ out_cnt, WaveSmem<E, D>& sm, int lane) {
  constexpr int DPL = D / 16;
  if (g.K == 0) {
    if (lane == 0) *out_cnt = 0;
    return;
  }
  double qv[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) qv[e] = sm.qbar[qcol(lane & 15, e)];
  const int L = g.L;
  // top level: causal -- the complete nodes before the ancestor that hold a
  // non-sink block; bidirectional -- every node holding a candidate
  int lo = g.j0 / g.span[L - 1];
  int M = g.causal ? max(0, qb / g.span[L - 1] - lo) : g.nodes[L - 1];
  int nchild = 0;                      // slots that are children of kept nodes
  int anc_first = g.causal ? lo : 0;   // first node of the contiguous tail of the pool
  for (int l = L - 1; l >= 0; --l) {
    // slot ids and validity need no scores
    int id[E];
    int nvalid = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int p = e * 64 + lane;
      const int n = p < M ? slot_node(p, nchild, g.f, sm.kept, anc_first) : INT_MAX;
      const bool valid = p < M && node_ok(g, l, n, qb, lo);
      id[e] = valid ? n : INT_MAX;
      nvalid += __popcll(__ballot(valid));
    }
    const int nk = min(g.K, nvalid);
    if (nvalid > g.K) {
#pragma unroll
      for (int e = 0; e < E; ++e) sm.node[e * 64 + lane] = id[e] != INT_MAX ? id[e] : -1;
      __builtin_amdgcn_wave_barrier();
      score_slots<E, D>(ps + (int64_t)g.off[l] * D, M, sm, qv, lane);
      __builtin_amdgcn_wave_barrier();
      // the slot ids come back from the table, so they need no registers while scoring
      uint64_t key[E];
#pragma unroll
      for (int e = 0; e < E; ++e) {
        id[e] = sm.node[e * 64 + lane];
        key[e] = id[e] >= 0 ? score_key(sm.sc[e * 64 + lane]) : 0ull;
      }
      wave_keep_best<E>(key, id, nk, sm.kept, lane);
    } else {
      // keep every valid slot, compacted in slot order
      int base = 0;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const unsigned long long m = __ballot(id[e] != INT_MAX);
        if (id[e] != INT_MAX) sm.kept[base + __popcll(m & ((1ull << lane) - 1))] = id[e];
        base += __popcll(m);
      }
    }
    __builtin_amdgcn_wave_barrier();
    if (l == 0) {
      for (int t = lane; t < nk; t += 64) {
        const int v = sm.kept[t];
        int r = 0;
        for (int u = 0; u < nk; ++u) r += (sm.kept[u] < v);
        out_idx[r] = v;
      }
      for (int t = nk + lane; t < g.K; t += 64) out_idx[t] = -1;
      if (lane == 0) *out_cnt = nk;
      return;
    }
    // next level's pool: children of the kept nodes, then (causal) the complete
    // children of the ancestor; invalid nodes are masked by node_ok
    nchild = nk * g.f;
    if (g.causal) {
      anc_first = (qb / g.span[l]) * g.f;
      M = nchild + (qb / g.span[l - 1] - anc_first);
    } else {
      anc_first = 0;
      M = nchild;
    }
    lo = g.j0 / g.span[l - 1];
  }
}

// ---------------------------------------------------------------------------
// Descent by a whole workgroup of NT threads for one query (decode): each level's
// pool is scored in rounds of loads (U nodes per 16-lane group), and the first
// wave keeps the best K with the same threshold search as the per-wave descent
// (E pool slots per lane cover the largest pool).

struct BlockSmem {
  double sc[kPoolMax];
  int id[kPoolMax];  // node held by each pool slot of the level, INT_MAX if none
  int kept[kMaxTopK];
  int wcnt[16];      // valid slots counted by each wave
};

template <int D, int NT, int U, int E>
__device__ void block_descend(const Geo& g, const float* __restrict__ ps, int qb, const double* qbar,
                              int32_t* __restrict__ out_idx, int32_t* __restrict__ out_cnt, BlockSmem& sm) {
  constexpr int DPL = D / 16;
  constexpr int NG = NT / 16;  // 16-lane groups
  constexpr int NWV = NT / 64;
  static_assert(NWV <= 16, "per-wave counts");
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int grp = tid >> 4;
  const int sub = tid & 15;
  if (g.K == 0) {
    if (tid == 0) *out_cnt = 0;
    return;
  }
  double qv[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) qv[e] = qbar[qcol(sub, e)];
  const int L = g.L;
  int lo = g.j0 / g.span[L - 1];
  int M = max(0, qb / g.span[L - 1] - lo);
  int nchild = 0, anc_first = lo;
  for (int l = L - 1; l >= 0; --l) {
    const float* lvl = ps + (int64_t)g.off[l] * D;
    // the level's pool as node ids (INT_MAX: no candidate), and its valid count
    int nv_local = 0;
    for (int p0 = 0; p0 < M; p0 += NT) {
      const int p = p0 + tid;
      const int n = p < M ? slot_node(p, nchild, g.f, sm.kept, anc_first) : INT_MAX;
      const bool valid = p < M && n >= lo;
      if (p < M) sm.id[p] = valid ? n : INT_MAX;
      nv_local += __popcll(__ballot(valid));
    }
    if (lane == 0) sm.wcnt[wave] = nv_local;
    __syncthreads();
    int nvalid = 0;
#pragma unroll
    for (int w = 0; w < NWV; ++w) nvalid += sm.wcnt[w];
    const int nk = min(g.K, nvalid);
    if (nvalid > g.K) {  // score the pool; a level with at most K valid slots keeps them all
      // slots without a node read a complete node of the pool (the first child of
      // the first kept node, or at the top level the first node of the ancestor
      // tail) so that no load is conditional; their scores are never used. A
      // complete node is never written by the append of a token of this query's
      // block, so that append may run beside this descent.
      const int stand_in = nchild > 0 ? sm.kept[0] * g.f : anc_first;
      for (int base = 0; base < M; base += NG * U) {
        float4 x[U][DPL / 4];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int p = base + u * NG + grp;
          const int n = p < M ? sm.id[p] : INT_MAX;
          const float4* row = reinterpret_cast<const float4*>(lvl + (int64_t)(n != INT_MAX ? n : stand_in) * D);
#pragma unroll
          for (int e4 = 0; e4 < DPL / 4; ++e4) x[u][e4] = row[e4 * 16 + sub];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          double acc = 0.0;
#pragma unroll
          for (int e4 = 0; e4 < DPL / 4; ++e4) {
            acc += qv[e4 * 4 + 0] * (double)x[u][e4].x;
            acc += qv[e4 * 4 + 1] * (double)x[u][e4].y;
            acc += qv[e4 * 4 + 2] * (double)x[u][e4].z;
            acc += qv[e4 * 4 + 3] * (double)x[u][e4].w;
          }
          acc = row16_sum(acc);
          const int p = base + u * NG + grp;
          if (sub == 0 && p < M) sm.sc[p] = acc;
        }
      }
    }
    __syncthreads();
    if (tid < 64) {  // the first wave keeps the level's best (M <= 64 E)
      int id[E];
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int p = e * 64 + tid;
        id[e] = p < M ? sm.id[p] : INT_MAX;
      }
      if (nvalid > g.K) {
        uint64_t key[E];
#pragma unroll
        for (int e = 0; e < E; ++e) key[e] = id[e] != INT_MAX ? score_key(sm.sc[e * 64 + tid]) : 0ull;
        wave_keep_best<E>(key, id, nk, sm.kept, tid);
      } else {
        // every valid slot, compacted in slot order
        int base = 0;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const unsigned long long m = __ballot(id[e] != INT_MAX);
          if (id[e] != INT_MAX) sm.kept[base + __popcll(m & ((1ull << tid) - 1))] = id[e];
          base += __popcll(m);
        }
      }
    }
    __syncthreads();
    if (l == 0) {
      for (int t = tid; t < nk; t += NT) {
        const int v = sm.kept[t];
        int r = 0;
        for (int u = 0; u < nk; ++u) r += (sm.kept[u] < v);
        out_idx[r] = v;
      }
      for (int t = nk + tid; t < g.K; t += NT) out_idx[t] = -1;
      if (tid == 0) *out_cnt = nk;
      return;
    }
    const int a_l = qb / g.span[l];
    const int a_below = qb / g.span[l - 1];
    nchild = nk * g.f;
    anc_first = a_l * g.f;
    M = nchild + (a_below - anc_first);
    lo = g.j0 / g.span[l - 1];
  }
}

}  // namespace pisa
