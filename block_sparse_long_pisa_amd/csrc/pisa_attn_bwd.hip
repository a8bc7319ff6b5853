// Backward pass of the sparse attention, the selection held constant (the PISA
// page, "Attention clairsemée PISA : noyaux Triton sans matrice de scores",
// says its kernels serve training as well as inference; the gradients are those
// of the exact softmax attention over each query's attended key set).
//
// For query row i with attended keys A(i), logits s = scale q_i.k_t, weights
// p = exp(s - lse_i) (lse from the forward), and dO_i the output gradient:
//   D_i   = dO_i . O_i                          (bwd_rowdot_kernel)
//   dP_it = dO_i . v_t,  dS_it = p_it (dP_it - D_i)
//   dQ_i  = scale sum_t dS_it k_t               (bwd_dq_kernel: query-centric, the
//                                               forward's walk and tiles)
//   dK_t  = scale sum_i dS_it q_i,  dV_t = sum_i p_it dO_i
//                                               (bwd_kv_kernel: key-centric)
// The key-centric pass needs, for every key block, the query blocks whose walk
// holds it: bwd_list_kernel builds those lists in query-block order (binary
// search in the ascending selections, no atomics, so results are
// deterministic). A list is cut into segments of kBwdSeg entries -- the sink
// block is attended by every query block -- each segment's partial sums land in
// the workspace, and bwd_kv_reduce adds them in order.
//
// All products run on bf16 matrix cores with fp32 accumulation; p and dS are
// rounded to bf16 before the products that consume them.
#include "pisa_attn_common.h"

namespace pisa {
namespace {

constexpr int kBwdSeg = 64;  // list entries (query blocks) per key-centric segment
constexpr int kListThreads = 256;

enum : int { kFull = 0, kSinkPart = 1, kLocal = 2 };

// ---------------------------------------------------------------------------
// D_i = dO_i . O_i, 16 lanes per row; beside it lse_i in log2 units, so that the
// key-centric pass takes p = exp2(s c - lse2) with one fused multiply-add

template <int D>
__global__ __launch_bounds__(256) void bwd_rowdot_kernel(const uint16_t* __restrict__ dout,
                                                         const uint16_t* __restrict__ out, const float* __restrict__ lse,
                                                         float* __restrict__ rowdot, float* __restrict__ lse2,
                                                         int64_t rows) {
  constexpr int PER = D / 16;  // bf16 per lane
  const int64_t r = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int sub = threadIdx.x & 15;
  const int64_t rr = r < rows ? r : rows - 1;
  float s = 0.f;
  if constexpr (PER == 8) {
    const uint4 a = *reinterpret_cast<const uint4*>(dout + rr * D + sub * 8);
    const uint4 o = *reinterpret_cast<const uint4*>(out + rr * D + sub * 8);
    const uint32_t av[4] = {a.x, a.y, a.z, a.w}, ov[4] = {o.x, o.y, o.z, o.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) s += bf16lo(av[e]) * bf16lo(ov[e]) + bf16hi(av[e]) * bf16hi(ov[e]);
  } else {
    const uint2 a = *reinterpret_cast<const uint2*>(dout + rr * D + sub * 4);
    const uint2 o = *reinterpret_cast<const uint2*>(out + rr * D + sub * 4);
    s = bf16lo(a.x) * bf16lo(o.x) + bf16hi(a.x) * bf16hi(o.x) + bf16lo(a.y) * bf16lo(o.y) + bf16hi(a.y) * bf16hi(o.y);
  }
#pragma unroll
  for (int sh = 1; sh < 16; sh <<= 1) s += __shfl_xor(s, sh);
  if (sub == 0 && r < rows) {
    rowdot[r] = s;
    lse2[r] = lse[r] * kLog2e;
  }
}

// ---------------------------------------------------------------------------
// dQ: query-centric. A workgroup serves NW waves x 32 query rows of one
// (batch, kv head, query block) unit and walks the unit's attended tiles as
// the forward does. K is staged with the transposing-read pitch (it is read
// both as rows, for S^T = K Q^T, and as columns, for dQ^T += K^T dS^T), V with
// the row pitch (dP^T = V dO^T).

template <int D, int BS>
struct DqState {
  bf16x8_t qf[D / 16];
  bf16x8_t df[D / 16];
  f32x16_t acc[D / 32];
  float lse2;  // this lane's query: lse in log2 units (+inf for a row past the sequence)
  float rd;    // this lane's query: D_i
  int offkt;   // transposing reads of the K tile
};

template <int D, int BS>
__device__ __forceinline__ void dq_tile(DqState<D, BS>& st, const uint16_t* ks, const uint16_t* vs, int nvalid,
                                        bool local, int key0, int qpos, int l32, int hi, float c, int wg_qmax) {
  constexpr int NDS = D / 16, NDB = D / 32;
  constexpr int KC = BS < 64 ? BS : 64;
  constexpr int NKB = KC / 32;
  constexpr int PK = TilePitch<D, BS>::K, PV = TilePitch<D, BS>::V;
#pragma unroll
  for (int ch = 0; ch < BS / KC; ++ch) {
    if (ch > 0 && (ch * KC >= nvalid || (local && key0 + ch * KC > wg_qmax))) break;
    f32x16_t s[NKB], dp[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kb][i] = dp[kb][i] = 0.f;
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds) {
        const int row = ch * KC + kb * 32 + l32, col = ds * 16 + hi * 8;
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_frag<PV>(ks, row, col), st.qf[ds], s[kb], 0, 0, 0);
        dp[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_frag<PK>(vs, row, col), st.df[ds], dp[kb], 0, 0, 0);
      }
    }
    // keys of this chunk past `lim` are masked (partial block, causal diagonal)
    const int lim = min(nvalid - 1, local ? qpos - key0 : BS - 1) - (ch * KC + hi * 4);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const bool on = kb * 32 + (i >> 2) * 8 + (i & 3) <= lim;
        const float p = on ? fast_exp2(fmaf(s[kb][i], c, -st.lse2)) : 0.f;
        s[kb][i] = p * (dp[kb][i] - st.rd);  // dS^T
      }
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        bf16x8_t b;
#pragma unroll
        for (int e = 0; e < 8; ++e) b[e] = (__bf16)s[kb][hh * 8 + e];
#pragma unroll
        for (int db = 0; db < NDB; ++db)
          st.acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_frag<PV>(ks, st.offkt, ch * KC + kb * 32 + hh * 16, db),
                                                               b, st.acc[db], 0, 0, 0);
      }
  }
}

template <int D, int BS, int NW>
__global__ __launch_bounds__(NW * 64) void bwd_dq_kernel(Geo g, const uint16_t* __restrict__ q,
                                                         const uint16_t* __restrict__ k,
                                                         const uint16_t* __restrict__ v,
                                                         const int32_t* __restrict__ idx,
                                                         const int32_t* __restrict__ cnt,
                                                         const uint16_t* __restrict__ dout,
                                                         const float* __restrict__ lse,
                                                         const float* __restrict__ rowdot, uint16_t* __restrict__ dq,
                                                         int parts) {
  constexpr int NT = NW * 64;
  constexpr int NDS = D / 16, NDB = D / 32;
  using TP = TilePitch<D, BS>;
  // stage s: V rows at the row pitch (VS*), K at the transposing pitch (KS*)
  __shared__ __attribute__((aligned(16))) uint16_t VS0[TP::KSIZE];
  __shared__ __attribute__((aligned(16))) uint16_t KS0[TP::VSIZE];
  __shared__ __attribute__((aligned(16))) uint16_t VS1[TP::KSIZE];
  __shared__ __attribute__((aligned(16))) uint16_t KS1[TP::VSIZE];
  __shared__ int sel[kMaxTopK];

  const int slabs = g.B * g.Hkv;
  const int wg = blockIdx.x;
  const int slab = wg % slabs;
  const int part = (wg / slabs) % parts;
  const int qb = g.nb - 1 - wg / (slabs * parts);
  const int b = slab / g.Hkv;
  const int kvh = slab % g.Hkv;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
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

  DqState<D, BS> st;
  const int64_t row = ((int64_t)b * g.Hq + h) * g.N + (qvalid ? qpos : 0);
#pragma unroll
  for (int ds = 0; ds < NDS; ++ds) {
    const uint4 uq = qvalid ? *reinterpret_cast<const uint4*>(q + row * D + ds * 16 + hi * 8) : make_uint4(0, 0, 0, 0);
    const uint4 ud = qvalid ? *reinterpret_cast<const uint4*>(dout + row * D + ds * 16 + hi * 8) : make_uint4(0, 0, 0, 0);
    st.qf[ds] = __builtin_bit_cast(bf16x8_t, uq);
    st.df[ds] = __builtin_bit_cast(bf16x8_t, ud);
  }
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) st.acc[db][i] = 0.f;
  st.lse2 = qvalid ? lse[row] * kLog2e : __builtin_inff();
  st.rd = qvalid ? rowdot[row] : 0.f;
  st.offkt = tr_offset<TP::V>(lane);
  const float c = g.scale * kLog2e;
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
  issue_tile<D, BS, NW>(vbase + (int64_t)j * BS * D, kbase + (int64_t)j * BS * D, min(BS, g.N - j * BS), VS0, KS0,
                        wave, lane, plan);
  for (int t = 0; t < walk.ntiles; t += 2) {
    wait_loads_and_sync();
    int j1 = 0, nv1 = 0;
    bool loc1 = false;
    if (t + 1 < walk.ntiles) {
      walk.at(t + 1, sel, g, qb, local_rows, j1, nv1, loc1);
      issue_tile<D, BS, NW>(vbase + (int64_t)j1 * BS * D, kbase + (int64_t)j1 * BS * D, min(BS, g.N - j1 * BS), VS1,
                            KS1, wave, lane, plan);
    }
    dq_tile<D, BS>(st, KS0, VS0, nvalid, local, j * BS, qpos, l32, hi, c, wg_qmax);
    if (t + 1 >= walk.ntiles) break;
    wait_loads_and_sync();
    if (t + 2 < walk.ntiles) {
      walk.at(t + 2, sel, g, qb, local_rows, j, nvalid, local);
      issue_tile<D, BS, NW>(vbase + (int64_t)j * BS * D, kbase + (int64_t)j * BS * D, min(BS, g.N - j * BS), VS0,
                            KS0, wave, lane, plan);
    }
    dq_tile<D, BS>(st, KS1, VS1, nv1, loc1, j1 * BS, qpos, l32, hi, c, wg_qmax);
  }

  if (qvalid) {
    uint16_t* drow = dq + row * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 16; i += 4) {
        const int d = db * 32 + (i >> 2) * 8 + hi * 4;
        uint2 w;
        w.x = pack_bf16x2(st.acc[db][i] * g.scale, st.acc[db][i + 1] * g.scale);
        w.y = pack_bf16x2(st.acc[db][i + 2] * g.scale, st.acc[db][i + 3] * g.scale);
        *reinterpret_cast<uint2*>(drow + d) = w;
      }
  }
}

// ---------------------------------------------------------------------------
// Lists: for key block j of a slab, the query blocks whose walk holds it, in
// query-block order, each with the kind of tile it is for that query block.

__device__ __forceinline__ bool sel_has(const int32_t* __restrict__ sel, int n, int j) {
  int lo = 0, hi = n;  // ascending selections
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (sel[mid] < j) lo = mid + 1; else hi = mid;
  }
  return lo < n && sel[lo] == j;
}

// -1 if query block qb does not attend key block j; otherwise the tile kind
// (the forward's walk: full sink blocks, the partial sink block unless
// selected, the selected blocks, the local block).
__device__ __forceinline__ int tile_kind(const Geo& g, const int32_t* __restrict__ idx, const int32_t* __restrict__ cnt,
                                         int slab, int j, int qb) {
  if (qb == j) return kLocal;
  if (qb < j) return -1;
  if (j < g.j0) return kFull;
  const int64_t unit = (int64_t)slab * g.nb + qb;
  const int n = min(max(cnt[unit], 0), g.K);
  const bool chosen = sel_has(idx + unit * g.K, n, j);
  if (j == g.j0 && g.sink > g.j0 * g.bs) return chosen ? kFull : kSinkPart;
  return chosen ? kFull : -1;
}

// One workgroup per (slab, key block). fill == 0: count the entries;
// fill == 1: write them (qb | kind << 28) from list_off on.
__global__ __launch_bounds__(kListThreads) void bwd_list_kernel(Geo g, const int32_t* __restrict__ idx,
                                                                const int32_t* __restrict__ cnt,
                                                                int32_t* __restrict__ counts,
                                                                const int32_t* __restrict__ list_off,
                                                                int32_t* __restrict__ lists, int fill) {
  __shared__ int wsum[kListThreads / 64];
  const int kbid = blockIdx.x;
  const int slab = kbid / g.nb;
  const int j = kbid % g.nb;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int base = 0;
  for (int qb0 = j; qb0 < g.nb; qb0 += kListThreads) {
    const int qb = qb0 + tid;
    const int kind = qb < g.nb ? tile_kind(g, idx, cnt, slab, j, qb) : -1;
    const unsigned long long m = __ballot(kind >= 0);
    if (lane == 0) wsum[wave] = __popcll(m);
    __syncthreads();
    int before = base, total = base;
    for (int w = 0; w < kListThreads / 64; ++w) {
      if (w < wave) before += wsum[w];
      total += wsum[w];
    }
    if (fill && kind >= 0) lists[list_off[kbid] + before + __popcll(m & ((1ull << lane) - 1))] = qb | (kind << 28);
    base = total;
    __syncthreads();
  }
  if (!fill && tid == 0) counts[kbid] = base;
}

// Exclusive scans of the list lengths and of the segment counts (one workgroup).
__global__ __launch_bounds__(1024) void bwd_scan_kernel(const int32_t* __restrict__ counts, int n,
                                                        int32_t* __restrict__ list_off, int32_t* __restrict__ seg_off) {
  __shared__ int s_l[1024], s_s[1024];
  __shared__ int carry_l, carry_s;
  if (threadIdx.x == 0) carry_l = carry_s = 0;
  __syncthreads();
  for (int base = 0; base < n; base += 1024) {
    const int i = base + threadIdx.x;
    const int cl = i < n ? counts[i] : 0;
    const int cs = (cl + kBwdSeg - 1) / kBwdSeg;
    s_l[threadIdx.x] = cl;
    s_s[threadIdx.x] = cs;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {  // inclusive Hillis-Steele scan
      const int al = threadIdx.x >= off ? s_l[threadIdx.x - off] : 0;
      const int as = threadIdx.x >= off ? s_s[threadIdx.x - off] : 0;
      __syncthreads();
      s_l[threadIdx.x] += al;
      s_s[threadIdx.x] += as;
      __syncthreads();
    }
    if (i < n) {
      list_off[i] = carry_l + s_l[threadIdx.x] - cl;
      seg_off[i] = carry_s + s_s[threadIdx.x] - cs;
    }
    __syncthreads();
    if (threadIdx.x == 1023) {
      carry_l += s_l[1023];
      carry_s += s_s[1023];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    list_off[n] = carry_l;
    seg_off[n] = carry_s;
  }
}

// ---------------------------------------------------------------------------
// dK, dV: key-centric. A workgroup serves one segment of one key block's list;
// wave w owns keys [32 w, 32 w + 32) of the block and keeps their K and V rows
// as matrix operands. For every (query block, head) of the segment the query
// rows and their output gradients are staged in LDS (Q at the row pitch, dO at
// the transposing pitch) and
//   S = Q K^T, dP = dO V^T (lane = key), p, dS,
//   dV^T += dO^T p, dK^T += Q^T dS   (d x keys, lane = key).

template <int D, int BS>
__device__ __forceinline__ void kv_tile(const bf16x8_t (&kf)[D / 16], const bf16x8_t (&vf)[D / 16],
                                        f32x16_t (&dk)[D / 32], f32x16_t (&dv)[D / 32], const uint16_t* qs,
                                        const uint16_t* os, const float* ls, const float* rs, bool mask, int rows,
                                        int rlo, int l32, int hi, int offq, int offo, float c) {
  constexpr int NDS = D / 16, NDB = D / 32;
  constexpr int QC = 32;  // query rows per chunk (one 32-row block keeps the registers in bounds)
  constexpr int PK = TilePitch<D, BS>::K, PV = TilePitch<D, BS>::V;
#pragma unroll
  for (int ch = 0; ch < BS / QC; ++ch) {
    if (ch > 0 && ch * QC >= rows) break;
    f32x16_t s, dp;
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = dp[i] = 0.f;
    // every LDS fragment of the chunk is requested before its first product: with
    // one wave per SIMD nothing else hides the LDS latency
    bf16x8_t fq[NDS], fo[NDS], tv[2][NDB], tq[2][NDB];
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
      const int row = ch * QC + l32, col = ds * 16 + hi * 8;
      fq[ds] = row_frag<PK>(qs, row, col);
      fo[ds] = row_frag<PV>(os, row, col);
    }
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        tv[hh][db] = tr_frag<PV>(os, offo, ch * QC + hh * 16, db);
        tq[hh][db] = tr_frag<PK>(qs, offq, ch * QC + hh * 16, db);
      }
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fq[ds], kf[ds], s, 0, 0, 0);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fo[ds], vf[ds], dp, 0, 0, 0);
    }
    // element i is query row r = ch*QC + (i/4)*8 + hi*4 + i%4; ls holds lse in
    // log2 units
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const float4 l4 = *reinterpret_cast<const float4*>(ls + ch * QC + i4 * 8 + hi * 4);
      const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) s[i4 * 4 + e] = fast_exp2(fmaf(s[i4 * 4 + e], c, -lv[e]));
    }
    if (mask) {  // uniform: only partial-sink, causal and ragged tiles; rows [rlo, rows) count for this key
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = ch * QC + (i >> 2) * 8 + hi * 4 + (i & 3);
        s[i] = r >= rlo && r < rows ? s[i] : 0.f;
      }
    }
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const float4 d4 = *reinterpret_cast<const float4*>(rs + ch * QC + i4 * 8 + hi * 4);
      const float dv4[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) dp[i4 * 4 + e] = s[i4 * 4 + e] * (dp[i4 * 4 + e] - dv4[e]);
    }
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      bf16x8_t pb, sb;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        pb[e] = (__bf16)s[hh * 8 + e];
        sb[e] = (__bf16)dp[hh * 8 + e];
      }
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tv[hh][db], pb, dv[db], 0, 0, 0);
        dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tq[hh][db], sb, dk[db], 0, 0, 0);
      }
    }
  }
}

// One (query block, head) stage. Whole tiles of full kind (every row and key
// counts) skip the mask; otherwise the rows that count for this lane's key are
// [rlo, rows): rlo = the key's own row on the causal diagonal, past the block
// for a key outside the sink (partial sink tile) or the sequence.
template <int D, int BS>
__device__ __forceinline__ void kv_stage(const bf16x8_t (&kf)[D / 16], const bf16x8_t (&vf)[D / 16],
                                         f32x16_t (&dk)[D / 32], f32x16_t (&dv)[D / 32], const uint16_t* qs,
                                         const uint16_t* os, const float* ls, const float* rs, const Geo& g, int qb,
                                         int kind, int j, int key, int l32, int hi, int offq, int offo, float c) {
  const int rows = min(BS, g.N - qb * BS);
  const bool mask = !(kind == kFull && rows == BS && (j + 1) * BS <= g.N);
  const bool key_ok = key < (kind == kSinkPart ? g.sink : g.N);
  const int rlo = !key_ok ? BS : kind == kLocal ? (key & (BS - 1)) : 0;
  kv_tile<D, BS>(kf, vf, dk, dv, qs, os, ls, rs, mask, rows, rlo, l32, hi, offq, offo, c);
}

// Issue the copies of one (query block, head) stage: Q and dO rows, and the
// rows' lse and D (64 floats per wave instruction; rows past the sequence
// re-read the last row, they are masked by `rows`).
template <int D, int BS, int NW>
__device__ __forceinline__ void issue_rows(const Geo& g, const uint16_t* q, const uint16_t* dout, const float* lse,
                                           const float* rowdot, int b, int h, int qb, uint16_t* qdst, uint16_t* odst,
                                           float* ldst, float* rdst, int wave, int lane,
                                           const DmaPlan<D, BS, NW>& plan) {
  const int64_t r0 = ((int64_t)b * g.Hq + h) * g.N + (int64_t)qb * BS;
  const int rows = min(BS, g.N - qb * BS);
  issue_tile<D, BS, NW>(q + r0 * D, dout + r0 * D, rows, qdst, odst, wave, lane, plan);
#pragma unroll
  for (int n = 0; n < (BS + 63) / 64; ++n) {
    if (n % NW == wave) {
      const int r = min(n * 64 + lane, rows - 1);
      __builtin_amdgcn_global_load_lds(lse + r0 + r, (lds_void_ptr)(ldst + n * 64), 4, 0, 0);
      __builtin_amdgcn_global_load_lds(rowdot + r0 + r, (lds_void_ptr)(rdst + n * 64), 4, 0, 0);
    }
  }
}

template <int D, int BS>
__global__ __launch_bounds__(BS / 32 * 64) void bwd_kv_kernel(Geo g, const uint16_t* __restrict__ q,
                                                              const uint16_t* __restrict__ k,
                                                              const uint16_t* __restrict__ v,
                                                              const uint16_t* __restrict__ dout,
                                                              const float* __restrict__ lse2,
                                                              const float* __restrict__ rowdot,
                                                              const int32_t* __restrict__ lists,
                                                              const int32_t* __restrict__ list_off,
                                                              const int32_t* __restrict__ seg_off, int nkb,
                                                              float* __restrict__ pdk, float* __restrict__ pdv) {
  constexpr int NW = BS / 32;
  constexpr int NDS = D / 16, NDB = D / 32;
  constexpr int LS = BS < 64 ? 64 : BS;  // lse / D slots per stage (whole 64-float copies)
  using TP = TilePitch<D, BS>;
  __shared__ __attribute__((aligned(16))) uint16_t Q0[TP::KSIZE];
  __shared__ __attribute__((aligned(16))) uint16_t O0[TP::VSIZE];
  __shared__ __attribute__((aligned(16))) uint16_t Q1[TP::KSIZE];
  __shared__ __attribute__((aligned(16))) uint16_t O1[TP::VSIZE];
  __shared__ __attribute__((aligned(16))) float L0[LS], R0[LS], L1[LS], R1[LS];

  const int w = blockIdx.x;
  if (w >= seg_off[nkb]) return;  // past the last segment (uniform)
  int lo = 0, hi_ = nkb - 1;      // the key block: last kb with seg_off[kb] <= w
  while (lo < hi_) {
    const int mid = (lo + hi_ + 1) >> 1;
    if (seg_off[mid] <= w) lo = mid; else hi_ = mid - 1;
  }
  const int kbid = lo;
  const int slab = kbid / g.nb;
  const int j = kbid % g.nb;
  const int b = slab / g.Hkv;
  const int kvh = slab % g.Hkv;
  const int e0 = list_off[kbid] + (w - seg_off[kbid]) * kBwdSeg;
  const int e1 = min(list_off[kbid + 1], e0 + kBwdSeg);
  const int npairs = (e1 - e0) * g.G;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int key = j * BS + wave * 32 + l32;
  const int64_t krow = ((int64_t)b * g.Hkv + kvh) * g.N + min(key, g.N - 1);
  bf16x8_t kf[NDS], vf[NDS];
#pragma unroll
  for (int ds = 0; ds < NDS; ++ds) {
    kf[ds] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(k + krow * D + ds * 16 + hi * 8));
    vf[ds] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(v + krow * D + ds * 16 + hi * 8));
  }
  f32x16_t dk[NDB], dv[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) dk[db][i] = dv[db][i] = 0.f;
  const int offq = tr_offset<TP::K>(lane);
  const int offo = tr_offset<TP::V>(lane);
  const float c = g.scale * kLog2e;
  DmaPlan<D, BS, NW> plan;
  plan.init(wave, lane);

  auto entry = [&](int t, int& qb, int& h, int& kind) {
    const int e = lists[e0 + t / g.G];
    qb = e & 0x0fffffff;
    kind = e >> 28;
    h = kvh * g.G + t % g.G;
  };
  int qb, h, kind;
  entry(0, qb, h, kind);
  issue_rows<D, BS, NW>(g, q, dout, lse2, rowdot, b, h, qb, Q0, O0, L0, R0, wave, lane, plan);
  for (int t = 0; t < npairs; t += 2) {
    wait_loads_and_sync();
    int qb1 = 0, h1 = 0, kind1 = 0;
    if (t + 1 < npairs) {
      entry(t + 1, qb1, h1, kind1);
      issue_rows<D, BS, NW>(g, q, dout, lse2, rowdot, b, h1, qb1, Q1, O1, L1, R1, wave, lane, plan);
    }
    kv_stage<D, BS>(kf, vf, dk, dv, Q0, O0, L0, R0, g, qb, kind, j, key, l32, hi, offq, offo, c);
    if (t + 1 >= npairs) break;
    wait_loads_and_sync();
    if (t + 2 < npairs) {
      entry(t + 2, qb, h, kind);
      issue_rows<D, BS, NW>(g, q, dout, lse2, rowdot, b, h, qb, Q0, O0, L0, R0, wave, lane, plan);
    }
    kv_stage<D, BS>(kf, vf, dk, dv, Q1, O1, L1, R1, g, qb1, kind1, j, key, l32, hi, offq, offo, c);
  }
  // partial sums of this segment: [segment][key of the block][d], fp32
  float* pk = pdk + ((int64_t)w * BS + wave * 32 + l32) * D;
  float* pv = pdv + ((int64_t)w * BS + wave * 32 + l32) * D;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; i += 4) {
      const int d = db * 32 + (i >> 2) * 8 + hi * 4;
      *reinterpret_cast<float4*>(pk + d) = make_float4(dk[db][i], dk[db][i + 1], dk[db][i + 2], dk[db][i + 3]);
      *reinterpret_cast<float4*>(pv + d) = make_float4(dv[db][i], dv[db][i + 1], dv[db][i + 2], dv[db][i + 3]);
    }
}

// dK = scale * (sum of the segments' partial sums), dV = sum, in segment order.
template <int D>
__global__ __launch_bounds__(256) void bwd_kv_reduce_kernel(Geo g, const int32_t* __restrict__ seg_off,
                                                            const float* __restrict__ pdk,
                                                            const float* __restrict__ pdv, uint16_t* __restrict__ dk,
                                                            uint16_t* __restrict__ dv) {
  const int kbid = blockIdx.x;
  const int slab = kbid / g.nb;
  const int j = kbid % g.nb;
  const int s0 = seg_off[kbid], s1 = seg_off[kbid + 1];
  const int rows = min(g.bs, g.N - j * g.bs);
  for (int e = threadIdx.x * 4; e < rows * D; e += 256 * 4) {
    const int r = e / D, d = e % D;
    float4 sk = make_float4(0.f, 0.f, 0.f, 0.f), sv = sk;
    for (int s = s0; s < s1; ++s) {
      const float4 a = *reinterpret_cast<const float4*>(pdk + ((int64_t)s * g.bs + r) * D + d);
      const float4 bb = *reinterpret_cast<const float4*>(pdv + ((int64_t)s * g.bs + r) * D + d);
      sk.x += a.x; sk.y += a.y; sk.z += a.z; sk.w += a.w;
      sv.x += bb.x; sv.y += bb.y; sv.z += bb.z; sv.w += bb.w;
    }
    const int64_t o = ((int64_t)slab * g.N + (int64_t)j * g.bs + r) * D + d;
    *reinterpret_cast<uint2*>(dk + o) =
        make_uint2(pack_bf16x2(sk.x * g.scale, sk.y * g.scale), pack_bf16x2(sk.z * g.scale, sk.w * g.scale));
    *reinterpret_cast<uint2*>(dv + o) = make_uint2(pack_bf16x2(sv.x, sv.y), pack_bf16x2(sv.z, sv.w));
  }
}

// ---------------------------------------------------------------------------
// workspace

struct BwdWs {
  float* rowdot;    // [B, Hq, N]
  float* lse2;      // [B, Hq, N]: lse * log2(e)
  int32_t* counts;  // [nkb]
  int32_t* list_off;  // [nkb + 1]
  int32_t* seg_off;   // [nkb + 1]
  int32_t* lists;     // [max_entries]
  float* pdk;         // [max_segs, bs, D]
  float* pdv;
};

struct BwdSizes {
  int64_t nkb, max_entries, max_segs;
};

BwdSizes bwd_sizes(const Geo& g) {
  BwdSizes z;
  z.nkb = (int64_t)g.B * g.Hkv * g.nb;
  // a query block's walk: full sink blocks, the partial sink block, K selected, the local block
  z.max_entries = z.nkb * (min(g.j0, g.nb) + 1 + g.K + 1);
  z.max_segs = z.nkb + (z.max_entries + kBwdSeg - 1) / kBwdSeg;
  return z;
}

size_t rnd(size_t x) { return (x + 255) & ~(size_t)255; }

BwdWs carve_bwd(const Geo& g, void* base) {
  const BwdSizes z = bwd_sizes(g);
  char* p = (char*)base;
  auto take = [&](size_t bytes) {
    char* r = p;
    p += rnd(bytes);
    return r;
  };
  BwdWs w;
  w.rowdot = (float*)take(sizeof(float) * (size_t)g.B * g.Hq * g.N);
  w.lse2 = (float*)take(sizeof(float) * (size_t)g.B * g.Hq * g.N);
  w.counts = (int32_t*)take(sizeof(int32_t) * z.nkb);
  w.list_off = (int32_t*)take(sizeof(int32_t) * (z.nkb + 1));
  w.seg_off = (int32_t*)take(sizeof(int32_t) * (z.nkb + 1));
  w.lists = (int32_t*)take(sizeof(int32_t) * z.max_entries);
  w.pdk = (float*)take(sizeof(float) * (size_t)z.max_segs * g.bs * g.D);
  w.pdv = (float*)take(sizeof(float) * (size_t)z.max_segs * g.bs * g.D);
  return w;
}

template <int D, int BS>
hipError_t launch_bwd_t(const Geo& g, const void* q, const void* k, const void* v, const int32_t* idx,
                        const int32_t* cnt, const void* out, const float* lse, const void* dout, void* dq, void* dk,
                        void* dv, void* wsb, hipStream_t s) {
  const BwdSizes z = bwd_sizes(g);
  BwdWs w = carve_bwd(g, wsb);
  const uint16_t *qt = (const uint16_t*)q, *kt = (const uint16_t*)k, *vt = (const uint16_t*)v;
  const uint16_t* dot = (const uint16_t*)dout;
  const int64_t rows = (int64_t)g.B * g.Hq * g.N;
  hipLaunchKernelGGL((bwd_rowdot_kernel<D>), dim3((unsigned)((rows + 15) / 16)), dim3(256), 0, s, dot,
                     (const uint16_t*)out, lse, w.rowdot, w.lse2, rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // dQ: the forward's workgroup shape (8, 4, 2 or 1 waves per part)
  const int waves = g.G * BS / 32;
  const int nw = waves % 8 == 0 ? 8 : waves % 4 == 0 ? 4 : waves % 2 == 0 ? 2 : 1;
  const int parts = waves / nw;
  const unsigned grid = (unsigned)((int64_t)g.nb * g.B * g.Hkv * parts);
  switch (nw) {
    case 8: hipLaunchKernelGGL((bwd_dq_kernel<D, BS, 8>), dim3(grid), dim3(512), 0, s, g, qt, kt, vt, idx, cnt, dot, lse, w.rowdot, (uint16_t*)dq, parts); break;
    case 4: hipLaunchKernelGGL((bwd_dq_kernel<D, BS, 4>), dim3(grid), dim3(256), 0, s, g, qt, kt, vt, idx, cnt, dot, lse, w.rowdot, (uint16_t*)dq, parts); break;
    case 2: hipLaunchKernelGGL((bwd_dq_kernel<D, BS, 2>), dim3(grid), dim3(128), 0, s, g, qt, kt, vt, idx, cnt, dot, lse, w.rowdot, (uint16_t*)dq, parts); break;
    default: hipLaunchKernelGGL((bwd_dq_kernel<D, BS, 1>), dim3(grid), dim3(64), 0, s, g, qt, kt, vt, idx, cnt, dot, lse, w.rowdot, (uint16_t*)dq, parts); break;
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_list_kernel, dim3((unsigned)z.nkb), dim3(kListThreads), 0, s, g, idx, cnt, w.counts,
                     (const int32_t*)nullptr, (int32_t*)nullptr, 0);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_scan_kernel, dim3(1), dim3(1024), 0, s, w.counts, (int)z.nkb, w.list_off, w.seg_off);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_list_kernel, dim3((unsigned)z.nkb), dim3(kListThreads), 0, s, g, idx, cnt, w.counts,
                     w.list_off, w.lists, 1);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_kv_kernel<D, BS>), dim3((unsigned)z.max_segs), dim3(BS / 32 * 64), 0, s, g, qt, kt, vt, dot,
                     w.lse2, w.rowdot, w.lists, w.list_off, w.seg_off, (int)z.nkb, w.pdk, w.pdv);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_kv_reduce_kernel<D>), dim3((unsigned)z.nkb), dim3(256), 0, s, g, w.seg_off, w.pdk, w.pdv,
                     (uint16_t*)dk, (uint16_t*)dv);
  return hipGetLastError();
}

template <int D>
hipError_t launch_bwd_d(const Geo& g, const void* q, const void* k, const void* v, const int32_t* idx,
                        const int32_t* cnt, const void* out, const float* lse, const void* dout, void* dq, void* dk,
                        void* dv, void* ws, hipStream_t s) {
  switch (g.bs) {
    case 32: return launch_bwd_t<D, 32>(g, q, k, v, idx, cnt, out, lse, dout, dq, dk, dv, ws, s);
    case 64: return launch_bwd_t<D, 64>(g, q, k, v, idx, cnt, out, lse, dout, dq, dk, dv, ws, s);
    default: return launch_bwd_t<D, 128>(g, q, k, v, idx, cnt, out, lse, dout, dq, dk, dv, ws, s);
  }
}

}  // namespace

size_t attn_bwd_workspace_bytes(const Geo& g) {
  const BwdSizes z = bwd_sizes(g);
  return 2 * rnd(sizeof(float) * (size_t)g.B * g.Hq * g.N) + rnd(sizeof(int32_t) * z.nkb) +
         2 * rnd(sizeof(int32_t) * (z.nkb + 1)) + rnd(sizeof(int32_t) * z.max_entries) +
         2 * rnd(sizeof(float) * (size_t)z.max_segs * g.bs * g.D);
}

hipError_t launch_attn_bwd(const Geo& g, const void* q, const void* k, const void* v, const int32_t* idx,
                           const int32_t* cnt, const void* out, const float* lse, const void* dout, void* dq, void* dk,
                           void* dv, void* ws, hipStream_t s) {
  return g.D == 128 ? launch_bwd_d<128>(g, q, k, v, idx, cnt, out, lse, dout, dq, dk, dv, ws, s)
                    : launch_bwd_d<64>(g, q, k, v, idx, cnt, out, lse, dout, dq, dk, dv, ws, s);
}

}  // namespace pisa
