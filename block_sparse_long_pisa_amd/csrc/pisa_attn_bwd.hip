// Backward pass of the sparse attention, the selection held constant (the PISA
// page, "Attention clairsemée PISA : noyaux Triton sans matrice de scores",
// says its kernels serve training as well as inference; the gradients are those
// of the exact softmax attention over each query's attended key set).
//
// For query row i with attended keys A(i), logits s = scale q_i.k_t, weights
// p = exp(s - lse_i) (lse from the forward), and dO_i the output gradient:
//   D_i   = dO_i . O_i                          (bwd_dq_kernel's prologue, which
//                                               also writes it for the key-centric pass)
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
// dQ: query-centric. A workgroup serves NW waves x 32 query rows of one
// (batch, kv head, query block) unit and walks the unit's attended tiles as
// the forward does. V is staged at the row pitch (dP^T = V dO^T). K is read both
// as rows (S^T = K Q^T) and as columns (dQ^T += K^T dS^T), and no padded pitch
// serves both without bank conflicts: at D = 128 its rows are unpadded 256-byte
// rows with the logical 16-byte unit u of row r at u ^ tile_swz(r), for which the
// bank-conflict counter of gfx950 reads zero on both reads; at D = 64 they are
// padded to the transposing pitch.

template <int D, int BS>
struct DqKLayout {
  static constexpr bool kSwz = D == 128;
  static constexpr int PITCH = kSwz ? D : TilePitch<D, BS>::V;  // elements per row
  static constexpr int SIZE = kSwz ? BS * D : TilePitch<D, BS>::VSIZE;
};

template <int D, int BS>
struct DqState {
  bf16x8_t qf[D / 16];
  bf16x8_t df[D / 16];
  f32x16_t acc[D / 32];
  float lse2;  // this lane's query: lse in log2 units (+inf for a row past the sequence)
  float rd;    // this lane's query: D_i
  // byte offsets into a K tile: row fragment of step ds (row l32 of a 32-row
  // block), transposing reads of slice db (rows of a 16-row block, first and
  // second eight)
  int offr[D / 16];
  int offtl[D / 32], offtu[D / 32];
  __device__ __forceinline__ void init_offsets(int lane) {
    using KL = DqKLayout<D, BS>;
    const int l32 = lane & 31, hi = lane >> 5;
    const int rr = hi * 4 + ((lane & 15) >> 2);
#pragma unroll
    for (int ds = 0; ds < D / 16; ++ds) {
      const int u = 2 * ds + hi;
      offr[ds] = KL::kSwz ? (l32 * D + ((u ^ tile_swz(l32)) * 8)) * 2 : (l32 * KL::PITCH + u * 8) * 2;
    }
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int col = 32 * db + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
      if (KL::kSwz) {
        offtl[db] = (rr * D + (((col >> 3) ^ tile_swz(rr)) * 8) + (col & 7)) * 2;
        offtu[db] = ((rr + 8) * D + (((col >> 3) ^ tile_swz(rr + 8)) * 8) + (col & 7)) * 2;
      } else {
        offtl[db] = (rr * KL::PITCH + col) * 2;
        offtu[db] = ((rr + 8) * KL::PITCH + col) * 2;
      }
    }
  }
};

// Per-lane source offsets of one wave's copies of a dQ stage: V rows at the row
// pitch (the forward's K plan) and K rows in DqKLayout.
template <int D, int BS, int NW>
struct DqPlan {
  using TP = TilePitch<D, BS>;
  using KL = DqKLayout<D, BS>;
  static constexpr int VN = (TP::KI + NW - 1) / NW;
  static constexpr int KCOP = KL::SIZE / 512;  // whole 1 KB copies of the K tile
  static constexpr int KN = (KCOP + NW - 1) / NW;
  uint32_t v[VN];  // byte offsets
  uint32_t k[KN];
  __device__ __forceinline__ void init(int wave, int lane) {
#pragma unroll
    for (int n = 0; n < VN; ++n) v[n] = 2u * unit_src<D, TP::KU>((wave + NW * n) * 64 + lane, BS);
#pragma unroll
    for (int n = 0; n < KN; ++n) {
      const int p = (wave + NW * n) * 64 + lane;
      if (KL::kSwz) {
        const int r = p / (D / 8);
        k[n] = 2u * (r * D + (((p % (D / 8)) ^ tile_swz(r)) * 8));
      } else {
        k[n] = 2u * unit_src<D, TP::VU>(p, BS);
      }
    }
  }
};

// Issue the copies of one dQ stage: V tile vt into vdst (row pitch), K tile kt
// into kdst (DqKLayout), through buffer resources bounded by the `rows_in_mem`
// rows in memory: the rows past a sequence's end come in as zeros (their keys
// are masked).
template <int D, int BS, int NW>
__device__ __forceinline__ void issue_dq_tile(const uint16_t* __restrict__ vt, const uint16_t* __restrict__ kt,
                                              int rows_in_mem, uint16_t* vdst, uint16_t* kdst, int wave,
                                              const DqPlan<D, BS, NW>& plan) {
  using PL = DqPlan<D, BS, NW>;
  constexpr int VI = TilePitch<D, BS>::KI;
  const __amdgpu_buffer_rsrc_t rv = tile_rsrc(vt, rows_in_mem * D * 2);
  const __amdgpu_buffer_rsrc_t rk = tile_rsrc(kt, rows_in_mem * D * 2);
#pragma unroll
  for (int n = 0; n < PL::VN; ++n) {
    const int i = wave + NW * n;
    if (n < VI / NW || i < VI)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void_ptr)(vdst + i * 512), 16, plan.v[n], 0, 0, 0);
  }
#pragma unroll
  for (int n = 0; n < PL::KN; ++n) {
    const int i = wave + NW * n;
    if (n < PL::KCOP / NW || i < PL::KCOP)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void_ptr)(kdst + i * 512), 16, plan.k[n], 0, 0, 0);
  }
}

template <int D, int BS>
__device__ __forceinline__ void dq_tile(DqState<D, BS>& st, const uint16_t* ks, const uint16_t* vs, int nvalid,
                                        bool local, int key0, int qpos, int l32, int hi, float c, int wg_qmax) {
  constexpr int NDS = D / 16, NDB = D / 32;
  // keys per chunk: 32 when the K tile carries per-lane offset tables (register room)
  constexpr int KC = DqKLayout<D, BS>::kSwz ? 32 : (BS < 64 ? BS : 64);
  constexpr int NKB = KC / 32;
  constexpr int PK = TilePitch<D, BS>::K, KP = DqKLayout<D, BS>::PITCH;
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
        const bf16x8_t kfr = *reinterpret_cast<const bf16x8_t*>(reinterpret_cast<const char*>(ks) +
                                                                (ch * KC + kb * 32) * KP * 2 + st.offr[ds]);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kfr, st.qf[ds], s[kb], 0, 0, 0);
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
        const char* kr = reinterpret_cast<const char*>(ks) + (ch * KC + kb * 32 + hh * 16) * KP * 2;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_ptr)(kr + st.offtl[db]));
          const v4i16_t up = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_ptr)(kr + st.offtu[db]));
          const v4i16_t a8[2] = {lo, up};
          st.acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a8), b, st.acc[db], 0, 0,
                                                               0);
        }
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
                                                         const uint16_t* __restrict__ out,
                                                         const float* __restrict__ lse, float* __restrict__ rowdot,
                                                         float* __restrict__ lse2, uint16_t* __restrict__ dq,
                                                         int parts) {
  constexpr int NT = NW * 64;
  constexpr int NDS = D / 16, NDB = D / 32;
  using TP = TilePitch<D, BS>;
  // stage s: V rows at the row pitch (VS*), K in the layout DqKLayout (KS*)
  __shared__ __attribute__((aligned(16))) uint16_t VS0[TP::KSIZE];
  __shared__ __attribute__((aligned(16))) uint16_t KS0[DqKLayout<D, BS>::SIZE];
  __shared__ __attribute__((aligned(16))) uint16_t VS1[TP::KSIZE];
  __shared__ __attribute__((aligned(16))) uint16_t KS1[DqKLayout<D, BS>::SIZE];
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
  // D_i = dO_i . O_i: this lane's half of the row, then the other half from
  // lane ^ 32. Each valid row belongs to one wave of one workgroup, which also
  // writes D_i and lse_i in log2 units for the key-centric pass.
  float rd = 0.f;
#pragma unroll
  for (int ds = 0; ds < NDS; ++ds) {
    const uint4 uo = qvalid ? *reinterpret_cast<const uint4*>(out + row * D + ds * 16 + hi * 8) : make_uint4(0, 0, 0, 0);
    const uint4 ud = __builtin_bit_cast(uint4, st.df[ds]);
    const uint32_t av[4] = {ud.x, ud.y, ud.z, ud.w}, ov[4] = {uo.x, uo.y, uo.z, uo.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) rd += bf16lo(av[e]) * bf16lo(ov[e]) + bf16hi(av[e]) * bf16hi(ov[e]);
  }
  rd += __shfl_xor(rd, 32);
  st.lse2 = qvalid ? lse[row] * kLog2e : __builtin_inff();
  st.rd = rd;
  if (qvalid && hi == 0) {
    rowdot[row] = rd;
    lse2[row] = st.lse2;
  }
  st.init_offsets(lane);
  const float c = g.scale * kLog2e;
  const int wg_qmax = qb * BS + (((part + 1) * NW - 1) / g.G) * 32 + 31;

  const uint16_t* kbase = k + ((int64_t)b * g.Hkv + kvh) * g.N * D;
  const uint16_t* vbase = v + ((int64_t)b * g.Hkv + kvh) * g.N * D;
  __syncthreads();
  const TileWalk walk = make_walk(g, qb, sel, nsel);
  DqPlan<D, BS, NW> plan;
  plan.init(wave, lane);

  int j, nvalid;
  bool local;
  walk.at(0, sel, g, qb, local_rows, j, nvalid, local);
  issue_dq_tile<D, BS, NW>(vbase + (int64_t)j * BS * D, kbase + (int64_t)j * BS * D, min(BS, g.N - j * BS), VS0, KS0,
                           wave, plan);
  for (int t = 0; t < walk.ntiles; t += 2) {
    wait_loads_and_sync();
    int j1 = 0, nv1 = 0;
    bool loc1 = false;
    if (t + 1 < walk.ntiles) {
      walk.at(t + 1, sel, g, qb, local_rows, j1, nv1, loc1);
      issue_dq_tile<D, BS, NW>(vbase + (int64_t)j1 * BS * D, kbase + (int64_t)j1 * BS * D, min(BS, g.N - j1 * BS),
                               VS1, KS1, wave, plan);
    }
    dq_tile<D, BS>(st, KS0, VS0, nvalid, local, j * BS, qpos, l32, hi, c, wg_qmax);
    if (t + 1 >= walk.ntiles) break;
    wait_loads_and_sync();
    if (t + 2 < walk.ntiles) {
      walk.at(t + 2, sel, g, qb, local_rows, j, nvalid, local);
      issue_dq_tile<D, BS, NW>(vbase + (int64_t)j * BS * D, kbase + (int64_t)j * BS * D, min(BS, g.N - j * BS), VS0,
                               KS0, wave, plan);
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
// dK, dV: key-centric. A workgroup of BS/16 waves serves one segment of one key
// block's list; wave w owns keys [16 w, 16 w + 16) of the block and keeps their
// K and V rows as the B operands of 16x16x32 matrix products (lane = key), so
// that its state leaves room for two waves per SIMD. For every (query block,
// head) of the segment the query rows Q and their output gradients dO are
// staged in LDS, and per 32-row chunk
//   S = Q K^T, dP = dO V^T   (rows = queries, lane = key),
//   p = exp2(S c - lse2), dS = p (dP - D),
//   dV^T += dO^T p, dK^T += Q^T dS   (rows = d, lane = key).
// The 32 query rows of a chunk enter the second pair of products in the order
// the first pair leaves them in the lanes: slot j of lane group g is row
// 4 g + j for j < 4 and row 16 + 4 g + j - 4 after, and the transposing reads of
// Q and dO take their rows in the same order.
//
// Tiles are unpadded, D/8 16-byte units per row, with the logical unit u of row
// r stored at u ^ kv_swz(r). In product step ds of S and dP, lane group g
// (lanes 16 g to 16 g + 15) takes the row unit (D/32) g + ds: the contraction
// over d visits the columns in that order, on both operands. With this layout
// the bank-conflict counter of gfx950 reads zero for the row fragments (16 rows
// at one unit per lane group) and for the transposing reads (4 rows x 32 bytes
// per lane group) at D = 128 and D = 64; with adjacent units per lane group
// instead, the row fragments conflict whatever the swizzle. D = 128: r mod 8 = k
// maps to 2k, plus one for the rows 4-7 of the first eight and 0-3 of the next.
// D = 64 (128-byte rows): 2k mod 8, XOR 3 for k >= 4, XOR 1 for the second eight
// rows.

typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <int D>
__device__ __forceinline__ int kv_swz(int r) {
  const int k = r & 7, h = (r >> 3) & 1;
  if constexpr (D == 128) return 2 * k + ((k >> 2) ^ h);
  else return ((2 * k) & 7) ^ (3 * (k >> 2)) ^ h;
}

// Per-lane source offsets (elements, row * D + col) of this wave's copies of a
// swizzled tile; NC copies of 64 units each.
template <int D, int BS, int NW>
struct KvPlan {
  static constexpr int UPR = D / 8;
  static constexpr int NC = BS * UPR / 64 / NW;
  uint32_t src[NC];  // bytes
  __device__ __forceinline__ void init(int wave, int lane) {
#pragma unroll
    for (int n = 0; n < NC; ++n) {
      const int p = (wave + NW * n) * 64 + lane;  // physical unit of the tile
      const int r = p / UPR;
      src[n] = 2u * (r * D + (((p % UPR) ^ kv_swz<D>(r)) * 8));
    }
  }
};

// Issue the copies of one (query block, head) stage: Q and dO rows (swizzled),
// and the rows' lse2 and D (64 floats per wave instruction). Q and dO come
// through buffer resources bounded by the rows in memory, so rows past the
// sequence arrive as zeros; their lse2 and D re-read the last row's. Those
// rows are masked by `rows`.
template <int D, int BS, int NW>
__device__ __forceinline__ void issue_kv_rows(const Geo& g, const uint16_t* q, const uint16_t* dout,
                                              const float* lse2, const float* rowdot, int b, int h, int qb,
                                              uint16_t* qdst, uint16_t* odst, float* ldst, float* rdst, int wave,
                                              int lane, const KvPlan<D, BS, NW>& plan) {
  using PL = KvPlan<D, BS, NW>;
  const int64_t r0 = ((int64_t)b * g.Hq + h) * g.N + (int64_t)qb * BS;
  const int rows = min(BS, g.N - qb * BS);
  const __amdgpu_buffer_rsrc_t rq = tile_rsrc(q + r0 * D, rows * D * 2);
  const __amdgpu_buffer_rsrc_t ro = tile_rsrc(dout + r0 * D, rows * D * 2);
#pragma unroll
  for (int n = 0; n < PL::NC; ++n) {
    const int i = wave + NW * n;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, (lds_void_ptr)(qdst + i * 512), 16, plan.src[n], 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ro, (lds_void_ptr)(odst + i * 512), 16, plan.src[n], 0, 0, 0);
  }
#pragma unroll
  for (int n = 0; n < (BS + 63) / 64; ++n) {
    if (n % NW == wave) {
      const uint32_t r = (uint32_t)min(n * 64 + lane, rows - 1);
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const char*>(lse2 + r0) + 4 * r, (lds_void_ptr)(ldst + n * 64),
                                       4, 0, 0);
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const char*>(rowdot + r0) + 4 * r,
                                       (lds_void_ptr)(rdst + n * 64), 4, 0, 0);
    }
  }
}

// Transposed fragment of a swizzled tile: rows (queries) 4 g + [0, 4) and
// 16 + 4 g + [0, 4) from row q0, columns [16 db, 16 db + 16), as the A operand
// (columns become rows) of a 16x16x32 product; `off` is this lane's byte offset
// for db (row 4 g + lane%16/4, its piece lane%4 of the 16-column slice).
template <int D>
__device__ __forceinline__ bf16x8_t kv_tr_frag(const uint16_t* tile, int off, int q0) {
  const char* base = reinterpret_cast<const char*>(tile) + q0 * D * 2 + off;
  const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_ptr)(base));
  const v4i16_t up = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_ptr)(base + 16 * D * 2));
  const v4i16_t a8[2] = {lo, up};
  return __builtin_bit_cast(bf16x8_t, a8);
}

template <int D, int BS>
__device__ __forceinline__ void kv_tile(const bf16x8_t (&kf)[D / 32], const bf16x8_t (&vf)[D / 32],
                                        f32x4_t (&dk)[D / 16], f32x4_t (&dv)[D / 16], const uint16_t* qs,
                                        const uint16_t* os, const float* ls, const float* rs, bool mask, int rows,
                                        int rlo, int g4, const int (&offr)[D / 32], const int (&offt)[D / 16],
                                        float c) {
  constexpr int NDS = D / 32, NDB = D / 16;
  constexpr int QC = 32;
#pragma unroll
  for (int ch = 0; ch < BS / QC; ++ch) {
    if (ch > 0 && ch * QC >= rows) break;
    const int q0 = ch * QC;
    f32x4_t s[2], dp[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) s[mb][i] = dp[mb][i] = 0.f;
    bf16x8_t fq[2][NDS], fo[2][NDS];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds) {
        const int o = (q0 + 16 * mb) * D * 2 + offr[ds];
        fq[mb][ds] = *reinterpret_cast<const bf16x8_t*>(reinterpret_cast<const char*>(qs) + o);
        fo[mb][ds] = *reinterpret_cast<const bf16x8_t*>(reinterpret_cast<const char*>(os) + o);
      }
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        s[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fq[mb][ds], kf[ds], s[mb], 0, 0, 0);
        dp[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fo[mb][ds], vf[ds], dp[mb], 0, 0, 0);
      }
    // element i of block mb is query row q0 + 16 mb + 4 g4 + i
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const int r0 = q0 + 16 * mb + 4 * g4;
      const float4 l4 = *reinterpret_cast<const float4*>(ls + r0);
      const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) s[mb][i] = fast_exp2(fmaf(s[mb][i], c, -lv[i]));
      if (mask) {  // uniform: partial-sink, causal and ragged tiles; rows [rlo, rows) count for this key
#pragma unroll
        for (int i = 0; i < 4; ++i) s[mb][i] = r0 + i >= rlo && r0 + i < rows ? s[mb][i] : 0.f;
      }
      const float4 d4 = *reinterpret_cast<const float4*>(rs + r0);
      const float dv4[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) dp[mb][i] = s[mb][i] * (dp[mb][i] - dv4[i]);
    }
    bf16x8_t pb, sb;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pb[i] = (__bf16)s[0][i];
      pb[4 + i] = (__bf16)s[1][i];
      sb[i] = (__bf16)dp[0][i];
      sb[4 + i] = (__bf16)dp[1][i];
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      dv[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv_tr_frag<D>(os, offt[db], q0), pb, dv[db], 0, 0, 0);
      dk[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv_tr_frag<D>(qs, offt[db], q0), sb, dk[db], 0, 0, 0);
    }
  }
}

// One (query block, head) stage. Whole tiles of full kind (every row and key
// counts) skip the mask; otherwise the rows that count for this lane's key are
// [rlo, rows): rlo = the key's own row on the causal diagonal, past the block
// for a key outside the sink (partial sink tile) or the sequence.
template <int D, int BS>
__device__ __forceinline__ void kv_stage(const bf16x8_t (&kf)[D / 32], const bf16x8_t (&vf)[D / 32],
                                         f32x4_t (&dk)[D / 16], f32x4_t (&dv)[D / 16], const uint16_t* qs,
                                         const uint16_t* os, const float* ls, const float* rs, const Geo& g, int qb,
                                         int kind, int j, int key, int g4, const int (&offr)[D / 32],
                                         const int (&offt)[D / 16], float c) {
  const int rows = min(BS, g.N - qb * BS);
  const bool mask = !(kind == kFull && rows == BS && (j + 1) * BS <= g.N);
  const bool key_ok = key < (kind == kSinkPart ? g.sink : g.N);
  const int rlo = !key_ok ? BS : kind == kLocal ? (key & (BS - 1)) : 0;
  kv_tile<D, BS>(kf, vf, dk, dv, qs, os, ls, rs, mask, rows, rlo, g4, offr, offt, c);
}

template <int D, int BS>
__global__ __launch_bounds__(BS / 16 * 64) void bwd_kv_kernel(Geo g, const uint16_t* __restrict__ q,
                                                              const uint16_t* __restrict__ k,
                                                              const uint16_t* __restrict__ v,
                                                              const uint16_t* __restrict__ dout,
                                                              const float* __restrict__ lse2,
                                                              const float* __restrict__ rowdot,
                                                              const int32_t* __restrict__ lists,
                                                              const int32_t* __restrict__ list_off,
                                                              const int32_t* __restrict__ seg_off, int nkb,
                                                              float* __restrict__ pdk, float* __restrict__ pdv,
                                                              uint16_t* __restrict__ dkout,
                                                              uint16_t* __restrict__ dvout) {
  constexpr int NW = BS / 16;
  constexpr int NDS = D / 32, NDB = D / 16;
  constexpr int LS = BS < 64 ? 64 : BS;  // lse2 / D slots per stage (whole 64-float copies)
  __shared__ __attribute__((aligned(16))) uint16_t Q0[BS * D];
  __shared__ __attribute__((aligned(16))) uint16_t O0[BS * D];
  __shared__ __attribute__((aligned(16))) uint16_t Q1[BS * D];
  __shared__ __attribute__((aligned(16))) uint16_t O1[BS * D];
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
  const int n16 = lane & 15;
  const int g4 = lane >> 4;
  const int key = j * BS + wave * 16 + n16;
  const int64_t krow = ((int64_t)b * g.Hkv + kvh) * g.N + min(key, g.N - 1);
  // K and V rows as B operands: key n16, in step ds the columns of unit
  // NDS g4 + ds, [8 (NDS g4 + ds), + 8)
  bf16x8_t kf[NDS], vf[NDS];
#pragma unroll
  for (int ds = 0; ds < NDS; ++ds) {
    const int col = (NDS * g4 + ds) * 8;
    kf[ds] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(k + krow * D + col));
    vf[ds] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(v + krow * D + col));
  }
  f32x4_t dk[NDB], dv[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) dk[db][i] = dv[db][i] = 0.f;
  // LDS byte offsets: row fragments (row n16 of a 16-row block, logical unit
  // NDS g4 + ds) and transposing reads (row 4 g4 + n16/4, piece n16%4 of the
  // 16-column slice db); the swizzle depends on the row mod 16 only
  int offr[NDS], offt[NDB];
#pragma unroll
  for (int ds = 0; ds < NDS; ++ds) offr[ds] = (n16 * D + (((NDS * g4 + ds) ^ kv_swz<D>(n16)) * 8)) * 2;
  {
    const int rr = 4 * g4 + (n16 >> 2), cc = n16 & 3;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
      offt[db] = (rr * D + (((2 * db + (cc >> 1)) ^ kv_swz<D>(rr)) * 8)) * 2 + (cc & 1) * 8;
  }
  const float c = g.scale * kLog2e;
  KvPlan<D, BS, NW> plan;
  plan.init(wave, lane);

  auto entry = [&](int t, int& qb, int& h, int& kind) {
    // one list entry for every lane: scalar, so row addresses form in scalar registers
    const int e = __builtin_amdgcn_readfirstlane(lists[e0 + t / g.G]);
    qb = e & 0x0fffffff;
    kind = e >> 28;
    h = kvh * g.G + t % g.G;
  };

  int qb, h, kind;
  entry(0, qb, h, kind);
  issue_kv_rows<D, BS, NW>(g, q, dout, lse2, rowdot, b, h, qb, Q0, O0, L0, R0, wave, lane, plan);
  for (int t = 0; t < npairs; t += 2) {
    wait_loads_and_sync();
    int qb1 = 0, h1 = 0, kind1 = 0;
    if (t + 1 < npairs) {
      entry(t + 1, qb1, h1, kind1);
      issue_kv_rows<D, BS, NW>(g, q, dout, lse2, rowdot, b, h1, qb1, Q1, O1, L1, R1, wave, lane, plan);
    }
    kv_stage<D, BS>(kf, vf, dk, dv, Q0, O0, L0, R0, g, qb, kind, j, key, g4, offr, offt, c);
    if (t + 1 >= npairs) break;
    wait_loads_and_sync();
    if (t + 2 < npairs) {
      entry(t + 2, qb, h, kind);
      issue_kv_rows<D, BS, NW>(g, q, dout, lse2, rowdot, b, h, qb, Q0, O0, L0, R0, wave, lane, plan);
    }
    kv_stage<D, BS>(kf, vf, dk, dv, Q1, O1, L1, R1, g, qb1, kind1, j, key, g4, offr, offt, c);
  }
  // lane holds key n16, columns 16 db + 4 g4 + [0, 4)
  if (seg_off[kbid + 1] - seg_off[kbid] == 1) {
    // the key block's only segment: dK and dV directly, as the reduce would
    // write them (its sum starts from +0.0)
    if (key < g.N) {
      uint16_t* ok = dkout + ((int64_t)slab * g.N + key) * D;
      uint16_t* ov = dvout + ((int64_t)slab * g.N + key) * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int d = db * 16 + g4 * 4;
        *reinterpret_cast<uint2*>(ok + d) = make_uint2(pack_bf16x2((0.f + dk[db][0]) * g.scale, (0.f + dk[db][1]) * g.scale),
                                                       pack_bf16x2((0.f + dk[db][2]) * g.scale, (0.f + dk[db][3]) * g.scale));
        *reinterpret_cast<uint2*>(ov + d) = make_uint2(pack_bf16x2(0.f + dv[db][0], 0.f + dv[db][1]),
                                                       pack_bf16x2(0.f + dv[db][2], 0.f + dv[db][3]));
      }
    }
    return;
  }
  // partial sums of this segment: [segment][key of the block][d], fp32
  float* pk = pdk + ((int64_t)w * BS + wave * 16 + n16) * D;
  float* pv = pdv + ((int64_t)w * BS + wave * 16 + n16) * D;
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    const int d = db * 16 + g4 * 4;
    *reinterpret_cast<float4*>(pk + d) = make_float4(dk[db][0], dk[db][1], dk[db][2], dk[db][3]);
    *reinterpret_cast<float4*>(pv + d) = make_float4(dv[db][0], dv[db][1], dv[db][2], dv[db][3]);
  }
}

// dK = scale * (sum of the segments' partial sums), dV = sum, in segment order,
// for the key blocks of more than one segment (the key-centric kernel writes a
// single segment's block itself).
template <int D>
__global__ __launch_bounds__(256) void bwd_kv_reduce_kernel(Geo g, const int32_t* __restrict__ seg_off,
                                                            const float* __restrict__ pdk,
                                                            const float* __restrict__ pdv, uint16_t* __restrict__ dk,
                                                            uint16_t* __restrict__ dv) {
  const int kbid = blockIdx.x;
  const int slab = kbid / g.nb;
  const int j = kbid % g.nb;
  const int s0 = seg_off[kbid], s1 = seg_off[kbid + 1];
  if (s1 - s0 == 1) return;
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
  const uint16_t* ot = (const uint16_t*)out;
  hipError_t e;
  // dQ: the forward's workgroup shape (8, 4, 2 or 1 waves per part)
  const int waves = g.G * BS / 32;
  const int nw = waves % 8 == 0 ? 8 : waves % 4 == 0 ? 4 : waves % 2 == 0 ? 2 : 1;
  const int parts = waves / nw;
  const unsigned grid = (unsigned)((int64_t)g.nb * g.B * g.Hkv * parts);
  switch (nw) {
    case 8: PISA_LAUNCH(g, (bwd_dq_kernel<D, BS, 8>), dim3(grid), dim3(512), 0, s, g, qt, kt, vt, idx, cnt, dot, ot, lse, w.rowdot, w.lse2, (uint16_t*)dq, parts); break;
    case 4: PISA_LAUNCH(g, (bwd_dq_kernel<D, BS, 4>), dim3(grid), dim3(256), 0, s, g, qt, kt, vt, idx, cnt, dot, ot, lse, w.rowdot, w.lse2, (uint16_t*)dq, parts); break;
    case 2: PISA_LAUNCH(g, (bwd_dq_kernel<D, BS, 2>), dim3(grid), dim3(128), 0, s, g, qt, kt, vt, idx, cnt, dot, ot, lse, w.rowdot, w.lse2, (uint16_t*)dq, parts); break;
    default: PISA_LAUNCH(g, (bwd_dq_kernel<D, BS, 1>), dim3(grid), dim3(64), 0, s, g, qt, kt, vt, idx, cnt, dot, ot, lse, w.rowdot, w.lse2, (uint16_t*)dq, parts); break;
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  PISA_LAUNCH(g, bwd_list_kernel, dim3((unsigned)z.nkb), dim3(kListThreads), 0, s, g, idx, cnt, w.counts,
                     (const int32_t*)nullptr, (int32_t*)nullptr, 0);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  PISA_LAUNCH(g, bwd_scan_kernel, dim3(1), dim3(1024), 0, s, w.counts, (int)z.nkb, w.list_off, w.seg_off);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  PISA_LAUNCH(g, bwd_list_kernel, dim3((unsigned)z.nkb), dim3(kListThreads), 0, s, g, idx, cnt, w.counts,
                     w.list_off, w.lists, 1);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  PISA_LAUNCH(g, (bwd_kv_kernel<D, BS>), dim3((unsigned)z.max_segs), dim3(BS / 16 * 64), 0, s, g, qt, kt, vt, dot,
                     w.lse2, w.rowdot, w.lists, w.list_off, w.seg_off, (int)z.nkb, w.pdk, w.pdv, (uint16_t*)dk,
                     (uint16_t*)dv);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  PISA_LAUNCH(g, (bwd_kv_reduce_kernel<D>), dim3((unsigned)z.nkb), dim3(256), 0, s, g, w.seg_off, w.pdk, w.pdv,
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
