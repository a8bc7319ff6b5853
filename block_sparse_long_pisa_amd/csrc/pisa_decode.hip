// One decode step: a new query token per sequence, its key and value already in
// the cache. Selection reuses the pyramid descent of "La sélection top-K guidée
// par la pyramide" with a one-token query block; attention over the attended
// blocks is split across workgroups and the partial results are merged with an
// online softmax, as the Pulsar Attention page merges per-host partial
// attentions ("Phase 2 : Encodage de la requête globale").
//
// Every sequence has its own cache length (one length for all, or a device
// array of them), so its own query block, local block and attended walk.
// Three launches on the caller's stream:
//   decode_select  one workgroup per (batch, kv head): fp64 mean of the group's
//                  query rows, descent, block list into the workspace;
//   decode_attn    (split, batch, kv head): streams its share of the K rows,
//                  keeps all its logits in LDS, then streams the V rows once;
//                  writes (max, sum, unnormalised output) per query head;
//   decode_merge   one workgroup per (batch, query head): merges the splits.
// The step is bound by HBM: it reads each attended K/V row exactly once.
#include <mutex>

#include "pisa_append.h"
#include "pisa_internal.h"
#include "pisa_select_common.h"

namespace pisa {
namespace {

// Workspace of the allocation-free decode entry point: one copy per GPU, held
// from the library's first use on that GPU until the process ends. Host code
// never passes this name to a kernel: on the host it is only a stand-in for the
// symbol, and the device address comes from hipGetSymbolAddress (scratch_ptr).
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

constexpr int kMaxDevices = 64;

constexpr int kDecThreads = 256;
constexpr int kTilesPerSplit = 6;
constexpr int kMaxGroup = 8;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct DecodeWs {
  int32_t* idx;  // [B*Hkv, K]
  int32_t* cnt;  // [B*Hkv]
  float* m;      // [B*Hkv, S, G]  log2-domain max
  float* l;      // [B*Hkv, S, G]
  float* o;      // [B*Hkv, S, G, D] unnormalised
};

// One workgroup of 512 threads per (batch, kv head): mean of the group's query
// rows, then the workgroup descent, with each level's pool scored in few rounds
// of loads (the decode pyramid comes from HBM) and the best K kept by the first
// wave's threshold search.
constexpr int kDecSelThreads = 512;

// Cache length of sequence b: from the per-sequence array when there is one.
// A length outside [1, capacity] marks a sequence that attends nothing.
__device__ __forceinline__ int seq_len_of(const Geo& g, const int32_t* lens, int len_all, int b, bool& valid) {
  const int len = lens != nullptr ? lens[b] : len_all;
  valid = len >= 1 && len <= g.N;
  return valid ? len : 1;
}

// With old_lens given, each workgroup first appends its slab's tokens
// [old_lens[b], lens[b]) to the pyramid (what pisa_pyramid_append does, rows
// staged kDecAppendRows at a time in the LDS the descent uses afterwards), then
// descends the updated pyramid: one launch fewer per serving step.
constexpr int kDecAppendRows = 64;

template <typename T, int D, int E>
__global__ __launch_bounds__(kDecSelThreads) void decode_select_kernel(Geo g, const T* __restrict__ q,
                                                                       const float* pyr,
                                                                       const int32_t* __restrict__ lens, int len_all,
                                                                       int32_t* __restrict__ idx,
                                                                       int32_t* __restrict__ cnt,
                                                                       const T* __restrict__ kc, float* pyr_w,
                                                                       const int32_t* __restrict__ old_lens) {
  // one LDS buffer: an append's key rows, then the descent's scratch and the query mean
  constexpr int kSmemBytes = (sizeof(BlockSmem) + 15) / 16 * 16;
  constexpr int kSelectBytes = kSmemBytes + D * (int)sizeof(double);
  constexpr int kAppendBytes = kAppendRowUnits<T, D, kDecAppendRows> * (int)sizeof(uint4);
  __shared__ __attribute__((aligned(16))) unsigned char buf[kSelectBytes > kAppendBytes ? kSelectBytes : kAppendBytes];
  BlockSmem& smem = *reinterpret_cast<BlockSmem*>(buf);
  double* qbar = reinterpret_cast<double*>(buf + kSmemBytes);
  const int slab = blockIdx.x;
  const int b = slab / g.Hkv;
  const int kvh = slab % g.Hkv;
  if (old_lens != nullptr) {  // uniform across the workgroup; ends with a barrier when it writes
    uint4* rows = reinterpret_cast<uint4*>(buf);
    if (g.pool == PISA_POOL_MAX)
      append_slab<T, D, true, kDecSelThreads, kDecAppendRows>(g, kc, pyr_w, slab, old_lens[b], lens[b], rows);
    else
      append_slab<T, D, false, kDecSelThreads, kDecAppendRows>(g, kc, pyr_w, slab, old_lens[b], lens[b], rows);
  }
  bool valid;
  const int qb = (seq_len_of(g, lens, len_all, b, valid) - 1) / g.bs;
  if (!valid) {  // uniform across the workgroup
    for (int t = threadIdx.x; t < g.K; t += kDecSelThreads) idx[(int64_t)slab * g.K + t] = -1;
    if (threadIdx.x == 0) cnt[slab] = 0;
    return;
  }
  for (int c = threadIdx.x; c < D; c += kDecSelThreads) {
    double s = 0.0;
    for (int hh = 0; hh < g.G; ++hh) {
      const T* row = q + ((int64_t)b * g.Hq + kvh * g.G + hh) * D;
      float x;
      if constexpr (sizeof(T) == 2) x = bf16_to_f32(((const uint16_t*)row)[c]);
      else x = ((const float*)row)[c];
      s += (double)x;
    }
    qbar[c] = s / (double)g.G;
  }
  __syncthreads();
  block_descend<D, kDecSelThreads, 8, E>(g, pyr + (int64_t)slab * g.off[g.L] * D, qb, qbar,
                                      idx + (int64_t)slab * g.K, cnt + slab, smem);
}

// Block walk of the decode token (position pos, block qb): full sink blocks,
// partial sink block, selected blocks, local block [qb*bs, pos].
__device__ __forceinline__ void decode_tile(const Geo& g, int qb, int pos, const int* sel, int nsel, int t, int& j,
                                            int& nvalid) {
  const int nfull = min(g.j0, qb);
  const bool tail = g.sink > g.j0 * g.bs && g.j0 < qb && !(nsel > 0 && sel[0] == g.j0);
  const int np = tail ? 1 : 0;
  if (t < nfull) {
    j = t;
    nvalid = g.bs;
  } else if (t < nfull + np) {
    j = g.j0;
    nvalid = g.sink - g.j0 * g.bs;
  } else if (t < nfull + np + nsel) {
    j = sel[t - nfull - np];
    nvalid = g.bs;
    if (j < 0 || j >= qb) {  // not a block this token may select: attend nothing
      j = qb;
      nvalid = 0;
    }
  } else {
    j = qb;
    nvalid = pos - qb * g.bs + 1;
  }
}

__device__ __forceinline__ int decode_ntiles(const Geo& g, int qb, const int* sel, int nsel) {
  const bool tail = g.sink > g.j0 * g.bs && g.j0 < qb && !(nsel > 0 && sel[0] == g.j0);
  return min(g.j0, qb) + (tail ? 1 : 0) + nsel + 1;
}

// Sum v[0, C) over the lanes of an aligned group of 2*S lanes (xor butterfly),
// halving the values each step: afterwards lane i of the group holds the sums
// of values [first, first + C / (2S)) with first = sum over steps of
// bit(i, s) * (half at that step). Once one value is left it is summed whole.
template <int C, int S>
__device__ __forceinline__ void butterfly(float* v, int lane) {
  if constexpr (S >= 1) {
    if constexpr (C > 1) {
      constexpr int H = C / 2;
      const bool up = (lane & S) != 0;
#pragma unroll
      for (int i = 0; i < H; ++i) {
        const float send = up ? v[i] : v[i + H];
        const float keep = up ? v[i + H] : v[i];
        v[i] = keep + __shfl_xor(send, S);
      }
      butterfly<H, S / 2>(v, lane);
    } else {
      v[0] += __shfl_xor(v[0], S);
      butterfly<1, S / 2>(v, lane);
    }
  }
}

// Index of the first value a lane holds after butterfly<C, S>.
template <int C, int S>
__device__ __forceinline__ int butterfly_first(int lane) {
  if constexpr (S >= 1 && C > 1) {
    return ((lane & S) ? C / 2 : 0) + butterfly_first<C / 2, S / 2>(lane);
  } else {
    return 0;
  }
}

template <typename T, int D, int G>
__global__ __launch_bounds__(kDecThreads) void decode_attn_kernel(Geo g, const T* __restrict__ q,
                                                                  const T* __restrict__ kc, const T* __restrict__ vc,
                                                                  const int32_t* __restrict__ lens, int len_all,
                                                                  int splits, DecodeWs ws) {
  constexpr int VEC = Wide<T>::kVec;
  constexpr int LPR = D / VEC;                // lanes per cache row
  constexpr int RP = kDecThreads / LPR;       // rows per pass of the workgroup
  constexpr int MAXK = kTilesPerSplit * 128;  // keys per split (bs <= 128)
  constexpr int RPT = 128 / RP;               // rows per thread per 128-key tile
  constexpr int NV = RPT * G;                 // partial dots per thread per tile
  constexpr int HOLD = NV >= LPR ? NV / LPR : 1;
  __shared__ float qs[G][D];
  __shared__ float sc[MAXK][G];  // logits, then weights 2^(logit - max), of this split's keys
  __shared__ int sel[kMaxTopK];
  __shared__ float red[kDecThreads / 64][G][D];
  __shared__ float mred[kDecThreads / 64][G];

  const int split = blockIdx.x;
  const int slab = blockIdx.y;
  const int b = slab / g.Hkv;
  const int kvh = slab % g.Hkv;
  const int tid = threadIdx.x;
  bool valid;
  const int pos = seq_len_of(g, lens, len_all, b, valid) - 1;
  const int qb = pos / g.bs;
  if (!valid) {  // an empty partial result (uniform across the workgroup)
    const int64_t pb0 = ((int64_t)slab * splits + split) * G;
    for (int e = tid; e < G * D; e += kDecThreads) ws.o[pb0 * D + e] = 0.f;
    if (tid < G) {
      ws.m[pb0 + tid] = -__builtin_inff();
      ws.l[pb0 + tid] = 0.f;
    }
    return;
  }
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = (tid % LPR) * VEC;
  const int rsub = tid / LPR;
  const int nsel = min(max(ws.cnt[slab], 0), g.K);
  for (int t = tid; t < nsel; t += kDecThreads) sel[t] = ws.idx[(int64_t)slab * g.K + t];
  for (int e = tid; e < G * D; e += kDecThreads) {
    const T* row = q + ((int64_t)b * g.Hq + kvh * G + e / D) * D;
    float x;
    if constexpr (sizeof(T) == 2) x = bf16_to_f32(((const uint16_t*)row)[e % D]);
    else x = ((const float*)row)[e % D];
    qs[e / D][e % D] = x;
  }
  __syncthreads();
  float qr[G][VEC];  // this lane's column slice of every head's query
#pragma unroll
  for (int hh = 0; hh < G; ++hh)
#pragma unroll
    for (int e = 0; e < VEC; ++e) qr[hh][e] = qs[hh][col + e];
  const int ntiles = decode_ntiles(g, qb, sel, nsel);
  const int t0 = split * kTilesPerSplit;
  const int t1 = min(ntiles, t0 + kTilesPerSplit);
  const T* kb = kc + (int64_t)slab * g.N * D;
  const T* vb = vc + (int64_t)slab * g.N * D;
  const float c = g.scale * kLog2e;

  // pass 1: logits of every key of this split; all of a tile's loads first
  int nkeys = 0;
  for (int t = t0; t < t1; ++t) {
    int j, nvalid;
    decode_tile(g, qb, pos, sel, nsel, t, j, nvalid);
    float x[RPT][VEC];
#pragma unroll
    for (int i = 0; i < RPT; ++i)  // unconditional loads (clamped rows): all in flight
      Wide<T>::widen(Wide<T>::stream(kb + ((int64_t)j * g.bs + min(rsub + i * RP, max(nvalid, 1) - 1)) * D + col), x[i]);
    float part[NV];
#pragma unroll
    for (int i = 0; i < RPT; ++i)
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < VEC; ++e) s = fmaf(qr[hh][e], x[i][e], s);
        part[i * G + hh] = s;
      }
    butterfly<NV, LPR / 2>(part, lane);
    const int first = butterfly_first<NV, LPR / 2>(lane);
    // with fewer sums than lanes, aligned runs of LPR / NV lanes hold the same sum
    if ((tid % (NV >= LPR ? 1 : LPR / NV)) == 0) {
#pragma unroll
      for (int e = 0; e < HOLD; ++e) {
        const int v = first + e;
        const int r = rsub + (v / G) * RP;
        if (r < g.bs) sc[nkeys + r][v % G] = r < nvalid ? part[e] * c : -__builtin_inff();
      }
    }
    nkeys += g.bs;
  }
  __syncthreads();
  // per-head max over the split, then the weights in place and their sums
  float mx[G], ls[G];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) mx[hh] = -__builtin_inff();
  for (int r = tid; r < nkeys; r += kDecThreads)
#pragma unroll
    for (int hh = 0; hh < G; ++hh) mx[hh] = fmaxf(mx[hh], sc[r][hh]);
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
#pragma unroll
    for (int sh = 1; sh < 64; sh <<= 1) mx[hh] = fmaxf(mx[hh], __shfl_xor(mx[hh], sh));
    if (lane == 0) mred[wave][hh] = mx[hh];
  }
  __syncthreads();
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    float m = mred[0][hh];
#pragma unroll
    for (int w = 1; w < kDecThreads / 64; ++w) m = fmaxf(m, mred[w][hh]);
    mx[hh] = m;
    ls[hh] = 0.f;
  }
  __syncthreads();  // everyone has read mred before it is reused for the sums
  for (int r = tid; r < nkeys; r += kDecThreads)
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      const float p = mx[hh] == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(sc[r][hh] - mx[hh]);
      sc[r][hh] = p;
      ls[hh] += p;
    }
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
#pragma unroll
    for (int sh = 1; sh < 64; sh <<= 1) ls[hh] += __shfl_xor(ls[hh], sh);
    if (lane == 0) mred[wave][hh] = ls[hh];
  }
  __syncthreads();
  // pass 2: stream V once, all of a tile's loads first
  float acc[G][VEC];
#pragma unroll
  for (int hh = 0; hh < G; ++hh)
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[hh][e] = 0.f;
  int base = 0;
  for (int t = t0; t < t1; ++t) {
    int j, nvalid;
    decode_tile(g, qb, pos, sel, nsel, t, j, nvalid);
    float x[RPT][VEC];
#pragma unroll
    for (int i = 0; i < RPT; ++i)  // unconditional loads (clamped rows): all in flight
      Wide<T>::widen(Wide<T>::stream(vb + ((int64_t)j * g.bs + min(rsub + i * RP, max(nvalid, 1) - 1)) * D + col), x[i]);
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int r = rsub + i * RP;
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        const float p = r < nvalid ? sc[base + min(r, g.bs - 1)][hh] : 0.f;
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[hh][e] = fmaf(p, x[i][e], acc[hh][e]);
      }
    }
    base += g.bs;
  }
  // sum the row slots: within the wave by shuffles, across waves in LDS
#pragma unroll
  for (int sh = LPR; sh < 64; sh <<= 1)
#pragma unroll
    for (int hh = 0; hh < G; ++hh)
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[hh][e] += __shfl_xor(acc[hh][e], sh);
  if (lane < LPR) {
#pragma unroll
    for (int hh = 0; hh < G; ++hh)
#pragma unroll
      for (int e = 0; e < VEC; ++e) red[wave][hh][col + e] = acc[hh][e];
  }
  __syncthreads();
  const int64_t pbase = ((int64_t)slab * splits + split) * G;
  for (int e = tid; e < G * D; e += kDecThreads) {
    const int hh = e / D, d = e % D;
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < kDecThreads / 64; ++w) s += red[w][hh][d];
    ws.o[(pbase + hh) * D + d] = s;
  }
  if (tid < G) {
    float l = 0.f;
#pragma unroll
    for (int w = 0; w < kDecThreads / 64; ++w) l += mred[w][tid];
    ws.m[pbase + tid] = mx[tid];
    ws.l[pbase + tid] = l;
  }
}

template <typename T, int D>
__global__ __launch_bounds__(D) void decode_merge_kernel(Geo g, int splits, DecodeWs ws, T* __restrict__ out,
                                                         float* __restrict__ lse) {
  const int bh = blockIdx.x;  // b * Hq + h
  const int b = bh / g.Hq;
  const int h = bh % g.Hq;
  const int slab = b * g.Hkv + h / g.G;
  const int hh = h % g.G;
  float mstar = -__builtin_inff();
  for (int s = 0; s < splits; ++s) mstar = fmaxf(mstar, ws.m[((int64_t)slab * splits + s) * g.G + hh]);
  float l = 0.f, o = 0.f;
  for (int s = 0; s < splits; ++s) {
    const int64_t p = ((int64_t)slab * splits + s) * g.G + hh;
    const float m = ws.m[p];
    const float w = m == -__builtin_inff() ? 0.f : exp2f(m - mstar);
    l += w * ws.l[p];
    o += w * ws.o[p * D + threadIdx.x];
  }
  const float val = l > 0.f ? o / l : 0.f;  // a sequence that attends nothing outputs zeros
  if constexpr (sizeof(T) == 2) ((uint16_t*)out)[(int64_t)bh * D + threadIdx.x] = (uint16_t)f32_to_bf16(val);
  else ((float*)out)[(int64_t)bh * D + threadIdx.x] = val;
  if (lse != nullptr && threadIdx.x == 0) lse[bh] = (mstar + log2f(l)) * kLn2;
}

DecodeWs carve(const Geo& g, void* base, int splits) {
  char* p = (char*)base;
  auto take = [&](size_t bytes) {
    char* r = p;
    p += (bytes + 255) & ~(size_t)255;
    return r;
  };
  const int64_t slabs = (int64_t)g.B * g.Hkv;
  DecodeWs w;
  w.idx = (int32_t*)take(sizeof(int32_t) * slabs * (g.K > 0 ? g.K : 1));
  w.cnt = (int32_t*)take(sizeof(int32_t) * slabs);
  w.m = (float*)take(sizeof(float) * slabs * splits * g.G);
  w.l = (float*)take(sizeof(float) * slabs * splits * g.G);
  w.o = (float*)take(sizeof(float) * slabs * splits * g.G * g.D);
  return w;
}

}  // namespace

// Device address of this GPU's scratch array, looked up once per device (with
// that device current) and kept.
hipError_t decode_scratch_ptr(void** ptr) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

// Worst-case block count of the walk: sink blocks, selected blocks, local block.
int decode_splits(const Geo& g, int /*cache_len*/) {
  const int sink_blocks = (g.sink + g.bs - 1) / g.bs;
  const int tiles = min(g.nb, sink_blocks + g.K + 1);
  return (tiles + kTilesPerSplit - 1) / kTilesPerSplit;
}

size_t decode_workspace_bytes(const Geo& g) {
  const int splits = decode_splits(g, g.N);
  const size_t slabs = (size_t)g.B * g.Hkv;
  auto r = [](size_t x) { return (x + 255) & ~(size_t)255; };
  return r(sizeof(int32_t) * slabs * (g.K > 0 ? g.K : 1)) + r(sizeof(int32_t) * slabs) +
         2 * r(sizeof(float) * slabs * splits * g.G) + r(sizeof(float) * slabs * splits * g.G * g.D);
}

template <typename T, int D>
static hipError_t launch_decode_d(const Geo& g, const void* q, const void* kc, const void* vc, const float* pyr,
                                  const int32_t* lens, int len_all, void* out, float* lse, int32_t* idx_out,
                                  int32_t* cnt_out, void* wsb, float* pyr_w, const int32_t* old_lens, hipStream_t s) {
  const int splits = decode_splits(g, len_all);
  DecodeWs ws = carve(g, wsb, splits);
  // the selection goes straight to the caller's buffers when they are given
  // (the same layouts, [B * Hkv, K] and [B * Hkv]) and the attention reads it
  // there: no copies after the step
  if (idx_out != nullptr && g.K > 0) ws.idx = idx_out;
  if (cnt_out != nullptr) ws.cnt = cnt_out;
  const int slabs = g.B * g.Hkv;
  {
    const int e = pool_slots_per_lane(g);
    const T* qt = (const T*)q;
    const T* kt = (const T*)kc;
    if (e <= 2)
      PISA_LAUNCH(g, (decode_select_kernel<T, D, 2>), dim3(slabs), dim3(kDecSelThreads), 0, s, g, qt, pyr, lens,
                  len_all, ws.idx, ws.cnt, kt, pyr_w, old_lens);
    else if (e <= 4)
      PISA_LAUNCH(g, (decode_select_kernel<T, D, 4>), dim3(slabs), dim3(kDecSelThreads), 0, s, g, qt, pyr, lens,
                  len_all, ws.idx, ws.cnt, kt, pyr_w, old_lens);
    else if (e <= 5)  // K = 32 at fanout 8: 263 slots (the ranking's bit counts run over fewer slot groups)
      PISA_LAUNCH(g, (decode_select_kernel<T, D, 5>), dim3(slabs), dim3(kDecSelThreads), 0, s, g, qt, pyr, lens,
                  len_all, ws.idx, ws.cnt, kt, pyr_w, old_lens);
    else if (e <= 6)
      PISA_LAUNCH(g, (decode_select_kernel<T, D, 6>), dim3(slabs), dim3(kDecSelThreads), 0, s, g, qt, pyr, lens,
                  len_all, ws.idx, ws.cnt, kt, pyr_w, old_lens);
    else if (e <= 8)
      PISA_LAUNCH(g, (decode_select_kernel<T, D, 8>), dim3(slabs), dim3(kDecSelThreads), 0, s, g, qt, pyr, lens,
                  len_all, ws.idx, ws.cnt, kt, pyr_w, old_lens);
    else
      PISA_LAUNCH(g, (decode_select_kernel<T, D, 16>), dim3(slabs), dim3(kDecSelThreads), 0, s, g, qt, pyr, lens,
                  len_all, ws.idx, ws.cnt, kt, pyr_w, old_lens);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 grid(splits, slabs);
  const T* qt = (const T*)q;
  const T* kt = (const T*)kc;
  const T* vt = (const T*)vc;
  switch (g.G) {
    case 1: PISA_LAUNCH(g, (decode_attn_kernel<T, D, 1>), grid, dim3(kDecThreads), 0, s, g, qt, kt, vt, lens, len_all, splits, ws); break;
    case 2: PISA_LAUNCH(g, (decode_attn_kernel<T, D, 2>), grid, dim3(kDecThreads), 0, s, g, qt, kt, vt, lens, len_all, splits, ws); break;
    case 4: PISA_LAUNCH(g, (decode_attn_kernel<T, D, 4>), grid, dim3(kDecThreads), 0, s, g, qt, kt, vt, lens, len_all, splits, ws); break;
    default: PISA_LAUNCH(g, (decode_attn_kernel<T, D, 8>), grid, dim3(kDecThreads), 0, s, g, qt, kt, vt, lens, len_all, splits, ws); break;
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  PISA_LAUNCH(g, (decode_merge_kernel<T, D>), dim3(g.B * g.Hq), dim3(D), 0, s, g, splits, ws, (T*)out, lse);
  return hipGetLastError();
}

hipError_t launch_decode(const Geo& g, const void* q, const void* kc, const void* vc, const float* pyr,
                         const int32_t* lens, int cache_len, void* out, float* lse, int32_t* idx, int32_t* cnt, void* ws,
                         hipStream_t s, float* pyr_w, const int32_t* old_lens) {
  if (g.dtype == PISA_BF16)
    return g.D == 128 ? launch_decode_d<uint16_t, 128>(g, q, kc, vc, pyr, lens, cache_len, out, lse, idx, cnt, ws,
                                                       pyr_w, old_lens, s)
                      : launch_decode_d<uint16_t, 64>(g, q, kc, vc, pyr, lens, cache_len, out, lse, idx, cnt, ws,
                                                      pyr_w, old_lens, s);
  return g.D == 128 ? launch_decode_d<float, 128>(g, q, kc, vc, pyr, lens, cache_len, out, lse, idx, cnt, ws, pyr_w,
                                                  old_lens, s)
                    : launch_decode_d<float, 64>(g, q, kc, vc, pyr, lens, cache_len, out, lse, idx, cnt, ws, pyr_w,
                                                 old_lens, s);
}

}  // namespace pisa
