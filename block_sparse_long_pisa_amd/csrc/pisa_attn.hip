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
// so every K/V tile staged in LDS feeds up to 256 rows. Per tile each wave
// computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (a lane then owns one
// query column), runs the online softmax in registers, and accumulates
// O^T += V^T P^T on the same matrix cores, with V stored transposed in LDS.
// fp32 path: plain VALU, one thread per query row.
#include "pisa_internal.h"

namespace pisa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Which key block a tile index refers to, and how many of its keys count.
struct TileWalk {
  int nfull_sink;    // blocks wholly inside the sink (before qb)
  int partial;       // 1 if the block holding the sink's end is attended as a sink tile
  int nsel;          // selected blocks
  int ntiles;        // + 1 local block
  __device__ __forceinline__ void at(int t, const int* sel, const Geo& g, int qb, int local_rows, int& j, int& nvalid,
                                     bool& local) const {
    local = false;
    if (t < nfull_sink) {
      j = t;
      nvalid = g.bs;
    } else if (t < nfull_sink + partial) {
      j = g.j0;
      nvalid = g.sink - g.j0 * g.bs;
    } else if (t < ntiles - 1) {
      j = sel[t - nfull_sink - partial];
      nvalid = g.bs;
      if (j < 0 || j >= qb) {  // not a block this unit may select: attend nothing from it
        j = qb;
        nvalid = 0;
      }
    } else {
      j = qb;
      nvalid = local_rows;
      local = true;
    }
  }
};

__device__ __forceinline__ TileWalk make_walk(const Geo& g, int qb, const int* sel, int nsel) {
  TileWalk w;
  w.nfull_sink = min(g.j0, qb);
  const bool sink_tail = g.sink > g.j0 * g.bs && g.j0 < qb;
  w.partial = (sink_tail && !(nsel > 0 && sel[0] == g.j0)) ? 1 : 0;
  w.nsel = nsel;
  w.ntiles = w.nfull_sink + w.partial + nsel + 1;
  return w;
}

__device__ __forceinline__ uint32_t word(const uint4& u, int p) {
  return p == 0 ? u.x : (p == 1 ? u.y : (p == 2 ? u.z : u.w));
}

template <int D, int BS, int NW>
__global__ __launch_bounds__(NW * 64) void attn_bf16_kernel(Geo g, const uint16_t* __restrict__ q,
                                                            const uint16_t* __restrict__ k,
                                                            const uint16_t* __restrict__ v,
                                                            const int32_t* __restrict__ idx,
                                                            const int32_t* __restrict__ cnt, uint16_t* __restrict__ out,
                                                            float* __restrict__ lse, int parts) {
  constexpr int NT = NW * 64;
  constexpr int KP = D + 8;   // K tile row pitch (bf16): 16-lane groups hit distinct banks
  constexpr int VP = BS + 4;  // V^T tile row pitch (bf16)
  constexpr int NKB = BS / 32;
  constexpr int NDS = D / 16;
  constexpr int NDB = D / 32;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[BS * KP];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[D * VP];
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
  const int wave = threadIdx.x >> 6;
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

  bf16x8_t qf[NDS];
  {
    const uint16_t* qrow = q + (((int64_t)b * g.Hq + h) * g.N + (qvalid ? qpos : 0)) * D;
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
      uint4 u = qvalid ? *reinterpret_cast<const uint4*>(qrow + ds * 16 + hi * 8) : make_uint4(0, 0, 0, 0);
      qf[ds] = __builtin_bit_cast(bf16x8_t, u);
    }
  }
  f32x16_t oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
  float m_run = -__builtin_inff();
  float l_run = 0.f;
  const float c = g.scale * kLog2e;

  const uint16_t* kbase = k + ((int64_t)b * g.Hkv + kvh) * g.N * D;
  const uint16_t* vbase = v + ((int64_t)b * g.Hkv + kvh) * g.N * D;
  __syncthreads();
  const TileWalk walk = make_walk(g, qb, sel, nsel);

  for (int t = 0; t < walk.ntiles; ++t) {
    int j, nvalid;
    bool local;
    walk.at(t, sel, g, qb, local_rows, j, nvalid, local);
    const int rows_in_mem = min(BS, g.N - j * BS);
    const uint16_t* kt = kbase + (int64_t)j * BS * D;
    const uint16_t* vt = vbase + (int64_t)j * BS * D;

    // stage K (row-major) and V (transposed) in LDS
    for (int ci = threadIdx.x; ci < BS * D / 8; ci += NT) {
      const int row = ci / (D / 8);
      const int cc = ci % (D / 8);
      uint4 u = row < rows_in_mem ? *reinterpret_cast<const uint4*>(kt + row * D + cc * 8) : make_uint4(0, 0, 0, 0);
      *reinterpret_cast<uint4*>(Ks + row * KP + cc * 8) = u;
    }
    for (int vb = threadIdx.x; vb < (BS / 4) * (D / 8); vb += NT) {
      const int kg = vb / (D / 8);
      const int dg = vb % (D / 8);
      uint4 r[4];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int row = kg * 4 + rr;
        r[rr] = row < rows_in_mem ? *reinterpret_cast<const uint4*>(vt + row * D + dg * 8) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t w0 = word(r[0], e >> 1), w1 = word(r[1], e >> 1);
        const uint32_t w2 = word(r[2], e >> 1), w3 = word(r[3], e >> 1);
        uint2 o2;
        if (e & 1) {
          o2.x = (w0 >> 16) | (w1 & 0xffff0000u);
          o2.y = (w2 >> 16) | (w3 & 0xffff0000u);
        } else {
          o2.x = (w0 & 0xffffu) | (w1 << 16);
          o2.y = (w2 & 0xffffu) | (w3 << 16);
        }
        *reinterpret_cast<uint2*>(Vt + (dg * 8 + e) * VP + kg * 4) = o2;
      }
    }
    __syncthreads();

    // S^T[key][query] for 32-key blocks; lane (l32, hi) owns query l32 and keys
    // kb*32 + (i/4)*8 + hi*4 + i%4 of accumulator element i
    f32x16_t sacc[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[kb][i] = 0.f;
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds) {
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(Ks + (kb * 32 + l32) * KP + ds * 16 + hi * 8);
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ds], sacc[kb], 0, 0, 0);
      }
    }
    if (local || nvalid < BS) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = kb * 32 + (i >> 2) * 8 + hi * 4 + (i & 3);
          const bool ok = key < nvalid && (!local || j * BS + key <= qpos);
          if (!ok) sacc[kb][i] = -__builtin_inff();
        }
    }
    // online softmax (log2 domain)
    float mx = -__builtin_inff();
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kb][i]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx * c);
    const float m_use = m_new == -__builtin_inff() ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_use);
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = exp2f(fmaf(sacc[kb][i], c, -m_use));
        sacc[kb][i] = p;
        rs += p;
      }
    rs += __shfl_xor(rs, 32);
    l_run = l_run * alpha + rs;
    m_run = m_new;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;

    // O^T[d][query] += V^T P^T over 16-key steps; B-operand slot (hi, e) of step
    // (kb, hh) holds key kb*32 + hh*16 + (e/4)*8 + hi*4 + e%4
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        bf16x8_t pb;
#pragma unroll
        for (int e = 0; e < 8; ++e) pb[e] = (__bf16)sacc[kb][hh * 8 + e];
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const uint16_t* vp = Vt + (db * 32 + l32) * VP + kb * 32 + hh * 16 + hi * 4;
          const uint2 lo = *reinterpret_cast<const uint2*>(vp);
          const uint2 up = *reinterpret_cast<const uint2*>(vp + 8);
          const bf16x8_t a = __builtin_bit_cast(bf16x8_t, make_uint4(lo.x, lo.y, up.x, up.y));
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, oacc[db], 0, 0, 0);
        }
      }
    }
    __syncthreads();
  }

  if (qvalid) {
    const float inv = 1.f / l_run;
    uint16_t* orow = out + (((int64_t)b * g.Hq + h) * g.N + qpos) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 16; i += 4) {
        const int d = db * 32 + (i >> 2) * 8 + hi * 4;
        uint2 w;
        w.x = pack_bf16x2(oacc[db][i] * inv, oacc[db][i + 1] * inv);
        w.y = pack_bf16x2(oacc[db][i + 2] * inv, oacc[db][i + 3] * inv);
        *reinterpret_cast<uint2*>(orow + d) = w;
      }
    if (lse != nullptr && hi == 0) lse[((int64_t)b * g.Hq + h) * g.N + qpos] = (m_run + log2f(l_run)) * kLn2;
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
