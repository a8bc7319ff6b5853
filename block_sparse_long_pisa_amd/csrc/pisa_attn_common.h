// Tile machinery shared by the forward and backward attention kernels
// ("Attention clairsemée PISA : noyaux Triton sans matrice de scores", section
// "Des noyaux Triton qui ne matérialisent rien"): the walk of one query block's
// attended key tiles, the padded LDS tile layouts, the asynchronous
// global->LDS copies that fill them, and the fragment reads the matrix cores
// take from them.
#pragma once

#include <limits.h>

#include "pisa_internal.h"

namespace pisa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// 2^x with the hardware's v_exp_f32 and no denormal range reduction: results
// below 2^-126 only ever weigh a softmax term that is negligible anyway.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Reductions across the two half-waves (lanes l and l ^ 32): v_permlane32_swap
// exchanges one half of its first operand with the other half of its second, so
// with x in both operands the two results hold x of both halves in every lane.
__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Which key block a tile index refers to, and how many of its keys count.
// Causal walk of query block qb: the sink blocks before qb, the partial sink
// block (unless selected), the selected blocks, the local block under the
// causal mask. Bidirectional walk: every full sink block but qb, the partial
// sink block (unless selected or qb), the selected blocks, the whole local block.
struct TileWalk {
  int nfull_sink;  // sink blocks attended whole
  int skip;        // the sink block index the walk steps over (qb, bidirectional), else INT_MAX
  int partial;     // 1 if the block holding the sink's end is attended as a sink tile
  int nsel;        // selected blocks
  int ntiles;      // + 1 local block
  bool causal;
  __device__ __forceinline__ void at(int t, const int* sel, const Geo& g, int qb, int local_rows, int& j, int& nvalid,
                                     bool& local) const {
    local = false;
    if (t < nfull_sink) {
      j = t + (t >= skip ? 1 : 0);
      nvalid = min(g.bs, g.N - j * g.bs);
    } else if (t < nfull_sink + partial) {
      j = g.j0;
      nvalid = min(g.sink, g.N) - g.j0 * g.bs;
    } else if (t < ntiles - 1) {
      j = sel[t - nfull_sink - partial];
      nvalid = min(g.bs, g.N - j * g.bs);
      if (j < 0 || j >= (causal ? qb : g.nb) || j == qb) {  // not a block this unit may select: attend nothing
        j = qb;
        nvalid = 0;
      }
    } else {
      j = qb;
      nvalid = local_rows;
      local = causal;
    }
    // every lane reads the same selection entry: make the block and its key
    // count scalar, so tile addresses are formed once per tile in scalar registers
    j = __builtin_amdgcn_readfirstlane(j);
    nvalid = __builtin_amdgcn_readfirstlane(nvalid);
  }
};

__device__ __forceinline__ TileWalk make_walk(const Geo& g, int qb, const int* sel, int nsel) {
  TileWalk w;
  w.causal = g.causal != 0;
  bool sink_tail;
  if (w.causal) {
    w.nfull_sink = min(g.j0, qb);
    w.skip = INT_MAX;
    sink_tail = g.sink > g.j0 * g.bs && g.j0 < qb;
  } else {
    const int jn = min(g.j0, g.nb);
    w.nfull_sink = jn - (qb < jn ? 1 : 0);
    w.skip = qb < jn ? qb : INT_MAX;
    sink_tail = g.sink > g.j0 * g.bs && g.j0 < g.nb && g.j0 != qb;
  }
  w.partial = (sink_tail && !(nsel > 0 && sel[0] == g.j0)) ? 1 : 0;
  w.nsel = nsel;
  w.ntiles = w.nfull_sink + w.partial + nsel + 1;
  return w;
}

// LDS tiles hold key rows with padded pitches chosen so that both read
// patterns are free of bank conflicts: K rows are D + 8 bf16 apart (16
// consecutive rows at one 16-byte chunk land on distinct banks), V rows D + 32
// apart (4 consecutive rows x 64 bytes, the transposing V^T reads, cover all
// banks once). Every read is then a per-lane base register plus an immediate.
// Swizzled tiles (SW, d = 128 only) are unpadded instead: 256-byte rows with the
// logical 16-byte unit u of row r stored at u ^ tile_swz(r), which keeps both
// patterns conflict-free with fewer bytes copied, at the price of a per-lane
// offset per read step.
template <int D, int BS = 128, bool SW = false>
struct TilePitch {
  static_assert(!SW || D == 128, "swizzled tiles have 256-byte rows");
  static constexpr int K = SW ? D : D + 8;   // bf16 elements per K row
  static constexpr int V = SW ? D : D + 32;  // bf16 elements per V row
  static constexpr int KU = K / 8;           // 16-byte units per K row
  static constexpr int VU = V / 8;
  // whole 1 KB wave copies per tile; the LDS arrays are sized to match
  static constexpr int KI = (BS * KU + 63) / 64;
  static constexpr int VI = (BS * VU + 63) / 64;
  static constexpr int KSIZE = KI * 512;  // bf16 elements
  static constexpr int VSIZE = VI * 512;
};

// The unit swizzle of unpadded 256-byte rows: it depends on r mod 16 only. For
// 16 rows read at one unit (row fragments) and for 8 rows read as 4 x 8-byte
// pieces of a 32-byte slice (transposing reads) it spreads the reads over all
// banks; the bank-conflict counter of gfx950 reads zero on both.
__device__ __forceinline__ int tile_swz(int r) { return 4 * (r & 3) + ((r >> 2) & 3); }

typedef __attribute__((address_space(3))) void* lds_void_ptr;
typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t* lds_v4i16_ptr;

// Source offset (elements) within a tile of the 16-byte unit u of a padded LDS
// tile; padding units (and the slack past the tile) re-read the row's first
// chunk, rows past `rows` re-read the last valid row (their keys are masked).
template <int D, int UPR>
__device__ __forceinline__ int unit_src(int u, int rows) {
  const int r = u / UPR, cu = u % UPR;
  return min(r, rows - 1) * D + (cu < D / 8 ? cu : 0) * 8;
}

// Per-lane source offsets, in bytes, of this wave's copies of a full tile
// (they do not change from tile to tile).
template <int D_, int BS_, int NW_, bool SW_ = false>
struct DmaPlan {
  static constexpr int D = D_, BS = BS_, NW = NW_;
  using TP = TilePitch<D, BS, SW_>;
  static constexpr int KN = (TP::KI + NW - 1) / NW;
  static constexpr int VN = (TP::VI + NW - 1) / NW;
  uint32_t k[KN];
  uint32_t v[VN];
  // source element offset of the physical unit p of a tile with UPR units per row
  template <int UPR>
  static __device__ __forceinline__ int src(int p) {
    if constexpr (SW_) {
      const int r = p / UPR;
      return r * D + ((p % UPR) ^ tile_swz(r)) * 8;
    } else {
      return unit_src<D, UPR>(p, BS);
    }
  }
  __device__ __forceinline__ void init(int wave, int lane) {
#pragma unroll
    for (int n = 0; n < KN; ++n) k[n] = 2u * src<TP::KU>((wave + NW * n) * 64 + lane);
#pragma unroll
    for (int n = 0; n < VN; ++n) v[n] = 2u * src<TP::VU>((wave + NW * n) * 64 + lane);
  }
};

// A buffer resource over one tile's rows in memory: `bytes` bounds it, and the
// hardware's range check fills the copies of units at or past that bound (the
// rows after a sequence's end, in its ragged last block) with zeros -- rows that
// the masks already exclude -- at no per-lane cost. A copy is then one 16-byte
// load per lane from the resource's scalar base plus this lane's 32-bit byte
// offset, with no per-lane 64-bit address arithmetic.
constexpr int kRawBufferWord3 = 0x00020000;  // word 3 of an untyped (raw) buffer resource
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const uint16_t* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base), 0, bytes, kRawBufferWord3);
}

// Issue the copies of one half of a tile -- its keys (KEYS) or its values -- of
// which `rows_in_mem` rows lie in memory. Each wave instruction fills 64
// consecutive 16-byte LDS units in row order; the first I / NW copies of every
// wave always exist.
template <bool KEYS, typename Plan>
__device__ __forceinline__ void issue_half(const uint16_t* __restrict__ src, int rows_in_mem, uint16_t* dst,
                                           int wave, const Plan& plan) {
  using TP = typename Plan::TP;
  constexpr int NW = Plan::NW;
  constexpr int N = KEYS ? Plan::KN : Plan::VN;
  constexpr int I = KEYS ? TP::KI : TP::VI;
  const uint32_t* off = KEYS ? plan.k : plan.v;
  const __amdgpu_buffer_rsrc_t r = tile_rsrc(src, rows_in_mem * Plan::D * 2);
#pragma unroll
  for (int n = 0; n < N; ++n) {
    const int i = wave + NW * n;
    if (n < I / NW || i < I)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_ptr)(dst + i * 512), 16, off[n], 0, 0, 0);
  }
}

// Issue the copies of one K and one V tile, keys first.
template <typename Plan>
__device__ __forceinline__ void issue_tile(const uint16_t* __restrict__ kt, const uint16_t* __restrict__ vt,
                                           int rows_in_mem, uint16_t* kdst, uint16_t* vdst, int wave,
                                           const Plan& plan) {
  issue_half<true>(kt, rows_in_mem, kdst, wave, plan);
  issue_half<false>(vt, rows_in_mem, vdst, wave, plan);
}

// Wait until at most N of this wave's vector memory loads are outstanding.
template <int N>
__device__ __forceinline__ void wait_loads() {
  static_assert(N >= 0 && N < 64, "vmcnt holds 6 bits");
  __builtin_amdgcn_s_waitcnt(0x0f70 | (N & 15) | ((N >> 4) << 14));  // expcnt, lgkmcnt left free
}

// A workgroup barrier after which every wave's LDS reads have completed. Unlike
// __syncthreads(), whose fence also waits for this wave's copies into LDS still
// in flight, it leaves those copies running.
__device__ __forceinline__ void lds_read_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ __forceinline__ void wait_loads_and_sync() {
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0) only (expcnt, lgkmcnt left free)
  __syncthreads();                            // ... and every other wave's
}

// K-fragment style read: 8 consecutive bf16 of row `row` of a tile with row
// pitch P (elements), starting at column c (the A operand of a 32x32x16 MFMA
// whose lane l holds row l % 32, columns 16 * step + 8 * (l / 32) ...).
template <int P>
__device__ __forceinline__ bf16x8_t row_frag(const uint16_t* tile, int row, int c) {
  return *reinterpret_cast<const bf16x8_t*>(tile + row * P + c);
}

// Byte offset of this lane's first transposing read in a tile of pitch P:
// lanes 4j..4j+3 of each 16-lane block supply row j's four 8-byte pieces of a
// 16-column slice (ds_read_b64_tr_b16), so the fragment holds a column.
template <int P>
__device__ __forceinline__ int tr_offset(int lane) {
  const int hi = lane >> 5;
  return ((hi * 4 + ((lane & 15) >> 2)) * P + 16 * ((lane >> 4) & 1) + 4 * (lane & 3)) * 2;
}

// Transposed fragment: rows [r, r + 16) of the tile, columns [32 * db, 32 * db + 32),
// as the A operand (columns become rows) of a 32x32x16 MFMA; `off` from tr_offset<P>.
template <int P>
__device__ __forceinline__ bf16x8_t tr_frag(const uint16_t* tile, int off, int r, int db) {
  const char* base = reinterpret_cast<const char*>(tile) + off + r * P * 2 + db * 64;
  const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_ptr)(base));
  const v4i16_t up = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_ptr)(base + 8 * P * 2));
  const v4i16_t a8[2] = {lo, up};
  return __builtin_bit_cast(bf16x8_t, a8);
}

}  // namespace
}  // namespace pisa
