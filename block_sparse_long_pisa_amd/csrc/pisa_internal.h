// Internal declarations of the PISA HIP library (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pisa.h"

namespace pisa {

constexpr int kMaxLevels = 8;
constexpr int kPoolMax = 1024;  // largest candidate pool scored at one level
constexpr int kMaxTopK = 256;

// Problem geometry derived on the host from pisa_problem and passed to every
// kernel by value. Node counts and offsets are per (batch, kv head) slab.
struct Geo {
  int B, Hq, Hkv, G, D;
  int N;        // tokens (prefill) or cache capacity (decode)
  int bs, nb;   // block size and number of (possibly partial) blocks
  int f, L, K;  // fanout, levels, top-k
  int sink, j0; // sink tokens; blocks wholly inside the sink
  int dtype;
  int causal;   // 1: causal; 0: the bidirectional variant
  int pool;     // PISA_POOL_MEAN or PISA_POOL_MAX
  int nodes[kMaxLevels];
  int off[kMaxLevels + 1];  // off[L] = nodes per slab
  int span[kMaxLevels];     // blocks under one node of level l (f^l)
  float scale;              // softmax scale
};

// ---------------------------------------------------------------------------
// bf16 helpers (bf16 is carried as raw uint16 bits)

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }
__device__ __forceinline__ float bf16lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16hi(uint32_t pair) { return __uint_as_float(pair & 0xffff0000u); }

// fp32 -> bf16, round to nearest even (inputs here are finite)
__device__ __forceinline__ uint32_t f32_to_bf16(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
}

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// 16 bytes of a read-once stream: marked non-temporal so they do not push
// reused data out of the caches.
__device__ __forceinline__ uint4 load_stream16(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Load 16 bytes and widen to fp32: 8 values for bf16, 4 for fp32.
template <typename T>
struct Wide;
// raw() fetches the 16 bytes, widen() converts them: issuing several raw()
// before any widen() keeps the loads in flight together.
template <>
struct Wide<uint16_t> {
  static constexpr int kVec = 8;
  __device__ __forceinline__ static uint4 raw(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ static uint4 stream(const uint16_t* p) { return load_stream16(p); }
  __device__ __forceinline__ static void widen(const uint4& u, float* out) {
    out[0] = bf16lo(u.x); out[1] = bf16hi(u.x);
    out[2] = bf16lo(u.y); out[3] = bf16hi(u.y);
    out[4] = bf16lo(u.z); out[5] = bf16hi(u.z);
    out[6] = bf16lo(u.w); out[7] = bf16hi(u.w);
  }
  __device__ __forceinline__ static void load(const uint16_t* p, float* out) { widen(raw(p), out); }
};
template <>
struct Wide<float> {
  static constexpr int kVec = 4;
  __device__ __forceinline__ static uint4 raw(const float* p) { return *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ static uint4 stream(const float* p) { return load_stream16(p); }
  __device__ __forceinline__ static void widen(const uint4& u, float* out) {
    out[0] = __uint_as_float(u.x); out[1] = __uint_as_float(u.y);
    out[2] = __uint_as_float(u.z); out[3] = __uint_as_float(u.w);
  }
  __device__ __forceinline__ static void load(const float* p, float* out) { widen(raw(p), out); }
};

// compute units of the current device (the runtime's cached attribute)
hipError_t device_cus(int* cus);

// Launch log: with PISA_LOG set to anything but 0 in the environment, every
// kernel launch is described on stderr (kernel, template arguments of its
// launcher, grid, workgroup, problem) just before it is enqueued.
bool log_launches();
void log_launch(const Geo& g, const char* kernel, const char* launcher, dim3 grid, dim3 block);
#define PISA_LAUNCH(g, kernel, grid, block, shmem, stream, ...)                                          \
  do {                                                                                                  \
    if (::pisa::log_launches()) ::pisa::log_launch(g, #kernel, __PRETTY_FUNCTION__, dim3(grid), dim3(block)); \
    hipLaunchKernelGGL(kernel, grid, block, shmem, stream, __VA_ARGS__);                                \
  } while (0)

// ---------------------------------------------------------------------------
// launchers (each lives beside its kernels)

hipError_t launch_build_pyramid(const Geo& g, const void* k, float* pyr, hipStream_t s);
hipError_t launch_select(const Geo& g, const void* q, const float* pyr, int32_t* idx, int32_t* cnt, hipStream_t s);
hipError_t launch_attn(const Geo& g, const void* q, const void* k, const void* v, const int32_t* idx,
                       const int32_t* cnt, void* out, float* lse, hipStream_t s);

// selection and attention in one launch (bf16, causal): idx and cnt nullable
hipError_t launch_select_attn(const Geo& g, const void* q, const void* k, const void* v, const float* pyr,
                              int32_t* idx, int32_t* cnt, void* out, float* lse, hipStream_t s);

// backward of the sparse attention (bf16): rowdot, dQ, key lists, dK/dV, reduce
size_t attn_bwd_workspace_bytes(const Geo& g);
hipError_t launch_attn_bwd(const Geo& g, const void* q, const void* k, const void* v, const int32_t* idx,
                           const int32_t* cnt, const void* out, const float* lse, const void* dout, void* dq, void* dk,
                           void* dv, void* ws, hipStream_t s);

// decode: selection of one token per (batch, kv head), split attention, merge
int decode_splits(const Geo& g, int cache_len);
size_t decode_workspace_bytes(const Geo& g);
// the allocation-free decode's workspace: a static device array per GPU
constexpr size_t kDecodeScratchBytes = (size_t)PISA_DECODE_SCRATCH_BYTES;
hipError_t decode_scratch_ptr(void** ptr);
// lens: per-sequence cache lengths on the device, or nullptr for cache_len everywhere;
// old_lens (device, with lens): the selection's launch also appends tokens
// [old_lens[b], lens[b]) to the pyramid, written through pyr_w (the same pyramid)
hipError_t launch_decode(const Geo& g, const void* q, const void* kc, const void* vc, const float* pyr,
                         const int32_t* lens, int cache_len, void* out, float* lse, int32_t* idx, int32_t* cnt, void* ws,
                         hipStream_t s, float* pyr_w = nullptr, const int32_t* old_lens = nullptr);

// pyramid update after tokens [old_lens[b], new_lens[b]) were written to the key cache
hipError_t launch_pyramid_append(const Geo& g, const void* k, float* pyr, const int32_t* old_lens,
                                 const int32_t* new_lens, hipStream_t s);

}  // namespace pisa
