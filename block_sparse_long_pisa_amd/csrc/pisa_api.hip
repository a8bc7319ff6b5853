// Host side of the C ABI: argument validation, problem geometry and launches.
// Every check runs on the host before any launch; a failing call launches and
// writes nothing.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <string>

#include "pisa_internal.h"

namespace {

thread_local std::string g_last_error;

pisa_status fail(pisa_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

pisa_status ok() {
  g_last_error.clear();
  return PISA_OK;
}

bool pow2_in(int x, int lo, int hi) { return x >= lo && x <= hi && (x & (x - 1)) == 0; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Validate the problem and derive its geometry.
pisa_status make_geo(const pisa_problem* p, pisa::Geo* g) {
  if (p == nullptr) return fail(PISA_ERR_NULL, "problem is NULL");
  if (p->dtype != PISA_F32 && p->dtype != PISA_BF16) return fail(PISA_ERR_UNSUPPORTED, "dtype %d", p->dtype);
  if (p->batch < 0 || p->heads_q <= 0 || p->heads_kv <= 0 || p->seq_len < 0)
    return fail(PISA_ERR_SHAPE, "batch %d, heads_q %d, heads_kv %d, seq_len %lld must be >= 0 / > 0", p->batch,
                p->heads_q, p->heads_kv, (long long)p->seq_len);
  if (p->heads_q % p->heads_kv != 0)
    return fail(PISA_ERR_SHAPE, "heads_q %d is not a multiple of heads_kv %d", p->heads_q, p->heads_kv);
  if (p->head_dim != 64 && p->head_dim != 128) return fail(PISA_ERR_UNSUPPORTED, "head_dim %d (64 or 128)", p->head_dim);
  if (!pow2_in(p->block_size, 32, 128)) return fail(PISA_ERR_UNSUPPORTED, "block_size %d (32, 64 or 128)", p->block_size);
  if (!pow2_in(p->fanout, 2, 16)) return fail(PISA_ERR_UNSUPPORTED, "fanout %d (2, 4, 8 or 16)", p->fanout);
  if (p->levels < 1) return fail(PISA_ERR_SHAPE, "levels %d < 1", p->levels);
  if (p->levels > pisa::kMaxLevels) return fail(PISA_ERR_UNSUPPORTED, "levels %d > %d", p->levels, pisa::kMaxLevels);
  if (p->top_k < 0) return fail(PISA_ERR_SHAPE, "top_k %d < 0", p->top_k);
  if (p->top_k > pisa::kMaxTopK) return fail(PISA_ERR_UNSUPPORTED, "top_k %d > %d", p->top_k, pisa::kMaxTopK);
  if ((int64_t)p->top_k * p->fanout + p->fanout - 1 > pisa::kPoolMax)
    return fail(PISA_ERR_UNSUPPORTED, "top_k * fanout + fanout - 1 = %d exceeds the %d-node pool",
                p->top_k * p->fanout + p->fanout - 1, pisa::kPoolMax);
  if (p->sink_len < 0) return fail(PISA_ERR_SHAPE, "sink_len %d < 0", p->sink_len);
  if (p->causal != 0 && p->causal != 1) return fail(PISA_ERR_UNSUPPORTED, "causal %d (0 or 1)", p->causal);
  if (p->pool != PISA_POOL_MEAN && p->pool != PISA_POOL_MAX) return fail(PISA_ERR_UNSUPPORTED, "pool %d", p->pool);
  if (!(p->sm_scale == p->sm_scale)) return fail(PISA_ERR_SHAPE, "sm_scale is NaN");
  if (p->seq_len > (int64_t)INT32_MAX - 256) return fail(PISA_ERR_SHAPE, "seq_len %lld too large", (long long)p->seq_len);
  if ((int64_t)p->batch * p->heads_kv > 65535 || (int64_t)p->batch * p->heads_q > INT32_MAX)
    return fail(PISA_ERR_SHAPE, "batch * heads too large");

  pisa::Geo& G = *g;
  G.B = p->batch;
  G.Hq = p->heads_q;
  G.Hkv = p->heads_kv;
  G.G = p->heads_q / p->heads_kv;
  G.D = p->head_dim;
  G.N = (int)p->seq_len;
  G.bs = p->block_size;
  G.nb = (int)((p->seq_len + p->block_size - 1) / p->block_size);
  G.f = p->fanout;
  G.L = p->levels;
  G.K = p->top_k;
  G.sink = p->sink_len;
  G.j0 = p->sink_len / p->block_size;
  G.dtype = p->dtype;
  G.causal = p->causal;
  G.pool = p->pool;
  G.scale = p->sm_scale > 0.f ? p->sm_scale : 1.0f / sqrtf((float)p->head_dim);
  int n = G.nb;
  int span = 1;
  G.off[0] = 0;
  for (int l = 0; l < pisa::kMaxLevels; ++l) {
    G.nodes[l] = l < G.L ? n : 0;
    G.span[l] = l < G.L ? span : 0;
    G.off[l + 1] = G.off[l] + G.nodes[l];
    if (l + 1 < G.L) {
      n = (n + G.f - 1) / G.f;
      span *= G.f;
    }
  }
  if (G.nb > 0 && G.nodes[G.L - 1] > pisa::kPoolMax)
    return fail(PISA_ERR_UNSUPPORTED, "top pyramid level holds %d nodes (> %d): use more levels", G.nodes[G.L - 1],
                pisa::kPoolMax);
  return PISA_OK;
}

bool empty(const pisa::Geo& g) { return g.B == 0 || g.N == 0; }

pisa_status hip_fail(hipError_t e, const char* what) {
  return fail(PISA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Checks shared by both decode entry points (cache_len checked by the caller).
pisa_status check_decode(const pisa::Geo& g, const void* q, const void* k_cache, const void* v_cache,
                         const float* pyramid, const void* out, const void* workspace, size_t workspace_bytes) {
  if (g.G != 1 && g.G != 2 && g.G != 4 && g.G != 8)
    return fail(PISA_ERR_UNSUPPORTED, "decode supports 1, 2, 4 or 8 query heads per kv head (got %d)", g.G);
  if (!g.causal) return fail(PISA_ERR_UNSUPPORTED, "decode is causal: the problem must have causal = 1");
  if (g.N < 1) return fail(PISA_ERR_SHAPE, "seq_len (the cache capacity) must be >= 1");
  if (q == nullptr || k_cache == nullptr || v_cache == nullptr || pyramid == nullptr || out == nullptr)
    return fail(PISA_ERR_NULL, "q, k_cache, v_cache, pyramid or out is NULL");
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(pyramid) || !aligned16(out))
    return fail(PISA_ERR_ALIGN, "q, caches, pyramid and out must be 16-byte aligned");
  const size_t need = pisa::decode_workspace_bytes(g);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(PISA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                workspace == nullptr ? (size_t)0 : workspace_bytes);
  if (((uintptr_t)workspace & 255u) != 0) return fail(PISA_ERR_ALIGN, "workspace must be 256-byte aligned");
  return PISA_OK;
}

}  // namespace

namespace pisa {

hipError_t device_cus(int* cus) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  return hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev);
}

bool log_launches() {
  static const bool on = [] {
    const char* e = getenv("PISA_LOG");
    return e != nullptr && *e != 0 && strcmp(e, "0") != 0;
  }();
  return on;
}

void log_launch(const Geo& g, const char* kernel, const char* launcher, dim3 grid, dim3 block) {
  // the launcher's template arguments, as its signature prints them: "[D = 128, ...]"
  const char* targs = strrchr(launcher, '[');
  fprintf(stderr,
          "[pisa] launch %s %s grid (%u, %u, %u) workgroup (%u, %u, %u) | B %d Hq %d Hkv %d N %d d %d bs %d f %d L %d "
          "K %d sink %d %s %s %s\n",
          kernel, targs ? targs : "", grid.x, grid.y, grid.z, block.x, block.y, block.z, g.B, g.Hq, g.Hkv, g.N, g.D,
          g.bs, g.f, g.L, g.K, g.sink, g.dtype == PISA_BF16 ? "bf16" : "f32", g.causal ? "causal" : "bidirectional",
          g.pool == PISA_POOL_MAX ? "max-pool" : "mean-pool");
}

}  // namespace pisa

extern "C" {

const char* pisa_status_string(pisa_status s) {
  // a C caller may pass any int: read its bits as one, since loading an enum
  // object that holds a value outside the enumeration is undefined in C++
  int v;
  memcpy(&v, &s, sizeof v);
  switch (v) {
    case PISA_OK: return "ok";
    case PISA_ERR_NULL: return "null pointer";
    case PISA_ERR_SHAPE: return "invalid shape";
    case PISA_ERR_UNSUPPORTED: return "unsupported";
    case PISA_ERR_WORKSPACE: return "workspace too small";
    case PISA_ERR_HIP: return "HIP error";
    case PISA_ERR_ALIGN: return "misaligned pointer";
  }
  return "unknown status";
}

const char* pisa_last_error(void) { return g_last_error.c_str(); }

int32_t pisa_version(void) { return 10000; }

pisa_status pisa_pyramid_layout(const pisa_problem* p, int64_t* level_offsets) {
  pisa::Geo g;
  pisa_status s = make_geo(p, &g);
  if (s != PISA_OK) return s;
  if (level_offsets == nullptr) return fail(PISA_ERR_NULL, "level_offsets is NULL");
  for (int l = 0; l <= g.L; ++l) level_offsets[l] = g.off[l];
  return ok();
}

pisa_status pisa_build_pyramid(const pisa_problem* p, const void* k, float* pyramid, hipStream_t stream) {
  pisa::Geo g;
  pisa_status s = make_geo(p, &g);
  if (s != PISA_OK) return s;
  if (empty(g)) return ok();
  if (k == nullptr || pyramid == nullptr) return fail(PISA_ERR_NULL, "k or pyramid is NULL");
  if (!aligned16(k) || !aligned16(pyramid)) return fail(PISA_ERR_ALIGN, "k and pyramid must be 16-byte aligned");
  hipError_t e = pisa::launch_build_pyramid(g, k, pyramid, stream);
  return e == hipSuccess ? ok() : hip_fail(e, "pisa_build_pyramid launch");
}

pisa_status pisa_select_topk(const pisa_problem* p, const void* q, const float* pyramid, int32_t* idx, int32_t* cnt,
                             hipStream_t stream) {
  pisa::Geo g;
  pisa_status s = make_geo(p, &g);
  if (s != PISA_OK) return s;
  if (empty(g)) return ok();
  if (q == nullptr || pyramid == nullptr || cnt == nullptr || (idx == nullptr && g.K > 0))
    return fail(PISA_ERR_NULL, "q, pyramid, idx or cnt is NULL");
  if (!aligned16(q) || !aligned16(pyramid)) return fail(PISA_ERR_ALIGN, "q and pyramid must be 16-byte aligned");
  hipError_t e = pisa::launch_select(g, q, pyramid, idx, cnt, stream);
  return e == hipSuccess ? ok() : hip_fail(e, "pisa_select_topk launch");
}

pisa_status pisa_sparse_attn_fwd(const pisa_problem* p, const void* q, const void* k, const void* v, const int32_t* idx,
                                 const int32_t* cnt, void* out, float* lse, hipStream_t stream) {
  pisa::Geo g;
  pisa_status s = make_geo(p, &g);
  if (s != PISA_OK) return s;
  if (empty(g)) return ok();
  if (q == nullptr || k == nullptr || v == nullptr || cnt == nullptr || out == nullptr || (idx == nullptr && g.K > 0))
    return fail(PISA_ERR_NULL, "q, k, v, idx, cnt or out is NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
    return fail(PISA_ERR_ALIGN, "q, k, v and out must be 16-byte aligned");
  hipError_t e = pisa::launch_attn(g, q, k, v, idx, cnt, out, lse, stream);
  return e == hipSuccess ? ok() : hip_fail(e, "pisa_sparse_attn_fwd launch");
}

pisa_status pisa_select_attend(const pisa_problem* p, const void* q, const void* k, const void* v,
                               const float* pyramid, int32_t* idx, int32_t* cnt, void* out, float* lse,
                               hipStream_t stream) {
  pisa::Geo g;
  pisa_status s = make_geo(p, &g);
  if (s != PISA_OK) return s;
  if (empty(g)) return ok();
  if (g.dtype != PISA_BF16) return fail(PISA_ERR_UNSUPPORTED, "the fused path is implemented for bf16 only");
  if (!g.causal) return fail(PISA_ERR_UNSUPPORTED, "the fused path is implemented for causal attention only");
  if (q == nullptr || k == nullptr || v == nullptr || pyramid == nullptr || out == nullptr)
    return fail(PISA_ERR_NULL, "q, k, v, pyramid or out is NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(pyramid) || !aligned16(out))
    return fail(PISA_ERR_ALIGN, "q, k, v, pyramid and out must be 16-byte aligned");
  hipError_t e = pisa::launch_select_attn(g, q, k, v, pyramid, idx, cnt, out, lse, stream);
  return e == hipSuccess ? ok() : hip_fail(e, "pisa_select_attend launch");
}

pisa_status pisa_sparse_attn_bwd_workspace_size(const pisa_problem* p, size_t* bytes) {
  pisa::Geo g;
  pisa_status s = make_geo(p, &g);
  if (s != PISA_OK) return s;
  if (bytes == nullptr) return fail(PISA_ERR_NULL, "bytes is NULL");
  *bytes = empty(g) ? 0 : pisa::attn_bwd_workspace_bytes(g);
  return ok();
}

pisa_status pisa_sparse_attn_bwd(const pisa_problem* p, const void* q, const void* k, const void* v, const int32_t* idx,
                                 const int32_t* cnt, const void* out, const float* lse, const void* dout, void* dq,
                                 void* dk, void* dv, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  pisa::Geo g;
  pisa_status s = make_geo(p, &g);
  if (s != PISA_OK) return s;
  if (empty(g)) return ok();
  if (g.dtype != PISA_BF16) return fail(PISA_ERR_UNSUPPORTED, "the backward pass is implemented for bf16 only");
  if (!g.causal) return fail(PISA_ERR_UNSUPPORTED, "the backward pass is implemented for causal attention only");
  if (q == nullptr || k == nullptr || v == nullptr || cnt == nullptr || out == nullptr || lse == nullptr ||
      dout == nullptr || dq == nullptr || dk == nullptr || dv == nullptr || (idx == nullptr && g.K > 0))
    return fail(PISA_ERR_NULL, "q, k, v, idx, cnt, out, lse, dout, dq, dk or dv is NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(dout) || !aligned16(dq) ||
      !aligned16(dk) || !aligned16(dv) || ((uintptr_t)lse & 3u) != 0)
    return fail(PISA_ERR_ALIGN, "tensors must be 16-byte aligned (lse 4-byte)");
  if ((int64_t)g.B * g.Hkv * g.nb > INT32_MAX / 2)
    return fail(PISA_ERR_UNSUPPORTED, "too many key blocks for the backward pass");
  const size_t need = pisa::attn_bwd_workspace_bytes(g);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(PISA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                workspace == nullptr ? (size_t)0 : workspace_bytes);
  if (((uintptr_t)workspace & 255u) != 0) return fail(PISA_ERR_ALIGN, "workspace must be 256-byte aligned");
  hipError_t e = pisa::launch_attn_bwd(g, q, k, v, idx, cnt, out, lse, dout, dq, dk, dv, workspace, stream);
  return e == hipSuccess ? ok() : hip_fail(e, "pisa_sparse_attn_bwd launch");
}

pisa_status pisa_decode_workspace_size(const pisa_problem* p, size_t* bytes) {
  pisa::Geo g;
  pisa_status s = make_geo(p, &g);
  if (s != PISA_OK) return s;
  if (bytes == nullptr) return fail(PISA_ERR_NULL, "bytes is NULL");
  *bytes = empty(g) ? 0 : pisa::decode_workspace_bytes(g);
  return ok();
}

pisa_status pisa_decode_step(const pisa_problem* p, const void* q, const void* k_cache, const void* v_cache,
                             const float* pyramid, int64_t cache_len, void* out, float* lse, int32_t* idx_out,
                             int32_t* cnt_out, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  pisa::Geo g;
  pisa_status s = make_geo(p, &g);
  if (s != PISA_OK) return s;
  if (g.B == 0) return ok();
  if (cache_len < 1 || cache_len > g.N)
    return fail(PISA_ERR_SHAPE, "cache_len %lld outside [1, seq_len = %d]", (long long)cache_len, g.N);
  s = check_decode(g, q, k_cache, v_cache, pyramid, out, workspace, workspace_bytes);
  if (s != PISA_OK) return s;
  hipError_t e = pisa::launch_decode(g, q, k_cache, v_cache, pyramid, nullptr, (int)cache_len, out, lse, idx_out,
                                     cnt_out, workspace, stream);
  return e == hipSuccess ? ok() : hip_fail(e, "pisa_decode_step launch");
}

pisa_status pisa_decode_step_ragged(const pisa_problem* p, const void* q, const void* k_cache, const void* v_cache,
                                    const float* pyramid, const int32_t* cache_lens, void* out, float* lse,
                                    int32_t* idx_out, int32_t* cnt_out, void* workspace, size_t workspace_bytes,
                                    hipStream_t stream) {
  pisa::Geo g;
  pisa_status s = make_geo(p, &g);
  if (s != PISA_OK) return s;
  if (g.B == 0) return ok();
  if (cache_lens == nullptr) return fail(PISA_ERR_NULL, "cache_lens is NULL");
  if (((uintptr_t)cache_lens & 3u) != 0) return fail(PISA_ERR_ALIGN, "cache_lens must be 4-byte aligned");
  s = check_decode(g, q, k_cache, v_cache, pyramid, out, workspace, workspace_bytes);
  if (s != PISA_OK) return s;
  hipError_t e = pisa::launch_decode(g, q, k_cache, v_cache, pyramid, cache_lens, 0, out, lse, idx_out, cnt_out,
                                     workspace, stream);
  return e == hipSuccess ? ok() : hip_fail(e, "pisa_decode_step_ragged launch");
}

pisa_status pisa_decode_step_ragged_append(const pisa_problem* p, const void* q, const void* k_cache,
                                           const void* v_cache, float* pyramid, const int32_t* old_lens,
                                           const int32_t* cache_lens, void* out, float* lse, int32_t* idx_out,
                                           int32_t* cnt_out, void* workspace, size_t workspace_bytes,
                                           hipStream_t stream) {
  pisa::Geo g;
  pisa_status s = make_geo(p, &g);
  if (s != PISA_OK) return s;
  if (g.B == 0) return ok();
  if (old_lens == nullptr || cache_lens == nullptr) return fail(PISA_ERR_NULL, "old_lens or cache_lens is NULL");
  if ((((uintptr_t)old_lens | (uintptr_t)cache_lens) & 3u) != 0)
    return fail(PISA_ERR_ALIGN, "old_lens and cache_lens must be 4-byte aligned");
  s = check_decode(g, q, k_cache, v_cache, pyramid, out, workspace, workspace_bytes);
  if (s != PISA_OK) return s;
  hipError_t e = pisa::launch_decode(g, q, k_cache, v_cache, pyramid, cache_lens, 0, out, lse, idx_out, cnt_out,
                                     workspace, stream, pyramid, old_lens);
  return e == hipSuccess ? ok() : hip_fail(e, "pisa_decode_step_ragged_append launch");
}

pisa_status pisa_decode_step_ragged_noalloc(const pisa_problem* p, const void* q, const void* k_cache,
                                            const void* v_cache, const float* pyramid, const int32_t* cache_lens,
                                            void* out, float* lse, int32_t* idx_out, int32_t* cnt_out,
                                            hipStream_t stream) {
  pisa::Geo g;
  pisa_status s = make_geo(p, &g);
  if (s != PISA_OK) return s;
  if (g.B == 0) return ok();
  if (cache_lens == nullptr) return fail(PISA_ERR_NULL, "cache_lens is NULL");
  if (((uintptr_t)cache_lens & 3u) != 0) return fail(PISA_ERR_ALIGN, "cache_lens must be 4-byte aligned");
  void* ws = nullptr;
  hipError_t e = pisa::decode_scratch_ptr(&ws);
  if (e != hipSuccess) return hip_fail(e, "pisa_decode_step_ragged_noalloc scratch lookup");
  // the problem and its buffers first (against the workspace it would need),
  // then whether that workspace fits the static one
  const size_t need = pisa::decode_workspace_bytes(g);
  s = check_decode(g, q, k_cache, v_cache, pyramid, out, ws, need);
  if (s != PISA_OK) return s;
  if (need > pisa::kDecodeScratchBytes)
    return fail(PISA_ERR_WORKSPACE, "this problem needs a %zu-byte decode workspace; the static one holds %zu bytes",
                need, pisa::kDecodeScratchBytes);
  e = pisa::launch_decode(g, q, k_cache, v_cache, pyramid, cache_lens, 0, out, lse, idx_out, cnt_out, ws, stream);
  return e == hipSuccess ? ok() : hip_fail(e, "pisa_decode_step_ragged_noalloc launch");
}

pisa_status pisa_pyramid_append(const pisa_problem* p, const void* k_cache, float* pyramid, const int32_t* old_lens,
                                const int32_t* new_lens, hipStream_t stream) {
  pisa::Geo g;
  pisa_status s = make_geo(p, &g);
  if (s != PISA_OK) return s;
  if (empty(g)) return ok();
  if (k_cache == nullptr || pyramid == nullptr || old_lens == nullptr || new_lens == nullptr)
    return fail(PISA_ERR_NULL, "k_cache, pyramid, old_lens or new_lens is NULL");
  if (!aligned16(k_cache) || !aligned16(pyramid)) return fail(PISA_ERR_ALIGN, "k_cache and pyramid must be 16-byte aligned");
  if ((((uintptr_t)old_lens | (uintptr_t)new_lens) & 3u) != 0)
    return fail(PISA_ERR_ALIGN, "old_lens and new_lens must be 4-byte aligned");
  hipError_t e = pisa::launch_pyramid_append(g, k_cache, pyramid, old_lens, new_lens, stream);
  return e == hipSuccess ? ok() : hip_fail(e, "pisa_pyramid_append launch");
}

}  // extern "C"
