/*
 * pisa.h -- C ABI of the PISA content-selected block-sparse attention library
 * for AMD Instinct MI355X (gfx950).
 *
 * What the library computes (sources are the pages' titles and sections):
 *
 *   "Attention clairsemée PISA : noyaux Triton sans matrice de scores"
 *     - "Une pyramide de clés plutôt qu'un tapis uniforme" and "Le pooling comme
 *       première réduction": keys are grouped into blocks, blocks into nodes,
 *       nodes into coarser nodes; each level summarises the level below by
 *       pooling (here: the arithmetic mean).
 *     - "La sélection top-K guidée par la pyramide": each query block keeps the
 *       K most relevant key blocks by descending the levels, pruning at the top
 *       and refining below, for O(N log N) work.
 *     - "Des noyaux Triton qui ne matérialisent rien": similarity, selection and
 *       aggregation never write the N x N score matrix to memory.
 *   "Dropping the Anchor: ... via Pulsar Attention"
 *     - "Phase 1 : Encodage statistique du contexte": a small fixed attention-sink
 *       prefix (64 tokens by default) keeps the softmax stable.
 *     - "Phase 2 : Encodage de la requête globale": partial attentions over
 *       disjoint key sets merge exactly with an online softmax.
 *
 * Conventions shared by every call:
 *   - All tensors are caller-owned device memory, contiguous, row-major, 16-byte
 *     aligned. The library never allocates or frees device memory and keeps no
 *     mutable global state, except the static per-GPU workspace of
 *     pisa_decode_step_ragged_noalloc; every other call is thread-safe.
 *   - Q, K, V, O use the layout [batch, heads, tokens, head_dim] in the problem's
 *     dtype (fp32 or bf16). The pyramid is fp32 [batch, heads_kv, nodes, head_dim]
 *     with the levels stored one after another, finest first
 *     (see pisa_pyramid_layout).
 *   - Calls are asynchronous on the given HIP stream (0 is the null stream).
 *     Arguments are validated on the host before anything is launched; on any
 *     error nothing is launched or written and a non-zero status is returned;
 *     pisa_last_error() then holds a description (per calling thread). A fault
 *     inside a kernel surfaces at the caller's next synchronisation.
 *   - An empty problem (batch == 0 or seq_len == 0) is valid and launches nothing.
 *   - Diagnostics: with the environment variable PISA_LOG set to anything but 0
 *     when the library is first used, every kernel launch is described on
 *     stderr (kernel, its template arguments, grid, workgroup and problem) just
 *     before it is enqueued; nothing else changes.
 */
#ifndef PISA_H
#define PISA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pisa_status {
  PISA_OK = 0,
  PISA_ERR_NULL = 1,        /* a required pointer is NULL */
  PISA_ERR_SHAPE = 2,       /* sizes are inconsistent or out of range */
  PISA_ERR_UNSUPPORTED = 3, /* a valid request this version does not implement */
  PISA_ERR_WORKSPACE = 4,   /* workspace missing or too small */
  PISA_ERR_HIP = 5,         /* the HIP runtime reported an error at launch */
  PISA_ERR_ALIGN = 6        /* a pointer is not 16-byte aligned */
} pisa_status;

typedef enum pisa_dtype { PISA_F32 = 0, PISA_BF16 = 1 } pisa_dtype;

/* How a pyramid node summarises its keys ("Le pooling comme première
 * réduction" names pooling without fixing the operator): the mean (the method's
 * default reading) or, as a variant, the element-wise maximum. */
typedef enum pisa_pool { PISA_POOL_MEAN = 0, PISA_POOL_MAX = 1 } pisa_pool;

/* Problem description, passed by const pointer to every call.
 *   heads_q % heads_kv == 0; the G = heads_q / heads_kv query heads of one KV
 *     head share one selection (grouped-query attention).
 *   seq_len: N for prefill; the cache capacity for decode. Any N >= 0: a last
 *     partial block is allowed.
 *   head_dim: 64 or 128.  block_size: 32, 64 or 128 tokens.
 *   fanout: 2, 4, 8 or 16 children per pyramid node.
 *   levels: 1..8 and counts the leaf-block level. The top level may hold at most
 *     1024 nodes and top_k * fanout + fanout - 1 <= 1024.
 *   top_k: >= 0 key blocks kept per query block (the beam width at every level).
 *   sink_len: >= 0 tokens of the always-attended prefix [0, sink_len).
 *   causal: 1, or 0 for the bidirectional variant: every block outside the
 *     sink except the query block's own is a candidate, the descent scores
 *     every node holding a candidate, and the query block is attended whole.
 *     Selection and the forward attention take 0; decode and the backward pass
 *     return PISA_ERR_UNSUPPORTED for it.
 *   sm_scale: softmax scale; <= 0 selects 1/sqrt(head_dim).
 *   dtype: PISA_F32 or PISA_BF16 for Q, K, V and O.
 *   pool: PISA_POOL_MEAN or PISA_POOL_MAX (node summaries of the pyramid). */
typedef struct pisa_problem {
  int32_t batch;
  int32_t heads_q;
  int32_t heads_kv;
  int32_t head_dim;
  int64_t seq_len;
  int32_t block_size;
  int32_t fanout;
  int32_t levels;
  int32_t top_k;
  int32_t sink_len;
  int32_t causal;
  float sm_scale;
  int32_t dtype;
  int32_t pool;
} pisa_problem;

/* Node offsets of each pyramid level ("Une pyramide de clés"). Host only, pure.
 *   level_offsets: host array of levels + 1 entries; entry l is the first node of
 *   level l within one (batch, kv head) slab, the last entry is the node count
 *   per slab. Level 0 has ceil(seq_len / block_size) nodes, level l has
 *   ceil(nodes_{l-1} / fanout). */
pisa_status pisa_pyramid_layout(const pisa_problem* p, int64_t* level_offsets);

/* Build the key pyramid ("Le pooling comme première réduction").
 *   k: [batch, heads_kv, seq_len, head_dim] keys.
 *   pyramid: fp32 [batch, heads_kv, nodes, head_dim], written in full.
 * Level 0 node j = the mean of key rows [j*bs, min(N, (j+1)*bs)), summed in fp64
 * and rounded once to fp32; level l node n = the mean of its (up to fanout)
 * children's stored fp32 values, summed in fp64 and rounded once to fp32. */
pisa_status pisa_build_pyramid(const pisa_problem* p, const void* k, float* pyramid, hipStream_t stream);

/* Select the top-K key blocks of every query block ("La sélection top-K guidée
 * par la pyramide").
 *   q: [batch, heads_q, seq_len, head_dim]; pyramid: from pisa_build_pyramid.
 *   idx: int32 [batch, heads_kv, n_blocks, top_k], selected blocks in ascending
 *        order, padded with -1.  cnt: int32 [batch, heads_kv, n_blocks].
 * The query representative of block qb is the mean of its rows over the G heads
 * of the KV group (fp64). From the top level down, every node lying wholly
 * before qb's ancestor at that level and holding at least one block outside the
 * sink is scored by the fp64 dot product of the representative with its fp32
 * summary; the K best (score descending, index ascending) are kept, and the next
 * level's pool is their children plus the complete children of qb's ancestor.
 * Blocks wholly inside [0, sink_len) and the block qb itself are never
 * candidates. */
pisa_status pisa_select_topk(const pisa_problem* p, const void* q, const float* pyramid, int32_t* idx, int32_t* cnt,
                             hipStream_t stream);

/* Exact softmax attention over the attended set ("Des noyaux Triton qui ne
 * matérialisent rien"; sink prefix from Pulsar "Phase 1").
 *   q: [batch, heads_q, seq_len, head_dim]; k, v: [batch, heads_kv, seq_len, head_dim];
 *   idx, cnt: from pisa_select_topk; out: like q;
 *   lse: nullable fp32 [batch, heads_q, seq_len], natural-log sum of exp(logits).
 * Query i of block qb attends to the key set
 *   ([0, sink_len) U selected blocks of qb U [qb*bs, i]) intersected with [0, i],
 * each key once, with logits sm_scale * q_i . k_t. No score matrix is written.
 * bf16 problems use bf16 matrix cores with fp32 accumulation (probabilities are
 * rounded to bf16 before the value product); fp32 problems compute in fp32. */
pisa_status pisa_sparse_attn_fwd(const pisa_problem* p, const void* q, const void* k, const void* v, const int32_t* idx,
                                 const int32_t* cnt, void* out, float* lse, hipStream_t stream);

/* Selection and attention fused in one launch (the PISA page, "Des noyaux
 * Triton qui ne matérialisent rien": similarity, selection and aggregation in
 * one pass). Computes what pisa_select_topk followed by pisa_sparse_attn_fwd
 * computes, from the same arguments:
 *   q, k, v: as for pisa_sparse_attn_fwd; pyramid: from pisa_build_pyramid;
 *   idx, cnt: nullable outputs, the selection as pisa_select_topk writes it;
 *   out, lse: as for pisa_sparse_attn_fwd (lse nullable).
 * Each workgroup of the attention grid computes its query block's mean and
 * descends the pyramid itself before attending, so no selection passes through
 * HBM. Implemented for bf16 causal problems; other problems return
 * PISA_ERR_UNSUPPORTED. The query mean adds the block's rows in another order than
 * pisa_select_topk, so the selection equals pisa_select_topk's bit for bit when
 * each column's fp64 sum is exact -- always when a column of the query block's
 * values spans at most 35 binades -- and, given the selection, out and lse equal
 * pisa_sparse_attn_fwd's bit for bit. The two-launch path (pisa_select_topk, then
 * pisa_sparse_attn_fwd) is the faster one on MI355X; this entry point is kept for
 * callers that must not hold the selection in memory. */
pisa_status pisa_select_attend(const pisa_problem* p, const void* q, const void* k, const void* v,
                               const float* pyramid, int32_t* idx, int32_t* cnt, void* out, float* lse,
                               hipStream_t stream);

/* Device workspace (bytes) that pisa_sparse_attn_bwd needs for this problem. */
pisa_status pisa_sparse_attn_bwd_workspace_size(const pisa_problem* p, size_t* bytes);

/* Gradients of the sparse attention with the selection held constant (the PISA
 * page, "Attention clairsemée PISA : noyaux Triton sans matrice de scores",
 * presents its kernels for training as well as inference).
 *   q, k, v, idx, cnt: as given to pisa_sparse_attn_fwd (idx ascending and
 *            distinct within a row, as pisa_select_topk writes it);
 *   out, lse: that call's output and its lse (lse is required here);
 *   dout: gradient of the loss with respect to out, like q;
 *   dq: like q; dk, dv: like k, v -- all written, none accumulated into;
 *   workspace: device memory of at least pisa_sparse_attn_bwd_workspace_size
 *              bytes, 256-byte aligned.
 * For query i with attended keys A(i), p = exp(sm_scale q_i.k_t - lse_i),
 * dS = p (dout_i.v_t - dout_i.out_i); dq_i = sm_scale sum_t dS k_t,
 * dk_t = sm_scale sum_i dS q_i, dv_t = sum_i p dout_i (key and value gradients
 * sum over the query heads of the group). bf16 only: fp32 problems return
 * PISA_ERR_UNSUPPORTED. Results are deterministic (no atomics). */
pisa_status pisa_sparse_attn_bwd(const pisa_problem* p, const void* q, const void* k, const void* v, const int32_t* idx,
                                 const int32_t* cnt, const void* out, const float* lse, const void* dout, void* dq,
                                 void* dk, void* dv, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Device workspace (bytes) that pisa_decode_step needs for this problem. */
pisa_status pisa_decode_workspace_size(const pisa_problem* p, size_t* bytes);

/* One decode step: a single new query token per sequence whose key and value are
 * already in the cache at position cache_len - 1 (Pulsar "Phase 2": partial
 * attentions merged by an online softmax).
 *   q: [batch, heads_q, head_dim]; k_cache, v_cache: [batch, heads_kv, seq_len, head_dim];
 *   pyramid: built by pisa_build_pyramid over the cache (nodes past the token's
 *            own ancestors are never read, so a pyramid of the full capacity works);
 *   cache_len: 1..seq_len, the same for every sequence;
 *   out: [batch, heads_q, head_dim]; lse: nullable fp32 [batch, heads_q];
 *   idx_out: nullable int32 [batch, heads_kv, top_k]; cnt_out: nullable int32 [batch, heads_kv];
 *            when given, the selection is written there and the attention of
 *            the same call reads it back, so they must not overlap any other
 *            buffer of the call;
 *   workspace: device memory of at least pisa_decode_workspace_size bytes.
 * Selection and attended set are those of a one-row query block at position
 * cache_len - 1. The attended blocks are split across workgroups and the
 * partial results merged. */
pisa_status pisa_decode_step(const pisa_problem* p, const void* q, const void* k_cache, const void* v_cache,
                             const float* pyramid, int64_t cache_len, void* out, float* lse, int32_t* idx_out,
                             int32_t* cnt_out, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* One decode step for a batch whose sequences have different cache lengths
 * (each sequence's new token sits at its own cache_lens[b] - 1). Same selection,
 * attended set and split-K merge as pisa_decode_step, per sequence.
 *   cache_lens: device int32 [batch], read by the kernels (so it may be produced
 *               on the device, e.g. by the step that appended the tokens);
 *   all other arguments, the workspace size included, as for pisa_decode_step.
 * The host cannot check device lengths: a sequence whose length lies outside
 * [1, seq_len] attends nothing -- its output is zeros, its lse -inf and its
 * selected-block count 0 -- and the call still succeeds. */
pisa_status pisa_decode_step_ragged(const pisa_problem* p, const void* q, const void* k_cache, const void* v_cache,
                                    const float* pyramid, const int32_t* cache_lens, void* out, float* lse,
                                    int32_t* idx_out, int32_t* cnt_out, void* workspace, size_t workspace_bytes,
                                    hipStream_t stream);

/* A serving step in the launches of one decode: the pyramid append of each
 * sequence's new tokens and the ragged decode at the new lengths (the PISA page,
 * "Le pooling comme première réduction": only the nodes holding new keys change;
 * the Pulsar page, "Phase 2 : Encodage de la requête globale": the split partial
 * attentions merged). Computes, bit for bit, what pisa_pyramid_append(p, k_cache,
 * pyramid, old_lens, cache_lens) followed by pisa_decode_step_ragged(p, q, ...,
 * cache_lens, ...) compute, for any lengths:
 *   pyramid: as for pisa_pyramid_append (updated in place) and then read as for
 *            pisa_decode_step_ragged;
 *   old_lens: device int32 [batch], the lengths the pyramid is up to date for;
 *   cache_lens: device int32 [batch], the new lengths (tokens [old_lens[b],
 *               cache_lens[b]) already in the caches), at which the step decodes;
 *   all other arguments as for pisa_decode_step_ragged.
 * The workgroup that selects for a (batch, kv head) first appends its tokens,
 * then descends the updated pyramid, so the step takes the decode's three
 * launches instead of four. Lengths are handled as by the two calls: a sequence
 * whose append would be skipped is not appended, and one whose cache_lens[b]
 * lies outside [1, seq_len] attends nothing. */
pisa_status pisa_decode_step_ragged_append(const pisa_problem* p, const void* q, const void* k_cache,
                                           const void* v_cache, float* pyramid, const int32_t* old_lens,
                                           const int32_t* cache_lens, void* out, float* lse, int32_t* idx_out,
                                           int32_t* cnt_out, void* workspace, size_t workspace_bytes,
                                           hipStream_t stream);

/* Largest decode workspace the allocation-free entry point can serve: 16 MiB
 * (workload of 64 sequences x 8 KV heads x 4 query heads per KV head, d = 128,
 * K = 32 needs about 6.5 MiB). */
#define PISA_DECODE_SCRATCH_BYTES (16u << 20)

/* pisa_decode_step_ragged for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, kernels and results (bit for bit) as pisa_decode_step_ragged,
 * without the workspace pair: the workspace is a static device array of
 * PISA_DECODE_SCRATCH_BYTES owned by the library, one per GPU, held from the
 * first call on that GPU until the process ends. The call allocates nothing.
 *   Returns PISA_ERR_WORKSPACE (nothing launched) when the problem needs more
 *   than PISA_DECODE_SCRATCH_BYTES (pisa_decode_workspace_size tells the need).
 *   Every call on one GPU shares that GPU's array and overwrites it; nothing in
 *   it has to start at zero. Calls that overlap on one GPU (other streams, other
 *   host threads) race on it and must be serialised by the caller. */
pisa_status pisa_decode_step_ragged_noalloc(const pisa_problem* p, const void* q, const void* k_cache,
                                            const void* v_cache, const float* pyramid, const int32_t* cache_lens,
                                            void* out, float* lse, int32_t* idx_out, int32_t* cnt_out,
                                            hipStream_t stream);

/* Bring the pyramid up to date after tokens were appended to the key cache
 * ("Le pooling comme première réduction": a node summarises its keys, so only
 * the nodes holding new keys change).
 *   k_cache: [batch, heads_kv, seq_len, head_dim], tokens [old_lens[b], new_lens[b])
 *            of sequence b already written;
 *   pyramid: fp32 [batch, heads_kv, nodes, head_dim] in the pisa_pyramid_layout
 *            of seq_len (the capacity), up to date for the first old_lens[b] tokens;
 *   old_lens, new_lens: device int32 [batch].
 * Every node whose tokens meet [old_lens[b], new_lens[b]) is recomputed over its
 * tokens before new_lens[b]: afterwards each node holding tokens before
 * new_lens[b] equals, bit for bit, what pisa_build_pyramid gives for a cache of
 * exactly new_lens[b] tokens. Other nodes are not written. A sequence with
 * old_lens[b] < 0, new_lens[b] > seq_len or old_lens[b] >= new_lens[b] is left
 * as it is. One workgroup per (batch, kv head): meant for the few tokens a
 * decode step appends; a long prompt is faster through pisa_build_pyramid.
 * Ordering: a decode at length n reads only complete nodes (wholly before the
 * block of its token n - 1), and appending that token writes only incomplete
 * ones, so the append of a step's token may be issued before or after that
 * step's decode, on the same stream or beside it on another; the decode of the
 * next step must follow it. */
pisa_status pisa_pyramid_append(const pisa_problem* p, const void* k_cache, float* pyramid, const int32_t* old_lens,
                                const int32_t* new_lens, hipStream_t stream);

/* Static text for a status code. */
const char* pisa_status_string(pisa_status s);

/* Detail of the last failing call on this thread ("" if none). */
const char* pisa_last_error(void);

/* Library version as major * 10000 + minor * 100 + patch. */
int32_t pisa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PISA_H */
