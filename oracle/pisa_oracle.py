"""Plain CPU oracle for PISA content-selected block-sparse attention.

TEST INFRASTRUCTURE. Only the tests, the package's smoke check and the
bench's CPU-baseline leg may import this module. The HIP library never calls
it and shares no code with it.

Everything is numpy, scores and softmax in fp64. The steps follow the PISA
page ("Attention clairsemée PISA : noyaux Triton sans matrice de scores"):

1. "Une pyramide de clés" / "Le pooling comme première réduction": keys are
   grouped into blocks, blocks into nodes of `fanout` blocks, and so on; each
   level summarises the level below by pooling. Pooling is the arithmetic
   mean. Summaries are stored as fp32: level 0 is the fp64 mean of the block's
   key rows rounded once; level l is the fp64 mean of its children's stored
   fp32 summaries, rounded once.
2. "La sélection top-K guidée par la pyramide": each query block scores the
   coarse summaries, keeps the best K nodes, and descends one level at a time
   into the children of what it kept, down to K key blocks.
3. "Des noyaux Triton qui ne matérialisent rien": exact softmax attention over
   the chosen keys only. The attended set also holds the attention-sink prefix
   (the Pulsar Attention page, "Phase 1 : Encodage statistique du contexte":
   a 64-token prefix by default) and the query's own block under a causal
   mask.
4. Decode is the same descent and attention for one new query token whose key
   and value are already in the cache (each sequence of a batch at its own
   cache length in `decode_ragged`). The online-softmax merge of partial
   results (Pulsar page, "Phase 2 : Encodage de la requête globale") is
   written out in `merge_partials`.

Readings where the pages are silent (each is also listed in the design notes):

* the query representative is the mean of the query block's rows over the
  heads that share one KV head; a node's score is the plain dot product of
  that mean with the node summary (no scale: it does not change the ranking);
* a node is a candidate only if it lies wholly before the query block's own
  ancestor at that level (complete and causal) and holds at least one block
  outside the sink; the ancestor itself is never scored, its complete
  children join the next level's pool;
* the beam keeps K nodes at every level (all of them when there are <= K);
* ties in score go to the lower index; selected blocks are emitted in
  ascending order, padded with -1;
* blocks lying wholly inside the sink are never candidates (they are always
  attended); the local block is never a candidate;
* the attended keys of query i in block qb form the set
  ([0, s) U selected blocks U [qb*bs, i]) intersected with [0, i]; a key in
  two of those ranges counts once.
"""

from __future__ import annotations

import math
from typing import List, Optional, Sequence

import numpy as np

__all__ = [
    "level_sizes",
    "build_pyramid",
    "query_block_means",
    "descend",
    "select",
    "selection_report",
    "attended_keys",
    "attend",
    "attend_block",
    "attend_backward",
    "decode",
    "decode_ragged",
    "merge_partials",
    "dense_causal_attention",
]


def level_sizes(n_blocks: int, fanout: int, levels: int) -> List[int]:
    """Nodes per level; level 0 holds the key blocks, a partial last node is kept."""
    sizes = [n_blocks]
    for _ in range(1, levels):
        sizes.append(-(-sizes[-1] // fanout))
    return sizes


# --------------------------------------------------------------------------
# 1. key pyramid


def _mean_groups(x: np.ndarray, group: int) -> np.ndarray:
    """Mean of consecutive groups of `group` rows along axis -2 (last group may be short), fp64."""
    n = x.shape[-2]
    ng = -(-n // group)
    pad = ng * group - n
    x64 = x.astype(np.float64)
    if pad:
        x64 = np.concatenate([x64, np.zeros(x64.shape[:-2] + (pad, x64.shape[-1]))], axis=-2)
    sums = x64.reshape(x64.shape[:-2] + (ng, group, x64.shape[-1])).sum(axis=-2)
    counts = np.full(ng, float(group))
    counts[-1] = n - (ng - 1) * group
    return sums / counts[:, None]


def _max_groups(x: np.ndarray, group: int) -> np.ndarray:
    """Element-wise max of consecutive groups of `group` rows along axis -2 (last group may be short)."""
    n = x.shape[-2]
    ng = -(-n // group)
    out = np.empty(x.shape[:-2] + (ng, x.shape[-1]), dtype=np.float64)
    for i in range(ng):
        out[..., i, :] = x[..., i * group:min(n, (i + 1) * group), :].astype(np.float64).max(axis=-2)
    return out


def build_pyramid(k: np.ndarray, block_size: int, fanout: int, levels: int, pool: str = "mean") -> List[np.ndarray]:
    """Key pyramid of a [B, H, N, d] key tensor: a list of fp32 arrays [B, H, nodes_l, d].

    pool "mean" (the default) summarises a node by the mean of its keys; "max"
    (a variant) by their element-wise maximum, which folds exactly level by level.
    """
    group = _mean_groups if pool == "mean" else _max_groups
    pyr = [group(k, block_size).astype(np.float32)]
    for _ in range(1, levels):
        pyr.append(group(pyr[-1], fanout).astype(np.float32))
    return pyr


# --------------------------------------------------------------------------
# 2. pyramid-guided top-K descent


def query_block_means(q: np.ndarray, heads_kv: int, block_size: int) -> np.ndarray:
    """Mean of each query block over its rows and the heads of its KV group: [B, Hkv, nb, d] fp64."""
    B, Hq, N, d = q.shape
    G = Hq // heads_kv
    per_head = _mean_groups(q, block_size)  # [B, Hq, nb, d]
    return per_head.reshape(B, heads_kv, G, -1, d).mean(axis=2)


def _top(nodes: Sequence[int], scores: np.ndarray, k: int) -> List[int]:
    """The k best nodes by (score descending, index ascending)."""
    order = sorted(range(len(nodes)), key=lambda i: (-scores[i], nodes[i]))
    return [nodes[i] for i in order[:k]]


def _descend_bidirectional(levels, qbar, qb, top_k, sink_len, block_size, fanout, trace):
    """Non-causal variant: the candidates are every block outside the sink except
    the query block itself; a node is scored if it holds a candidate, so the top
    level starts with all of them and each level expands the kept nodes only."""
    L = len(levels)
    nb = levels[0].shape[0]
    j0 = sink_len // block_size
    span = [fanout ** l for l in range(L)]

    def useful(n: int, l: int) -> bool:
        lo, hi = max(n * span[l], j0), min((n + 1) * span[l], nb)
        return hi - lo - (1 if lo <= qb < hi else 0) > 0

    pool = [n for n in range(levels[L - 1].shape[0]) if useful(n, L - 1)]
    for l in range(L - 1, -1, -1):
        scores = levels[l][pool].astype(np.float64) @ qbar if pool else np.zeros(0)
        kept = _top(pool, scores, top_k)
        if trace is not None:
            trace.append(dict(level=l, pool=list(pool), scores=scores, kept=list(kept)))
        if l == 0:
            return sorted(kept)
        below = levels[l - 1].shape[0]
        pool = sorted(c for n in kept for c in range(n * fanout, min((n + 1) * fanout, below)) if useful(c, l - 1))
    raise AssertionError("unreachable")


def descend(levels: Sequence[np.ndarray], qbar: np.ndarray, qb: int, top_k: int, sink_len: int,
            block_size: int, fanout: int, trace: Optional[list] = None, causal: bool = True) -> List[int]:
    """Selected key blocks (ascending) for query block `qb`.

    `levels[l]` is the [nodes_l, d] pyramid level of one (batch, KV head);
    `qbar` the fp64 query representative. If `trace` is a list, one dict per
    level (pool, scores, kept) is appended to it. causal=False: the
    bidirectional variant (`_descend_bidirectional`).
    """
    if not causal:
        return _descend_bidirectional(levels, qbar, qb, top_k, sink_len, block_size, fanout, trace)
    L = len(levels)
    j0 = sink_len // block_size  # blocks wholly inside the sink
    span = [fanout ** l for l in range(L)]  # blocks under one node of level l
    anc = [qb // s for s in span]  # ancestor of qb at each level

    def useful(n: int, l: int) -> bool:  # holds at least one block outside the sink
        return (n + 1) * span[l] > j0

    pool = [n for n in range(anc[L - 1]) if useful(n, L - 1)]
    for l in range(L - 1, -1, -1):
        scores = levels[l][pool].astype(np.float64) @ qbar if pool else np.zeros(0)
        kept = _top(pool, scores, top_k)
        if trace is not None:
            trace.append(dict(level=l, pool=list(pool), scores=scores, kept=list(kept)))
        if l == 0:
            return sorted(kept)
        nxt = [c for n in kept for c in range(n * fanout, (n + 1) * fanout)]
        nxt += list(range(anc[l] * fanout, anc[l - 1]))  # complete children of the ancestor
        pool = sorted(c for c in nxt if useful(c, l - 1))
    raise AssertionError("unreachable")


def selection_report(trace: list, top_k: int, fanout: int, targets: Sequence[int] = ()) -> dict:
    """Self-report of one descent, from its `trace` (see `descend`).

    gaps: for every level whose pool held more than `top_k` nodes, the margin
      between the K-th and (K+1)-th best scores, i.e. how far the keep/prune
      boundary was from a tie (0.0 for a tie broken by index);
    pruned: for every target block, the level at which its ancestor was scored
      and not kept, or None when that never happened (the block was selected, or
      never scored).
    """
    gaps = {}
    for t in trace:
        if len(t["pool"]) > top_k:
            order = sorted(range(len(t["pool"])), key=lambda i: (-t["scores"][i], t["pool"][i]))
            gaps[t["level"]] = float(t["scores"][order[top_k - 1]] - t["scores"][order[top_k]])
    pruned = {}
    for j in targets:
        pruned[j] = None
        for t in trace:
            a = j // fanout ** t["level"]
            if a in t["pool"] and a not in t["kept"]:
                pruned[j] = t["level"]
                break
    return dict(gaps=gaps, pruned=pruned)


def select(pyramid: Sequence[np.ndarray], qbar: np.ndarray, top_k: int, sink_len: int, block_size: int,
           fanout: int, traces: Optional[dict] = None, causal: bool = True):
    """Selection for every (batch, KV head, query block).

    Returns idx int32 [B, Hkv, nb, K] (ascending, -1 padded) and cnt int32 [B, Hkv, nb].
    """
    B, Hkv, nb, _ = qbar.shape
    idx = np.full((B, Hkv, nb, top_k), -1, np.int32)
    cnt = np.zeros((B, Hkv, nb), np.int32)
    for b in range(B):
        for g in range(Hkv):
            lv = [p[b, g] for p in pyramid]
            for qb in range(nb):
                tr = [] if traces is not None else None
                sel = descend(lv, qbar[b, g, qb], qb, top_k, sink_len, block_size, fanout, tr, causal)
                cnt[b, g, qb] = len(sel)
                idx[b, g, qb, :len(sel)] = sel
                if traces is not None:
                    traces[(b, g, qb)] = tr
    return idx, cnt


# --------------------------------------------------------------------------
# 3. exact attention over the attended set


def attended_keys(i: int, sel: Sequence[int], sink_len: int, block_size: int, causal: bool = True,
                  n: Optional[int] = None) -> np.ndarray:
    """Sorted key positions attended by the query at absolute position i.

    Causal: ([0, sink) U selected blocks U [qb*bs, i]) intersected with [0, i].
    Non-causal (sequence length n): [0, sink) U selected blocks U the whole block
    qb, intersected with [0, n).
    """
    qb = i // block_size
    if causal:
        keys = set(range(min(sink_len, i + 1)))
        for j in sel:
            keys.update(range(j * block_size, (j + 1) * block_size))
        keys.update(range(qb * block_size, i + 1))
        return np.array(sorted(t for t in keys if t <= i), dtype=np.int64)
    keys = set(range(min(sink_len, n)))
    for j in sel:
        keys.update(range(j * block_size, min(n, (j + 1) * block_size)))
    keys.update(range(qb * block_size, min(n, (qb + 1) * block_size)))
    return np.array(sorted(keys), dtype=np.int64)


def _softmax_rows(s: np.ndarray):
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    z = e.sum(axis=-1, keepdims=True)
    return e / z, (m + np.log(z))[..., 0]


def attend_block(q_rows: np.ndarray, k: np.ndarray, v: np.ndarray, row0: int, sel: Sequence[int],
                 sink_len: int, block_size: int, sm_scale: float, causal: bool = True):
    """Attention for consecutive query rows q_rows[r] at positions row0 + r (all in one block).

    k, v: [N, d] of the query's KV head. Returns (o fp64 [R, d], lse fp64 [R]).
    """
    R = q_rows.shape[0]
    last = row0 + R - 1
    keys = attended_keys(last, sel, sink_len, block_size, causal, k.shape[0])  # superset for every row
    s = sm_scale * (q_rows.astype(np.float64) @ k[keys].astype(np.float64).T)
    if causal:
        pos = row0 + np.arange(R)[:, None]
        s = np.where(keys[None, :] <= pos, s, -np.inf)  # key position <= query position
    w, lse = _softmax_rows(s)
    return w @ v[keys].astype(np.float64), lse


def attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, idx: np.ndarray, cnt: np.ndarray, sink_len: int,
           block_size: int, sm_scale: float, blocks: Optional[Sequence] = None, causal: bool = True):
    """Sparse attention output o [B, Hq, N, d] fp64 and lse [B, Hq, N].

    `blocks`, if given, is a list of (b, g, qb) units to compute; other rows stay NaN.
    """
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    nb = -(-N // block_size)
    o = np.full((B, Hq, N, d), np.nan)
    lse = np.full((B, Hq, N), np.nan)
    units = blocks if blocks is not None else [(b, g, qb) for b in range(B) for g in range(Hkv) for qb in range(nb)]
    for (b, g, qb) in units:
        sel = idx[b, g, qb, :cnt[b, g, qb]].tolist()
        r0, r1 = qb * block_size, min(N, (qb + 1) * block_size)
        for h in range(g * G, (g + 1) * G):
            o[b, h, r0:r1], lse[b, h, r0:r1] = attend_block(q[b, h, r0:r1], k[b, g], v[b, g], r0, sel,
                                                             sink_len, block_size, sm_scale, causal)
    return o, lse


def attend_backward(q: np.ndarray, k: np.ndarray, v: np.ndarray, idx: np.ndarray, cnt: np.ndarray,
                    dout: np.ndarray, sink_len: int, block_size: int, sm_scale: float,
                    units: Optional[Sequence] = None):
    """Gradients of L = sum(dout * o) for o = attend(q, k, v, idx, cnt), the selection held constant.

    `units`, if given, is a list of (b, g, qb) query-block units whose terms are
    summed (dq rows of other units stay 0; dk and dv then hold only these units'
    contributions -- exact for a key block when every unit attending it is listed).

    Per query row i with attended keys A(i): s_t = sm_scale q_i.k_t, p = softmax_A(i)(s),
    o_i = sum_t p_t v_t. Then dv_t += p_t dout_i, dp_t = dout_i.v_t,
    ds_t = p_t (dp_t - sum_u p_u dp_u), dq_i = sm_scale sum_t ds_t k_t and
    dk_t += sm_scale ds_t q_i; key and value gradients of a KV head sum over the
    query heads that share it. Returns dq, dk, dv (fp64, shapes of q, k, v).
    """
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    nb = -(-N // block_size)
    dq = np.zeros((B, Hq, N, d))
    dk = np.zeros((B, Hkv, N, d))
    dv = np.zeros((B, Hkv, N, d))
    todo = units if units is not None else [(b, g, qb) for b in range(B) for g in range(Hkv) for qb in range(nb)]
    for (b, g, qb) in todo:
        sel = idx[b, g, qb, :cnt[b, g, qb]].tolist()
        r0, r1 = qb * block_size, min(N, (qb + 1) * block_size)
        keys = attended_keys(r1 - 1, sel, sink_len, block_size)
        kk, vv = k[b, g, keys].astype(np.float64), v[b, g, keys].astype(np.float64)
        pos = np.arange(r0, r1)[:, None]
        for h in range(g * G, (g + 1) * G):
            qq = q[b, h, r0:r1].astype(np.float64)
            do = dout[b, h, r0:r1].astype(np.float64)
            s = sm_scale * (qq @ kk.T)
            s = np.where(keys[None, :] <= pos, s, -np.inf)
            p, _ = _softmax_rows(s)
            dp = do @ vv.T
            ds = p * (dp - np.sum(p * dp, axis=1, keepdims=True))
            dq[b, h, r0:r1] = sm_scale * (ds @ kk)
            np.add.at(dk[b, g], keys, sm_scale * (ds.T @ qq))
            np.add.at(dv[b, g], keys, p.T @ do)
    return dq, dk, dv


# --------------------------------------------------------------------------
# 4. decode: one new query token per sequence


def decode(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray, pyramid: Sequence[np.ndarray],
           cache_len: int, top_k: int, sink_len: int, block_size: int, fanout: int, sm_scale: float,
           batches: Optional[Sequence[int]] = None):
    """One decode step.

    q [B, Hq, d]; caches [B, Hkv, cap, d]; the new token sits at cache_len - 1.
    Returns o [B, Hq, d] fp64, lse [B, Hq], idx int32 [B, Hkv, K], cnt int32 [B, Hkv].
    """
    B, Hq, d = q.shape
    Hkv = k_cache.shape[1]
    G = Hq // Hkv
    i = cache_len - 1
    qb = i // block_size
    o = np.full((B, Hq, d), np.nan)
    lse = np.full((B, Hq), np.nan)
    idx = np.full((B, Hkv, top_k), -1, np.int32)
    cnt = np.zeros((B, Hkv), np.int32)
    for b in (batches if batches is not None else range(B)):
        for g in range(Hkv):
            qbar = q[b, g * G:(g + 1) * G].astype(np.float64).mean(axis=0)
            sel = descend([p[b, g] for p in pyramid], qbar, qb, top_k, sink_len, block_size, fanout)
            cnt[b, g] = len(sel)
            idx[b, g, :len(sel)] = sel
            keys = attended_keys(i, sel, sink_len, block_size)
            kk = k_cache[b, g, keys].astype(np.float64)
            vv = v_cache[b, g, keys].astype(np.float64)
            for h in range(g * G, (g + 1) * G):
                w, l = _softmax_rows(sm_scale * (q[b, h].astype(np.float64) @ kk.T)[None, :])
                o[b, h] = (w @ vv)[0]
                lse[b, h] = l[0]
    return o, lse, idx, cnt


def decode_ragged(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray, pyramid: Sequence[np.ndarray],
                  cache_lens: Sequence[int], top_k: int, sink_len: int, block_size: int, fanout: int,
                  sm_scale: float, batches: Optional[Sequence[int]] = None):
    """One decode step where sequence b's cache holds cache_lens[b] tokens, its new token last.

    Each sequence is the single-sequence decode at its own length. A length
    outside [1, capacity] attends nothing: output 0, lse -inf, no blocks (the
    empty-sum reading of the softmax). Returns o, lse, idx, cnt like `decode`.
    """
    B, Hq, d = q.shape
    cap = k_cache.shape[2]
    o = np.full((B, Hq, d), np.nan)
    lse = np.full((B, Hq), np.nan)
    idx = np.full((B, k_cache.shape[1], top_k), -1, np.int32)
    cnt = np.zeros((B, k_cache.shape[1]), np.int32)
    for b in (batches if batches is not None else range(B)):
        n = int(cache_lens[b])
        if not 1 <= n <= cap:
            o[b] = 0.0
            lse[b] = -np.inf
            continue
        ob, lb, ib, cb = decode(q[b:b + 1], k_cache[b:b + 1], v_cache[b:b + 1], [lv[b:b + 1] for lv in pyramid], n,
                                top_k, sink_len, block_size, fanout, sm_scale)
        o[b], lse[b], idx[b], cnt[b] = ob[0], lb[0], ib[0], cb[0]
    return o, lse, idx, cnt


def merge_partials(parts):
    """Online-softmax merge of partial attentions over disjoint key sets.

    Each part is (m, l, o): the max logit, the sum of exp(logit - m) and the
    normalised output over that part. Returns the merged (m, l, o).
    """
    m = max(p[0] for p in parts)
    ls = [p[1] * math.exp(p[0] - m) for p in parts]
    l = sum(ls)
    o = sum(w * np.asarray(p[2], dtype=np.float64) for w, p in zip(ls, parts)) / l
    return m, l, o


# --------------------------------------------------------------------------
# dense reference (the definition on the linear-attention explainer page,
# "Le Problème du Coût Quadratique de l'Attention Classique", with a causal mask)


def dense_causal_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, sm_scale: float):
    """Dense causal softmax attention for small inputs: o [B, Hq, N, d] fp64, lse [B, Hq, N]."""
    B, Hq, N, d = q.shape
    G = Hq // k.shape[1]
    o = np.empty((B, Hq, N, d))
    lse = np.empty((B, Hq, N))
    mask = np.tril(np.ones((N, N), dtype=bool))
    for b in range(B):
        for h in range(Hq):
            s = sm_scale * (q[b, h].astype(np.float64) @ k[b, h // G].astype(np.float64).T)
            s = np.where(mask, s, -np.inf)
            w, lse[b, h] = _softmax_rows(s)
            o[b, h] = w @ v[b, h // G].astype(np.float64)
    return o, lse
