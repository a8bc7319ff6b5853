"""Pins for the oracle's exact attention over the attended set and its decode step.

The attended-set rule comes from the PISA page ("Des noyaux Triton qui ne
matérialisent rien": similarity, selection and aggregation without writing the
score matrix) plus the Pulsar page's attention-sink prefix ("Phase 1"); the
dense definition from the linear-attention explainer ("Le Problème du Coût
Quadratique de l'Attention Classique"); the merge from the Pulsar page's
"Phase 2" online-softmax fusion.
"""

import math

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

import gen
from oracle import (attend, attended_keys, build_pyramid, decode, decode_ragged, dense_causal_attention,
                    merge_partials, query_block_means, select)


def _sdpa(q, k, v, mask, scale):
    """torch's CPU SDPA in fp64 with a boolean mask [B or 1, H or 1, N, N]; GQA heads expanded."""
    G = q.shape[1] // k.shape[1]
    kt = torch.from_numpy(np.repeat(k.astype(np.float64), G, axis=1))
    vt = torch.from_numpy(np.repeat(v.astype(np.float64), G, axis=1))
    qt = torch.from_numpy(q.astype(np.float64))
    m = None if mask is None else torch.from_numpy(mask)
    out = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, is_causal=mask is None,
                                                           scale=scale)
    return out.numpy()


def _case(seed, B, Hq, Hkv, N, d):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, N, d)).astype(np.float32)
    k = rng.standard_normal((B, Hkv, N, d)).astype(np.float32)
    v = rng.standard_normal((B, Hkv, N, d)).astype(np.float32)
    return q, k, v


def _mask_from_sets(N, bs, sink, idx, cnt):
    """Boolean [B, Hkv, N, N] mask of attended keys built from the set rule, for torch."""
    B, Hkv = cnt.shape[:2]
    m = np.zeros((B, Hkv, N, N), dtype=bool)
    for b in range(B):
        for g in range(Hkv):
            for i in range(N):
                sel = idx[b, g, i // bs, :cnt[b, g, i // bs]].tolist()
                m[b, g, i, attended_keys(i, sel, sink, bs)] = True
    return m


@pytest.mark.parametrize("sink", [0, 16, 40])
def test_all_blocks_selected_is_dense_causal_attention(sink):
    B, Hq, Hkv, N, d, bs, f, L = 2, 4, 2, 256, 16, 16, 2, 3
    q, k, v = _case(1, B, Hq, Hkv, N, d)
    pyr = build_pyramid(k, bs, f, L)
    idx, cnt = select(pyr, query_block_means(q, Hkv, bs), N // bs, sink, bs, f)
    scale = 1 / math.sqrt(d)
    o, lse = attend(q, k, v, idx, cnt, sink, bs, scale)
    ref = _sdpa(q, k, v, None, scale)
    assert np.max(np.abs(o - ref)) < 1e-12
    od, lsed = dense_causal_attention(q, k, v, scale)
    assert np.max(np.abs(o - od)) < 1e-12 and np.max(np.abs(lse - lsed)) < 1e-12


@pytest.mark.parametrize("K,sink,N", [(2, 16, 320), (0, 24, 256), (3, 0, 250), (1, 64, 300)])
def test_fixed_selection_is_masked_sdpa(K, sink, N):
    # N = 250, 300 leave a ragged last block
    B, Hq, Hkv, d, bs, f, L = 1, 6, 2, 8, 32, 2, 3
    q, k, v = _case(K + N, B, Hq, Hkv, N, d)
    pyr = build_pyramid(k, bs, f, L)
    idx, cnt = select(pyr, query_block_means(q, Hkv, bs), K, sink, bs, f)
    scale = 0.3
    o, lse = attend(q, k, v, idx, cnt, sink, bs, scale)
    mask = np.repeat(_mask_from_sets(N, bs, sink, idx, cnt), Hq // Hkv, axis=1)
    ref = _sdpa(q, k, v, mask, scale)
    assert np.max(np.abs(o - ref)) < 1e-12
    # lse against an independent log-sum-exp over the masked logits
    G = Hq // Hkv
    for h in range(Hq):
        s = scale * (q[0, h].astype(np.float64) @ k[0, h // G].astype(np.float64).T)
        s = np.where(mask[0, h], s, -np.inf)
        assert np.max(np.abs(lse[0, h] - logsumexp(s, axis=1))) < 1e-12


def test_zero_k_is_sink_plus_local_window():
    B, Hq, Hkv, N, d, bs, f, L, sink = 1, 2, 1, 192, 8, 32, 2, 2, 20
    q, k, v = _case(3, B, Hq, Hkv, N, d)
    pyr = build_pyramid(k, bs, f, L)
    idx, cnt = select(pyr, query_block_means(q, Hkv, bs), 0, sink, bs, f)
    assert np.all(cnt == 0)
    o, _ = attend(q, k, v, idx, cnt, sink, bs, 0.25)
    i = np.arange(N)[:, None]
    t = np.arange(N)[None, :]
    mask = ((t < sink) | (t >= (i // bs) * bs)) & (t <= i)
    ref = _sdpa(q, k, v, mask[None, None].repeat(Hq, 1), 0.25)
    assert np.max(np.abs(o - ref)) < 1e-12


def test_outputs_are_convex_combinations_of_attended_values():
    c = gen.workload(1)
    p = c["problem"]
    q, k, v, _ = gen.host_inputs(p, c["seed"], c["value_scale"], c["plant"])
    pyr = build_pyramid(k, p.block_size, p.fanout, p.levels)
    idx, cnt = select(pyr, query_block_means(q, 1, p.block_size), p.top_k, p.sink_len, p.block_size, p.fanout)
    o, _ = attend(q, k, v, idx, cnt, p.sink_len, p.block_size, p.scale)
    assert np.array_equal(o[0, 0, 0], v[0, 0, 0].astype(np.float64))  # row 0 sees only key 0
    for i in range(0, p.seq_len, 37):
        qb = i // p.block_size
        keys = attended_keys(i, idx[0, 0, qb, :cnt[0, 0, qb]].tolist(), p.sink_len, p.block_size)
        vv = v[0, 0, keys].astype(np.float64)
        assert np.all(o[0, 0, i] >= vv.min(0) - 1e-12) and np.all(o[0, 0, i] <= vv.max(0) + 1e-12)


def test_attended_keys_are_a_set():
    # sink overlaps selected block 0 and the local block: each key once
    assert attended_keys(70, [0], 100, 64).tolist() == list(range(0, 71))
    assert attended_keys(5, [], 64, 64).tolist() == list(range(6))
    assert attended_keys(130, [0], 16, 64).tolist() == list(range(64)) + list(range(128, 131))
    assert attended_keys(130, [], 16, 64).tolist() == list(range(16)) + list(range(128, 131))


def test_merge_partials_recovers_one_softmax():
    rng = np.random.default_rng(5)
    s = rng.standard_normal(300) * 3
    vals = rng.standard_normal((300, 4))
    w = np.exp(s - s.max())
    direct = (w / w.sum()) @ vals
    for nparts in (1, 2, 7):
        cuts = np.sort(rng.choice(np.arange(1, 300), nparts - 1, replace=False))
        parts = []
        for seg in np.split(np.arange(300), cuts):
            m = s[seg].max()
            e = np.exp(s[seg] - m)
            parts.append((m, e.sum(), (e / e.sum()) @ vals[seg]))
        m, l, o = merge_partials(parts)
        assert np.max(np.abs(o - direct)) < 1e-13
        assert abs(m + math.log(l) - logsumexp(s)) < 1e-12


@pytest.mark.parametrize("cache_len", [256, 250, 33, 1])
def test_decode_all_blocks_is_last_row_of_dense(cache_len):
    B, Hq, Hkv, cap, d, bs, f, L, sink = 2, 4, 2, 256, 16, 32, 2, 3, 16
    rng = np.random.default_rng(cache_len)
    qfull = rng.standard_normal((B, Hq, cap, d)).astype(np.float32)
    k = rng.standard_normal((B, Hkv, cap, d)).astype(np.float32)
    v = rng.standard_normal((B, Hkv, cap, d)).astype(np.float32)
    pyr = build_pyramid(k, bs, f, L)
    qtok = qfull[:, :, cache_len - 1]
    o, lse, idx, cnt = decode(qtok, k, v, pyr, cache_len, cap // bs, sink, bs, f, 0.25)
    od, lsed = dense_causal_attention(qfull[:, :, :cache_len], k[:, :, :cache_len], v[:, :, :cache_len], 0.25)
    assert np.max(np.abs(o - od[:, :, -1])) < 1e-12
    assert np.max(np.abs(lse - lsed[:, :, -1])) < 1e-12


def test_decode_selection_matches_prefill_rule_for_single_row_block():
    # One query row per block: the decode descent is the prefill descent of a block
    # whose representative is the mean of that row over the group's heads.
    B, Hq, Hkv, cap, d, bs, f, L, K, sink = 1, 4, 2, 1024, 8, 16, 4, 3, 3, 16
    _, k, v = _case(9, B, Hkv, Hkv, cap, d)
    q = np.random.default_rng(10).standard_normal((B, Hq, d)).astype(np.float32)
    pyr = build_pyramid(k, bs, f, L)
    for cache_len in (1024, 700, 17):
        _, _, idx, cnt = decode(q, k, v, pyr, cache_len, K, sink, bs, f, 0.3)
        qb = (cache_len - 1) // bs
        qfake = np.zeros((B, Hq, cap, d), np.float32)
        qfake[:, :, qb * bs] = q  # a block whose only non-zero row is the token...
        qbar = query_block_means(qfake, Hkv, bs) * bs  # ...scaled back to the row mean
        sidx, scnt = select(pyr, qbar, K, sink, bs, f)
        assert np.array_equal(idx, sidx[:, :, qb]) and np.array_equal(cnt, scnt[:, :, qb])


def test_ragged_decode_all_blocks_is_each_sequence_s_dense_last_row():
    # every sequence at its own length: with K covering every block, row b is the
    # last row of dense causal attention over that sequence's first len_b tokens
    B, Hq, Hkv, cap, d, bs, f, L, sink = 4, 4, 2, 256, 16, 32, 2, 3, 16
    lens = [256, 1, 97, 33]
    rng = np.random.default_rng(21)
    qfull = rng.standard_normal((B, Hq, cap, d)).astype(np.float32)
    k = rng.standard_normal((B, Hkv, cap, d)).astype(np.float32)
    v = rng.standard_normal((B, Hkv, cap, d)).astype(np.float32)
    pyr = build_pyramid(k, bs, f, L)
    qtok = np.stack([qfull[b, :, lens[b] - 1] for b in range(B)])
    o, lse, idx, cnt = decode_ragged(qtok, k, v, pyr, lens, cap // bs, sink, bs, f, 0.25)
    for b, n in enumerate(lens):
        od, lsed = dense_causal_attention(qfull[b:b + 1, :, :n], k[b:b + 1, :, :n], v[b:b + 1, :, :n], 0.25)
        assert np.max(np.abs(o[b] - od[0, :, -1])) < 1e-12
        assert np.max(np.abs(lse[b] - lsed[0, :, -1])) < 1e-12
        assert np.all(cnt[b] == max(0, (n - 1) // bs - sink // bs))  # every earlier block outside the sink


def test_ragged_decode_out_of_range_lengths_attend_nothing():
    B, Hq, Hkv, cap, d = 3, 2, 1, 64, 8
    rng = np.random.default_rng(5)
    q = rng.standard_normal((B, Hq, d)).astype(np.float32)
    k = rng.standard_normal((B, Hkv, cap, d)).astype(np.float32)
    pyr = build_pyramid(k, 16, 2, 2)
    o, lse, idx, cnt = decode_ragged(q, k, k, pyr, [0, 65, -3], 2, 0, 16, 2, 0.5)
    assert np.all(o == 0.0) and np.all(lse == -np.inf) and np.all(cnt == 0) and np.all(idx == -1)
