"""Pins for the oracle's variants: max-pooled node summaries and non-causal
(bidirectional) selection and attention."""

import numpy as np
import pytest
import torch

from oracle import attend, attended_keys, build_pyramid, descend, level_sizes, query_block_means, select


def test_max_pyramid_closed_forms_and_brute_force():
    # constant keys: every summary is the constant; a ramp: a node's maximum is
    # its last existing row; in general, the element-wise max over the node's tokens
    N, d, bs, f, L = 1000, 3, 32, 4, 3
    const = np.full((1, 1, N, d), 0.25, np.float32)
    for lv in build_pyramid(const, bs, f, L, pool="max"):
        assert np.all(lv == np.float32(0.25))
    ramp = np.tile(np.arange(N, dtype=np.float32)[:, None], (1, d))[None, None]
    sizes = level_sizes(-(-N // bs), f, L)
    for l, lv in enumerate(build_pyramid(ramp, bs, f, L, pool="max")):
        span = bs * f ** l
        want = [min(N, (n + 1) * span) - 1 for n in range(sizes[l])]
        assert lv[0, 0, :, 0].tolist() == want
    rng = np.random.default_rng(3)
    k = rng.standard_normal((2, 2, N, d)).astype(np.float32)
    pyr = build_pyramid(k, bs, f, L, pool="max")
    for l in range(L):
        span = bs * f ** l
        for n in range(sizes[l]):
            assert np.array_equal(pyr[l][:, :, n], k[:, :, n * span:min(N, (n + 1) * span)].max(axis=2))


def _candidates(nb, qb, j0):
    return [j for j in range(j0, nb) if j != qb]


def test_bidirectional_k_at_least_all_blocks_selects_every_candidate():
    nb, bs, f, L = 40, 8, 4, 3
    rng = np.random.default_rng(4)
    k = rng.standard_normal((1, 1, nb * bs, 5)).astype(np.float32)
    lv = [p[0, 0] for p in build_pyramid(k, bs, f, L)]
    for qb in (0, 17, 39):
        for sink in (0, 8, 20):
            sel = descend(lv, rng.standard_normal(5), qb, nb, sink, bs, f, causal=False)
            assert sel == _candidates(nb, qb, sink // bs)


def test_bidirectional_equals_brute_force_when_the_top_level_fits_the_beam():
    # top level of 4 nodes, K = 4: nothing is pruned above the leaves, so the
    # descent is the exhaustive top-K over every candidate block
    nb, bs, f, L, K = 16, 16, 4, 2, 4
    rng = np.random.default_rng(6)
    q = rng.standard_normal((1, 1, nb * bs, 8)).astype(np.float32)
    k = rng.standard_normal((1, 1, nb * bs, 8)).astype(np.float32)
    pyr = build_pyramid(k, bs, f, L)
    qbar = query_block_means(q, 1, bs)
    for sink in (0, 16, 40):
        idx, cnt = select(pyr, qbar, K, sink, bs, f, causal=False)
        for qb in range(nb):
            cand = _candidates(nb, qb, sink // bs)
            sc = {j: float(pyr[0][0, 0, j].astype(np.float64) @ qbar[0, 0, qb]) for j in cand}
            best = sorted(sorted(cand, key=lambda j: (-sc[j], j))[:K])
            assert idx[0, 0, qb, :cnt[0, 0, qb]].tolist() == best


def _sdpa(q, k, v, mask, scale):
    G = q.shape[1] // k.shape[1]
    m = None if mask is None else torch.from_numpy(np.repeat(mask, G, axis=1))
    return torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q.astype(np.float64)), torch.from_numpy(np.repeat(k.astype(np.float64), G, axis=1)),
        torch.from_numpy(np.repeat(v.astype(np.float64), G, axis=1)), attn_mask=m, scale=scale).numpy()


@pytest.mark.parametrize("sink", [0, 12])
def test_non_causal_all_blocks_is_dense_bidirectional_attention(sink):
    B, Hq, Hkv, N, d, bs = 1, 4, 2, 75, 8, 16
    rng = np.random.default_rng(8)
    q, k, v = (rng.standard_normal((B, h, N, d)).astype(np.float32) for h in (Hq, Hkv, Hkv))
    pyr = build_pyramid(k, bs, 2, 3)
    idx, cnt = select(pyr, query_block_means(q, Hkv, bs), 8, sink, bs, 2, causal=False)
    o, _ = attend(q, k, v, idx, cnt, sink, bs, 0.4, causal=False)
    assert np.max(np.abs(o - _sdpa(q, k, v, None, 0.4))) < 1e-12


def test_non_causal_fixed_selection_is_masked_sdpa():
    B, Hq, Hkv, N, d, bs, sink = 2, 2, 1, 90, 8, 16, 10
    rng = np.random.default_rng(9)
    q, k, v = (rng.standard_normal((B, h, N, d)).astype(np.float32) for h in (Hq, Hkv, Hkv))
    pyr = build_pyramid(k, bs, 2, 3, pool="max")
    idx, cnt = select(pyr, query_block_means(q, Hkv, bs), 2, sink, bs, 2, causal=False)
    mask = np.zeros((B, Hkv, N, N), bool)
    for b in range(B):
        for i in range(N):
            sel = idx[b, 0, i // bs, :cnt[b, 0, i // bs]].tolist()
            mask[b, 0, i, attended_keys(i, sel, sink, bs, causal=False, n=N)] = True
    o, _ = attend(q, k, v, idx, cnt, sink, bs, 0.6, causal=False)
    assert np.max(np.abs(o - _sdpa(q, k, v, mask, 0.6))) < 1e-12
