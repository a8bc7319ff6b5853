"""Pins for the oracle's key pyramid (PISA page, "Une pyramide de clés" and
"Le pooling comme première réduction": each level pools the one below; the
pooling is the mean)."""

import math

import numpy as np
import pytest

import gen
from oracle import build_pyramid, level_sizes, query_block_means


def test_level_sizes():
    assert level_sizes(1024, 8, 4) == [1024, 128, 16, 2]
    assert level_sizes(8192, 8, 5) == [8192, 1024, 128, 16, 2]
    assert level_sizes(16, 4, 2) == [16, 4]
    assert level_sizes(13, 4, 3) == [13, 4, 1]  # partial last nodes are kept


def test_constant_keys_give_constant_summaries():
    k = np.full((1, 2, 96, 8), 0.375, np.float32)
    for lvl in build_pyramid(k, 16, 2, 3):
        assert np.all(lvl == np.float32(0.375))


def test_ramp_closed_form():
    # K[t, c] = t + c: a node covering tokens [a, b) has mean (a + b - 1) / 2 + c, exact in fp32.
    N, d, bs, f, L = 1024, 4, 16, 4, 4
    t = np.arange(N, dtype=np.float64)[:, None] + np.arange(d)[None, :]
    k = t.astype(np.float32)[None, None]
    pyr = build_pyramid(k, bs, f, L)
    for l, lvl in enumerate(pyr):
        w = bs * f ** l
        for n in range(lvl.shape[2]):
            expect = (n * w + (n + 1) * w - 1) / 2.0 + np.arange(d)
            assert np.array_equal(lvl[0, 0, n], expect.astype(np.float32)), (l, n)


def test_ragged_tail_closed_form():
    # N = 1000 is not a multiple of bs = 64: the last block holds 40 tokens and
    # the last level-1 node 3 full blocks + that partial one.
    N, bs, f = 1000, 64, 4
    k = np.arange(N, dtype=np.float32)[None, None, :, None].repeat(2, axis=3)
    pyr = build_pyramid(k, bs, f, 2)
    assert pyr[0].shape[2] == 16 and pyr[1].shape[2] == 4
    assert pyr[0][0, 0, 15, 0] == np.float32((960 + 999) / 2.0)
    children = pyr[0][0, 0, 12:16, 0].astype(np.float64)
    assert pyr[1][0, 0, 3, 0] == np.float32(children.mean())


def test_against_token_means_brute_force():
    rng = np.random.default_rng(7)
    k = rng.standard_normal((2, 3, 640, 16)).astype(np.float32)
    bs, f, L = 32, 4, 3
    pyr = build_pyramid(k, bs, f, L)
    bound = None
    for l, lvl in enumerate(pyr):
        w = bs * f ** l
        # one round-to-nearest per level: |fl(x) - x| <= 2^-24 |x|, plus the
        # children's own errors carried through their mean
        here = 2.0 ** -24 * np.abs(lvl.astype(np.float64))
        if bound is not None:
            nch = bound.shape[2]
            padded = np.concatenate([bound, np.zeros(bound.shape[:2] + (lvl.shape[2] * f - nch, bound.shape[3]))], 2)
            sums = padded.reshape(bound.shape[:2] + (lvl.shape[2], f, bound.shape[3])).sum(3)
            counts = np.array([min(f, nch - n * f) for n in range(lvl.shape[2])], float)
            here = here + sums / counts[:, None]
        bound = here
        for n in range(lvl.shape[2]):
            tok = k[:, :, n * w:min(640, (n + 1) * w)].astype(np.float64).mean(axis=2)
            err = np.abs(lvl[:, :, n].astype(np.float64) - tok)
            assert np.all(err <= bound[:, :, n] * (1 + 1e-9) + 1e-15), (l, n)


def test_each_level_is_the_rounded_mean_of_its_children():
    rng = np.random.default_rng(3)
    k = gen.round_to_bf16(rng.standard_normal((1, 2, 2048, 32)) / 8)
    pyr = build_pyramid(k, 64, 8, 3)
    for l in (1, 2):
        below = pyr[l - 1][0, 1].astype(np.float64)
        for n in range(pyr[l].shape[2]):
            ch = below[n * 8:(n + 1) * 8]
            exact = np.array([math.fsum(ch[:, c]) for c in range(ch.shape[1])]) / ch.shape[0]
            assert np.array_equal(pyr[l][0, 1, n], exact.astype(np.float32))


def test_block_sums_are_exact_on_generated_inputs():
    # The fp64 sum of a block's bf16 keys is exact here, so any summation order
    # (CPU or GPU) gives the same fp32 summary: compare with an exactly rounded sum.
    c = gen.workload(2)
    p = c["problem"].replace(heads_q=2, heads_kv=2, seq_len=4096)
    q, k, v, _ = gen.host_inputs(p, c["seed"], c["value_scale"], c["plant"])
    pyr = build_pyramid(k, p.block_size, p.fanout, p.levels)
    bs = p.block_size
    for h in range(2):
        for j in range(0, 64, 7):
            rows = k[0, h, j * bs:(j + 1) * bs].astype(np.float64)
            exact = np.array([math.fsum(rows[:, c_]) for c_ in range(rows.shape[1])]) / bs
            assert np.array_equal(pyr[0][0, h, j], exact.astype(np.float32))


def test_query_block_means_brute_force():
    rng = np.random.default_rng(11)
    q = rng.standard_normal((1, 4, 100, 3)).astype(np.float32)
    m = query_block_means(q, 2, 32)  # G = 2, last block has 4 rows
    assert m.shape == (1, 2, 4, 3)
    for g in range(2):
        for qb in range(4):
            rows = q[0, 2 * g:2 * g + 2, qb * 32:min(100, qb * 32 + 32)].astype(np.float64)
            acc = np.zeros(3)
            n = 0
            for h in range(rows.shape[0]):
                for r in range(rows.shape[1]):
                    acc += rows[h, r]
                    n += 1
            assert np.allclose(m[0, g, qb], acc / n, rtol=0, atol=1e-15)
