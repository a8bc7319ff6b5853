"""Pins for the oracle's pyramid-guided top-K descent (PISA page, "La
sélection top-K guidée par la pyramide")."""

import numpy as np
import pytest

import gen
from oracle import build_pyramid, descend, query_block_means, select, selection_report


def _blocks_keys(means, bs):
    """d = 1 keys whose block j holds the constant means[j]."""
    return np.repeat(np.asarray(means, np.float32), bs)[None, None, :, None]


def _brute_force(levels0, qbar, qb, top_k, j0):
    cand = list(range(j0, qb))
    scores = [float(levels0[j].astype(np.float64) @ qbar) for j in cand]
    order = sorted(range(len(cand)), key=lambda i: (-scores[i], cand[i]))
    return sorted(cand[i] for i in order[:top_k])


def test_hand_worked_descent():
    # 8 blocks of 2 tokens, d = 1, fanout 2, 3 levels, K = 2, query block 7, q̄ = +1.
    # Block means 5 1 2 9 3 3 0 (block 7 is the local block).
    # level 2: ancestor of 7 is node 1, pool {node 0}.
    # level 1: pool = children of node 0 {0, 1} + ancestor child {2}; means 3, 5.5, 3;
    #          keep node 1 (5.5) and, on the tie at 3, node 0 (lower index).
    # level 0: pool {0, 1, 2, 3} + ancestor child {6}; best two are 9 (block 3), 5 (block 0).
    k = _blocks_keys([5, 1, 2, 9, 3, 3, 0, 7], 2)
    lv = [p[0, 0] for p in build_pyramid(k, 2, 2, 3)]
    tr = []
    assert descend(lv, np.array([1.0]), 7, 2, 0, 2, 2, tr) == [0, 3]
    assert [t["pool"] for t in tr] == [[0], [0, 1, 2], [0, 1, 2, 3, 6]]
    assert tr[1]["kept"] == [1, 0]
    # with a 2-token sink, block 0 is always attended and never a candidate
    assert descend(lv, np.array([1.0]), 7, 2, 2, 2, 2) == [2, 3]
    # a negative query mean reverses the ranking: level 1 keeps nodes 0 and 2
    # (tie at -3 goes to the lower index), level 0 pool {0, 1, 4, 5, 6}
    assert descend(lv, np.array([-1.0]), 7, 2, 0, 2, 2) == [1, 6]


def test_hand_worked_pruning_differs_from_brute_force():
    # Block 4 = 8 is the second best block, but its node (blocks 4, 5; mean -1) is pruned.
    k = _blocks_keys([5, 1, 2, 9, 8, -10, 0, 7], 2)
    lv = [p[0, 0] for p in build_pyramid(k, 2, 2, 3)]
    assert descend(lv, np.array([1.0]), 7, 2, 0, 2, 2) == [0, 3]
    assert _brute_force(lv[0], np.array([1.0]), 7, 2, 0) == [3, 4]


def test_selection_report_on_the_hand_worked_pruning():
    # level 1 scores the nodes (5, 1) -> 3, (2, 9) -> 5.5, (8, -10) -> -1 and keeps two:
    # boundary margin 3 - (-1) = 4; level 0 scores blocks {0, 1, 2, 3, 6} = 5, 1, 2, 9, 0:
    # margin 5 - 2 = 3. Block 4's node is dropped at level 1; block 3 is selected.
    k = _blocks_keys([5, 1, 2, 9, 8, -10, 0, 7], 2)
    lv = [p[0, 0] for p in build_pyramid(k, 2, 2, 3)]
    tr = []
    assert descend(lv, np.array([1.0]), 7, 2, 0, 2, 2, tr) == [0, 3]
    rep = selection_report(tr, 2, 2, targets=[4, 3, 5])
    assert rep["gaps"] == {1: 4.0, 0: 3.0}
    assert rep["pruned"] == {4: 1, 3: None, 5: 1}


def test_selection_report_names_the_level_that_drops_a_planted_block():
    # deep random trees: a block the brute force ranks first but the descent
    # misses is reported pruned at some level >= 1; a selected block never is
    N, d, bs, f, L, K = 4096, 8, 16, 4, 4, 2
    q, k, pyr, qbar = _random_case(7, N, d, bs, f, L)
    lv = [p[0, 0] for p in pyr]
    seen = 0
    for qb in range(1, 256):
        tr = []
        sel = descend(lv, qbar[0, 0, qb], qb, K, 0, bs, f, tr)
        bf = _brute_force(lv[0], qbar[0, 0, qb], qb, K, 0)
        rep = selection_report(tr, K, f, targets=bf)
        for j in bf:
            if j in sel:
                assert rep["pruned"][j] is None
            else:
                assert rep["pruned"][j] is not None and rep["pruned"][j] >= 1
                seen += 1
        assert all(g >= 0.0 for g in rep["gaps"].values())
    assert seen > 0


def _random_case(seed, N, d, bs, f, L, Hq=1, Hkv=1):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((1, Hq, N, d)).astype(np.float32)
    k = rng.standard_normal((1, Hkv, N, d)).astype(np.float32)
    return q, k, build_pyramid(k, bs, f, L), query_block_means(q, Hkv, bs)


def test_config1_shape_descent_is_exhaustive():
    # 16 blocks, fanout 4, 2 levels, K = 4: the top level never holds more than
    # 3 complete nodes, so nothing is pruned and the descent equals brute force.
    c = gen.workload(1)
    p = c["problem"]
    q, k, v, man = gen.host_inputs(p, c["seed"], c["value_scale"], c["plant"])
    pyr = build_pyramid(k, p.block_size, p.fanout, p.levels)
    qbar = query_block_means(q, p.heads_kv, p.block_size)
    idx, cnt = select(pyr, qbar, p.top_k, p.sink_len, p.block_size, p.fanout)
    j0 = p.sink_len // p.block_size
    for qb in range(p.n_blocks):
        bf = _brute_force(pyr[0][0, 0], qbar[0, 0, qb], qb, p.top_k, j0)
        assert idx[0, 0, qb, :cnt[0, 0, qb]].tolist() == bf
        assert cnt[0, 0, qb] == min(p.top_k, max(0, qb - j0))
        assert np.all(idx[0, 0, qb, cnt[0, 0, qb]:] == -1)
    # every surviving planted block is selected (margin-separated)
    for n in man["needles"]:
        if n["survived"]:
            assert n["target"] in idx[0, 0, n["qb"]].tolist()


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_deep_descent_matches_brute_force_when_winners_survive(seed):
    N, d, bs, f, L, K = 4096, 8, 16, 4, 4, 2
    q, k, pyr, qbar = _random_case(seed, N, d, bs, f, L)
    lv = [p[0, 0] for p in pyr]
    agree = pruned = 0
    for qb in range(1, 256):
        tr = []
        sel = descend(lv, qbar[0, 0, qb], qb, K, 0, bs, f, tr)
        bf = _brute_force(lv[0], qbar[0, 0, qb], qb, K, 0)
        # the result is always the top-K of the final pool
        final = tr[-1]
        assert sel == sorted(final["kept"])
        ok = all(
            any(j // f ** t["level"] in t["kept"] for t in tr if t["level"] == lvl)
            for j in bf
            for lvl in range(1, L)
        )
        if ok:
            assert sel == bf
            agree += 1
        else:
            pruned += 1
    assert agree > 0 and pruned > 0  # both branches exercised


def test_k_at_least_all_blocks_selects_every_candidate():
    N, d, bs, f, L = 2048, 8, 32, 4, 3
    q, k, pyr, qbar = _random_case(5, N, d, bs, f, L, Hq=4, Hkv=2)
    nb = N // bs
    for sink in (0, 32, 64, 100):
        idx, cnt = select(pyr, qbar, nb, sink, bs, f)
        j0 = sink // bs
        for g in range(2):
            for qb in range(nb):
                assert idx[0, g, qb, :cnt[0, g, qb]].tolist() == list(range(j0, max(j0, qb)))


def test_selection_ignores_blocks_after_the_query_block():
    N, d, bs, f, L, K = 2048, 8, 16, 4, 4, 3
    rng = np.random.default_rng(9)
    q, k, pyr, qbar = _random_case(4, N, d, bs, f, L)
    for qb in (5, 37, 64, 100, 127):
        base = descend([p[0, 0] for p in pyr], qbar[0, 0, qb], qb, K, 0, bs, f)
        k2 = k.copy()
        k2[0, 0, qb * bs:] = rng.standard_normal(k2[0, 0, qb * bs:].shape) * 5  # refill the future
        pyr2 = build_pyramid(k2, bs, f, L)
        assert descend([p[0, 0] for p in pyr2], qbar[0, 0, qb], qb, K, 0, bs, f) == base
        k3 = k.copy()  # permute the blocks after qb
        tail = k3[0, 0, (qb + 1) * bs:].reshape(-1, bs, d)
        k3[0, 0, (qb + 1) * bs:] = tail[rng.permutation(len(tail))].reshape(-1, d)
        pyr3 = build_pyramid(k3, bs, f, L)
        assert descend([p[0, 0] for p in pyr3], qbar[0, 0, qb], qb, K, 0, bs, f) == base


def test_decode_reads_no_pyramid_node_holding_its_own_token():
    # A decode at length n scores only complete nodes, wholly before the block of
    # its token n - 1; that token's append touches only its leaf and the leaf's
    # ancestors, none of them complete. So the pyramid of the prefix without the
    # token serves the decode as well, and a serving loop may run the append of a
    # step beside that step's decode (lengths on and across block boundaries).
    from oracle import decode_ragged

    B, Hq, Hkv, cap, d, bs, f, L, K, s = 3, 4, 2, 1024, 16, 16, 4, 3, 5, 16
    rng = np.random.default_rng(21)
    q = rng.standard_normal((B, Hq, d)).astype(np.float32)
    k = rng.standard_normal((B, Hkv, cap, d)).astype(np.float32)
    v = rng.standard_normal((B, Hkv, cap, d)).astype(np.float32)
    most = 0
    for lens in ((16 * 7 + 1, 16 * 8, 300), (16 * 8 + 1, 513, 1024), (17, 16, 1)):
        before, after = k.copy(), k.copy()
        for b, n in enumerate(lens):
            before[b, :, n - 1:] = 0.0  # the prefix without the token
            after[b, :, n:] = 0.0       # with it
        pb, pa = build_pyramid(before, bs, f, L), build_pyramid(after, bs, f, L)
        assert any(not np.array_equal(x, y) for x, y in zip(pb, pa))  # the appended token changes the pyramid
        ob, lb, ib, cb = decode_ragged(q, after, v, pb, lens, K, s, bs, f, 0.25)
        oa, la, ia, ca = decode_ragged(q, after, v, pa, lens, K, s, bs, f, 0.25)
        assert np.array_equal(ib, ia) and np.array_equal(cb, ca)
        assert np.array_equal(ob, oa) and np.array_equal(lb, la)
        most = max(most, int(ca.max()))
    assert most == K  # the longer sequences select a full set


def test_equal_blocks_tie_to_lower_index():
    N, d, bs, f, L = 1024, 4, 16, 4, 3
    rng = np.random.default_rng(2)
    k = np.zeros((1, 1, N, d), np.float32)
    hot = rng.standard_normal(d).astype(np.float32)
    # three identical blocks in different nodes: their level-1 nodes tie exactly too
    for j in (3, 9, 21):
        k[0, 0, j * bs:(j + 1) * bs] = hot
    pyr = build_pyramid(k, bs, f, L)
    qbar = hot.astype(np.float64)
    assert descend([p[0, 0] for p in pyr], qbar, 63, 1, 0, bs, f) == [3]
    assert descend([p[0, 0] for p in pyr], qbar, 63, 2, 0, bs, f) == [3, 9]


def test_scored_nodes_do_not_grow_with_n():
    # With enough levels that the top holds <= f nodes, each level scores at most
    # K*f + f - 1 nodes, whatever N is (no quadratic indexer).
    K, f, bs, d = 2, 4, 16, 4
    for N, L in ((4096, 4), (16384, 5), (65536, 6)):
        _, _, pyr, qbar = _random_case(N, N, d, bs, f, L)
        lv = [p[0, 0] for p in pyr]
        nb = N // bs
        for qb in (nb // 2, nb - 1):
            tr = []
            descend(lv, qbar[0, 0, qb], qb, K, 0, bs, f, tr)
            assert len(tr[0]["pool"]) <= f
            assert all(len(t["pool"]) <= K * f + f - 1 for t in tr)
            assert sum(len(t["pool"]) for t in tr) <= f + (L - 1) * (K * f + f - 1)


def test_zero_k_and_first_blocks():
    _, _, pyr, qbar = _random_case(1, 512, 4, 16, 2, 3)
    lv = [p[0, 0] for p in pyr]
    assert descend(lv, qbar[0, 0, 20], 20, 0, 0, 16, 2) == []
    assert descend(lv, qbar[0, 0, 0], 0, 3, 0, 16, 2) == []
    assert descend(lv, qbar[0, 0, 1], 1, 3, 0, 16, 2) == [0]
    assert descend(lv, qbar[0, 0, 1], 1, 3, 16, 16, 2) == []  # block 0 is all sink
