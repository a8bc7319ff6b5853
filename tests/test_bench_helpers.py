"""The bench's algorithmic-work counts agree with the oracle's attended sets and descent pools."""

import numpy as np

import bench
import gen
import oracle


def test_attended_pairs_counts_every_attended_key_once():
    p = gen.Problem(1, 4, 2, 1000, 16, 32, 4, 3, 3, 40, "f32")
    q, k, v, _ = gen.host_inputs(p, 1, 1.0, ("uniform_pairs", 4))
    pyr = oracle.build_pyramid(k, p.block_size, p.fanout, p.levels)
    idx, cnt = oracle.select(pyr, oracle.query_block_means(q, p.heads_kv, p.block_size), p.top_k, p.sink_len,
                             p.block_size, p.fanout)
    brute = 0
    for g in range(p.heads_kv):
        for i in range(p.seq_len):
            qb = i // p.block_size
            brute += len(oracle.attended_keys(i, idx[0, g, qb, :cnt[0, g, qb]].tolist(), p.sink_len, p.block_size))
    assert bench.attended_pairs(p, idx, cnt) == brute * p.group


def test_decode_scored_nodes_match_the_descent_pools():
    p = gen.Problem(1, 4, 1, 131072, 8, 128, 8, 4, 32, 64, "f32")
    rng = np.random.default_rng(0)
    levels = [rng.standard_normal((n, 8)).astype(np.float32) for n in oracle.level_sizes(p.n_blocks, 8, 4)]
    tr = []
    oracle.descend(levels, rng.standard_normal(8), p.n_blocks - 1, 32, 64, 128, 8, tr)
    assert sum(len(t["pool"]) for t in tr) == bench.decode_scored_nodes(p, p.seq_len) == 1 + 15 + 127 + 263
