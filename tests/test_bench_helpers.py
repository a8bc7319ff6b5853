"""The bench's algorithmic-work counts agree with the oracle's attended sets and descent pools; its
measured-traffic table holds only for the sources it was taken on."""

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


def test_append_bytes_single_token_by_hand():
    # one token at position 1000 (block 7 of 128-token blocks, fanout 8, 4 levels):
    # the leaf re-reads rows 896..1000; level 1 node 0 reads its 8 present children,
    # level 2 node 0 reads its 1 present child, level 3 node 0 its 1
    p = gen.workload(4)["problem"]
    rows = 1001 - 7 * 128
    written = 4  # one node per level
    read = 8 + 1 + 1
    want = p.heads_kv * (rows * p.head_dim * 2 + (read + written) * p.head_dim * 4)
    assert bench.append_bytes(p, [1000], [1001]) == want
    assert bench.append_bytes(p, [5], [5]) == 0 and bench.append_bytes(p, [-1], [3]) == 0


def test_bidirectional_pairs_count_every_attended_key_once():
    p = gen.Problem(1, 4, 2, 1000, 16, 32, 4, 3, 3, 40, "f32", causal=False)
    q, k, v, _ = gen.host_inputs(p, 1, 1.0, ("uniform_pairs", 4))
    pyr = oracle.build_pyramid(k, p.block_size, p.fanout, p.levels)
    idx, cnt = oracle.select(pyr, oracle.query_block_means(q, p.heads_kv, p.block_size), p.top_k, p.sink_len,
                             p.block_size, p.fanout, causal=False)
    brute = 0
    for g in range(p.heads_kv):
        for i in range(p.seq_len):
            qb = i // p.block_size
            sel = idx[0, g, qb, :cnt[0, g, qb]].tolist()
            brute += len(oracle.attended_keys(i, sel, p.sink_len, p.block_size, causal=False, n=p.seq_len))
    assert bench.attended_pairs_bidirectional(p, idx, cnt) == brute * p.group


def test_median_ms_takes_the_median_of_event_intervals():
    class Ev:
        def __init__(self, t):
            self.t = t

        def elapsed_time(self, other):
            return other.t - self.t

    pairs = [(Ev(0.0), Ev(d)) for d in (5.0, 1.0, 100.0, 2.0, 3.0)]
    assert bench.median_ms(pairs) == 3.0e-3


def test_measured_traffic_holds_only_for_the_sources_it_was_taken_on(monkeypatch):
    import hashlib
    import os

    import bench

    files = ("pisa_pool.hip", "pisa_internal.h")
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(bench.ROOT, "block_sparse_long_pisa_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    table = {"x": (files, h.hexdigest()[:16], 100.0, 10.0), "y": (files, "0" * 16, 100.0, 10.0)}
    monkeypatch.setattr(bench, "MEASURED_TRAFFIC", table)
    monkeypatch.setattr(bench, "COPY_SCALE", {"fetch": 2.0, "write": 1.0})
    assert bench.measured_traffic("x") == 1024 * (100 * 2 + 10)
    assert bench.measured_traffic("y") is None  # another source
    assert bench.measured_traffic("w2/x") is None  # never measured
