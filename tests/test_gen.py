"""The seeded generator: determinism, rounding, planting records."""

import numpy as np
import torch

import gen


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 3.4e38, 1e-40], np.float32)])
    ours = gen.round_to_bf16(x)
    theirs = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(ours, theirs)
    assert np.array_equal(gen.round_to_bf16(ours), ours)


def test_host_inputs_are_deterministic_and_sliceable():
    c = gen.workload(2)
    p = c["problem"].replace(heads_q=3, heads_kv=3, seq_len=1024)
    a = gen.host_inputs(p, c["seed"], c["value_scale"], c["plant"])
    b = gen.host_inputs(p, c["seed"], c["value_scale"], c["plant"])
    for x, y in zip(a[:3], b[:3]):
        assert np.array_equal(x, y)
    # head 1 alone (a child stream) equals head 1 of the full draw, planting aside
    p1 = p.replace(heads_q=2, heads_kv=2)
    c1 = gen.host_inputs(p1, c["seed"], c["value_scale"], None)
    assert np.array_equal(c1[0][0, 1], a[0][0, 1])
    assert np.all(gen.round_to_bf16(a[1]) == a[1])


def test_planting_writes_the_query_block_mean_plus_small_noise():
    c = gen.workload(3)
    p = c["problem"].replace(seq_len=8192)
    q, k, v, man = gen.host_inputs(p, c["seed"], c["value_scale"], c["plant"])
    assert len(man["needles"]) == 16 * p.heads_kv
    G, bs = p.group, p.block_size
    for n in man["needles"]:
        if not n["survived"]:
            continue
        b, g, qb, t = n["b"], n["g"], n["qb"], n["target"]
        assert 0 <= t < qb
        target = q[b, g * G:(g + 1) * G, qb * bs:(qb + 1) * bs].astype(np.float64).mean(axis=(0, 1))
        dev = k[b, g, t * bs:(t + 1) * bs].astype(np.float64) - target
        assert abs(dev.std() - 0.1) < 0.01 and abs(dev.mean()) < 0.01


def test_star_import_names_exist():
    ns = {}
    exec("from gen import *", ns)
    for name in gen.__all__:
        assert name in ns, name
