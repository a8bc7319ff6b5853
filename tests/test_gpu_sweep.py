"""A seeded sweep over problem configurations, against the oracle.

Each case draws, from a seed of its own, one point of the space the library
accepts: head size, block size, fanout, GQA group size, batch and kv heads, a
ragged sequence length, pyramid depth (deeper than the blocks need included),
K, sink length (none, one token, part of a block, whole blocks), causal or
bidirectional, mean or max summaries, bf16 or fp32. Every case runs the whole
prefill through the C ABI -- pyramid, selection, attention -- and compares it
with the oracle: the pyramid and the selection bit for bit, the outputs within
the dtype's bar. Causal bf16 cases also run the fused launch, which must equal
the two launches bit for bit, and the backward pass against the oracle's fp64
gradients; causal cases whose group size the decode takes also run one decode
step at a drawn cache length.
"""

import math

import numpy as np
import pytest

import gen
import oracle
from parity import (assert_outputs_close, assert_pyramid_equal, assert_selection_equal, cprob, gpu_prefill,
                    grads_close, log, oracle_attend, oracle_select, to_dev, to_host)

torch = pytest.importorskip("torch")

P = gen.Problem
N_CASES = 48


def sweep_case(i: int):
    """Case i of the sweep: (problem, planting scheme, input seed)."""
    rng = np.random.default_rng([20261203, i])
    d = int(rng.choice([64, 128]))
    bs = int(rng.choice([32, 64, 128]))
    f = int(rng.choice([2, 4, 8, 16]))
    group = int(rng.choice([1, 2, 3, 4, 8]))
    hkv = int(rng.integers(1, 3))
    batch = 1 if group * hkv > 4 else int(rng.integers(1, 3))
    n = int(rng.integers(1, 48 * bs + 1))
    levels = int(rng.integers(1, 6))
    top_k = int(rng.integers(0, 41))
    sink = int(rng.choice([0, 1, bs // 2, bs, bs + 7, 3 * bs]))
    causal = bool(rng.random() < 0.7)
    pool = "max" if rng.random() < 0.3 else "mean"
    dtype = "f32" if rng.random() < 0.2 else "bf16"
    p = P(batch, group * hkv, hkv, n, d, bs, f, levels, top_k, sink, dtype, causal=causal, pool=pool)
    return p, ("uniform_pairs", 2), 100 + i


def test_sweep_spans_the_space():
    """(Host only.) The drawn cases reach every value of every axis, and both sides of each switch."""
    cases = [sweep_case(i)[0] for i in range(N_CASES)]
    assert {p.head_dim for p in cases} == {64, 128}
    assert {p.block_size for p in cases} == {32, 64, 128}
    assert {p.fanout for p in cases} == {2, 4, 8, 16}
    assert {p.heads_q // p.heads_kv for p in cases} == {1, 2, 3, 4, 8}
    assert {p.causal for p in cases} == {True, False}
    assert {p.pool for p in cases} == {"mean", "max"}
    assert {p.dtype for p in cases} == {"bf16", "f32"}
    assert any(p.top_k == 0 for p in cases) and any(p.sink_len == 0 for p in cases)
    assert any(p.seq_len % p.block_size for p in cases)
    # a pyramid deeper than its blocks need: some level above the first holds one node
    assert any(len([s for s in oracle.level_sizes(p.n_blocks, p.fanout, p.levels) if s == 1]) > 1 for p in cases)


@pytest.mark.gpu
@pytest.mark.parametrize("i", range(N_CASES))
def test_sweep_case(i):
    import block_sparse_long_pisa_amd as pisa

    p, plant, seed = sweep_case(i)
    log(f"sweep case {i}: {p}")
    q, k, v, _ = gen.host_inputs(p, seed, 1.0 / math.sqrt(p.head_dim), plant)
    qd, kd, vd = to_dev(q, p.dtype), to_dev(k, p.dtype), to_dev(v, p.dtype)
    levels, gi, gc, out, lse = gpu_prefill(p, qd, kd, vd)
    pyr, oi, oc = oracle_select(p, q, k)
    assert_pyramid_equal(levels, pyr)
    assert_selection_equal(gi, gc, oi, oc)
    o, ol = oracle_attend(p, q, k, v, oi, oc)
    err = assert_outputs_close(p, to_host(out), o, lse, ol)
    log(f"  prefill max abs err {err:.2e}")

    cp = cprob(p)
    if p.dtype == "bf16" and p.causal:
        dpyr = pisa.build_pyramid(cp, kd)
        fo, fl, fi, fc = pisa.select_attend(cp, qd, kd, vd, dpyr, want_lse=True, want_idx=True)
        torch.cuda.synchronize()
        assert np.array_equal(to_host(fc), gc) and np.array_equal(to_host(fi), gi), "fused selection differs"
        assert torch.equal(fo, out) and np.array_equal(to_host(fl), lse), "fused output differs"
        log("  fused launch equals the two launches")
        do = gen.round_to_bf16(np.random.default_rng([20261203, i, 2]).standard_normal(q.shape).astype(np.float32))
        bout, blse, bidx, bcnt, _ = pisa.prefill(cp, qd, kd, vd, want_lse=True)
        grads = pisa.sparse_attn_bwd(cp, qd, kd, vd, bidx, bcnt, bout, blse, to_dev(do, "bf16"))
        torch.cuda.synchronize()
        want = oracle.attend_backward(q, k, v, oi, oc, do, p.sink_len, p.block_size, p.scale)
        res = [grads_close(n, to_host(g), w) for n, g, w in zip(("dq", "dk", "dv"), grads, want)]
        log("  backward " + ", ".join(f"{n}: max {a:.2e} of max|g|, rel L2 {b:.2e}"
                                      for n, (a, b) in zip(("dq", "dk", "dv"), res)))

    if p.causal and p.heads_q // p.heads_kv in (1, 2, 4, 8):
        pdec = p.replace(decode=True)
        cache_len = int(np.random.default_rng([20261203, i, 1]).integers(1, p.seq_len + 1))
        qh, kh, vh, _ = gen.host_decode_inputs(pdec, seed, 1.0 / math.sqrt(p.head_dim), cache_len)
        kc, vc = to_dev(kh, p.dtype), to_dev(vh, p.dtype)
        dpyr = pisa.build_pyramid(cp, kc)
        dout, dlse, didx, dcnt = pisa.decode_step(cp, to_dev(qh, p.dtype), kc, vc, dpyr, cache_len, want_lse=True,
                                                  want_idx=True)
        torch.cuda.synchronize()
        opyr = oracle.build_pyramid(kh, p.block_size, p.fanout, p.levels, pool=p.pool)
        do, dl, di, dc = oracle.decode(qh, kh, vh, opyr, cache_len, p.top_k, p.sink_len, p.block_size, p.fanout,
                                       p.scale)
        assert np.array_equal(to_host(dcnt), dc)
        if p.top_k:
            assert np.array_equal(to_host(didx), di)
        derr = assert_outputs_close(p, to_host(dout), do, to_host(dlse), dl)
        log(f"  decode at cache length {cache_len}: max abs err {derr:.2e}")
