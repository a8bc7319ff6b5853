"""GPU parity at the library's limits.

* top_k at its maximum (256) with the deepest pyramid (8 levels, fanout 2): at
  8192 tokens and block 32 every earlier block is a candidate, so this also
  reaches the largest kept set;
* the level-0 pool at its maximum: K = 255, fanout 4, 255 * 4 + 3 = 1023 slots
  (the 16-slot ranking of both the per-wave and the workgroup descents);
* the decode step at both.

Selections bit-exact against the oracle; outputs on every row at the small size,
on sampled query blocks at the large one.
"""

import math

import numpy as np
import pytest

import gen
import oracle
from parity import assert_outputs_close, assert_selection_equal, cprob, log, oracle_select, to_dev, to_host

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

P = gen.Problem

MAX_K = P(1, 2, 1, 8192, 64, 32, 2, 8, 256, 32, "bf16")
MAX_POOL = P(1, 4, 1, 65536, 64, 64, 4, 3, 255, 64, "bf16")


def _prefill(pisa, p, seed):
    q, k, v, man = gen.host_inputs(p, seed, 1.0 / math.sqrt(p.head_dim), ("uniform_pairs", 4))
    cp = cprob(p)
    out, lse, idx, cnt, _ = pisa.prefill(cp, to_dev(q, p.dtype), to_dev(k, p.dtype), to_dev(v, p.dtype),
                                         want_lse=True)
    torch.cuda.synchronize()
    _, oi, oc = oracle_select(p, q, k)
    assert_selection_equal(to_host(idx), to_host(cnt), oi, oc)
    return q, k, v, oi, oc, to_host(out), to_host(lse)


def test_max_top_k_deepest_pyramid():
    import block_sparse_long_pisa_amd as pisa

    p = MAX_K
    log(f"limits: max top_k, 8 levels: {p}")
    q, k, v, oi, oc, out, lse = _prefill(pisa, p, 31)
    assert oc.max() == p.n_blocks - 2  # the last block keeps every earlier one but the sink's
    o, ol = oracle.attend(q, k, v, oi, oc, p.sink_len, p.block_size, p.scale)
    err = assert_outputs_close(p, out, o, lse, ol)
    log(f"  largest count {int(oc.max())}, max abs err {err:.2e}")


def test_max_pool():
    import block_sparse_long_pisa_amd as pisa

    p = MAX_POOL
    log(f"limits: level-0 pool of 1023 slots: {p}")
    q, k, v, oi, oc, out, lse = _prefill(pisa, p, 32)
    assert oc.max() == p.top_k
    nb = p.n_blocks
    units = sorted({(0, 0, qb) for qb in (0, 1, 2, 255, 256, 257, 300, 700, nb - 2, nb - 1)})
    o, ol = oracle.attend(q, k, v, oi, oc, p.sink_len, p.block_size, p.scale, blocks=units)
    err = assert_outputs_close(p, out, o, lse, ol)
    log(f"  {oc.size} selections bit-exact; sampled outputs max abs err {err:.2e}")


@pytest.mark.parametrize("base,cache_lens", [(MAX_K, (8192, 5000)), (MAX_POOL, (65536, 40000))])
def test_decode_at_the_limits(base, cache_lens):
    import block_sparse_long_pisa_amd as pisa

    p = base.replace(batch=2, decode=True)
    for cache_len in cache_lens:
        log(f"limits, decode: {p}, cache_len {cache_len}")
        q, k, v, _ = gen.host_decode_inputs(p, 40 + cache_len, 1.0 / math.sqrt(p.head_dim), cache_len)
        cp = cprob(p)
        kd, vd = to_dev(k, p.dtype), to_dev(v, p.dtype)
        pyr = pisa.build_pyramid(cp, kd)
        out, lse, idx, cnt = pisa.decode_step(cp, to_dev(q, p.dtype), kd, vd, pyr, cache_len, want_lse=True,
                                              want_idx=True)
        torch.cuda.synchronize()
        opyr = oracle.build_pyramid(k, p.block_size, p.fanout, p.levels)
        o, ol, oi, oc = oracle.decode(q, k, v, opyr, cache_len, p.top_k, p.sink_len, p.block_size, p.fanout, p.scale)
        assert np.array_equal(to_host(cnt), oc) and np.array_equal(to_host(idx), oi)
        err = assert_outputs_close(p, to_host(out), o, to_host(lse), ol)
        log(f"  counts {oc.reshape(-1).tolist()}, max abs err {err:.2e}")
