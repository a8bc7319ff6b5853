"""GPU parity of the selection across candidate-pool sizes.

The per-wave descent gives each lane ceil(pool / 64) pool slots, rounded up to
one of the instantiated counts (1-6, 8, 10, 12, 16), and the decode descent
rounds to 2, 4, 5, 6, 8 or 16. The top-K search skips slot groups past a level's
pool. These cases choose K with fanout 8, so that the level-0 pool K*8 + 7
lands in every slot count, and check every selection bit for bit against the
oracle. The ragged last block (27 rows) also takes the query mean's general
path.
"""

import math

import numpy as np
import pytest

import gen
import oracle
from parity import assert_pyramid_equal, assert_selection_equal, cprob, log, oracle_select, split_levels, to_dev, to_host

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

P = gen.Problem

# K -> level-0 pool K*8+7 -> slots per lane
PREFILL_K = {1: 1, 8: 2, 16: 3, 24: 4, 32: 5, 40: 6, 56: 8, 72: 10, 88: 12, 120: 16}


@pytest.mark.parametrize("K", list(PREFILL_K))
def test_selection_for_each_pool_slot_count(K):
    import block_sparse_long_pisa_amd as pisa

    p = P(1, 4, 2, 32768 - 5, 64, 32, 8, 3, K, 64, "bf16")
    assert math.ceil((K * 8 + 7) / 64) <= PREFILL_K[K]
    log(f"pool slots: K={K}, level-0 pool {K * 8 + 7}: {p}")
    q, k, _, _ = gen.host_inputs(p, 100 + K, 1.0 / math.sqrt(p.head_dim), ("uniform_pairs", 4))
    cp = cprob(p)
    qd, kd = to_dev(q, p.dtype), to_dev(k, p.dtype)
    pyr = pisa.build_pyramid(cp, kd)
    idx, cnt = pisa.select_topk(cp, qd, pyr)
    torch.cuda.synchronize()
    opyr, oi, oc = oracle_select(p, q, k)
    assert_pyramid_equal(split_levels(to_host(pyr), pisa.pyramid_layout(cp)), opyr)
    gi, gc = to_host(idx), to_host(cnt)
    assert_selection_equal(gi, gc, oi, oc)
    log(f"  {oc.size} selections bit-exact, largest count {int(oc.max())}")


# decode: K -> slots per lane of the workgroup descent
DECODE_K = {8: 2, 24: 4, 32: 5, 40: 6, 56: 8, 120: 16}


@pytest.mark.parametrize("K", list(DECODE_K))
def test_decode_selection_for_each_pool_slot_count(K):
    import block_sparse_long_pisa_amd as pisa

    p = P(4, 4, 2, 32768, 64, 32, 8, 3, K, 64, "bf16", decode=True)
    lens = [32768, 20001, 9000, 31000]
    log(f"decode pool slots: K={K}: {p}, lengths {lens}")
    q, k, v, _ = gen.host_decode_inputs(p, 200 + K, 1.0 / math.sqrt(p.head_dim), p.seq_len)
    cp = cprob(p)
    kd, vd = to_dev(k, p.dtype), to_dev(v, p.dtype)
    pyr = pisa.build_pyramid(cp, kd)
    dl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    _, _, idx, cnt = pisa.decode_step_ragged(cp, to_dev(q, p.dtype), kd, vd, pyr, dl, want_idx=True)
    torch.cuda.synchronize()
    opyr = oracle.build_pyramid(k, p.block_size, p.fanout, p.levels)
    _, _, oi, oc = oracle.decode_ragged(q, k, v, opyr, lens, p.top_k, p.sink_len, p.block_size, p.fanout, p.scale)
    assert np.array_equal(to_host(cnt), oc) and np.array_equal(to_host(idx), oi)
    log(f"  counts {oc.reshape(-1).tolist()}")
