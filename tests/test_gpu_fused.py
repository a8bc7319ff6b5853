"""GPU parity of the fused selection + attention (one launch) against the oracle.

* small cases spanning several tiles, ragged tails and the degenerate shapes:
  the selection bit-exact against the oracle's, the outputs within the dtype's
  bar;
* the full-size bf16 workloads (32K MHA, 128K GQA, 1M one-group): every
  selection bit-exact against the oracle's, outputs on sampled query blocks;
* in every case the fused launch also equals the two-launch path (selection,
  then sparse attention) bit for bit, as the header promises.
"""

import math

import numpy as np
import pytest

import gen
import oracle
from parity import assert_outputs_close, assert_selection_equal, cprob, log, oracle_select, to_dev, to_host
from test_gpu_full import _sample_units
from test_gpu_parity import SHAPES, SMALL

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

CASES = [n for n, (p, _, _) in SMALL.items() if p.dtype == "bf16"]


def _both(pisa, cp, q, k, v):
    """Fused and two-launch results on the same pyramid."""
    pyr = pisa.build_pyramid(cp, k)
    fo, fl, fi, fc = pisa.select_attend(cp, q, k, v, pyr, want_lse=True, want_idx=True)
    si, sc = pisa.select_topk(cp, q, pyr)
    so, sl = pisa.sparse_attn_fwd(cp, q, k, v, si, sc, want_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(fc, sc) and torch.equal(fi, si), "fused selection differs from pisa_select_topk"
    assert torch.equal(fo, so) and torch.equal(fl, sl), "fused output differs from pisa_sparse_attn_fwd"
    return fo, fl, fi, fc


@pytest.mark.parametrize("name", CASES)
def test_fused_parity(name):
    import block_sparse_long_pisa_amd as pisa

    p, plant, scale = SMALL[name]
    log(f"fused case {name}: {p}")
    s = scale if scale is not None else 1.0 / math.sqrt(p.head_dim)
    q, k, v, _ = gen.host_inputs(p, 11, s, plant)
    cp = cprob(p)
    out, lse, idx, cnt = _both(pisa, cp, to_dev(q, p.dtype), to_dev(k, p.dtype), to_dev(v, p.dtype))
    _, oi, oc = oracle_select(p, q, k)
    assert_selection_equal(to_host(idx), to_host(cnt), oi, oc)
    o, ol = oracle.attend(q, k, v, oi, oc, p.sink_len, p.block_size, p.scale)
    err = assert_outputs_close(p, to_host(out), o, to_host(lse), ol)
    log(f"  max abs err {err:.2e}")


@pytest.mark.parametrize("d,bs,nw", SHAPES)
def test_fused_every_attention_shape(d, bs, nw):
    import block_sparse_long_pisa_amd as pisa

    G = nw * 32 // bs
    p = gen.Problem(1, 2 * G, 2, 11 * bs + 37, d, bs, 4, 2, 3, 64, "bf16")
    log(f"fused shape d={d} bs={bs} waves={nw}: {p}")
    q, k, v, _ = gen.host_inputs(p, 23, 1.0 / math.sqrt(d), ("uniform_pairs", 2))
    out, lse, idx, cnt = _both(pisa, cprob(p), to_dev(q, p.dtype), to_dev(k, p.dtype), to_dev(v, p.dtype))
    _, oi, oc = oracle_select(p, q, k)
    assert_selection_equal(to_host(idx), to_host(cnt), oi, oc)
    o, ol = oracle.attend(q, k, v, oi, oc, p.sink_len, p.block_size, p.scale)
    err = assert_outputs_close(p, to_host(out), o, to_host(lse), ol)
    log(f"  max abs err {err:.2e}")


def test_fused_without_selection_outputs():
    import block_sparse_long_pisa_amd as pisa

    p = SMALL["gqa_ragged"][0]
    q, k, v, _ = gen.host_inputs(p, 5, 1.0 / math.sqrt(p.head_dim), ("uniform_pairs", 4))
    cp = cprob(p)
    qd, kd, vd = to_dev(q, p.dtype), to_dev(k, p.dtype), to_dev(v, p.dtype)
    pyr = pisa.build_pyramid(cp, kd)
    a = pisa.select_attend(cp, qd, kd, vd, pyr)[0]
    b = pisa.select_attend(cp, qd, kd, vd, pyr, want_idx=True)[0]
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("workload_id", [2, 3, 5])
def test_fused_full_size(workload_id):
    import block_sparse_long_pisa_amd as pisa

    c = gen.workload(workload_id)
    p = c["problem"]
    log(f"fused, config {workload_id}: {c['name']}")
    q, k, v, man = gen.device_inputs(p, c["seed"], c["value_scale"], c["plant"], device="cuda")
    cp = cprob(p)
    out, lse, idx, cnt = _both(pisa, cp, q, k, v)
    gi, gc = to_host(idx), to_host(cnt)
    qh, kh, vh = to_host(q), to_host(k), to_host(v)
    del q, k, v
    log("  GPU done (fused equals the two-launch path); oracle selection")
    _, oi, oc = oracle_select(p, qh, kh)
    assert_selection_equal(gi, gc, oi, oc)
    units = _sample_units(p, man, n_random=8)
    o, ol = oracle.attend(qh, kh, vh, oi, oc, p.sink_len, p.block_size, p.scale, blocks=units)
    err = assert_outputs_close(p, to_host(out), o, to_host(lse), ol)
    log(f"  {oc.size} selections bit-exact; sampled outputs max abs err {err:.2e}")
