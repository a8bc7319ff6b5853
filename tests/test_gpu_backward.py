"""GPU parity of the backward pass (dq, dk, dv with the selection held constant)
against the oracle's fp64 gradients.

The HIP selection is first checked bit-exact against the oracle's; the oracle's
gradients then use its own selection, so no oracle input comes from the HIP path.

Tolerance (bf16 inputs): the products take p and dS rounded to bf16 (relative
2^-9 each), D_i = dO_i.O_i uses the forward's bf16 output, and the gradients are
rounded to bf16 on output (relative 2^-9 ~ 2e-3). Summed over hundreds to
thousands of keys the per-term roundings largely cancel, so the bar is a
per-tensor relative L2 error of 1e-2 and a max-abs error of 1e-2 of the tensor's
largest gradient.
"""

import math

import numpy as np
import pytest

import gen
import oracle
from parity import cprob, grads_close, log, oracle_select, to_dev, to_host

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

P = gen.Problem

CASES = {
    "gqa_ragged": (P(2, 8, 2, 4000, 128, 128, 4, 3, 4, 64, "bf16"), ("uniform_pairs", 4)),
    "mha_bs64_ragged": (P(1, 4, 4, 3000, 128, 64, 8, 2, 6, 64, "bf16"), ("uniform_pairs", 4)),
    "d64_bs32_partial_sink": (P(1, 4, 1, 2065, 64, 32, 4, 3, 3, 40, "bf16"), ("uniform_pairs", 4)),
    "group8": (P(1, 16, 2, 2048, 128, 128, 4, 2, 3, 64, "bf16"), ("uniform_pairs", 4)),
    "wide_sink_bs32": (P(1, 4, 4, 1500, 64, 32, 4, 3, 4, 100, "bf16"), ("uniform_pairs", 4)),
    "d128_bs32": (P(1, 4, 2, 1000, 128, 32, 2, 4, 5, 32, "bf16"), ("log_distance", 8)),
    "k0": (P(1, 4, 2, 1500, 128, 64, 4, 2, 0, 64, "bf16"), None),
    "shorter_than_block": (P(1, 2, 1, 50, 128, 64, 4, 2, 4, 64, "bf16"), None),
    # d = 64 at blocks 128 and 64 (the key-centric swizzle over several 32-row
    # chunks and 8 or 4 waves); an odd group (the query-centric pass at 2 waves)
    "d64_bs128_ragged": (P(1, 4, 2, 3100, 64, 128, 4, 3, 4, 64, "bf16"), ("uniform_pairs", 4)),
    "d64_bs64_group3": (P(1, 6, 2, 2500, 64, 64, 4, 2, 5, 64, "bf16"), ("uniform_pairs", 4)),
}


def _run(p, plant, seed=17, sharp=False):
    import block_sparse_long_pisa_amd as pisa

    s = (1.0, 1.0, 1.0 / math.sqrt(p.head_dim)) if sharp else 1.0 / math.sqrt(p.head_dim)
    q, k, v, _ = gen.host_inputs(p, seed, s, plant)
    rng = np.random.default_rng(seed + 1)
    do = gen.round_to_bf16(rng.standard_normal(q.shape).astype(np.float32))
    cp = cprob(p)
    qd, kd, vd, dod = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"), to_dev(do, "bf16")
    out, lse, idx, cnt, pyr = pisa.prefill(cp, qd, kd, vd, want_lse=True)
    dq, dk, dv = pisa.sparse_attn_bwd(cp, qd, kd, vd, idx, cnt, out, lse, dod)
    torch.cuda.synchronize()
    _, oi, oc = oracle_select(p, q, k)
    assert np.array_equal(to_host(cnt), oc)
    if p.top_k:
        assert np.array_equal(to_host(idx), oi)
    want = oracle.attend_backward(q, k, v, oi, oc, do, p.sink_len, p.block_size, p.scale)
    res = [grads_close(n, to_host(g), w) for n, g, w in zip(("dq", "dk", "dv"), (dq, dk, dv), want)]
    return res


@pytest.mark.parametrize("name", list(CASES))
def test_backward_parity(name):
    p, plant = CASES[name]
    log(f"backward case {name}: {p}")
    res = _run(p, plant)
    log("  " + ", ".join(f"{n}: max {a:.2e} of max|g|, rel L2 {b:.2e}" for n, (a, b) in zip(("dq", "dk", "dv"), res)))


def test_backward_parity_sharp_logits():
    # unit-spread logits: peaked attention, large dS
    p = P(1, 8, 2, 4096, 128, 128, 8, 3, 8, 64, "bf16")
    log(f"backward sharp case: {p}")
    res = _run(p, ("uniform_depth", 8), seed=5, sharp=True)
    log("  " + ", ".join(f"{n}: max {a:.2e}, rel L2 {b:.2e}" for n, (a, b) in zip(("dq", "dk", "dv"), res)))


def test_backward_dense_reduction():
    # K covering every block: the gradients of dense causal attention
    p = P(1, 4, 2, 1024, 128, 64, 4, 2, 16, 64, "bf16")
    _run(p, None, seed=9)


def test_backward_is_deterministic():
    import block_sparse_long_pisa_amd as pisa

    p = P(1, 8, 2, 4096, 128, 128, 4, 3, 4, 64, "bf16")
    q, k, v, _ = gen.host_inputs(p, 3, 1.0 / math.sqrt(p.head_dim), ("uniform_pairs", 4))
    cp = cprob(p)
    qd, kd, vd = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    dod = torch.randn_like(qd)
    out, lse, idx, cnt, _ = pisa.prefill(cp, qd, kd, vd, want_lse=True)
    a = pisa.sparse_attn_bwd(cp, qd, kd, vd, idx, cnt, out, lse, dod)
    b = pisa.sparse_attn_bwd(cp, qd, kd, vd, idx, cnt, out, lse, dod)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)
