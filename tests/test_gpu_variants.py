"""GPU parity of the variants: non-causal (bidirectional) selection and attention,
and max-pooled node summaries -- each against the oracle, pyramid and selection
bit-exact, outputs within the dtype's bar; decode and pyramid append with max
summaries; the variants the library does not implement fail on the host."""

import math

import numpy as np
import pytest

import gen
import oracle
from parity import (assert_outputs_close, assert_pyramid_equal, assert_selection_equal, cprob, gpu_prefill, log,
                    oracle_attend, oracle_select, split_levels, to_dev, to_host)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

P = gen.Problem
SHARP = (1.0, 1.0, 1.0 / math.sqrt(128))

CASES = {
    "bidir_gqa_ragged": (P(2, 8, 2, 4000, 128, 128, 4, 3, 4, 64, "bf16", causal=False), ("uniform_pairs", 4), None),
    "bidir_fp32": (P(1, 2, 1, 700, 64, 64, 2, 3, 2, 0, "f32", causal=False), ("uniform_pairs", 2), 1.0),
    "bidir_wide_sink_bs32": (P(1, 4, 4, 2048, 64, 32, 4, 3, 4, 100, "bf16", causal=False), ("uniform_pairs", 4),
                             None),
    "bidir_sink_beyond_n": (P(1, 2, 1, 50, 128, 32, 4, 2, 4, 64, "bf16", causal=False), None, None),
    "bidir_sharp": (P(1, 8, 2, 8192, 128, 128, 8, 3, 8, 64, "bf16", causal=False), ("uniform_depth", 8), SHARP),
    "max_gqa_ragged": (P(2, 8, 2, 4000, 128, 128, 4, 3, 4, 64, "bf16", pool="max"), ("uniform_pairs", 4), None),
    "max_fp32_deep": (P(1, 4, 2, 3000, 64, 32, 2, 5, 5, 40, "f32", pool="max"), ("log_distance", 8), 1.0),
    "bidir_max_mha_bs64": (P(1, 4, 4, 3000, 128, 64, 8, 2, 6, 64, "bf16", causal=False, pool="max"),
                           ("uniform_pairs", 4), None),
}


@pytest.mark.parametrize("name", list(CASES))
def test_variant_prefill_parity(name):
    p, plant, scale = CASES[name]
    log(f"variant case {name}: {p}")
    s = scale if scale is not None else 1.0 / math.sqrt(p.head_dim)
    q, k, v, _ = gen.host_inputs(p, 23, s, plant)
    levels, gi, gc, out, lse = gpu_prefill(p, to_dev(q, p.dtype), to_dev(k, p.dtype), to_dev(v, p.dtype))
    pyr, oi, oc = oracle_select(p, q, k)
    assert_pyramid_equal(levels, pyr)
    assert_selection_equal(gi, gc, oi, oc)
    o, ol = oracle_attend(p, q, k, v, oi, oc)
    err = assert_outputs_close(p, to_host(out), o, lse, ol)
    log(f"  max abs err {err:.2e}")


def test_bidirectional_all_blocks_is_dense_attention():
    p = P(1, 4, 2, 1000, 128, 64, 4, 2, 16, 64, "bf16", causal=False)
    q, k, v, _ = gen.host_inputs(p, 2, SHARP, None)
    levels, gi, gc, out, lse = gpu_prefill(p, to_dev(q, p.dtype), to_dev(k, p.dtype), to_dev(v, p.dtype))
    j0 = p.sink_len // p.block_size  # every block past the sink is a candidate, the query's own aside
    want = np.array([p.n_blocks - j0 - (1 if qb >= j0 else 0) for qb in range(p.n_blocks)])
    assert np.all(gc == want[None, None, :])
    G = p.group
    qt = torch.from_numpy(q.astype(np.float64))
    kt = torch.from_numpy(np.repeat(k.astype(np.float64), G, axis=1))
    vt = torch.from_numpy(np.repeat(v.astype(np.float64), G, axis=1))
    dense = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=p.scale).numpy()
    assert_outputs_close(p, to_host(out), dense)


def test_max_pool_decode_and_append():
    import block_sparse_long_pisa_amd as pisa

    p = P(3, 8, 2, 4096, 128, 128, 4, 3, 4, 64, "bf16", decode=True, pool="max")
    q, k, v, _ = gen.host_decode_inputs(p, 31, 1.0 / math.sqrt(128), 3000)
    cp = cprob(p)
    kd, vd = to_dev(k, p.dtype), to_dev(v, p.dtype)
    pyr = pisa.build_pyramid(cp, kd)
    opyr = oracle.build_pyramid(k, p.block_size, p.fanout, p.levels, pool="max")
    assert_pyramid_equal(split_levels(to_host(pyr), pisa.pyramid_layout(cp)), opyr)
    for n in (3000, 129):
        out, lse, idx, cnt = pisa.decode_step(cp, to_dev(q, p.dtype), kd, vd, pyr, n, want_lse=True, want_idx=True)
        torch.cuda.synchronize()
        o, ol, oi, oc = oracle.decode(q, k, v, opyr, n, p.top_k, p.sink_len, p.block_size, p.fanout, p.scale)
        assert np.array_equal(to_host(cnt), oc) and np.array_equal(to_host(idx), oi)
        assert_outputs_close(p, to_host(out), o, to_host(lse), ol)
    # append: tokens [old, new) of each sequence; nodes holding tokens before new equal a fresh max build
    old, new = [100, 2000, 4000], [101, 2300, 4096]
    pisa.pyramid_append(cp, kd, pyr, torch.tensor(old, dtype=torch.int32, device="cuda"),
                        torch.tensor(new, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    levels = split_levels(to_host(pyr), pisa.pyramid_layout(cp))
    for b in range(p.batch):
        want = oracle.build_pyramid(k[b:b + 1, :, :new[b]], p.block_size, p.fanout, p.levels, pool="max")
        for l, w in enumerate(want):
            assert np.array_equal(levels[l][b:b + 1, :, :w.shape[2]].view(np.uint32), w.view(np.uint32))


def test_unimplemented_variants_fail_on_the_host():
    import block_sparse_long_pisa_amd as pisa

    p = P(1, 4, 2, 1024, 128, 64, 4, 2, 4, 64, "bf16", decode=True, causal=False)
    cp = cprob(p)
    q = torch.zeros((1, 4, 128), dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros((1, 2, 1024, 128), dtype=torch.bfloat16, device="cuda")
    pyr = pisa.build_pyramid(cp, kc)
    with pytest.raises(pisa.PisaError, match="unsupported"):
        pisa.decode_step(cp, q, kc, kc, pyr, 100)
    qf = torch.zeros((1, 4, 1024, 128), dtype=torch.bfloat16, device="cuda")
    out, lse, idx, cnt, _ = pisa.prefill(cp, qf, kc, kc, want_lse=True)
    with pytest.raises(pisa.PisaError, match="unsupported"):
        pisa.sparse_attn_bwd(cp, qf, kc, kc, idx, cnt, out, lse, qf)
