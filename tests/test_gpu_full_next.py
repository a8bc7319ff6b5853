"""Full-size parity of the serving path, the backward pass and the variants, at
the shapes the bench times (inputs drawn on the GPU, copied to the host for the
oracle; outputs compared on samples the oracle computes unit by unit).

* backward, 128K GQA workload: dq on sampled query blocks; dk and dv on
  sampled key blocks, each with every unit that attends it summed by the oracle;
* variants on the same workload: every pyramid summary and every selection
  bit-exact, outputs on sampled query blocks;
* serving, 64 x 128K decode workload at ragged lengths: one appended token per
  sequence, then a ragged decode; the appended pyramid nodes and the decode of
  sampled sequences against the oracle.
"""

import numpy as np
import pytest

import gen
import oracle
from parity import (assert_outputs_close, assert_pyramid_equal, assert_selection_equal, cprob, grads_close, log,
                    split_levels, to_host)
from test_gpu_full import _sample_units

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.mark.timeout(900)
def test_full_backward_128k_gqa():
    import block_sparse_long_pisa_amd as pisa

    c = gen.workload(3)
    p = c["problem"]
    log(f"backward at full size: {c['name']}")
    q, k, v, man = gen.device_inputs(p, c["seed"], c["value_scale"], c["plant"], device="cuda")
    cp = cprob(p)
    out, lse, idx, cnt, _ = pisa.prefill(cp, q, k, v, want_lse=True)
    gen_do = torch.Generator(device="cuda")
    gen_do.manual_seed(77)
    dout = torch.randn(q.shape, generator=gen_do, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    dq, dk, dv = pisa.sparse_attn_bwd(cp, q, k, v, idx, cnt, out, lse, dout)
    torch.cuda.synchronize()
    qh, kh, vh, doh = to_host(q), to_host(k), to_host(v), to_host(dout)
    gdq, gdk, gdv = to_host(dq), to_host(dk), to_host(dv)
    gi, gc = to_host(idx), to_host(cnt)
    del q, k, v, dout, dq, dk, dv, out, lse
    log("  GPU done; oracle selection")
    o_levels = oracle.build_pyramid(kh, p.block_size, p.fanout, p.levels)
    oi, oc = oracle.select(o_levels, oracle.query_block_means(qh, p.heads_kv, p.block_size), p.top_k, p.sink_len,
                           p.block_size, p.fanout)
    assert_selection_equal(gi, gc, oi, oc)
    G, bs, nb = p.group, p.block_size, p.n_blocks
    units = _sample_units(p, man, n_random=6)
    want = oracle.attend_backward(qh, kh, vh, oi, oc, doh, p.sink_len, bs, p.scale, units=units)
    for (b, g, qb) in units:
        rows = slice(qb * bs, min(p.seq_len, (qb + 1) * bs))
        heads = slice(g * G, (g + 1) * G)
        grads_close(f"dq unit {(b, g, qb)}", gdq[b, heads, rows], want[0][b, heads, rows])
    log(f"  dq of {len(units)} sampled query blocks within the bar")
    rng = np.random.default_rng(5)
    for _ in range(3):
        g, j = int(rng.integers(p.heads_kv)), int(rng.integers(1, nb - 1))
        attending = [(0, g, qb) for qb in range(j, nb) if qb == j or j in oi[0, g, qb, :oc[0, g, qb]].tolist()]
        _, wk, wv = oracle.attend_backward(qh, kh, vh, oi, oc, doh, p.sink_len, bs, p.scale, units=attending)
        keys = slice(j * bs, (j + 1) * bs)
        a = grads_close(f"dk block {(g, j)}", gdk[0, g, keys], wk[0, g, keys])
        bb = grads_close(f"dv block {(g, j)}", gdv[0, g, keys], wv[0, g, keys])
        log(f"  key block {j} of kv head {g}: {len(attending)} attending blocks; dk rel L2 {a[1]:.2e}, "
            f"dv rel L2 {bb[1]:.2e}")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("causal,pool", [(False, "mean"), (True, "max")])
def test_full_variants_128k_gqa(causal, pool):
    import block_sparse_long_pisa_amd as pisa

    c = gen.workload(3)
    p = c["problem"].replace(causal=causal, pool=pool)
    log(f"variant causal={causal} pool={pool} at full size: {c['name']}")
    q, k, v, man = gen.device_inputs(p, c["seed"], c["value_scale"], c["plant"], device="cuda")
    cp = cprob(p)
    out, lse, idx, cnt, pyr = pisa.prefill(cp, q, k, v, want_lse=True)
    torch.cuda.synchronize()
    g_levels = split_levels(to_host(pyr), pisa.pyramid_layout(cp))
    gi, gc = to_host(idx), to_host(cnt)
    qh, kh, vh = to_host(q), to_host(k), to_host(v)
    o_levels = oracle.build_pyramid(kh, p.block_size, p.fanout, p.levels, pool=pool)
    assert_pyramid_equal(g_levels, o_levels)
    oi, oc = oracle.select(o_levels, oracle.query_block_means(qh, p.heads_kv, p.block_size), p.top_k, p.sink_len,
                           p.block_size, p.fanout, causal=causal)
    assert_selection_equal(gi, gc, oi, oc)
    log(f"  pyramid and {oc.size} selections bit-exact")
    units = _sample_units(p, man, n_random=8)
    o, ol = oracle.attend(qh, kh, vh, oi, oc, p.sink_len, p.block_size, p.scale, blocks=units, causal=causal)
    err = assert_outputs_close(p, to_host(out), o, to_host(lse), ol)
    log(f"  sampled outputs: max abs err {err:.2e}")


@pytest.mark.timeout(900)
def test_full_serving_64x128k_ragged():
    import block_sparse_long_pisa_amd as pisa

    c = gen.workload(4)
    p = c["problem"]
    log(f"serving at full size: {c['name']}, ragged lengths")
    qd, kc, vc, _ = gen.device_decode_inputs(p, c["seed"], c["value_scale"], p.seq_len, device="cuda")
    cp = cprob(p)
    pyr = pisa.build_pyramid(cp, kc)
    rng = np.random.default_rng(11)
    old = rng.integers(p.seq_len // 2, p.seq_len, size=p.batch).astype(np.int32)
    new = old + 1
    pisa.pyramid_append(cp, kc, pyr, torch.from_numpy(old).cuda(), torch.from_numpy(new).cuda())
    out, lse, idx, cnt = pisa.decode_step_ragged(cp, qd, kc, vc, pyr, torch.from_numpy(new).cuda(), want_lse=True,
                                                 want_idx=True)
    torch.cuda.synchronize()
    offs = pisa.pyramid_layout(cp)
    qh = to_host(qd)
    oh, lh, gi, gc = to_host(out), to_host(lse), to_host(idx), to_host(cnt)
    for b in (0, 17, 42, 63):
        n = int(new[b])
        kb, vb = to_host(kc[b:b + 1]), to_host(vc[b:b + 1])
        g_levels = split_levels(to_host(pyr[b:b + 1]), offs)
        prefix = oracle.build_pyramid(kb[:, :, :n], p.block_size, p.fanout, p.levels)
        for l, w in enumerate(prefix):  # every node holding a token before n, as a fresh build of n tokens
            assert np.array_equal(g_levels[l][:, :, :w.shape[2]].view(np.uint32), w.view(np.uint32)), (b, l)
        o, ol, oi, oc = oracle.decode_ragged(qh[b:b + 1], kb, vb, prefix, [n], p.top_k, p.sink_len, p.block_size,
                                             p.fanout, p.scale)
        assert np.array_equal(gc[b:b + 1], oc) and np.array_equal(gi[b:b + 1], oi)
        err = assert_outputs_close(p, oh[b:b + 1], o, lh[b:b + 1], ol)
        log(f"  sequence {b} at length {n}: appended pyramid bit-exact, max abs err {err:.2e}")
