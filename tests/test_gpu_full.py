"""Parity at the workloads' full sizes, in the launch configuration the bench times.

Inputs are drawn on the GPU (gen.device_inputs) and copied to the host for the
oracle. Every pyramid summary and every selection is compared; attention
outputs are compared on sampled query blocks (the planted ones, the first and
last blocks, a seeded random sample and several hundred units spread evenly over
all of them), decode on sampled sequences.
"""

import math

import numpy as np
import pytest

import gen
import oracle
from parity import (assert_outputs_close, assert_pyramid_equal, assert_selection_equal, cprob, log, split_levels,
                    to_dev, to_host)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _sample_units(p, man, n_random=12, seed=0, n_spread=0):
    """Planted units, the first and last blocks, a seeded random sample, and
    n_spread units evenly spaced over all (batch, kv head, query block) units --
    over every slab and block position, and so over the attention's persistent
    workgroups and their item orders."""
    rng = np.random.default_rng(seed)
    units = set()
    for n in man["needles"][:12]:
        units.add((n["b"], n["g"], n["qb"]))
    nb = p.n_blocks
    for g in range(min(p.heads_kv, 2)):
        units.update({(0, g, 0), (0, g, 1), (0, g, nb - 1)})
    for _ in range(n_random):
        units.add((int(rng.integers(p.batch)), int(rng.integers(p.heads_kv)), int(rng.integers(nb))))
    if n_spread:
        total = p.batch * p.heads_kv * nb
        step = max(1, total // n_spread) | 1  # odd: the blocks of every slab fall at varied positions
        for u in range(step // 2, total, step):
            units.add((u // (p.heads_kv * nb), (u // nb) % p.heads_kv, u % nb))
    return sorted(units)


# units checked against the oracle per workload beyond the planted, edge and
# random ones (the oracle's cost per unit grows with the rows and keys it attends)
SPREAD = {2: 512, 3: 256, 5: 64}


@pytest.mark.timeout(900)
@pytest.mark.parametrize("workload_id", [1, 2, 3, 5])
def test_full_prefill(workload_id):
    import block_sparse_long_pisa_amd as pisa

    c = gen.workload(workload_id)
    p = c["problem"]
    log(f"workload {workload_id}: {c['name']}")
    if workload_id == 1:
        qh, kh, vh, man = gen.host_inputs(p, c["seed"], c["value_scale"], c["plant"])
        q, k, v = to_dev(qh, p.dtype), to_dev(kh, p.dtype), to_dev(vh, p.dtype)
    else:
        q, k, v, man = gen.device_inputs(p, c["seed"], c["value_scale"], c["plant"], device="cuda")
    cp = cprob(p)
    out, lse, idx, cnt, pyr = pisa.prefill(cp, q, k, v, want_lse=True)
    torch.cuda.synchronize()
    offs = pisa.pyramid_layout(cp)
    g_levels = split_levels(to_host(pyr), offs)
    gi, gc = to_host(idx), to_host(cnt)
    del pyr
    if workload_id != 1:
        qh, kh, vh = to_host(q), to_host(k), to_host(v)
    log("  GPU done; oracle pyramid")
    o_levels = oracle.build_pyramid(kh, p.block_size, p.fanout, p.levels)
    assert_pyramid_equal(g_levels, o_levels)
    log("  pyramid bit-exact; oracle selection of every query block")
    qbar = oracle.query_block_means(qh, p.heads_kv, p.block_size)
    traces = {}
    oi, oc = oracle.select(o_levels, qbar, p.top_k, p.sink_len, p.block_size, p.fanout, traces=traces)
    assert_selection_equal(gi, gc, oi, oc)
    # how close the keep/prune boundaries came to a tie, against the scores' size:
    # exact equality is meaningful because the smallest margin is far above the
    # rounding of an fp64 dot product of d terms (~d * 2^-53 relative)
    rel = [g / max(abs(t["scores"]).max(), 1e-300) for tr in traces.values()
           for t in tr if len(t["pool"]) > p.top_k
           for g in [oracle.selection_report([t], p.top_k, p.fanout)["gaps"][t["level"]]]]
    if rel:
        assert min(rel) > 1e3 * p.head_dim * 2.0 ** -53, f"a boundary within rounding of a tie: {min(rel):.2e}"
    dropped = sum(1 for n in man["needles"] if n["survived"] and oracle.selection_report(
        traces[(n["b"], n["g"], n["qb"])], p.top_k, p.fanout, [n["target"]])["pruned"][n["target"]] is not None)
    log(f"  {oc.size} selections bit-exact; smallest relative boundary margin "
        f"{min(rel) if rel else float('nan'):.2e}; planted blocks dropped by coarse levels: {dropped}; "
        "oracle attention on sampled blocks")
    units = _sample_units(p, man, n_spread=SPREAD[workload_id]) if workload_id != 1 else None
    o, ol = oracle.attend(qh, kh, vh, oi, oc, p.sink_len, p.block_size, p.scale, blocks=units)
    err = assert_outputs_close(p, to_host(out), o, to_host(lse), ol)
    found = sum(1 for n in man["needles"] if n["survived"] and n["target"] in oi[n["b"], n["g"], n["qb"]].tolist())
    log(f"  {len(units) if units else 'all'} units: max abs err {err:.2e}; planted blocks selected: "
        f"{found}/{sum(n['survived'] for n in man['needles'])}")


@pytest.mark.timeout(900)
def test_full_decode():
    import block_sparse_long_pisa_amd as pisa

    c = gen.workload(4)
    p = c["problem"]
    cache_len = p.seq_len
    log(f"config 4: {c['name']}")
    q, kc, vc, man = gen.device_decode_inputs(p, c["seed"], c["value_scale"], cache_len, device="cuda")
    cp = cprob(p)
    pyr = pisa.build_pyramid(cp, kc)
    out, lse, idx, cnt = pisa.decode_step(cp, q, kc, vc, pyr, cache_len, want_lse=True, want_idx=True)
    torch.cuda.synchronize()
    offs = pisa.pyramid_layout(cp)
    qh = to_host(q)
    oh, lh, gi, gc = to_host(out), to_host(lse), to_host(idx), to_host(cnt)
    for b in sorted({0, 17, 42, 63} | set(range(2, p.batch, 4))):  # 19 of the 64 sequences
        log(f"  sequence {b}")
        kb, vb = to_host(kc[b:b + 1]), to_host(vc[b:b + 1])
        g_levels = split_levels(to_host(pyr[b:b + 1]), offs)
        o_levels = oracle.build_pyramid(kb, p.block_size, p.fanout, p.levels)
        assert_pyramid_equal(g_levels, o_levels)
        o, ol, oi, oc = oracle.decode(qh[b:b + 1], kb, vb, o_levels, cache_len, p.top_k, p.sink_len, p.block_size,
                                      p.fanout, p.scale)
        assert np.array_equal(gc[b:b + 1], oc) and np.array_equal(gi[b:b + 1], oi)
        err = assert_outputs_close(p, oh[b:b + 1], o, lh[b:b + 1], ol)
        planted = [n for n in man["needles"] if n["b"] == b]
        found = sum(1 for n in planted if n["target"] in oi[0, n["g"]].tolist())
        log(f"    max abs err {err:.2e}; planted blocks selected {found}/{len(planted)}")


@pytest.mark.timeout(300)
def test_million_token_prefill_holds_no_score_matrix():
    """No N x N score matrix, nor any buffer beyond the call's own: at 1M tokens
    (one GQA group, 4 query heads), the prefill's peak device memory is the
    inputs, the outputs (out, lse), the pyramid, the selection (idx, cnt) and
    nothing else -- torch's allocator sees only those, and the driver's free
    memory drops by no more than what torch itself reserved (the library
    allocates nothing of its own)."""
    import block_sparse_long_pisa_amd as pisa

    c = gen.workload(5)
    p = c["problem"]
    cp = cprob(p)
    q, k, v, _ = gen.device_inputs(p, c["seed"], c["value_scale"], c["plant"], device="cuda")
    # load the library's code objects with one small call first
    small = gen.Problem(1, 4, 1, 4096, 128, 128, 8, 3, 8, 64, "bf16")
    qs, ks, vs, _ = gen.device_inputs(small, 5, c["value_scale"], None, device="cuda")
    pisa.prefill(cprob(small), qs, ks, vs, want_lse=True)
    del qs, ks, vs
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    reserved0 = torch.cuda.memory_reserved()
    free0 = torch.cuda.mem_get_info()[0]
    out, lse, idx, cnt, pyr = pisa.prefill(cp, q, k, v, want_lse=True)
    torch.cuda.synchronize()
    peak = torch.cuda.max_memory_allocated() - base
    nodes = pisa.pyramid_layout(cp)[-1]
    nb = p.n_blocks
    expected = (q.numel() * 2                                        # out
                + p.batch * p.heads_q * p.seq_len * 4                # lse
                + p.batch * p.heads_kv * nodes * p.head_dim * 4      # pyramid
                + p.batch * p.heads_kv * nb * (p.top_k + 1) * 4)     # idx, cnt
    allowance = 2 << 20  # allocator rounding of the five buffers
    log(f"  peak {peak / 2**20:.1f} MiB above the inputs; outputs, pyramid and selection {expected / 2**20:.1f} MiB")
    assert peak <= expected + allowance
    drop = free0 - torch.cuda.mem_get_info()[0]
    grown = torch.cuda.memory_reserved() - reserved0
    assert drop <= grown + allowance, f"device memory fell by {drop} bytes, torch reserved {grown}"
    dense = p.batch * p.heads_q * p.seq_len * p.seq_len * 2  # one bf16 score matrix
    assert peak < dense // 1000
    del out, lse, idx, cnt, pyr
