"""GPU parity of the serving path: decode over a batch of sequences with different
cache lengths, and the pyramid kept up to date as tokens are appended.

* ragged decode: every sequence against the oracle's single-sequence decode at
  its own length (selected blocks bit-exact, outputs within the dtype's bar);
  out-of-range lengths attend nothing (zeros, lse -inf, no blocks);
* pyramid append: every node holding a token before the new length equals,
  bit for bit, the oracle's pyramid of exactly that many tokens; every node the
  append does not reach keeps its old value;
* a short serving loop (append the new token, update the pyramid, decode) checked
  step by step against the oracle;
* the append of a step run before, after and beside that step's decode: the same
  results bit for bit;
* the append and the decode in one call (pisa_decode_step_ragged_append) against
  the two calls, bit for bit.
"""

import math

import numpy as np
import pytest

import gen
import oracle
from parity import assert_outputs_close, cprob, log, split_levels, to_dev, to_host

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

P = gen.Problem

RAGGED = {
    "gqa4_bs64": (P(8, 8, 2, 3000, 128, 64, 4, 3, 6, 64, "bf16"), [1, 63, 64, 65, 1500, 3000, 0, 2999]),
    "gqa4_bs128_deep": (P(4, 16, 4, 8192, 128, 128, 8, 3, 16, 64, "bf16"), [8192, 129, 5000, 8193]),
    "group8_d64": (P(3, 16, 2, 2048, 64, 32, 4, 3, 5, 40, "bf16"), [2048, 40, 1000]),
    "fp32_group1": (P(4, 2, 2, 700, 64, 32, 4, 2, 3, 40, "f32"), [700, 1, 33, -5]),
    "k0": (P(2, 4, 1, 1024, 128, 128, 4, 2, 0, 64, "bf16"), [1024, 300]),
}


def _scale(p):
    return 1.0 if p.dtype == "f32" else 1.0 / math.sqrt(p.head_dim)


def _check_decode(p, lens, out, lse, idx, cnt, o, ol, oi, oc):
    valid = np.array([1 <= n <= p.seq_len for n in lens])
    assert np.array_equal(to_host(cnt), oc)
    if p.top_k:
        assert np.array_equal(to_host(idx), oi)
    go, gl = to_host(out), to_host(lse)
    if valid.any():
        mask = np.zeros(go.shape[:2], bool)
        mask[valid] = True
        err = assert_outputs_close(p, go, o, gl, ol, rows_mask=mask)
    else:
        err = 0.0
    if (~valid).any():
        assert np.all(go[~valid] == 0.0) and np.all(np.isneginf(gl[~valid]))
    return err


@pytest.mark.parametrize("name", list(RAGGED))
def test_ragged_decode_parity(name):
    import block_sparse_long_pisa_amd as pisa

    p, lens = RAGGED[name]
    p = p.replace(decode=True)
    log(f"ragged decode case {name}: {p}, lengths {lens}")
    q, k, v, _ = gen.host_decode_inputs(p, 40 + len(lens), _scale(p), p.seq_len)
    cp = cprob(p)
    kd, vd = to_dev(k, p.dtype), to_dev(v, p.dtype)
    pyr = pisa.build_pyramid(cp, kd)
    dl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    out, lse, idx, cnt = pisa.decode_step_ragged(cp, to_dev(q, p.dtype), kd, vd, pyr, dl, want_lse=True,
                                                 want_idx=True)
    torch.cuda.synchronize()
    opyr = oracle.build_pyramid(k, p.block_size, p.fanout, p.levels)
    o, ol, oi, oc = oracle.decode_ragged(q, k, v, opyr, lens, p.top_k, p.sink_len, p.block_size, p.fanout, p.scale)
    err = _check_decode(p, lens, out, lse, idx, cnt, o, ol, oi, oc)
    log(f"  max abs err {err:.2e}")


def test_uniform_lengths_match_the_scalar_decode_bit_for_bit():
    import block_sparse_long_pisa_amd as pisa

    p = P(3, 8, 2, 4096, 128, 128, 4, 3, 4, 64, "bf16", decode=True)
    q, k, v, _ = gen.host_decode_inputs(p, 77, _scale(p), 3000)
    cp = cprob(p)
    qd, kd, vd = to_dev(q, p.dtype), to_dev(k, p.dtype), to_dev(v, p.dtype)
    pyr = pisa.build_pyramid(cp, kd)
    a = pisa.decode_step(cp, qd, kd, vd, pyr, 3000, want_lse=True, want_idx=True)
    dl = torch.full((p.batch,), 3000, dtype=torch.int32, device="cuda")
    b = pisa.decode_step_ragged(cp, qd, kd, vd, pyr, dl, want_lse=True, want_idx=True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def _node_meets(l, n, p, lo, hi):
    """Does node n of level l hold a token in [lo, hi)?"""
    span = p.block_size * p.fanout ** l
    return n * span < hi and (n + 1) * span > lo


def _check_prefix_pyramid(p, gpu_levels, k, b, n):
    """Nodes holding tokens before n equal the oracle pyramid of the first n tokens of sequence b."""
    want = oracle.build_pyramid(k[b:b + 1, :, :n], p.block_size, p.fanout, p.levels)
    for l, w in enumerate(want):
        got = gpu_levels[l][b:b + 1, :, :w.shape[2]]
        bad = np.argwhere(got.view(np.uint32) != w.view(np.uint32))
        assert bad.size == 0, f"sequence {b}, length {n}, level {l}: {len(bad)} summaries differ"


APPEND = {
    "bf16_bs64_ragged_cap": (P(6, 4, 2, 2000, 128, 64, 4, 3, 4, 64, "bf16"),
                             [0, 5, 63, 64, 127, 1999], [1, 6, 64, 65, 400, 2000]),
    "f32_d64_fanout2_deep": (P(4, 2, 1, 1500, 64, 32, 2, 5, 3, 32, "f32"),
                             [31, 0, 700, 1499], [32, 1500, 701, 1499]),
    "bf16_one_level": (P(2, 2, 2, 1024, 128, 128, 4, 1, 2, 64, "bf16"), [100, 1000], [101, 1024]),
    # one leaf deep in a fanout-16 tree: 15 complete siblings at each of its three
    # coarser levels, and a leaf just past a level-2 node boundary
    "bf16_fanout16_many_siblings": (P(2, 1, 1, 131072, 128, 32, 16, 4, 4, 64, "bf16"), [131070, 4096],
                                    [131071, 4097]),
}


@pytest.mark.parametrize("name", list(APPEND))
def test_pyramid_append_equals_a_fresh_build_of_the_prefix(name):
    import block_sparse_long_pisa_amd as pisa

    p, old, new = APPEND[name]
    log(f"append case {name}: {p}, {old} -> {new}")
    q, k, v, _ = gen.host_decode_inputs(p.replace(decode=True), 13, _scale(p), p.seq_len)
    cp = cprob(p)
    kd = to_dev(k, p.dtype)
    offs = pisa.pyramid_layout(cp)
    pyr = pisa.build_pyramid(cp, kd)  # over the whole capacity: stale wherever a node meets [old, new)
    before = split_levels(to_host(pyr), offs)
    pisa.pyramid_append(cp, kd, pyr, torch.tensor(old, dtype=torch.int32, device="cuda"),
                        torch.tensor(new, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    after = split_levels(to_host(pyr), offs)
    for b in range(p.batch):
        if new[b] > old[b]:
            _check_prefix_pyramid(p, after, k, b, new[b])
        for l in range(p.levels):
            for n in range(after[l].shape[2]):
                if not (new[b] > old[b] and _node_meets(l, n, p, old[b], new[b])):
                    assert np.array_equal(after[l][b, :, n].view(np.uint32), before[l][b, :, n].view(np.uint32)), \
                        f"sequence {b}: node {n} of level {l} was written but holds no appended token"


def test_serving_loop_append_then_decode():
    """Each step: the new token's K/V land in the cache, the pyramid is updated,
    and the batch decodes at its new lengths -- against the oracle every step."""
    import block_sparse_long_pisa_amd as pisa

    p = P(4, 8, 2, 1200, 128, 64, 4, 3, 4, 64, "bf16", decode=True)
    start = [1, 130, 700, 1195]
    steps = 4
    q, k, v, _ = gen.host_decode_inputs(p, 91, _scale(p), p.seq_len)
    cp = cprob(p)
    kd, vd = to_dev(k, p.dtype), to_dev(v, p.dtype)
    # the caches hold garbage past each sequence's length until a token is appended
    for b, n in enumerate(start):
        kd[b, :, n:] = 7.0
        vd[b, :, n:] = -7.0
    pyr = pisa.build_pyramid(cp, kd)
    lens = list(start)
    ws = torch.empty(max(1, pisa.decode_workspace_size(cp)), dtype=torch.uint8, device="cuda")
    rng = np.random.default_rng(3)
    qs = gen.round_to_bf16((rng.standard_normal((steps, p.batch, p.heads_q, p.head_dim)) /
                            math.sqrt(p.head_dim)).astype(np.float32))
    for s in range(steps):
        old = list(lens)
        lens = [n + 1 for n in lens]
        for b, n in enumerate(lens):  # the new token's key and value
            kd[b, :, n - 1] = to_dev(k[b, :, n - 1], p.dtype)
            vd[b, :, n - 1] = to_dev(v[b, :, n - 1], p.dtype)
        pisa.pyramid_append(cp, kd, pyr, torch.tensor(old, dtype=torch.int32, device="cuda"),
                            torch.tensor(lens, dtype=torch.int32, device="cuda"))
        dl = torch.tensor(lens, dtype=torch.int32, device="cuda")
        out, lse, idx, cnt = pisa.decode_step_ragged(cp, to_dev(qs[s], p.dtype), kd, vd, pyr, dl, want_lse=True,
                                                     want_idx=True, workspace=ws)
        torch.cuda.synchronize()
        kh, vh = to_host(kd), to_host(vd)
        opyr = oracle.build_pyramid(kh, p.block_size, p.fanout, p.levels)
        # the oracle reads only complete nodes before each token's ancestors, so a
        # pyramid of the capacity (garbage included) serves every length
        o, ol, oi, oc = oracle.decode_ragged(qs[s], kh, vh, opyr, lens, p.top_k, p.sink_len, p.block_size, p.fanout,
                                             p.scale)
        err = _check_decode(p.replace(seq_len=p.seq_len), lens, out, lse, idx, cnt, o, ol, oi, oc)
        levels = split_levels(to_host(pyr), pisa.pyramid_layout(cp))
        for b, n in enumerate(lens):
            _check_prefix_pyramid(p, levels, kh, b, n)
        log(f"  step {s}: lengths {lens}, max abs err {err:.2e}")


def test_append_may_run_beside_the_decode_of_its_step():
    """The decode at length n scores only complete pyramid nodes, and the append
    of its token n - 1 writes only that token's leaf and its ancestors, none of
    them complete: so the append of a step may run after, or beside, that step's
    decode (the next decode must follow it). Three orders of the same loop --
    append then decode, decode then append, and the append on a second stream
    beside the decode -- give the same results bit for bit, with lengths that
    cross block boundaries."""
    import block_sparse_long_pisa_amd as pisa

    p = P(4, 8, 2, 1200, 128, 64, 4, 3, 4, 64, "bf16", decode=True)
    start = [62, 127, 640, 1190]
    steps = 4
    q, k, v, _ = gen.host_decode_inputs(p, 93, _scale(p), p.seq_len)
    cp = cprob(p)
    rng = np.random.default_rng(5)
    qs = [to_dev(gen.round_to_bf16((rng.standard_normal((p.batch, p.heads_q, p.head_dim)) /
                                    math.sqrt(p.head_dim)).astype(np.float32)), p.dtype) for _ in range(steps)]
    lens = [[n + s for n in start] for s in range(steps + 1)]
    lens_d = [torch.tensor(l, dtype=torch.int32, device="cuda") for l in lens]
    kd, vd = to_dev(k, p.dtype), to_dev(v, p.dtype)  # every token's key and value already in the cache

    def run(order):
        # a build over the whole capacity: the nodes a decode reads (complete ones)
        # are exact, and each append brings its token's nodes to the prefix state
        pyr = pisa.build_pyramid(cp, kd)
        ws = torch.empty(max(1, pisa.decode_workspace_size(cp)), dtype=torch.uint8, device="cuda")
        side = torch.cuda.Stream()
        res = []
        appended = torch.cuda.Event()
        for s in range(steps):
            if order == "append_first":
                pisa.pyramid_append(cp, kd, pyr, lens_d[s], lens_d[s + 1])
                r = pisa.decode_step_ragged(cp, qs[s], kd, vd, pyr, lens_d[s + 1], want_lse=True, want_idx=True,
                                            workspace=ws)
            elif order == "decode_first":
                r = pisa.decode_step_ragged(cp, qs[s], kd, vd, pyr, lens_d[s + 1], want_lse=True, want_idx=True,
                                            workspace=ws)
                pisa.pyramid_append(cp, kd, pyr, lens_d[s], lens_d[s + 1])
            else:  # the append on a second stream, beside the decode
                main = torch.cuda.current_stream()
                side.wait_stream(main)
                with torch.cuda.stream(side):
                    pisa.pyramid_append(cp, kd, pyr, lens_d[s], lens_d[s + 1])
                    appended.record(side)
                r = pisa.decode_step_ragged(cp, qs[s], kd, vd, pyr, lens_d[s + 1], want_lse=True, want_idx=True,
                                            workspace=ws)
                main.wait_event(appended)  # the next decode follows this append
            res.append([to_host(x).copy() for x in r])
        torch.cuda.synchronize()
        return res, to_host(pyr)

    a, pa = run("append_first")
    b, pb = run("decode_first")
    c, pc = run("beside")
    assert np.array_equal(pa, pb) and np.array_equal(pa, pc)
    for s in range(steps):
        for x, y, z in zip(a[s], b[s], c[s]):
            assert np.array_equal(x, y) and np.array_equal(x, z), f"step {s}"
    log(f"  lengths {lens[0]} -> {lens[-1]}: three orders identical, counts {a[-1][3].reshape(-1).tolist()}")


ONE_CALL = {
    "gqa4_bs64_mean": P(4, 8, 2, 1200, 128, 64, 4, 3, 4, 64, "bf16", decode=True),
    "gqa4_bs64_max": P(4, 8, 2, 1200, 128, 64, 4, 3, 4, 64, "bf16", decode=True, pool="max"),
    "fp32_group1_bs32": P(4, 2, 2, 700, 64, 32, 4, 3, 3, 40, "f32", decode=True),
    "group8_bs128": P(2, 16, 2, 2048, 128, 128, 8, 2, 6, 64, "bf16", decode=True),
}


@pytest.mark.parametrize("name", list(ONE_CALL))
def test_append_and_decode_in_one_call_match_the_two_calls(name):
    """pisa_decode_step_ragged_append against pisa_pyramid_append followed by
    pisa_decode_step_ragged: outputs, lse, selections and the whole pyramid equal
    bit for bit after every step. The steps append one token (the append beside
    the descent), several tokens across a block boundary (the selecting workgroup
    appends first), nothing (equal lengths), and a length past the capacity
    (nothing appended, nothing attended)."""
    import block_sparse_long_pisa_amd as pisa

    p = ONE_CALL[name]
    log(f"one-call append + decode {name}: {p}")
    cap, bs = p.seq_len, p.block_size
    q, k, v, _ = gen.host_decode_inputs(p, 71, _scale(p), cap)
    cp = cprob(p)
    kd, vd = to_dev(k, p.dtype), to_dev(v, p.dtype)
    start = [bs - 2, 2 * bs - 1, cap // 2, cap - 6][:p.batch] + [bs + 3] * max(0, p.batch - 4)
    deltas = [[1] * p.batch, [3] * p.batch, [1, 0, 1, 2][:p.batch] + [1] * max(0, p.batch - 4),
              [1] * (p.batch - 1) + [7], [bs + 1] * (p.batch - 1) + [0]]
    lens = [start]
    for d in deltas:
        lens.append([n + x for n, x in zip(lens[-1], d)])
    lens_d = [torch.tensor(l, dtype=torch.int32, device="cuda") for l in lens]
    rng = np.random.default_rng(6)
    tdt = torch.bfloat16 if p.dtype == "bf16" else torch.float32
    qs = [torch.from_numpy(gen.round_to_bf16((rng.standard_normal((p.batch, p.heads_q, p.head_dim)) *
                                              _scale(p)).astype(np.float32))).to(tdt).cuda() for _ in deltas]
    pyr_a = pisa.build_pyramid(cp, kd)  # the whole capacity: the nodes a decode reads are exact
    pyr_b = pyr_a.clone()
    ws = torch.empty(max(1, pisa.decode_workspace_size(cp)), dtype=torch.uint8, device="cuda")
    for s in range(len(deltas)):
        pisa.pyramid_append(cp, kd, pyr_a, lens_d[s], lens_d[s + 1])
        ra = pisa.decode_step_ragged(cp, qs[s], kd, vd, pyr_a, lens_d[s + 1], want_lse=True, want_idx=True,
                                     workspace=ws)
        ra = [to_host(x).copy() for x in ra]
        rb = pisa.decode_step_ragged_append(cp, qs[s], kd, vd, pyr_b, lens_d[s], lens_d[s + 1], want_lse=True,
                                            want_idx=True, workspace=ws)
        rb = [to_host(x).copy() for x in rb]
        torch.cuda.synchronize()
        for n, x, y in zip(("out", "lse", "idx", "cnt"), ra, rb):
            assert np.array_equal(x, y), f"step {s}: {n} differs"
        assert torch.equal(pyr_a, pyr_b), f"step {s}: pyramid differs"
    log(f"  lengths {lens[0]} -> {lens[-1]}: one call equals two, step by step")


def test_append_matches_the_build_bit_for_bit_on_keys_spanning_many_binades():
    """fp32 keys whose columns mix values near 1e4, 1 and 1e-12 (over 50 binades):
    the fp64 column sums of a block are then inexact, so only the same order of
    additions makes two summaries agree. The append must equal, bit for bit, a
    fresh build over exactly the appended prefix, and both stay within one fp32
    unit in the last place of the oracle (whose numpy sums add in another order)."""
    import block_sparse_long_pisa_amd as pisa

    p = P(3, 2, 2, 1000, 128, 128, 4, 3, 4, 64, "f32")
    rng = np.random.default_rng(77)
    k = rng.standard_normal((p.batch, p.heads_kv, p.seq_len, p.head_dim))
    scale = rng.choice(np.array([1e4, 1.0, 1e-12]), size=k.shape, p=[0.05, 0.45, 0.5])
    k = (k * scale).astype(np.float32)
    old, new = [0, 130, 900], [127, 385, 1000]
    cp = cprob(p)
    kd = to_dev(k, p.dtype)
    offs = pisa.pyramid_layout(cp)
    pyr = pisa.build_pyramid(cp, kd)
    pisa.pyramid_append(cp, kd, pyr, torch.tensor(old, dtype=torch.int32, device="cuda"),
                        torch.tensor(new, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    after = split_levels(to_host(pyr), offs)
    for b in range(p.batch):
        n = new[b]
        pb = p.replace(batch=1, seq_len=n)
        cpb = cprob(pb)
        fresh = split_levels(to_host(pisa.build_pyramid(cpb, to_dev(k[b:b + 1, :, :n], p.dtype))),
                             pisa.pyramid_layout(cpb))
        want = oracle.build_pyramid(k[b:b + 1, :, :n], p.block_size, p.fanout, p.levels)
        for l in range(p.levels):
            got = after[l][b:b + 1, :, :fresh[l].shape[2]]
            assert np.array_equal(got.view(np.uint32), fresh[l].view(np.uint32)), f"sequence {b}, level {l}"
            np.testing.assert_allclose(got, want[l], rtol=2.0 ** -22, atol=0.0)
