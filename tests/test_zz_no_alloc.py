"""The allocation-free decode entry point (pisa_decode_step_ragged_noalloc),
called through the C ABI: its workspace is the library's static per-GPU array.

Two calls in a row, the second on a smaller batch and shorter caches, each
compared bit for bit with pisa_decode_step_ragged on a caller workspace (the
same kernels, so the same bits), and the first also with the oracle; and a
problem too large for the static workspace is refused on the host.
"""

import math

import numpy as np
import pytest

import gen
import oracle
from parity import assert_outputs_close, cprob, log, to_dev, to_host

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

P = gen.Problem


def _run_both(p, lens, seed):
    import block_sparse_long_pisa_amd as pisa

    q, k, v, _ = gen.host_decode_inputs(p, seed, 1.0 / math.sqrt(p.head_dim), p.seq_len)
    cp = cprob(p)
    qd, kd, vd = to_dev(q, p.dtype), to_dev(k, p.dtype), to_dev(v, p.dtype)
    pyr = pisa.build_pyramid(cp, kd)
    dl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    ref = pisa.decode_step_ragged(cp, qd, kd, vd, pyr, dl, want_lse=True, want_idx=True)
    out = torch.full_like(qd, 7.0)
    lse = torch.full((p.batch, p.heads_q), 7.0, dtype=torch.float32, device="cuda")
    idx = torch.full((p.batch, p.heads_kv, p.top_k), 7, dtype=torch.int32, device="cuda")
    cnt = torch.full((p.batch, p.heads_kv), 7, dtype=torch.int32, device="cuda")
    pisa.decode_step_ragged_noalloc(cp, qd, kd, vd, pyr, dl, out, lse, idx, cnt)
    torch.cuda.synchronize()
    for name, a, b in zip(("out", "lse", "idx", "cnt"), (out, lse, idx, cnt), ref):
        assert torch.equal(a, b), f"{name} differs from pisa_decode_step_ragged"
    return q, k, v, (out, lse, idx, cnt)


def test_noalloc_decode_two_calls_second_smaller():
    first = P(8, 8, 2, 4096, 128, 128, 4, 3, 8, 64, "bf16", decode=True)
    lens1 = [4096, 1, 129, 3000, 4095, 2048, 640, 77]
    log(f"no-alloc decode call 1: {first}, lengths {lens1}")
    q, k, v, (out, lse, idx, cnt) = _run_both(first, lens1, 91)
    opyr = oracle.build_pyramid(k, first.block_size, first.fanout, first.levels)
    o, ol, oi, oc = oracle.decode_ragged(q, k, v, opyr, lens1, first.top_k, first.sink_len, first.block_size,
                                         first.fanout, first.scale)
    assert np.array_equal(to_host(cnt), oc) and np.array_equal(to_host(idx), oi)
    err = assert_outputs_close(first, to_host(out), o, to_host(lse), ol)
    log(f"  call 1 max abs err against the oracle {err:.2e}")

    second = P(3, 8, 2, 1024, 128, 128, 4, 3, 8, 64, "bf16", decode=True)
    lens2 = [1024, 200, 513]
    log(f"no-alloc decode call 2 (smaller): {second}, lengths {lens2}")
    _run_both(second, lens2, 92)


def test_noalloc_decode_refuses_a_problem_beyond_the_static_workspace():
    import block_sparse_long_pisa_amd as pisa

    # 512 (sequence, kv head) units x 11 splits x 8 query heads x d = 128 fp32 partials: 23 MB
    p = P(32, 128, 16, 2112, 128, 32, 4, 3, 64, 64, "bf16", decode=True)
    cp = cprob(p)
    assert pisa.decode_workspace_size(cp) > pisa.DECODE_SCRATCH_BYTES
    dev = "cuda"
    q = torch.zeros((p.batch, p.heads_q, p.head_dim), dtype=torch.bfloat16, device=dev)
    kc = torch.zeros((p.batch, p.heads_kv, p.seq_len, p.head_dim), dtype=torch.bfloat16, device=dev)
    nodes = pisa.pyramid_layout(cp)[-1]
    pyr = torch.zeros((p.batch, p.heads_kv, nodes, p.head_dim), dtype=torch.float32, device=dev)
    lens = torch.full((p.batch,), p.seq_len, dtype=torch.int32, device=dev)
    out = torch.full_like(q, 3.0)
    with pytest.raises(pisa.PisaError) as e:
        pisa.decode_step_ragged_noalloc(cp, q, kc, kc, pyr, lens, out)
    assert e.value.status == 4
    torch.cuda.synchronize()
    assert bool((out == 3.0).all()), "a refused call must write nothing"
