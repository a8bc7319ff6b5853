"""Pins for the oracle's backward pass of the sparse attention (selection held
constant): torch autograd of its own fp64 SDPA for the dense and the masked
case, and central finite differences of the oracle's forward."""

import numpy as np
import pytest
import torch

from oracle import attend, attend_backward, attended_keys, build_pyramid, query_block_means, select


def _case(seed, B, Hq, Hkv, N, d):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, N, d))
    k = rng.standard_normal((B, Hkv, N, d))
    v = rng.standard_normal((B, Hkv, N, d))
    do = rng.standard_normal((B, Hq, N, d))
    return q, k, v, do


def _autograd(q, k, v, do, mask, scale):
    """Gradients by torch autograd of fp64 SDPA (mask None -> causal); GQA by repeating the KV heads."""
    G = q.shape[1] // k.shape[1]
    qt = torch.tensor(q, requires_grad=True)
    kt = torch.tensor(k, requires_grad=True)
    vt = torch.tensor(v, requires_grad=True)
    kr = kt.repeat_interleave(G, dim=1)
    vr = vt.repeat_interleave(G, dim=1)
    m = None if mask is None else torch.from_numpy(np.repeat(mask, G, axis=1))
    o = torch.nn.functional.scaled_dot_product_attention(qt, kr, vr, attn_mask=m, is_causal=mask is None, scale=scale)
    (o * torch.from_numpy(do)).sum().backward()
    return qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy()


def _selection(q, k, bs, f, L, K, sink):
    pyr = build_pyramid(k.astype(np.float32), bs, f, L)
    return select(pyr, query_block_means(q.astype(np.float32), k.shape[1], bs), K, sink, bs, f)


@pytest.mark.parametrize("sink", [0, 8, 20])
def test_all_blocks_selected_is_dense_causal_autograd(sink):
    B, Hq, Hkv, N, d, bs = 1, 4, 2, 70, 8, 16
    q, k, v, do = _case(1, B, Hq, Hkv, N, d)
    idx, cnt = _selection(q, k, bs, 2, 3, 8, sink)  # K = 8 >= every earlier block
    got = attend_backward(q, k, v, idx, cnt, do, sink, bs, 0.3)
    want = _autograd(q, k, v, do, None, 0.3)
    for a, b in zip(got, want):
        assert np.max(np.abs(a - b)) < 1e-11


@pytest.mark.parametrize("K,sink", [(1, 0), (2, 12), (0, 16)])
def test_fixed_selection_is_masked_sdpa_autograd(K, sink):
    B, Hq, Hkv, N, d, bs = 2, 2, 1, 90, 8, 16
    q, k, v, do = _case(2 + K, B, Hq, Hkv, N, d)
    idx, cnt = _selection(q, k, bs, 2, 3, K, sink)
    mask = np.zeros((B, Hkv, N, N), dtype=bool)
    for b in range(B):
        for i in range(N):
            sel = idx[b, 0, i // bs, :cnt[b, 0, i // bs]].tolist()
            mask[b, 0, i, attended_keys(i, sel, sink, bs)] = True
    got = attend_backward(q, k, v, idx, cnt, do, sink, bs, 0.5)
    want = _autograd(q, k, v, do, mask, 0.5)
    for a, b in zip(got, want):
        assert np.max(np.abs(a - b)) < 1e-11


def test_central_differences_of_the_forward():
    # L(x) = sum(do * attend(x)); dL/dx_e ~ (L(x + h e) - L(x - h e)) / 2h, with the
    # selection computed once and held fixed
    B, Hq, Hkv, N, d, bs, sink, scale = 1, 2, 1, 40, 4, 8, 4, 0.7
    q, k, v, do = _case(7, B, Hq, Hkv, N, d)
    idx, cnt = _selection(q, k, bs, 2, 2, 2, sink)
    dq, dk, dv = attend_backward(q, k, v, idx, cnt, do, sink, bs, scale)

    def loss(q_, k_, v_):
        o, _ = attend(q_, k_, v_, idx, cnt, sink, bs, scale)
        return float(np.sum(do * o))

    rng = np.random.default_rng(0)
    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for _ in range(12):
            e = tuple(int(rng.integers(0, n)) for n in x.shape)
            xp, xm = x.copy(), x.copy()
            xp[e] += h
            xm[e] -= h
            args_p = {"q": (xp, k, v), "k": (q, xp, v), "v": (q, k, xp)}[name]
            args_m = {"q": (xm, k, v), "k": (q, xm, v), "v": (q, k, xm)}[name]
            fd = (loss(*args_p) - loss(*args_m)) / (2 * h)
            assert abs(fd - g[e]) < 1e-6 * max(1.0, abs(g[e])), (name, e, fd, g[e])
