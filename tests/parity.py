"""Helpers for the GPU parity tests: run the HIP path through the C ABI, run the
oracle on the same inputs, compare. The oracle never sees a HIP result."""

from __future__ import annotations

import math
import sys
from typing import Optional, Sequence

import numpy as np

import block_sparse_long_pisa_amd as pisa
import gen
import oracle

BF16_MAX_ABS = 2e-3  # bf16 inputs: max-abs error of outputs against the fp64 oracle
F32_MAX_ABS = 1e-5  # fp32 inputs
BF16_ROW_REL = 1e-2  # per-row relative L2 (bf16), a sharper internal gate
LSE_ABS = {"bf16": 1e-3, "f32": 1e-5}


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def cprob(p: gen.Problem):
    return pisa.problem(p.batch, p.heads_q, p.heads_kv, p.seq_len, p.head_dim, p.block_size, p.fanout, p.levels,
                        p.top_k, p.sink_len, p.dtype, sm_scale=p.sm_scale, causal=int(p.causal), pool=p.pool)


def to_dev(x: np.ndarray, dtype: str):
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16 if dtype == "bf16" else torch.float32).cuda()


def to_host(t) -> np.ndarray:
    import torch

    return t.detach().to(torch.float32).cpu().numpy() if t.dtype in (torch.bfloat16, torch.float16) else t.detach().cpu().numpy()


def split_levels(pyr: np.ndarray, offs: Sequence[int]):
    return [pyr[:, :, offs[l]:offs[l + 1]] for l in range(len(offs) - 1)]


def gpu_prefill(p: gen.Problem, q, k, v, want_lse=True):
    """q, k, v: device tensors. Returns host arrays (levels, idx, cnt, out, lse)."""
    import torch

    cp = cprob(p)
    out, lse, idx, cnt, pyr = pisa.prefill(cp, q, k, v, want_lse=want_lse)
    torch.cuda.synchronize()
    offs = pisa.pyramid_layout(cp)
    return split_levels(to_host(pyr), offs), to_host(idx), to_host(cnt), out, (to_host(lse) if lse is not None else None)


def oracle_select(p: gen.Problem, q: np.ndarray, k: np.ndarray):
    pyr = oracle.build_pyramid(k, p.block_size, p.fanout, p.levels, pool=p.pool)
    qbar = oracle.query_block_means(q, p.heads_kv, p.block_size)
    idx, cnt = oracle.select(pyr, qbar, p.top_k, p.sink_len, p.block_size, p.fanout, causal=p.causal)
    return pyr, idx, cnt


def oracle_attend(p: gen.Problem, q, k, v, idx, cnt, blocks=None):
    return oracle.attend(q, k, v, idx, cnt, p.sink_len, p.block_size, p.scale, blocks=blocks, causal=p.causal)


def assert_pyramid_equal(gpu_levels, ora_levels):
    for l, (a, b) in enumerate(zip(gpu_levels, ora_levels)):
        assert a.shape == b.shape, (l, a.shape, b.shape)
        bad = np.argwhere(a.view(np.uint32) != b.view(np.uint32))
        assert bad.size == 0, f"level {l}: {len(bad)} summaries differ, first at {bad[0].tolist()}"


def assert_selection_equal(gi, gc, oi, oc):
    assert np.array_equal(gc, oc), f"cnt differs at {np.argwhere(gc != oc)[:5].tolist()}"
    bad = np.argwhere(np.any(gi != oi, axis=-1))
    assert bad.size == 0, f"{len(bad)} selections differ, first unit {bad[0].tolist()}: gpu {gi[tuple(bad[0])]} oracle {oi[tuple(bad[0])]}"


def assert_outputs_close(p: gen.Problem, o_gpu: np.ndarray, o_ora: np.ndarray, lse_gpu=None, lse_ora=None,
                         rows_mask: Optional[np.ndarray] = None):
    """Compare where the oracle computed (non-NaN)."""
    m = ~np.isnan(o_ora[..., 0]) if rows_mask is None else rows_mask
    a, b = o_gpu[m].astype(np.float64), o_ora[m]
    err = np.abs(a - b).max() if a.size else 0.0
    tol = BF16_MAX_ABS if p.dtype == "bf16" else F32_MAX_ABS
    assert err <= tol, f"max abs error {err:.3e} > {tol:.0e}"
    if p.dtype == "bf16" and a.size:
        rel = np.linalg.norm(a - b, axis=-1) / np.maximum(np.linalg.norm(b, axis=-1), 1e-30)
        assert rel.max() <= BF16_ROW_REL, f"row relative L2 {rel.max():.3e} > {BF16_ROW_REL}"
    if lse_gpu is not None and lse_ora is not None:
        d = np.abs(lse_gpu[m].astype(np.float64) - lse_ora[m]).max() if a.size else 0.0
        assert d <= LSE_ABS[p.dtype], f"lse error {d:.3e}"
    return err


GRAD_REL_L2 = 1e-2  # backward (bf16): per-tensor relative L2 error
GRAD_MAX_REL = 1e-2  # backward (bf16): max-abs error as a fraction of the tensor's largest gradient


def grads_close(name: str, got: np.ndarray, want: np.ndarray):
    """Backward bar: p and dS enter the products rounded to bf16 (relative 2^-9
    each), D_i uses the forward's bf16 output and the gradients are rounded to
    bf16 on output; summed over many keys the roundings largely cancel, so the bar
    is relative to the whole tensor. Returns (max error / max |want|, relative L2)."""
    g = got.astype(np.float64)
    err = np.abs(g - want)
    scale = np.abs(want).max()
    rel = np.linalg.norm(g - want) / max(np.linalg.norm(want), 1e-30)
    assert err.max() <= GRAD_MAX_REL * scale, f"{name}: max abs error {err.max():.3e} > {GRAD_MAX_REL} x {scale:.3e}"
    assert rel <= GRAD_REL_L2, f"{name}: relative L2 error {rel:.3e} > {GRAD_REL_L2}"
    return err.max() / max(scale, 1e-300), rel
