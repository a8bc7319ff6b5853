"""Python binding of the PISA block-sparse attention library (libpisa.so, gfx950).

Argument marshalling only: every step runs in the HIP library. Tensors are
torch device tensors (torch provides memory and the current stream); the
library itself never allocates. If the library is missing the import of this
module still works, but every call raises: there is no CPU fallback.
"""

from __future__ import annotations

import ctypes
import math
import os
from typing import List, Optional, Sequence, Tuple

__all__ = [
    "PisaError",
    "Problem",
    "F32",
    "BF16",
    "POOL_MEAN",
    "POOL_MAX",
    "EXPORTED_SYMBOLS",
    "library_path",
    "load_library",
    "problem",
    "pyramid_layout",
    "build_pyramid",
    "select_topk",
    "sparse_attn_fwd",
    "select_attend",
    "sparse_attn_bwd_workspace_size",
    "sparse_attn_bwd",
    "decode_workspace_size",
    "decode_step",
    "decode_step_ragged",
    "decode_step_ragged_noalloc",
    "decode_step_ragged_append",
    "DECODE_SCRATCH_BYTES",
    "pyramid_append",
    "prefill",
]

F32, BF16 = 0, 1
_STATUS = {0: "ok", 1: "null pointer", 2: "invalid shape", 3: "unsupported", 4: "workspace too small",
           5: "HIP error", 6: "misaligned pointer"}
EXPORTED_SYMBOLS = [
    "pisa_pyramid_layout",
    "pisa_build_pyramid",
    "pisa_select_topk",
    "pisa_sparse_attn_fwd",
    "pisa_select_attend",
    "pisa_sparse_attn_bwd_workspace_size",
    "pisa_sparse_attn_bwd",
    "pisa_decode_workspace_size",
    "pisa_decode_step",
    "pisa_decode_step_ragged",
    "pisa_decode_step_ragged_noalloc",
    "pisa_decode_step_ragged_append",
    "pisa_pyramid_append",
    "pisa_status_string",
    "pisa_last_error",
    "pisa_version",
]


class PisaError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str = ""):
        self.status = status
        super().__init__(f"{where}: {_STATUS.get(status, status)} ({detail})" if detail else f"{where}: {status}")


class Problem(ctypes.Structure):
    """Mirror of `pisa_problem` in include/pisa.h."""

    _fields_ = [
        ("batch", ctypes.c_int32),
        ("heads_q", ctypes.c_int32),
        ("heads_kv", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("seq_len", ctypes.c_int64),
        ("block_size", ctypes.c_int32),
        ("fanout", ctypes.c_int32),
        ("levels", ctypes.c_int32),
        ("top_k", ctypes.c_int32),
        ("sink_len", ctypes.c_int32),
        ("causal", ctypes.c_int32),
        ("sm_scale", ctypes.c_float),
        ("dtype", ctypes.c_int32),
        ("pool", ctypes.c_int32),
    ]

    @property
    def n_blocks(self) -> int:
        return -(-self.seq_len // self.block_size)

    @property
    def group(self) -> int:
        return self.heads_q // self.heads_kv


POOL_MEAN, POOL_MAX = 0, 1


def problem(batch, heads_q, heads_kv, seq_len, head_dim, block_size, fanout, levels, top_k, sink_len, dtype,
            sm_scale=0.0, causal=1, pool=POOL_MEAN) -> Problem:
    d = {"f32": F32, "bf16": BF16}.get(dtype, dtype)
    pl = {"mean": POOL_MEAN, "max": POOL_MAX}.get(pool, pool)
    return Problem(batch, heads_q, heads_kv, head_dim, seq_len, block_size, fanout, levels, top_k, sink_len,
                   int(causal), sm_scale, d, pl)


# ---------------------------------------------------------------------------
# library loading


def library_path() -> str:
    """The in-tree libpisa.so, or the file PISA_LIBRARY names (e.g. the host-sanitised build)."""
    return os.environ.get("PISA_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib",
                                                          "libpisa.so")


_lib = None


def load_library():
    """Load libpisa.so (built by block_sparse_long_pisa_amd.build); raises if it is absent."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise PisaError(-1, "load_library", f"{path} is missing: run `python -m block_sparse_long_pisa_amd.build`")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER(Problem)
    vp, i32p, i64p, f32p = ctypes.c_void_p, ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int64), ctypes.c_void_p
    sig = {
        "pisa_pyramid_layout": [P, i64p],
        "pisa_build_pyramid": [P, vp, vp, vp],
        "pisa_select_topk": [P, vp, vp, vp, vp, vp],
        "pisa_sparse_attn_fwd": [P, vp, vp, vp, vp, vp, vp, vp, vp],
        "pisa_select_attend": [P, vp, vp, vp, vp, vp, vp, vp, vp, vp],
        "pisa_decode_workspace_size": [P, ctypes.POINTER(ctypes.c_size_t)],
        "pisa_sparse_attn_bwd_workspace_size": [P, ctypes.POINTER(ctypes.c_size_t)],
        "pisa_sparse_attn_bwd": [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp],
        "pisa_decode_step": [P, vp, vp, vp, vp, ctypes.c_int64, vp, vp, vp, vp, vp, ctypes.c_size_t, vp],
        "pisa_decode_step_ragged": [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp],
        "pisa_decode_step_ragged_noalloc": [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp],
        "pisa_decode_step_ragged_append": [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp],
        "pisa_pyramid_append": [P, vp, vp, vp, vp, vp],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    lib.pisa_status_string.argtypes = [ctypes.c_int]
    lib.pisa_status_string.restype = ctypes.c_char_p
    lib.pisa_last_error.argtypes = []
    lib.pisa_last_error.restype = ctypes.c_char_p
    lib.pisa_version.argtypes = []
    lib.pisa_version.restype = ctypes.c_int32
    _lib = lib
    return lib


def _check(status: int, where: str):
    if status != 0:
        detail = load_library().pisa_last_error().decode(errors="replace")
        raise PisaError(status, where, detail)


# ---------------------------------------------------------------------------
# tensor helpers (torch is imported lazily: only device memory and streams)


def _torch():
    import torch

    return torch


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(t) -> int:
    torch = _torch()
    return torch.cuda.current_stream(t.device).cuda_stream


def _tdtype(p: Problem):
    torch = _torch()
    return torch.bfloat16 if p.dtype == BF16 else torch.float32


def _expect(t, shape: Sequence[int], dtype, name: str):
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (no CPU path exists)")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def pyramid_layout(p: Problem) -> List[int]:
    lib = load_library()
    offs = (ctypes.c_int64 * (p.levels + 1))()
    _check(lib.pisa_pyramid_layout(ctypes.byref(p), offs), "pisa_pyramid_layout")
    return list(offs)


def build_pyramid(p: Problem, k, pyramid=None):
    """fp32 pyramid [B, Hkv, nodes, d] of keys k [B, Hkv, N, d]."""
    torch = _torch()
    lib = load_library()
    nodes = pyramid_layout(p)[-1]
    _expect(k, (p.batch, p.heads_kv, p.seq_len, p.head_dim), _tdtype(p), "k")
    if pyramid is None:
        pyramid = torch.empty((p.batch, p.heads_kv, nodes, p.head_dim), dtype=torch.float32, device=k.device)
    _expect(pyramid, (p.batch, p.heads_kv, nodes, p.head_dim), torch.float32, "pyramid")
    _check(lib.pisa_build_pyramid(ctypes.byref(p), _ptr(k), _ptr(pyramid), _stream(k)), "pisa_build_pyramid")
    return pyramid


def select_topk(p: Problem, q, pyramid, idx=None, cnt=None):
    """Selected blocks idx int32 [B, Hkv, nb, K] (ascending, -1 padded) and cnt int32 [B, Hkv, nb]."""
    torch = _torch()
    lib = load_library()
    nodes = pyramid_layout(p)[-1]
    nb = p.n_blocks
    _expect(q, (p.batch, p.heads_q, p.seq_len, p.head_dim), _tdtype(p), "q")
    _expect(pyramid, (p.batch, p.heads_kv, nodes, p.head_dim), torch.float32, "pyramid")
    if idx is None:
        idx = torch.empty((p.batch, p.heads_kv, nb, p.top_k), dtype=torch.int32, device=q.device)
    if cnt is None:
        cnt = torch.empty((p.batch, p.heads_kv, nb), dtype=torch.int32, device=q.device)
    _expect(idx, (p.batch, p.heads_kv, nb, p.top_k), torch.int32, "idx")
    _expect(cnt, (p.batch, p.heads_kv, nb), torch.int32, "cnt")
    _check(lib.pisa_select_topk(ctypes.byref(p), _ptr(q), _ptr(pyramid), _ptr(idx) if p.top_k else None, _ptr(cnt),
                                _stream(q)), "pisa_select_topk")
    return idx, cnt


def sparse_attn_fwd(p: Problem, q, k, v, idx, cnt, out=None, lse=None, want_lse: bool = False):
    """Attention output [B, Hq, N, d] (and fp32 lse [B, Hq, N] if requested)."""
    torch = _torch()
    lib = load_library()
    nb = p.n_blocks
    dt = _tdtype(p)
    _expect(q, (p.batch, p.heads_q, p.seq_len, p.head_dim), dt, "q")
    _expect(k, (p.batch, p.heads_kv, p.seq_len, p.head_dim), dt, "k")
    _expect(v, (p.batch, p.heads_kv, p.seq_len, p.head_dim), dt, "v")
    _expect(idx, (p.batch, p.heads_kv, nb, p.top_k), torch.int32, "idx")
    _expect(cnt, (p.batch, p.heads_kv, nb), torch.int32, "cnt")
    if out is None:
        out = torch.empty_like(q)
    _expect(out, tuple(q.shape), dt, "out")
    if lse is None and want_lse:
        lse = torch.empty((p.batch, p.heads_q, p.seq_len), dtype=torch.float32, device=q.device)
    if lse is not None:
        _expect(lse, (p.batch, p.heads_q, p.seq_len), torch.float32, "lse")
    _check(lib.pisa_sparse_attn_fwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(idx) if p.top_k else None,
                                    _ptr(cnt), _ptr(out), _ptr(lse), _stream(q)), "pisa_sparse_attn_fwd")
    return out, lse


def select_attend(p: Problem, q, k, v, pyramid, idx=None, cnt=None, out=None, lse=None, want_lse: bool = False,
                  want_idx: bool = False):
    """Selection and attention in one launch (bf16, causal). Returns (out, lse, idx, cnt); idx and cnt are
    written only when given or requested."""
    torch = _torch()
    lib = load_library()
    nb = p.n_blocks
    dt = _tdtype(p)
    _expect(q, (p.batch, p.heads_q, p.seq_len, p.head_dim), dt, "q")
    _expect(k, (p.batch, p.heads_kv, p.seq_len, p.head_dim), dt, "k")
    _expect(v, (p.batch, p.heads_kv, p.seq_len, p.head_dim), dt, "v")
    _expect(pyramid, (p.batch, p.heads_kv, pyramid_layout(p)[-1], p.head_dim), torch.float32, "pyramid")
    if want_idx and idx is None:
        idx = torch.empty((p.batch, p.heads_kv, nb, p.top_k), dtype=torch.int32, device=q.device)
    if want_idx and cnt is None:
        cnt = torch.empty((p.batch, p.heads_kv, nb), dtype=torch.int32, device=q.device)
    if idx is not None:
        _expect(idx, (p.batch, p.heads_kv, nb, p.top_k), torch.int32, "idx")
    if cnt is not None:
        _expect(cnt, (p.batch, p.heads_kv, nb), torch.int32, "cnt")
    if out is None:
        out = torch.empty_like(q)
    _expect(out, tuple(q.shape), dt, "out")
    if lse is None and want_lse:
        lse = torch.empty((p.batch, p.heads_q, p.seq_len), dtype=torch.float32, device=q.device)
    if lse is not None:
        _expect(lse, (p.batch, p.heads_q, p.seq_len), torch.float32, "lse")
    _check(lib.pisa_select_attend(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(pyramid),
                                  _ptr(idx) if (idx is not None and p.top_k) else None, _ptr(cnt), _ptr(out),
                                  _ptr(lse), _stream(q)), "pisa_select_attend")
    return out, lse, idx, cnt


def prefill(p: Problem, q, k, v, want_lse: bool = False):
    """The whole prefill path: pyramid, selection, attention. Returns (out, lse, idx, cnt, pyramid)."""
    pyr = build_pyramid(p, k)
    idx, cnt = select_topk(p, q, pyr)
    out, lse = sparse_attn_fwd(p, q, k, v, idx, cnt, want_lse=want_lse)
    return out, lse, idx, cnt, pyr


def sparse_attn_bwd_workspace_size(p: Problem) -> int:
    lib = load_library()
    n = ctypes.c_size_t(0)
    _check(lib.pisa_sparse_attn_bwd_workspace_size(ctypes.byref(p), ctypes.byref(n)),
           "pisa_sparse_attn_bwd_workspace_size")
    return n.value


def sparse_attn_bwd(p: Problem, q, k, v, idx, cnt, out, lse, dout, dq=None, dk=None, dv=None, workspace=None):
    """Gradients (dq, dk, dv) of the sparse attention for output gradient dout; the selection is held constant."""
    torch = _torch()
    lib = load_library()
    dt = _tdtype(p)
    nb = p.n_blocks
    _expect(q, (p.batch, p.heads_q, p.seq_len, p.head_dim), dt, "q")
    _expect(k, (p.batch, p.heads_kv, p.seq_len, p.head_dim), dt, "k")
    _expect(v, (p.batch, p.heads_kv, p.seq_len, p.head_dim), dt, "v")
    _expect(cnt, (p.batch, p.heads_kv, nb), torch.int32, "cnt")
    if p.top_k:
        _expect(idx, (p.batch, p.heads_kv, nb, p.top_k), torch.int32, "idx")
    _expect(out, tuple(q.shape), dt, "out")
    _expect(lse, (p.batch, p.heads_q, p.seq_len), torch.float32, "lse")
    _expect(dout, tuple(q.shape), dt, "dout")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _expect(dq, tuple(q.shape), dt, "dq")
    _expect(dk, tuple(k.shape), dt, "dk")
    _expect(dv, tuple(v.shape), dt, "dv")
    if workspace is None:
        workspace = torch.empty(max(1, sparse_attn_bwd_workspace_size(p)), dtype=torch.uint8, device=q.device)
    _check(lib.pisa_sparse_attn_bwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(idx) if p.top_k else None,
                                    _ptr(cnt), _ptr(out), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
                                    _ptr(workspace), workspace.numel(), _stream(q)), "pisa_sparse_attn_bwd")
    return dq, dk, dv


def decode_workspace_size(p: Problem) -> int:
    lib = load_library()
    n = ctypes.c_size_t(0)
    _check(lib.pisa_decode_workspace_size(ctypes.byref(p), ctypes.byref(n)), "pisa_decode_workspace_size")
    return n.value


def decode_step(p: Problem, q, k_cache, v_cache, pyramid, cache_len: int, out=None, lse=None, want_lse=False,
                idx_out=None, cnt_out=None, want_idx=False, workspace=None):
    """One decode step. q [B, Hq, d]; caches [B, Hkv, cap, d]. Returns (out, lse, idx, cnt)."""
    torch = _torch()
    lib = load_library()
    dt = _tdtype(p)
    nodes = pyramid_layout(p)[-1]
    _expect(q, (p.batch, p.heads_q, p.head_dim), dt, "q")
    _expect(k_cache, (p.batch, p.heads_kv, p.seq_len, p.head_dim), dt, "k_cache")
    _expect(v_cache, (p.batch, p.heads_kv, p.seq_len, p.head_dim), dt, "v_cache")
    _expect(pyramid, (p.batch, p.heads_kv, nodes, p.head_dim), torch.float32, "pyramid")
    if out is None:
        out = torch.empty_like(q)
    _expect(out, tuple(q.shape), dt, "out")
    if lse is None and want_lse:
        lse = torch.empty((p.batch, p.heads_q), dtype=torch.float32, device=q.device)
    if idx_out is None and want_idx and p.top_k:
        idx_out = torch.empty((p.batch, p.heads_kv, p.top_k), dtype=torch.int32, device=q.device)
    if cnt_out is None and want_idx:
        cnt_out = torch.empty((p.batch, p.heads_kv), dtype=torch.int32, device=q.device)
    if workspace is None:
        workspace = torch.empty(max(1, decode_workspace_size(p)), dtype=torch.uint8, device=q.device)
    _check(lib.pisa_decode_step(ctypes.byref(p), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(pyramid), int(cache_len),
                                _ptr(out), _ptr(lse), _ptr(idx_out), _ptr(cnt_out), _ptr(workspace),
                                workspace.numel(), _stream(q)), "pisa_decode_step")
    return out, lse, idx_out, cnt_out


def decode_step_ragged(p: Problem, q, k_cache, v_cache, pyramid, cache_lens, out=None, lse=None, want_lse=False,
                       idx_out=None, cnt_out=None, want_idx=False, workspace=None):
    """One decode step with a cache length per sequence: cache_lens int32 [B] on the device.

    Returns (out, lse, idx, cnt) as decode_step does.
    """
    torch = _torch()
    lib = load_library()
    dt = _tdtype(p)
    nodes = pyramid_layout(p)[-1]
    _expect(q, (p.batch, p.heads_q, p.head_dim), dt, "q")
    _expect(k_cache, (p.batch, p.heads_kv, p.seq_len, p.head_dim), dt, "k_cache")
    _expect(v_cache, (p.batch, p.heads_kv, p.seq_len, p.head_dim), dt, "v_cache")
    _expect(pyramid, (p.batch, p.heads_kv, nodes, p.head_dim), torch.float32, "pyramid")
    _expect(cache_lens, (p.batch,), torch.int32, "cache_lens")
    if out is None:
        out = torch.empty_like(q)
    _expect(out, tuple(q.shape), dt, "out")
    if lse is None and want_lse:
        lse = torch.empty((p.batch, p.heads_q), dtype=torch.float32, device=q.device)
    if idx_out is None and want_idx and p.top_k:
        idx_out = torch.empty((p.batch, p.heads_kv, p.top_k), dtype=torch.int32, device=q.device)
    if cnt_out is None and want_idx:
        cnt_out = torch.empty((p.batch, p.heads_kv), dtype=torch.int32, device=q.device)
    if workspace is None:
        workspace = torch.empty(max(1, decode_workspace_size(p)), dtype=torch.uint8, device=q.device)
    _check(lib.pisa_decode_step_ragged(ctypes.byref(p), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(pyramid),
                                       _ptr(cache_lens), _ptr(out), _ptr(lse), _ptr(idx_out), _ptr(cnt_out),
                                       _ptr(workspace), workspace.numel(), _stream(q)), "pisa_decode_step_ragged")
    return out, lse, idx_out, cnt_out


def decode_step_ragged_append(p: Problem, q, k_cache, v_cache, pyramid, old_lens, cache_lens, out=None, lse=None,
                              want_lse=False, idx_out=None, cnt_out=None, want_idx=False, workspace=None):
    """pyramid_append(p, k_cache, pyramid, old_lens, cache_lens) then decode_step_ragged at cache_lens, in the
    launches of one decode step (the pyramid is updated in place). Returns (out, lse, idx, cnt)."""
    torch = _torch()
    lib = load_library()
    dt = _tdtype(p)
    nodes = pyramid_layout(p)[-1]
    _expect(q, (p.batch, p.heads_q, p.head_dim), dt, "q")
    _expect(k_cache, (p.batch, p.heads_kv, p.seq_len, p.head_dim), dt, "k_cache")
    _expect(v_cache, (p.batch, p.heads_kv, p.seq_len, p.head_dim), dt, "v_cache")
    _expect(pyramid, (p.batch, p.heads_kv, nodes, p.head_dim), torch.float32, "pyramid")
    _expect(old_lens, (p.batch,), torch.int32, "old_lens")
    _expect(cache_lens, (p.batch,), torch.int32, "cache_lens")
    if out is None:
        out = torch.empty_like(q)
    _expect(out, tuple(q.shape), dt, "out")
    if lse is None and want_lse:
        lse = torch.empty((p.batch, p.heads_q), dtype=torch.float32, device=q.device)
    if idx_out is None and want_idx and p.top_k:
        idx_out = torch.empty((p.batch, p.heads_kv, p.top_k), dtype=torch.int32, device=q.device)
    if cnt_out is None and want_idx:
        cnt_out = torch.empty((p.batch, p.heads_kv), dtype=torch.int32, device=q.device)
    if workspace is None:
        workspace = torch.empty(max(1, decode_workspace_size(p)), dtype=torch.uint8, device=q.device)
    _check(lib.pisa_decode_step_ragged_append(ctypes.byref(p), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(pyramid),
                                              _ptr(old_lens), _ptr(cache_lens), _ptr(out), _ptr(lse), _ptr(idx_out),
                                              _ptr(cnt_out), _ptr(workspace), workspace.numel(), _stream(q)),
           "pisa_decode_step_ragged_append")
    return out, lse, idx_out, cnt_out


DECODE_SCRATCH_BYTES = 16 << 20  # PISA_DECODE_SCRATCH_BYTES in include/pisa.h


def decode_step_ragged_noalloc(p: Problem, q, k_cache, v_cache, pyramid, cache_lens, out, lse=None, idx_out=None,
                               cnt_out=None):
    """decode_step_ragged with the library's static per-GPU workspace: nothing is
    allocated, so every output buffer (out; lse, idx_out, cnt_out if wanted) is
    the caller's. Calls on one GPU share the workspace: overlapping calls race."""
    torch = _torch()
    lib = load_library()
    dt = _tdtype(p)
    nodes = pyramid_layout(p)[-1]
    _expect(q, (p.batch, p.heads_q, p.head_dim), dt, "q")
    _expect(k_cache, (p.batch, p.heads_kv, p.seq_len, p.head_dim), dt, "k_cache")
    _expect(v_cache, (p.batch, p.heads_kv, p.seq_len, p.head_dim), dt, "v_cache")
    _expect(pyramid, (p.batch, p.heads_kv, nodes, p.head_dim), torch.float32, "pyramid")
    _expect(cache_lens, (p.batch,), torch.int32, "cache_lens")
    _expect(out, tuple(q.shape), dt, "out")
    if lse is not None:
        _expect(lse, (p.batch, p.heads_q), torch.float32, "lse")
    if idx_out is not None:
        _expect(idx_out, (p.batch, p.heads_kv, p.top_k), torch.int32, "idx_out")
    if cnt_out is not None:
        _expect(cnt_out, (p.batch, p.heads_kv), torch.int32, "cnt_out")
    _check(lib.pisa_decode_step_ragged_noalloc(ctypes.byref(p), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(pyramid),
                                               _ptr(cache_lens), _ptr(out), _ptr(lse), _ptr(idx_out), _ptr(cnt_out),
                                               _stream(q)), "pisa_decode_step_ragged_noalloc")
    return out, lse, idx_out, cnt_out


def pyramid_append(p: Problem, k_cache, pyramid, old_lens, new_lens):
    """Update `pyramid` in place after tokens [old_lens[b], new_lens[b]) were written to k_cache."""
    torch = _torch()
    lib = load_library()
    nodes = pyramid_layout(p)[-1]
    _expect(k_cache, (p.batch, p.heads_kv, p.seq_len, p.head_dim), _tdtype(p), "k_cache")
    _expect(pyramid, (p.batch, p.heads_kv, nodes, p.head_dim), torch.float32, "pyramid")
    _expect(old_lens, (p.batch,), torch.int32, "old_lens")
    _expect(new_lens, (p.batch,), torch.int32, "new_lens")
    _check(lib.pisa_pyramid_append(ctypes.byref(p), _ptr(k_cache), _ptr(pyramid), _ptr(old_lens), _ptr(new_lens),
                                   _stream(k_cache)), "pisa_pyramid_append")
    return pyramid
