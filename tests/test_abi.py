"""The C ABI: the library loads, exports what include/pisa.h declares, and validates
arguments on the host (no GPU needed: nothing here reaches a launch)."""

import ctypes
import os
import re

import pytest

import block_sparse_long_pisa_amd as pisa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

OK, ENULL, ESHAPE, EUNSUP, EWS, EHIP, EALIGN = range(7)


def _declared():
    src = open(os.path.join(ROOT, "include", "pisa.h")).read()
    return sorted(set(re.findall(r"\b(pisa_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(pisa.library_path()):
        pytest.fail("libpisa.so is not built: run python -m block_sparse_long_pisa_amd.build")
    return pisa.load_library()


def test_exports_every_declared_symbol(lib):
    declared = _declared()
    assert set(declared) == set(pisa.EXPORTED_SYMBOLS)
    for name in declared:
        assert hasattr(lib, name), name
    assert lib.pisa_version() == 10000


def test_struct_layout_matches_header():
    # int32 x4, int64, int32 x6, float, int32 x2 -> 60 bytes padded to 64 (int64 alignment)
    assert ctypes.sizeof(pisa.Problem) == 64
    assert pisa.Problem.seq_len.offset == 16
    assert pisa.Problem.dtype.offset == 52
    assert pisa.Problem.pool.offset == 56
    fields = re.search(r"typedef struct pisa_problem \{(.*?)\} pisa_problem;", open(os.path.join(ROOT, "include", "pisa.h")).read(),
                       re.S).group(1)
    names = re.findall(r"(?:int32_t|int64_t|float)\s+(\w+);", fields)
    assert names == [f[0] for f in pisa.Problem._fields_]


def _p(**kw):
    base = dict(batch=1, heads_q=4, heads_kv=2, seq_len=1024, head_dim=128, block_size=64, fanout=4, levels=3,
                top_k=4, sink_len=64, dtype="bf16")
    base.update(kw)
    return pisa.problem(**base)


def test_layout_offsets(lib):
    assert pisa.pyramid_layout(_p()) == [0, 16, 20, 21]
    assert pisa.pyramid_layout(_p(seq_len=131072, block_size=128, fanout=8, levels=4)) == [0, 1024, 1152, 1168, 1170]
    assert pisa.pyramid_layout(_p(seq_len=1000, block_size=64, fanout=4, levels=3)) == [0, 16, 20, 21]
    assert pisa.pyramid_layout(_p(seq_len=0)) == [0, 0, 0, 0]


@pytest.mark.parametrize("kw,status", [
    (dict(heads_q=3, heads_kv=2), ESHAPE),
    (dict(batch=-1), ESHAPE),
    (dict(seq_len=-5), ESHAPE),
    (dict(head_dim=96), EUNSUP),
    (dict(block_size=48), EUNSUP),
    (dict(block_size=256), EUNSUP),
    (dict(fanout=3), EUNSUP),
    (dict(levels=0), ESHAPE),
    (dict(levels=9), EUNSUP),
    (dict(top_k=-1), ESHAPE),
    (dict(top_k=300), EUNSUP),
    (dict(top_k=257, fanout=2), EUNSUP),  # one past the largest kept set
    (dict(top_k=256, fanout=4), EUNSUP),  # level-0 pool 1027 > 1024
    (dict(top_k=128, fanout=16), EUNSUP),
    (dict(sink_len=-1), ESHAPE),
    (dict(causal=2), EUNSUP),
    (dict(pool=2), EUNSUP),
    (dict(dtype=7), EUNSUP),
    (dict(seq_len=1 << 20, block_size=32, levels=1), EUNSUP),  # top level too wide
])
def test_invalid_problems_are_rejected_on_the_host(lib, kw, status):
    p = _p(**kw)
    offs = (ctypes.c_int64 * 16)()
    assert lib.pisa_pyramid_layout(ctypes.byref(p), offs) == status
    assert lib.pisa_last_error() != b""
    fake = ctypes.c_void_p(4096)
    assert lib.pisa_build_pyramid(ctypes.byref(p), fake, fake, None) == status
    assert lib.pisa_select_topk(ctypes.byref(p), fake, fake, fake, fake, None) == status
    assert lib.pisa_sparse_attn_fwd(ctypes.byref(p), fake, fake, fake, fake, fake, fake, None, None) == status
    n = ctypes.c_size_t(0)
    assert lib.pisa_decode_workspace_size(ctypes.byref(p), ctypes.byref(n)) == status


@pytest.mark.parametrize("kw", [
    dict(top_k=256, fanout=2, levels=8, block_size=32, seq_len=8192),  # largest kept set, deepest pyramid
    dict(top_k=255, fanout=4, levels=3, seq_len=65536),                # level-0 pool of 1023 slots
])
def test_problems_at_the_limits_are_accepted(lib, kw):
    p = _p(**kw)
    offs = (ctypes.c_int64 * 16)()
    assert lib.pisa_pyramid_layout(ctypes.byref(p), offs) == 0, lib.pisa_last_error()
    n = ctypes.c_size_t(0)
    assert lib.pisa_decode_workspace_size(ctypes.byref(p), ctypes.byref(n)) == 0
    assert n.value > 0


def test_null_and_misaligned_pointers(lib):
    p = _p()
    fake = ctypes.c_void_p(4096)
    odd = ctypes.c_void_p(4098)
    assert lib.pisa_build_pyramid(None, fake, fake, None) == ENULL
    assert lib.pisa_build_pyramid(ctypes.byref(p), None, fake, None) == ENULL
    assert lib.pisa_build_pyramid(ctypes.byref(p), odd, fake, None) == EALIGN
    assert lib.pisa_select_topk(ctypes.byref(p), fake, fake, None, fake, None) == ENULL
    assert lib.pisa_sparse_attn_fwd(ctypes.byref(p), fake, fake, fake, fake, None, fake, None, None) == ENULL
    assert lib.pisa_sparse_attn_fwd(ctypes.byref(p), fake, odd, fake, fake, fake, fake, None, None) == EALIGN
    assert lib.pisa_pyramid_layout(ctypes.byref(p), None) == ENULL
    assert b"NULL" in lib.pisa_last_error()


def test_empty_problems_launch_nothing(lib):
    for kw in (dict(batch=0), dict(seq_len=0)):
        p = _p(**kw)
        assert lib.pisa_build_pyramid(ctypes.byref(p), None, None, None) == OK
        assert lib.pisa_select_topk(ctypes.byref(p), None, None, None, None, None) == OK
        assert lib.pisa_sparse_attn_fwd(ctypes.byref(p), None, None, None, None, None, None, None, None) == OK
    n = ctypes.c_size_t(99)
    assert lib.pisa_decode_workspace_size(ctypes.byref(_p(batch=0)), ctypes.byref(n)) == OK and n.value == 0


def test_decode_validation(lib):
    p = _p(seq_len=4096)
    n = ctypes.c_size_t(0)
    assert lib.pisa_decode_workspace_size(ctypes.byref(p), ctypes.byref(n)) == OK and n.value > 0
    fake = ctypes.c_void_p(4096)
    ws = ctypes.c_void_p(1 << 20)

    def call(cache_len, ws_ptr=ws, ws_bytes=n.value, prob=p):
        return lib.pisa_decode_step(ctypes.byref(prob), fake, fake, fake, fake, cache_len, fake, None, None, None,
                                    ws_ptr, ws_bytes, None)

    assert call(0) == ESHAPE
    assert call(4097) == ESHAPE
    assert call(100, ws_ptr=None) == EWS
    assert call(100, ws_bytes=n.value - 1) == EWS
    assert call(100, ws_ptr=ctypes.c_void_p((1 << 20) + 16)) == EALIGN
    assert call(100, prob=_p(seq_len=4096, heads_q=6, heads_kv=2)) == EUNSUP  # G = 3
    assert call(100, prob=_p(seq_len=4096, heads_q=32, heads_kv=2)) == EUNSUP  # G = 16


def test_ragged_decode_and_append_validation(lib):
    p = _p(seq_len=4096)
    n = ctypes.c_size_t(0)
    assert lib.pisa_decode_workspace_size(ctypes.byref(p), ctypes.byref(n)) == OK
    fake = ctypes.c_void_p(4096)
    ws = ctypes.c_void_p(1 << 20)

    def ragged(lens=fake, ws_ptr=ws, ws_bytes=n.value, prob=p, q=fake):
        return lib.pisa_decode_step_ragged(ctypes.byref(prob), q, fake, fake, fake, lens, fake, None, None, None,
                                           ws_ptr, ws_bytes, None)

    assert ragged(lens=None) == ENULL
    assert ragged(lens=ctypes.c_void_p(4098)) == EALIGN
    assert ragged(q=None) == ENULL
    assert ragged(ws_bytes=n.value - 1) == EWS
    assert ragged(prob=_p(seq_len=4096, heads_q=6, heads_kv=2)) == EUNSUP
    assert ragged(prob=_p(batch=0)) == OK  # empty batch: nothing to do

    def append(k=fake, pyr=fake, old=fake, new=fake, prob=p):
        return lib.pisa_pyramid_append(ctypes.byref(prob), k, pyr, old, new, None)

    assert append(old=None) == ENULL
    assert append(pyr=None) == ENULL
    assert append(new=ctypes.c_void_p(4097)) == EALIGN
    assert append(k=ctypes.c_void_p(4100)) == EALIGN
    assert append(prob=_p(seq_len=0)) == OK
    assert lib.pisa_pyramid_append(None, fake, fake, fake, fake, None) == ENULL

    def both(old=fake, lens=fake, pyr=fake, ws_bytes=n.value, prob=p):
        return lib.pisa_decode_step_ragged_append(ctypes.byref(prob), fake, fake, fake, pyr, old, lens, fake, None,
                                                  None, None, ws, ws_bytes, None)

    assert both(old=None) == ENULL
    assert both(lens=None) == ENULL
    assert both(pyr=None) == ENULL
    assert both(old=ctypes.c_void_p(4098)) == EALIGN
    assert both(ws_bytes=n.value - 1) == EWS
    assert both(prob=_p(seq_len=4096, heads_q=6, heads_kv=2)) == EUNSUP
    assert both(prob=_p(batch=0)) == OK


def test_backward_validation(lib):
    p = _p(seq_len=4096)
    n = ctypes.c_size_t(0)
    assert lib.pisa_sparse_attn_bwd_workspace_size(ctypes.byref(p), ctypes.byref(n)) == OK and n.value > 0
    assert lib.pisa_sparse_attn_bwd_workspace_size(ctypes.byref(p), None) == ENULL
    fake = ctypes.c_void_p(4096)
    ws = ctypes.c_void_p(1 << 20)

    def bwd(prob=p, lse=fake, dq=fake, ws_ptr=ws, ws_bytes=n.value, k=fake):
        return lib.pisa_sparse_attn_bwd(ctypes.byref(prob), fake, k, fake, fake, fake, fake, lse, fake, dq, fake, fake,
                                        ws_ptr, ws_bytes, None)

    assert bwd(lse=None) == ENULL
    assert bwd(dq=None) == ENULL
    assert bwd(k=ctypes.c_void_p(4104)) == EALIGN
    assert bwd(ws_bytes=n.value - 1) == EWS
    assert bwd(ws_ptr=ctypes.c_void_p((1 << 20) + 64)) == EALIGN
    assert bwd(prob=_p(seq_len=4096, dtype=pisa.F32)) == EUNSUP
    assert bwd(prob=_p(batch=0)) == OK


def test_fused_validation(lib):
    p = _p(seq_len=4096)
    fake = ctypes.c_void_p(4096)

    def fused(prob=p, pyr=fake, out=fake, k=fake, idx=fake, cnt=fake):
        return lib.pisa_select_attend(ctypes.byref(prob), fake, k, fake, pyr, idx, cnt, out, None, None)

    assert fused(pyr=None) == ENULL
    assert fused(out=None) == ENULL
    assert fused(k=ctypes.c_void_p(4104)) == EALIGN
    assert fused(pyr=ctypes.c_void_p(4100)) == EALIGN
    assert fused(prob=_p(seq_len=4096, dtype=pisa.F32)) == EUNSUP
    assert fused(prob=_p(seq_len=4096, causal=0)) == EUNSUP
    assert fused(prob=_p(batch=0)) == OK
    assert lib.pisa_select_attend(None, fake, fake, fake, fake, None, None, fake, None, None) == ENULL


def test_status_strings(lib):
    for s in range(7):
        assert lib.pisa_status_string(s)
    assert lib.pisa_status_string(42) == b"unknown status"


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(pisa, "_lib", None)
    monkeypatch.setattr(pisa, "library_path", lambda: str(tmp_path / "libpisa.so"))
    with pytest.raises(pisa.PisaError):
        pisa.load_library()
