"""Seeded synthetic inputs for the PISA block-sparse attention path.

This module is shared test and bench infrastructure. It draws Q, K and V,
plants "needle" key blocks, and records where it planted them. It holds none
of the method's arithmetic: no pooling, scoring, selection or attention.
Both the CPU oracle and the HIP path receive exactly the arrays made here.

Workload recipe (the pages print no dataset that fits one GPU; these stand in
for the long-context needle-retrieval workloads the Pulsar and SSA pages
evaluate on):

* Q, K, V are i.i.d. N(0, 1), scaled by 1/sqrt(d) for the bf16 workloads
  (a "sharp" test variant leaves Q and K unscaled, so logits have unit
  spread, and keeps V at 1/sqrt(d)).
  Values are drawn in fp64, rounded to fp32, then (bf16 workloads) rounded to
  bf16 with round-to-nearest-even.
* A planted block (a "needle") for query block qb of KV group g overwrites
  every row of key block t with  mean(Q rows of qb over the heads of g)
  + 0.1 * N(0, 1), rounded to the tensor dtype. V is untouched.

Two sources of randomness exist:

* ``host``: numpy PCG64 with ``SeedSequence([seed, tensor_id, b, h])`` child
  streams, so any (tensor, b, h) slice can be rebuilt on its own.
* ``device``: torch's generator on the GPU, for the workloads too large to
  draw on the host (a 32 GiB decode cache). Tests copy the slices they check
  back to the host for the oracle.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Tuple

import numpy as np

__all__ = [
    "Problem",
    "WORKLOADS",
    "workload",
    "round_to_bf16",
    "bf16_bits",
    "host_inputs",
    "host_decode_inputs",
    "device_inputs",
    "device_decode_inputs",
]

# tensor ids for the child seed streams
_TQ, _TK, _TV, _TPLANT, _TNOISE = 0, 1, 2, 100, 101


@dataclasses.dataclass(frozen=True)
class Problem:
    """Shape of one PISA problem (all sizes in elements / tokens / blocks)."""

    batch: int
    heads_q: int
    heads_kv: int
    seq_len: int  # prefill length N, or decode cache capacity
    head_dim: int
    block_size: int
    fanout: int
    levels: int  # counts the leaf-block level
    top_k: int
    sink_len: int
    dtype: str  # "f32" or "bf16"
    sm_scale: float = 0.0  # <= 0 means 1/sqrt(head_dim)
    decode: bool = False
    causal: bool = True    # False: the bidirectional variant
    pool: str = "mean"     # "mean", or the "max" variant of node summaries

    @property
    def group(self) -> int:
        return self.heads_q // self.heads_kv

    @property
    def n_blocks(self) -> int:
        return -(-self.seq_len // self.block_size)

    @property
    def scale(self) -> float:
        return self.sm_scale if self.sm_scale > 0 else 1.0 / math.sqrt(self.head_dim)

    def replace(self, **kw) -> "Problem":
        return dataclasses.replace(self, **kw)


# The five workloads: shapes, seeds and planting schemes.
WORKLOADS: Dict[int, dict] = {
    1: dict(
        name="tiny fp32 causal single head, N=1024",
        problem=Problem(1, 1, 1, 1024, 64, 64, 4, 2, 4, 64, "f32"),
        seed=0,
        value_scale=1.0,
        plant="every_block",
    ),
    2: dict(
        name="prefill bf16 causal MHA, N=32768, 32 heads",
        problem=Problem(1, 32, 32, 32768, 128, 64, 8, 3, 16, 64, "bf16"),
        seed=1,
        value_scale=None,  # 1/sqrt(d)
        plant=("uniform_pairs", 8),
    ),
    3: dict(
        name="prefill bf16 causal GQA 32q/8kv, N=131072",
        problem=Problem(1, 32, 8, 131072, 128, 128, 8, 4, 32, 64, "bf16"),
        seed=2,
        value_scale=None,
        plant=("uniform_depth", 16),
    ),
    4: dict(
        name="decode bf16 GQA 32q/8kv, 64 sequences x 131072-token cache",
        problem=Problem(64, 32, 8, 131072, 128, 128, 8, 4, 32, 64, "bf16", decode=True),
        seed=3,
        value_scale=None,
        plant=("decode_one", 1),
    ),
    5: dict(
        name="prefill bf16 causal one GQA group 4q/1kv, N=1048576",
        problem=Problem(1, 4, 1, 1048576, 128, 128, 8, 5, 64, 64, "bf16"),
        seed=4,
        value_scale=None,
        plant=("log_distance", 32),
    ),
}


def workload(i: int) -> dict:
    c = dict(WORKLOADS[i])
    if c["value_scale"] is None:
        c["value_scale"] = 1.0 / math.sqrt(c["problem"].head_dim)
    return c


# --------------------------------------------------------------------------
# rounding helpers (input construction only)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round to the nearest bf16 (ties to even); returns fp32 holding bf16 values."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    nan = np.isnan(f)
    out = (r & 0xFFFFFFFF).astype(np.uint32).view(np.float32)
    if nan.any():
        out = np.where(nan, np.float32(np.nan), out)
    return out.reshape(np.shape(x))


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """The upper 16 bits of fp32 values that are already bf16-representable."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def _to_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64).astype(np.float32)
    return round_to_bf16(x) if dtype == "bf16" else x


def _scales(value_scale):
    """One scale for Q, K and V, or a (q, k, v) triple."""
    if isinstance(value_scale, (tuple, list)):
        return tuple(float(x) for x in value_scale)
    return (float(value_scale),) * 3


def _rng(seed: int, *keys: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, *keys])))


# --------------------------------------------------------------------------
# planting plans: lists of (b, g, qb, target) chosen from the plan's own stream


def _j0(p: Problem) -> int:
    return p.sink_len // p.block_size


def plan_needles(p: Problem, seed: int, plant) -> List[Tuple[int, int, int, int]]:
    """Return planting events (b, g, qb, target) in the order they are applied."""
    nb, j0 = p.n_blocks, _j0(p)
    out: List[Tuple[int, int, int, int]] = []
    if plant is None:
        return out
    if plant == "every_block":
        for b in range(p.batch):
            for g in range(p.heads_kv):
                rng = _rng(seed, _TPLANT, b, g)
                for qb in range(j0 + 1, nb):
                    t = int(rng.integers(j0, qb))
                    out.append((b, g, qb, t))
        return out
    kind, count = plant
    for b in range(p.batch):
        for g in range(p.heads_kv):
            rng = _rng(seed, _TPLANT, b, g)
            if nb - j0 < 2:
                continue
            for _ in range(count):
                if kind == "uniform_pairs":
                    qb = int(rng.integers(j0 + 1, nb))
                    t = int(rng.integers(j0, qb))
                elif kind == "uniform_depth":
                    t = int(rng.integers(j0, nb - 1))
                    qb = int(rng.integers(t + 1, nb))
                elif kind == "log_distance":
                    qb = int(rng.integers(j0 + 1, nb))
                    span = qb - j0
                    dist = int(math.floor(math.exp(rng.uniform(0.0, math.log(span + 1)))))
                    dist = min(max(dist, 1), span)
                    t = qb - dist
                elif kind == "decode_one":
                    qb = (p.seq_len - 1) // p.block_size
                    if qb <= j0:
                        continue
                    t = int(rng.integers(j0, qb))
                else:
                    raise ValueError(f"unknown planting scheme {kind!r}")
                out.append((b, g, qb, t))
    return out


def _survivors(events):
    """A later plant into the same (b, g, target) overwrites an earlier one."""
    last = {}
    for e in events:
        last[(e[0], e[1], e[3])] = e
    kept = set(last.values())
    return [dict(b=b, g=g, qb=qb, target=t, survived=(b, g, qb, t) in kept) for (b, g, qb, t) in events]


# --------------------------------------------------------------------------
# host (numpy) generation


def host_inputs(p: Problem, seed: int, value_scale: float, plant=None):
    """Q, K, V as fp32 numpy arrays [B, H, N, d] holding dtype-representable values.

    Returns (q, k, v, manifest).
    """
    B, Hq, Hkv, N, d = p.batch, p.heads_q, p.heads_kv, p.seq_len, p.head_dim
    sq, sk, sv = _scales(value_scale)
    q = np.empty((B, Hq, N, d), np.float32)
    k = np.empty((B, Hkv, N, d), np.float32)
    v = np.empty((B, Hkv, N, d), np.float32)
    for b in range(B):
        for h in range(Hq):
            q[b, h] = _to_dtype(_rng(seed, _TQ, b, h).standard_normal((N, d)) * sq, p.dtype)
        for h in range(Hkv):
            k[b, h] = _to_dtype(_rng(seed, _TK, b, h).standard_normal((N, d)) * sk, p.dtype)
            v[b, h] = _to_dtype(_rng(seed, _TV, b, h).standard_normal((N, d)) * sv, p.dtype)
    events = plan_needles(p, seed, plant)
    G, bs = p.group, p.block_size
    noise_rng = {}
    for (b, g, qb, t) in events:
        r0, r1 = qb * bs, min(N, (qb + 1) * bs)
        target = q[b, g * G:(g + 1) * G, r0:r1].astype(np.float64).mean(axis=(0, 1))
        key = (b, g)
        if key not in noise_rng:
            noise_rng[key] = _rng(seed, _TNOISE, b, g)
        t0, t1 = t * bs, min(N, (t + 1) * bs)
        noise = noise_rng[key].standard_normal((t1 - t0, d))
        k[b, g, t0:t1] = _to_dtype(target[None, :] + 0.1 * noise, p.dtype)
    return q, k, v, dict(needles=_survivors(events))


def host_decode_inputs(p: Problem, seed: int, value_scale: float, cache_len: int, plant=("decode_one", 1)):
    """Decode inputs on the host: q [B, Hq, d], k/v cache [B, Hkv, cap, d].

    The new token's key and value are already in the cache at position
    cache_len - 1.
    """
    B, Hq, Hkv, cap, d = p.batch, p.heads_q, p.heads_kv, p.seq_len, p.head_dim
    sq, sk, sv = _scales(value_scale)
    q = np.empty((B, Hq, d), np.float32)
    k = np.empty((B, Hkv, cap, d), np.float32)
    v = np.empty((B, Hkv, cap, d), np.float32)
    for b in range(B):
        for h in range(Hq):
            q[b, h] = _to_dtype(_rng(seed, _TQ, b, h).standard_normal(d) * sq, p.dtype)
        for h in range(Hkv):
            k[b, h] = _to_dtype(_rng(seed, _TK, b, h).standard_normal((cap, d)) * sk, p.dtype)
            v[b, h] = _to_dtype(_rng(seed, _TV, b, h).standard_normal((cap, d)) * sv, p.dtype)
    events = plan_needles(p.replace(seq_len=cache_len), seed, plant)
    G, bs = p.group, p.block_size
    for (b, g, qb, t) in events:
        target = q[b, g * G:(g + 1) * G].astype(np.float64).mean(axis=0)
        noise = _rng(seed, _TNOISE, b, g).standard_normal((bs, d))
        k[b, g, t * bs:(t + 1) * bs] = _to_dtype(target[None, :] + 0.1 * noise, p.dtype)
    return q, k, v, dict(needles=_survivors(events))


# --------------------------------------------------------------------------
# device (torch) generation for the full-size workloads


def _torch_gen(device, seed: int, *keys: int):
    import torch

    s = np.random.SeedSequence([seed, *keys]).generate_state(2, np.uint32)
    g = torch.Generator(device=device)
    g.manual_seed(int(s[0]) << 32 | int(s[1]))
    return g


def _randn_into(out, device, seed, keys, value_scale, chunk_rows=1 << 22):
    import torch

    g = _torch_gen(device, seed, *keys)
    flat = out.view(-1, out.shape[-1])
    for r0 in range(0, flat.shape[0], chunk_rows):
        r1 = min(flat.shape[0], r0 + chunk_rows)
        x = torch.randn((r1 - r0, flat.shape[1]), generator=g, device=device, dtype=torch.float32)
        flat[r0:r1].copy_(x.mul_(value_scale))  # the copy rounds to the tensor dtype (RNE)


def _tdtype(p: Problem):
    import torch

    return torch.bfloat16 if p.dtype == "bf16" else torch.float32


def device_inputs(p: Problem, seed: int, value_scale: float, plant=None, device="cuda"):
    """Q, K, V drawn on `device` with torch's generator; returns (q, k, v, manifest)."""
    import torch

    B, Hq, Hkv, N, d = p.batch, p.heads_q, p.heads_kv, p.seq_len, p.head_dim
    dt = _tdtype(p)
    q = torch.empty((B, Hq, N, d), dtype=dt, device=device)
    k = torch.empty((B, Hkv, N, d), dtype=dt, device=device)
    v = torch.empty((B, Hkv, N, d), dtype=dt, device=device)
    sq, sk, sv = _scales(value_scale)
    _randn_into(q, device, seed, (_TQ,), sq)
    _randn_into(k, device, seed, (_TK,), sk)
    _randn_into(v, device, seed, (_TV,), sv)
    events = plan_needles(p, seed, plant)
    G, bs = p.group, p.block_size
    gn = _torch_gen(device, seed, _TNOISE)
    for (b, g, qb, t) in events:
        r0, r1 = qb * bs, min(N, (qb + 1) * bs)
        target = q[b, g * G:(g + 1) * G, r0:r1].double().mean(dim=(0, 1))
        t0, t1 = t * bs, min(N, (t + 1) * bs)
        noise = torch.randn((t1 - t0, d), generator=gn, device=device, dtype=torch.float64)
        k[b, g, t0:t1] = (target[None, :] + 0.1 * noise).float().to(dt)
    return q, k, v, dict(needles=_survivors(events))


def device_decode_inputs(p: Problem, seed: int, value_scale: float, cache_len: int, plant=("decode_one", 1), device="cuda"):
    """Decode inputs drawn on `device`: q [B, Hq, d], k/v cache [B, Hkv, cap, d]."""
    import torch

    B, Hq, Hkv, cap, d = p.batch, p.heads_q, p.heads_kv, p.seq_len, p.head_dim
    dt = _tdtype(p)
    q = torch.empty((B, Hq, d), dtype=dt, device=device)
    k = torch.empty((B, Hkv, cap, d), dtype=dt, device=device)
    v = torch.empty((B, Hkv, cap, d), dtype=dt, device=device)
    sq, sk, sv = _scales(value_scale)
    _randn_into(q, device, seed, (_TQ,), sq)
    for b in range(B):  # per sequence, to bound the fp32 temporaries
        _randn_into(k[b], device, seed, (_TK, b), sk)
        _randn_into(v[b], device, seed, (_TV, b), sv)
    events = plan_needles(p.replace(seq_len=cache_len), seed, plant)
    G, bs = p.group, p.block_size
    gn = _torch_gen(device, seed, _TNOISE)
    for (b, g, qb, t) in events:
        target = q[b, g * G:(g + 1) * G].double().mean(dim=0)
        noise = torch.randn((bs, d), generator=gn, device=device, dtype=torch.float64)
        k[b, g, t * bs:(t + 1) * bs] = (target[None, :] + 0.1 * noise).float().to(dt)
    return q, k, v, dict(needles=_survivors(events))
