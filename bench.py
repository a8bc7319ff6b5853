#!/usr/bin/env python3
"""Throughput of the PISA block-sparse attention path on one MI355X.

A step is one pass of the whole prefill path -- key pyramid, top-K selection,
sparse attention -- over the 128K-token GQA workload (B=1, 32 query heads on 8
KV heads, N=131072, d=128, bf16, block 128, fanout 8, 4 levels, K=32, 64-token
sink, one local block). Inputs are synthetic (seeded), drawn on the GPU and
resident in HBM before the timed region. Beside it the decode workload (64
sequences x 131072-token cache, one new token each) is timed per step.

Prints one JSON line on stdout; progress goes to stderr.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12  # B/s, MI355X
BF16_PEAK = 2.5e15  # flop/s, dense bf16 matrix cores

# HBM traffic per launch on the 128K prefill and the 64 x 128K decode (and, keyed
# "w2/..." and "w5/...", on the 32K and 1M prefills), from two rocprofv3 --pmc runs
# (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch). Each counter is scaled by what
# it reads for a plain device copy of 1 GiB into 1 GiB: FETCH_SIZE reports
# 524337.5 KiB for the copy's 1 GiB of reads, WRITE_SIZE 1048576 KiB for its
# writes. A figure holds only for the kernel source it was taken on: the sources
# are hashed at run time and a changed kernel reports null.
COPY_SCALE = {"fetch": 1048576.0 / 524337.5, "write": 1048576.0 / 1048576.0}
MEASURED_TRAFFIC = {
    # step: (sources, sha256 prefix of their bytes in this order, FETCH_SIZE KiB, WRITE_SIZE KiB)
    "attention": (("pisa_attn.hip", "pisa_attn_fwd.h", "pisa_attn_common.h", "pisa_internal.h"), "661f4e2286e61980",
                  5855513.3, 1048576.9),
    "pyramid": (("pisa_pool.hip", "pisa_internal.h"), "3bf04d0514e54278",
                131123.5 + 275.7, 4608.2 + 72.0),  # leaf and level 1, then levels 2 and up
    "select": (("pisa_select.hip", "pisa_select_common.h", "pisa_internal.h"), "e9aeb64bfaa4b868",
               526688.7, 1056.0),
    # select + split attention + merge of the plain decode step (its first four dispatches of each)
    "decode": (("pisa_decode.hip", "pisa_select_common.h", "pisa_internal.h", "pisa_append.h"), "d8dca548eff013a9",
               50290.3 + 550539.7 + 3601.3, 80.0 + 6336.0 + 512.0),
    # the 32K MHA (w2) and 1M one-group (w5) prefills, from the same runs
    "w2/attention": (("pisa_attn.hip", "pisa_attn_fwd.h", "pisa_attn_common.h", "pisa_internal.h"), "661f4e2286e61980",
                     2448433.1, 263290.1),
    "w2/pyramid": (("pisa_pool.hip", "pisa_internal.h"), "3bf04d0514e54278", 131123.2 + 531.7, 9216.0 + 128.0),
    "w2/select": (("pisa_select.hip", "pisa_select_common.h", "pisa_internal.h"), "e9aeb64bfaa4b868",
                  135745.9, 1088.5),
    "w5/attention": (("pisa_attn.hip", "pisa_attn_fwd.h", "pisa_attn_common.h", "pisa_internal.h"), "661f4e2286e61980",
                     15704745.0, 1049570.2),
    "w5/pyramid": (("pisa_pool.hip", "pisa_internal.h"), "3bf04d0514e54278", 131123.9 + 8.9 + 275.7, 4608.2 + 1.0 + 72.0),
    "w5/select": (("pisa_select.hip", "pisa_select_common.h", "pisa_internal.h"), "e9aeb64bfaa4b868",
                  543207.3, 2125.9),
}


def measured_traffic(step):
    """Scaled HBM bytes (read + written) of one launch of `step` ("attention", or "w2/attention" for another
    workload), or None if it was not measured or its kernel changed since."""
    import hashlib

    if step not in MEASURED_TRAFFIC:
        return None
    files, digest, fetch_kib, write_kib = MEASURED_TRAFFIC[step]
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "block_sparse_long_pisa_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    if not h.hexdigest().startswith(digest):
        return None
    return round(1024.0 * (fetch_kib * COPY_SCALE["fetch"] + write_kib * COPY_SCALE["write"]))


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# algorithmic work (what the method must move or compute; masked work excluded)


def attended_pairs(p, idx, cnt):
    """Sum over query rows of |attended keys| for a prefill (numpy, exact integers)."""
    import numpy as np

    bs, s, N, G = p.block_size, p.sink_len, p.seq_len, p.group
    nb = p.n_blocks
    j0 = s // bs
    qb = np.arange(nb)
    rows = np.minimum(bs, N - qb * bs).astype(np.int64)
    s_eff = np.minimum(s, qb * bs)
    total = 0
    for b in range(cnt.shape[0]):
        for g in range(cnt.shape[1]):
            c = cnt[b, g].astype(np.int64)
            first = idx[b, g, :, 0] if idx.shape[-1] else np.full(nb, -1)
            has_j0 = (c > 0) & (first == j0)
            overlap = np.where(has_j0 & (j0 * bs < s_eff), np.minimum(s_eff, (j0 + 1) * bs) - j0 * bs, 0)
            before = c * bs + s_eff - overlap
            total += int(np.sum(rows * before + rows * (rows + 1) // 2)) * G
    return total


def attended_pairs_bidirectional(p, idx, cnt):
    """Sum over query rows of |attended keys| for the non-causal variant (exact integers)."""
    import numpy as np

    bs, N, G = p.block_size, p.seq_len, p.group
    s = min(p.sink_len, N)
    j0 = p.sink_len // bs
    nb = p.n_blocks
    size = np.minimum(bs, N - np.arange(nb) * bs).astype(np.int64)  # keys per block
    sink_in = np.clip(np.minimum(s, (np.arange(nb) + 1) * bs) - np.arange(nb) * bs, 0, None)  # keys of block j in the sink
    total = 0
    for b in range(cnt.shape[0]):
        for g in range(cnt.shape[1]):
            for qb in range(nb):
                sel = idx[b, g, qb, :cnt[b, g, qb]]
                keys = s + int(size[sel].sum() - sink_in[sel].sum()) + int(size[qb] - sink_in[qb])
                total += int(size[qb]) * keys
    return total * G


def pyramid_bytes(p, nodes):
    elt = 2 if p.dtype == "bf16" else 4
    return p.batch * p.heads_kv * p.seq_len * p.head_dim * elt + p.batch * p.heads_kv * nodes * p.head_dim * 4


def select_bytes(p, nodes):
    elt = 2 if p.dtype == "bf16" else 4
    nb = p.n_blocks
    return (p.batch * p.heads_q * p.seq_len * p.head_dim * elt + p.batch * p.heads_kv * nodes * p.head_dim * 4 +
            p.batch * p.heads_kv * nb * (p.top_k + 1) * 4)


def decode_scored_nodes(p, cache_len):
    """Pool sizes of the descent for the decode token (no sink filtering needed at these shapes)."""
    f, L, K, bs = p.fanout, p.levels, p.top_k, p.block_size
    qb = (cache_len - 1) // bs
    j0 = p.sink_len // bs
    span = [f ** l for l in range(L)]
    anc = [qb // s for s in span]
    pool = max(0, anc[L - 1] - j0 // span[L - 1])
    total = pool
    for l in range(L - 1, 0, -1):
        kept = min(K, pool)
        pool = kept * f + (anc[l - 1] - anc[l] * f)
        total += pool
    return total


def decode_bytes(p, cache_len, cnt):
    """K/V rows attended + pyramid rows scored + q + out, for one step.

    cache_len: one length for every sequence, or a list of per-sequence lengths.
    """
    bs, s, d = p.block_size, p.sink_len, p.head_dim
    lens = [int(cache_len)] * cnt.shape[0] if isinstance(cache_len, (int, np_int_types())) else list(cache_len)
    total_keys = 0
    summaries = 0
    for b in range(cnt.shape[0]):
        pos = lens[b] - 1
        qb = pos // bs
        for g in range(cnt.shape[1]):
            c = int(cnt[b, g])
            total_keys += c * bs + min(s, qb * bs) + (pos - qb * bs + 1)  # sink overlap with block 0 ignored
        summaries += p.heads_kv * decode_scored_nodes(p, lens[b]) * d * 4
    kv = total_keys * d * 2 * 2
    qo = 2 * p.batch * p.heads_q * d * 2
    return kv + summaries + qo


def np_int_types():
    import numpy as np

    return np.integer


def append_bytes(p, old_lens, new_lens):
    """Key rows read and pyramid nodes read and written by one pyramid append."""
    bs, f, d, L = p.block_size, p.fanout, p.head_dim, p.levels
    elt = 2 if p.dtype == "bf16" else 4
    total = 0
    for a, z in zip(old_lens, new_lens):
        if not 0 <= a < z <= p.seq_len:
            continue
        j0, j1 = a // bs, (z - 1) // bs
        rows = z - j0 * bs  # rows of the affected leaves
        nodes_read, nodes_written = 0, j1 - j0 + 1
        present = j1 + 1
        lo, hi = j0, j1
        for _ in range(1, L):
            na, nz = lo // f, hi // f
            nodes_read += sum(min(f, present - n * f) for n in range(na, nz + 1))
            nodes_written += nz - na + 1
            lo, hi, present = na, nz, -(-present // f)
        total += p.heads_kv * (rows * d * elt + (nodes_read + nodes_written) * d * 4)
    return total


# ---------------------------------------------------------------------------
# what this GPU reaches on plain library work (context for the peaks)


def achievable_probes(torch, dev, reps=10):
    """A large device copy (torch copy_, 2 GiB into 2 GiB; read + write bytes) and
    a dense bf16 GEMM (torch matmul, 8192^3). Reported beside the published peaks,
    which stay the denominators of every fraction."""
    x = torch.ones(1 << 29, dtype=torch.float32, device=dev)
    y = torch.empty_like(x)
    a = torch.randn((8192, 8192), device=dev, dtype=torch.float32).to(torch.bfloat16)
    bm = torch.randn((8192, 8192), device=dev, dtype=torch.float32).to(torch.bfloat16)
    for _ in range(3):
        y.copy_(x)
        torch.matmul(a, bm)
    torch.cuda.synchronize()
    e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    e[0].record()
    for _ in range(reps):
        y.copy_(x)
    e[1].record()
    for _ in range(reps):
        torch.matmul(a, bm)
    e[2].record()
    torch.cuda.synchronize()
    t_read = e[0].elapsed_time(e[1]) * 1e-3 / reps
    t_gemm = e[1].elapsed_time(e[2]) * 1e-3 / reps
    copy_bw = 2 * x.numel() * 4 / t_read
    gemm = 2.0 * 8192 ** 3 / t_gemm
    del x, y, a, bm
    torch.cuda.empty_cache()
    log(f"probes: device copy {copy_bw / 1e9:.0f} GB/s (read + write), bf16 GEMM {gemm / 1e12:.0f} TFLOP/s")
    return {
        "copy_GB/s": copy_bw / 1e9, "copy_frac": copy_bw / HBM_PEAK,
        "bf16_gemm_TFLOP/s": gemm / 1e12, "bf16_gemm_frac": gemm / BF16_PEAK,
        "what": "torch copy_ of 2 GiB into 2 GiB (bytes read + written); torch matmul of two 8192x8192 bf16 "
                "matrices",
    }


# ---------------------------------------------------------------------------
# CPU oracle on a bounded sample


def cpu_baseline(p, q, k, v, seed_units=0):
    """Time the oracle (numpy fp64) on a sample of the prefill workload and scale to tokens/s."""
    import numpy as np
    import torch

    import oracle

    try:
        from threadpoolctl import threadpool_info

        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    t_all = time.perf_counter()
    G, bs, nb = p.group, p.block_size, p.n_blocks
    # the oracle sees one KV head at a time: Q of its group, its K and V
    n_heads = p.heads_kv
    qh = [q[:, g * G:(g + 1) * G].float().cpu().numpy() for g in range(1)]
    kh = [k[:, g:g + 1].float().cpu().numpy() for g in range(n_heads)]
    vh = [v[:, g:g + 1].float().cpu().numpy() for g in range(1)]
    # stage 1: pyramid of n_heads KV heads (full length)
    t0 = time.perf_counter()
    pyr = [oracle.build_pyramid(kk, bs, p.fanout, p.levels) for kk in kh]
    t_pyr = (time.perf_counter() - t0) / n_heads * p.heads_kv
    # stage 2: selection of a sample of query blocks
    t0 = time.perf_counter()
    qbar = [oracle.query_block_means(qq, 1, bs) for qq in qh]
    t_qbar = (time.perf_counter() - t0) * p.heads_kv
    rng = np.random.default_rng(seed_units)
    sel_units = np.sort(rng.choice(nb, min(nb, 1024), replace=False))
    sels = {}
    t0 = time.perf_counter()
    for qb in sel_units:
        lv = [lvl[0, 0] for lvl in pyr[0]]
        sels[int(qb)] = oracle.descend(lv, qbar[0][0, 0, qb], int(qb), p.top_k, p.sink_len, bs, p.fanout)
    t_sel = (time.perf_counter() - t0) / len(sel_units) * nb * p.heads_kv + t_qbar
    # stage 3: attention for the same sample of units (all G heads, all rows)
    att_units = sel_units
    t0 = time.perf_counter()
    for qb in att_units:
        sel = sels[int(qb)]
        r0, r1 = int(qb) * bs, min(p.seq_len, (int(qb) + 1) * bs)
        for h in range(G):
            oracle.attend_block(qh[0][0, h, r0:r1], kh[0][0, 0], vh[0][0, 0], r0, sel, p.sink_len, bs, p.scale)
    t_att = (time.perf_counter() - t0) / len(att_units) * nb * p.heads_kv
    total = t_pyr + t_sel + t_att
    return dict(
        value=p.batch * p.seq_len / total,
        unit="tokens/s",
        cores=int(threads),
        kind="oracle",
        sample=(f"pyramid of {n_heads}/{p.heads_kv} KV heads (full length), selection of {len(sel_units)} query "
                f"blocks and attention of {len(att_units)} query blocks x {G} heads of KV head 0, each stage scaled "
                f"to all {nb * p.heads_kv} units; stage seconds extrapolated: pyramid {t_pyr:.1f}, selection "
                f"{t_sel:.1f}, attention {t_att:.1f}; sample wall time {time.perf_counter() - t_all:.1f} s"),
    )


# ---------------------------------------------------------------------------


def median_ms(pairs):
    """Median of event intervals (start, end) in seconds."""
    import numpy as np

    return float(np.median([a.elapsed_time(b) for a, b in pairs])) * 1e-3


def prefill_buffers(p, cp, dev):
    import torch

    import block_sparse_long_pisa_amd as pisa

    nodes = pisa.pyramid_layout(cp)[-1]
    nb = p.n_blocks
    pyr = torch.empty((p.batch, p.heads_kv, nodes, p.head_dim), dtype=torch.float32, device=dev)
    idx = torch.empty((p.batch, p.heads_kv, nb, p.top_k), dtype=torch.int32, device=dev)
    cnt = torch.empty((p.batch, p.heads_kv, nb), dtype=torch.int32, device=dev)
    return nodes, pyr, idx, cnt


def time_prefill(p, cp, q, k, v, pyr, idx, cnt, out, steps, warmup):
    """Wall time per step over `steps` steps (after `warmup`), then the median
    HIP-event time of each kernel over `steps` more steps. Events are recorded on
    torch's current stream, the stream the binding launches on."""
    import torch

    import block_sparse_long_pisa_amd as pisa

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        pisa.build_pyramid(cp, k, pyr)
        if ev is not None:
            ev[1].record()
        pisa.select_topk(cp, q, pyr, idx, cnt)
        if ev is not None:
            ev[2].record()
        pisa.sparse_attn_fwd(cp, q, k, v, idx, cnt, out)
        if ev is not None:
            ev[3].record()

    torch.cuda.synchronize()
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    for e in evs:
        step(e)
    torch.cuda.synchronize()
    t_pool = median_ms([(e[0], e[1]) for e in evs])
    t_sel = median_ms([(e[1], e[2]) for e in evs])
    t_att = median_ms([(e[2], e[3]) for e in evs])
    return elapsed / steps, t_pool, t_sel, t_att


def kernel_lines(p, nodes, idx, cnt, t_pool, t_sel, t_att, workload=None):
    idx_h, cnt_h = idx.cpu().numpy(), cnt.cpu().numpy()
    pairs = attended_pairs(p, idx_h, cnt_h)
    flops = 4.0 * p.head_dim * pairs
    b_pool = pyramid_bytes(p, nodes)
    b_sel = select_bytes(p, nodes)
    tr = (lambda step: measured_traffic(f"{workload}/{step}")) if workload else measured_traffic
    return flops, pairs, {
        "pyramid": {"ms": t_pool * 1e3, "bound": "hbm", "bytes": b_pool, "GB/s": b_pool / t_pool / 1e9,
                    "frac": b_pool / t_pool / HBM_PEAK, "traffic": tr("pyramid")},
        "select": {"ms": t_sel * 1e3, "bound": "hbm", "bytes": b_sel, "GB/s": b_sel / t_sel / 1e9,
                   "frac": b_sel / t_sel / HBM_PEAK, "traffic": tr("select")},
        "attention": {"ms": t_att * 1e3, "bound": "mfma", "flops": flops, "TFLOP/s": flops / t_att / 1e12,
                      "frac": flops / t_att / BF16_PEAK, "attended_pairs": pairs, "traffic": tr("attention")},
    }


WORKLOAD_TEXT = {
    2: "PISA prefill, bf16 causal MHA 32 heads, N=32768, d=128, block 64, fanout 8, 3 levels, K=16, 64-token sink, "
       "1 local block; 8 planted (query block, target) pairs per head",
    3: "PISA prefill, bf16 causal GQA 32q/8kv heads, N=131072, d=128, block 128, fanout 8, 4 levels, K=32, "
       "64-token sink, 1 local block; planted needles at 16 depths per KV head",
    5: "PISA prefill, bf16 causal one GQA group 4q/1kv heads, N=1048576, d=128, block 128, fanout 8, 5 levels, "
       "K=64, 64-token sink, 1 local block; 32 planted needles at log-uniform distances",
}


def run_other_prefill(wid, args, dev):
    """One more prefill workload timed like the headline one (its own line under
    `workloads`, not the headline value)."""
    import torch

    import block_sparse_long_pisa_amd as pisa
    import gen

    cfg = gen.workload(wid)
    p = cfg["problem"]
    cp = pisa.problem(p.batch, p.heads_q, p.heads_kv, p.seq_len, p.head_dim, p.block_size, p.fanout, p.levels,
                      p.top_k, p.sink_len, p.dtype)
    log(f"generating {cfg['name']} on the GPU")
    q, k, v, _ = gen.device_inputs(p, cfg["seed"], cfg["value_scale"], cfg["plant"], device=dev)
    nodes, pyr, idx, cnt = prefill_buffers(p, cp, dev)
    out = torch.empty_like(q)
    steps = args.workload_steps
    t_step, t_pool, t_sel, t_att = time_prefill(p, cp, q, k, v, pyr, idx, cnt, out, steps, args.warmup)
    flops, pairs, kernels = kernel_lines(p, nodes, idx, cnt, t_pool, t_sel, t_att, workload=f"w{wid}")
    log(f"workload {wid}: {t_step * 1e3:.3f} ms/step: pyramid {t_pool * 1e3:.3f} ms "
        f"({kernels['pyramid']['frac'] * 100:.0f}% HBM), select {t_sel * 1e3:.3f} ms "
        f"({kernels['select']['frac'] * 100:.0f}% HBM), attention {t_att * 1e3:.3f} ms "
        f"({kernels['attention']['frac'] * 100:.1f}% MFMA)")
    del q, k, v, out, pyr, idx, cnt
    torch.cuda.empty_cache()
    return {
        "workload": WORKLOAD_TEXT[wid],
        "seed": cfg["seed"],
        "steps": steps,
        "ms_per_step": t_step * 1e3,
        "tokens_per_s": p.batch * p.seq_len / t_step,
        "kernel_sum_ms": (t_pool + t_sel + t_att) * 1e3,
        "tokens_per_s_kernels": p.batch * p.seq_len / (t_pool + t_sel + t_att),
        "kernels": kernels,
    }


def run_prefill(args, dev):
    import numpy as np
    import torch

    import block_sparse_long_pisa_amd as pisa
    import gen

    cfg = gen.workload(3)
    p = cfg["problem"]
    cp = pisa.problem(p.batch, p.heads_q, p.heads_kv, p.seq_len, p.head_dim, p.block_size, p.fanout, p.levels,
                      p.top_k, p.sink_len, p.dtype)
    log(f"generating {cfg['name']} on the GPU")
    q, k, v, _ = gen.device_inputs(p, cfg["seed"], cfg["value_scale"], cfg["plant"], device=dev)
    nodes, pyr, idx, cnt = prefill_buffers(p, cp, dev)
    nb = p.n_blocks
    out = torch.empty_like(q)
    log(f"warmup {args.warmup}, timing {args.steps} steps")
    t_step, t_pool, t_sel, t_att = time_prefill(p, cp, q, k, v, pyr, idx, cnt, out, args.steps, args.warmup)
    elapsed = t_step * args.steps
    ms_per_step = t_step * 1e3
    flops, pairs, kernels = kernel_lines(p, nodes, idx, cnt, t_pool, t_sel, t_att)
    log(f"prefill {ms_per_step:.3f} ms/step: pyramid {t_pool * 1e3:.3f} ms, select {t_sel * 1e3:.3f} ms, "
        f"attention {t_att * 1e3:.3f} ms ({flops / t_att / 1e12:.1f} TFLOP/s)")

    result = {
        "metric": "sparse-attn prefill tokens/s @128K + decode µs/step; % HBM & MFMA peak",
        "value": p.batch * p.seq_len / (elapsed / args.steps),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "PISA prefill, bf16 causal GQA 32q/8kv heads, N=131072, d=128, block 128, fanout 8, "
                        "4 levels, K=32, 64-token sink, 1 local block; planted needles at 16 depths per KV head",
            "batch": p.batch, "seq_len": p.seq_len, "heads_q": p.heads_q, "heads_kv": p.heads_kv,
            "head_dim": p.head_dim, "block_size": p.block_size, "fanout": p.fanout, "levels": p.levels,
            "top_k": p.top_k, "sink_len": p.sink_len, "seed": cfg["seed"],
        },
        "roofline": {
            "kernel": "attn_bf16_kernel (sparse attention)",
            "bound": "mfma",
            "achieved": flops / t_att / 1e12,
            "peak": BF16_PEAK / 1e12,
            "unit": "TFLOP/s",
            "frac": flops / t_att / BF16_PEAK,
            "traffic": measured_traffic("attention"),
            "algorithmic_flops_per_launch": flops,
            "avg_launch_ms": t_att * 1e3,
        },
        "kernels": kernels,
    }

    if args.fused:
        # the fused selection + attention (one launch) on the same pyramid, beside
        # the two launches it replaces
        pisa.build_pyramid(cp, k, pyr)
        for _ in range(args.warmup):
            pisa.select_attend(cp, q, k, v, pyr, idx, cnt, out)
        torch.cuda.synchronize()
        fe = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.fused_steps)]
        for e in fe:
            e[0].record()
            pisa.select_attend(cp, q, k, v, pyr, idx, cnt, out)
            e[1].record()
        torch.cuda.synchronize()
        t_fu = median_ms([(e[0], e[1]) for e in fe])
        log(f"fused select+attend {t_fu * 1e3:.3f} ms, against select + attention {(t_sel + t_att) * 1e3:.3f} ms")
        result["fused"] = {
            "workload": "the same prefill: pisa_select_attend (query mean, descent and attention in one launch) "
                        "on the built pyramid",
            "ms": t_fu * 1e3,
            "two_launch_ms": (t_sel + t_att) * 1e3,
            "step_ms": (t_pool + t_fu) * 1e3,
            "tokens_per_s": p.batch * p.seq_len / (t_pool + t_fu),
            "TFLOP/s": flops / t_fu / 1e12,
            "frac": flops / t_fu / BF16_PEAK,
        }

    if args.variants:
        # the variants on the same inputs: bidirectional (mean summaries) and
        # causal with max-pooled summaries; one step = pyramid, selection, attention
        result["variants"] = {}
        for name, causal, pool in (("bidirectional", 0, "mean"), ("max_pool", 1, "max")):
            vp = pisa.problem(p.batch, p.heads_q, p.heads_kv, p.seq_len, p.head_dim, p.block_size, p.fanout,
                              p.levels, p.top_k, p.sink_len, p.dtype, causal=causal, pool=pool)

            def vstep(ev=None):
                if ev is not None:
                    ev[0].record()
                pisa.build_pyramid(vp, k, pyr)
                pisa.select_topk(vp, q, pyr, idx, cnt)
                if ev is not None:
                    ev[1].record()
                pisa.sparse_attn_fwd(vp, q, k, v, idx, cnt, out)
                if ev is not None:
                    ev[2].record()

            for _ in range(args.warmup):
                vstep()
            torch.cuda.synchronize()
            ve = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.variant_steps)]
            for e in ve:
                vstep(e)
            torch.cuda.synchronize()
            t_ps = median_ms([(e[0], e[1]) for e in ve])
            t_at = median_ms([(e[1], e[2]) for e in ve])
            ih, ch = idx.cpu().numpy(), cnt.cpu().numpy()
            vpairs = attended_pairs(p, ih, ch) if causal else attended_pairs_bidirectional(p, ih, ch)
            vfl = 4.0 * p.head_dim * vpairs
            log(f"variant {name}: {(t_ps + t_at) * 1e3:.3f} ms/step (pyramid+select {t_ps * 1e3:.3f} ms, "
                f"attention {t_at * 1e3:.3f} ms, {vfl / t_at / 1e12:.1f} TFLOP/s)")
            result["variants"][name] = {
                "causal": bool(causal), "pool": pool,
                "ms_per_step": (t_ps + t_at) * 1e3,
                "tokens_per_s": p.batch * p.seq_len / (t_ps + t_at),
                "pyramid_select_ms": t_ps * 1e3,
                "attention_ms": t_at * 1e3,
                "attention_TFLOP/s": vfl / t_at / 1e12,
                "attention_frac": vfl / t_at / BF16_PEAK,
            }

    if args.backward:
        # backward of the same attention: the forward's output and lse, an output
        # gradient, then dq, dk, dv (selection held constant)
        lse = torch.empty((p.batch, p.heads_q, p.seq_len), dtype=torch.float32, device=dev)
        pisa.sparse_attn_fwd(cp, q, k, v, idx, cnt, out, lse)
        dout = torch.randn_like(q)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        bws = torch.empty(pisa.sparse_attn_bwd_workspace_size(cp), dtype=torch.uint8, device=dev)
        for _ in range(args.warmup):
            pisa.sparse_attn_bwd(cp, q, k, v, idx, cnt, out, lse, dout, dq, dk, dv, workspace=bws)
        torch.cuda.synchronize()
        be = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.backward_steps)]
        for e in be:
            e[0].record()
            pisa.sparse_attn_bwd(cp, q, k, v, idx, cnt, out, lse, dout, dq, dk, dv, workspace=bws)
            e[1].record()
        torch.cuda.synchronize()
        t_bwd = median_ms([(e[0], e[1]) for e in be])
        bflops = 10.0 * p.head_dim * pairs  # S, dP, dV, dK, dQ products over the attended pairs
        log(f"backward {t_bwd * 1e3:.3f} ms ({bflops / t_bwd / 1e12:.1f} TFLOP/s)")
        result["backward"] = {
            "workload": "gradients dq, dk, dv of the same 128K GQA sparse attention (selection held constant)",
            "ms": t_bwd * 1e3,
            "steps": args.backward_steps,
            "bound": "mfma",
            "algorithmic_flops": bflops,
            "TFLOP/s": bflops / t_bwd / 1e12,
            "frac": bflops / t_bwd / BF16_PEAK,
            "workspace_bytes": bws.numel(),
        }
        del dout, dq, dk, dv, bws, lse

    if args.probes:
        result["achievable"] = achievable_probes(torch, dev)

    if args.copy_calibration:
        a = torch.empty(1 << 29, dtype=torch.int16, device=dev)
        bcopy = torch.empty_like(a)
        torch.cuda.synchronize()
        bcopy.copy_(a)
        torch.cuda.synchronize()
        result["copy_calibration_bytes"] = 2 * a.numel() * 2
        del a, bcopy

    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a sample")
        result["cpu_baseline"] = cpu_baseline(p, q, k, v)
    del q, k, v, out, pyr
    torch.cuda.empty_cache()

    return result


def run_decode(args, dev):
    import torch

    import block_sparse_long_pisa_amd as pisa
    import gen

    dcfg = gen.workload(4)
    dp = dcfg["problem"]
    dcp = pisa.problem(dp.batch, dp.heads_q, dp.heads_kv, dp.seq_len, dp.head_dim, dp.block_size, dp.fanout,
                       dp.levels, dp.top_k, dp.sink_len, dp.dtype)
    cache_len = dp.seq_len
    log(f"generating {dcfg['name']} on the GPU")
    dq, kc, vc, _ = gen.device_decode_inputs(dp, dcfg["seed"], dcfg["value_scale"], cache_len, device=dev)
    dpyr = pisa.build_pyramid(dcp, kc)  # built once over the cache, not timed
    ws = torch.empty(pisa.decode_workspace_size(dcp), dtype=torch.uint8, device=dev)
    dout = torch.empty_like(dq)
    didx = torch.empty((dp.batch, dp.heads_kv, dp.top_k), dtype=torch.int32, device=dev)
    dcnt = torch.empty((dp.batch, dp.heads_kv), dtype=torch.int32, device=dev)
    for _ in range(args.warmup):
        pisa.decode_step(dcp, dq, kc, vc, dpyr, cache_len, out=dout, idx_out=didx, cnt_out=dcnt, workspace=ws)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(args.decode_steps):
        pisa.decode_step(dcp, dq, kc, vc, dpyr, cache_len, out=dout, idx_out=didx, cnt_out=dcnt, workspace=ws)
    e1.record()
    torch.cuda.synchronize()
    t_dec = (time.perf_counter() - t0) / args.decode_steps
    t_dec_ev = e0.elapsed_time(e1) * 1e-3 / args.decode_steps
    db = decode_bytes(dp, cache_len, dcnt.cpu().numpy())
    log(f"decode {t_dec * 1e6:.1f} us/step ({db / t_dec_ev / 1e9:.0f} GB/s)")
    decode = {
        "workload": "PISA decode, bf16 GQA 32q/8kv, 64 sequences x 131072-token cache, one new token each, "
                    "block 128, fanout 8, 4 levels, K=32, 64-token sink",
        "us_per_step": t_dec * 1e6,
        "us_per_step_events": t_dec_ev * 1e6,
        "tokens_per_s": dp.batch / t_dec,
        "steps": args.decode_steps,
        "bound": "hbm",
        "bytes_per_step": db,
        "GB/s": db / t_dec_ev / 1e9,
        "frac": db / t_dec_ev / HBM_PEAK,
        "traffic": measured_traffic("decode"),
    }

    # serving step: every sequence at its own length; each step appends one token
    # per sequence (its key and value are already in the cache), updates the
    # pyramid and decodes the batch at the new lengths
    import numpy as np

    nsteps = args.decode_steps + args.warmup
    rng = np.random.default_rng(dcfg["seed"])
    # lengths for two loops of nsteps steps (appended first, then beside the decode)
    base = rng.integers(dp.seq_len // 2, dp.seq_len - 2 * nsteps, size=dp.batch)
    lens_h = np.stack([base + s for s in range(2 * nsteps + 1)]).astype(np.int32)
    lens_d = torch.from_numpy(lens_h).to(dev)

    def serve(s, ev=None):
        if ev is not None:
            ev[0].record()
        pisa.pyramid_append(dcp, kc, dpyr, lens_d[s], lens_d[s + 1])
        if ev is not None:
            ev[1].record()
        pisa.decode_step_ragged(dcp, dq, kc, vc, dpyr, lens_d[s + 1], out=dout, idx_out=didx, cnt_out=dcnt,
                                workspace=ws)
        if ev is not None:
            ev[2].record()

    for s in range(args.warmup):
        serve(s)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.decode_steps)]
    t0 = time.perf_counter()
    for i in range(args.decode_steps):
        serve(args.warmup + i, evs[i])
    torch.cuda.synchronize()
    t_srv = (time.perf_counter() - t0) / args.decode_steps
    t_app = median_ms([(e[0], e[1]) for e in evs])
    t_rdec = median_ms([(e[1], e[2]) for e in evs])
    last = args.warmup + args.decode_steps - 1
    rb = decode_bytes(dp, lens_h[last + 1].tolist(), dcnt.cpu().numpy())
    ab = append_bytes(dp, lens_h[last].tolist(), lens_h[last + 1].tolist())
    log(f"serving step {t_srv * 1e6:.1f} us (append {t_app * 1e6:.1f} us, ragged decode {t_rdec * 1e6:.1f} us, "
        f"{rb / t_rdec / 1e9:.0f} GB/s)")

    # The same loop with each step's append and decode in one call
    # (pisa_decode_step_ragged_append): the append runs in the selection's launch.
    def serve_one_call(s):
        pisa.decode_step_ragged_append(dcp, dq, kc, vc, dpyr, lens_d[s], lens_d[s + 1], out=dout, idx_out=didx,
                                       cnt_out=dcnt, workspace=ws)

    for s in range(nsteps, nsteps + args.warmup):
        serve_one_call(s)
    torch.cuda.synchronize()
    e0.record()
    t0 = time.perf_counter()
    for i in range(args.decode_steps):
        serve_one_call(nsteps + args.warmup + i)
    e1.record()
    torch.cuda.synchronize()
    t_one = (time.perf_counter() - t0) / args.decode_steps
    t_one_ev = e0.elapsed_time(e1) * 1e-3 / args.decode_steps
    log(f"serving step in one call (append in the selection's launch) {t_one * 1e6:.1f} us")
    decode["serving"] = {
        "workload": "64 sequences at lengths uniform in [65536, 131072), one token appended per sequence per step: "
                    "pyramid append then ragged decode",
        "us_per_step": t_srv * 1e6,
        "append_us": t_app * 1e6,
        "decode_us": t_rdec * 1e6,
        "tokens_per_s": dp.batch / t_srv,
        "decode_bytes": rb,
        "append_bytes": ab,
        "decode_GB/s": rb / t_rdec / 1e9,
        "decode_frac": rb / t_rdec / HBM_PEAK,
        "one_call": {
            "workload": "the same serving loop, each step's append and decode in one call "
                        "(pisa_decode_step_ragged_append: the append runs in the selection's launch)",
            "us_per_step": t_one * 1e6,
            "us_per_step_events": t_one_ev * 1e6,
            "tokens_per_s": dp.batch / t_one,
        },
    }
    return decode


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--decode-steps", type=int, default=50)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--only", choices=["prefill", "decode", "w2", "w5"], default=None,
                    help="run one workload only (profiling); the JSON line then lacks the others")
    ap.add_argument("--workloads", dest="workloads", action="store_true", default=True,
                    help="also time the 32K MHA and the 1M single-group prefill workloads (default)")
    ap.add_argument("--no-workloads", dest="workloads", action="store_false")
    ap.add_argument("--workload-steps", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--backward", dest="backward", action="store_true", default=True,
                    help="also time the backward pass on the prefill workload (default)")
    ap.add_argument("--no-backward", dest="backward", action="store_false")
    ap.add_argument("--backward-steps", type=int, default=5)
    ap.add_argument("--variants", dest="variants", action="store_true", default=True,
                    help="also time the bidirectional and max-pool variants on the prefill workload (default)")
    ap.add_argument("--no-variants", dest="variants", action="store_false")
    ap.add_argument("--variant-steps", type=int, default=5)
    ap.add_argument("--fused", dest="fused", action="store_true", default=True,
                    help="also time the fused selection + attention on the prefill workload (default)")
    ap.add_argument("--no-fused", dest="fused", action="store_false")
    ap.add_argument("--fused-steps", type=int, default=5)
    ap.add_argument("--probes", dest="probes", action="store_true", default=True,
                    help="also measure a plain stream read and a dense bf16 GEMM on this GPU (default)")
    ap.add_argument("--no-probes", dest="probes", action="store_false")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain 1 GiB device copy (counter calibration for rocprofv3 --pmc runs)")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}): the library runs on one GPU; run with --gpus 1", flush=True)
        return 2

    import numpy as np
    import torch

    import block_sparse_long_pisa_amd as pisa
    import gen

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.only == "decode":
        result = {"metric": "decode µs/step (profiling run)", "decode": run_decode(args, dev)}
    elif args.only in ("w2", "w5"):
        wid = int(args.only[1])
        result = {"metric": f"prefill workload {wid} (profiling run)", "workload": run_other_prefill(wid, args, dev)}
    else:
        result = run_prefill(args, dev)
        if args.only is None:
            if args.workloads:
                result["workloads"] = {f"w{w}": run_other_prefill(w, args, dev) for w in (2, 5)}
            if not args.no_decode:
                result["decode"] = run_decode(args, dev)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
