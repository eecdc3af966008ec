#!/usr/bin/env python3
"""Benchmark of the quantized paged KV cache on one MI355X.

A step is one decode step of the workload: quantize-on-write of the step's
new token of every sequence, then paged decode attention of every sequence
over its whole cache, both in one launch (kvq_decode_step; ``--unfused``
runs kvq_reshape_and_cache then kvq_paged_decode_attention instead).
The default workload is the INT8 per-token-head symmetric decode (batch 32,
32 q / 8 kv heads, head_dim 128, block 64, seq_lens ~U[1024, 8192], 4 outlier
channels x10); --config selects the others.  The cache is built once (untimed)
and copied into enough replicas (>= 1.2 GB in total) that steps cycle through
memory larger than the 256 MB Infinity Cache.

Prints ONE JSON line.  ``value`` is decode effective KV GB/s of the whole
step: the algorithmic bytes decode reads (packed codes + fp32 scale/zero of
attended tokens, plus queries, outputs and block-table entries) divided by
the step time, steps launched back to back (``--graph`` replays each from a
HIP graph instead).  ``roofline`` is the step's kernel alone: after the
timed steps, ``steps`` back-to-back launches between two HIP events on the
stream it runs on, divided by ``steps``; its algorithmic bytes add the new
tokens' write (bf16 rows read, codes + meta + slots).  ``decode_only`` is
kvq_paged_decode_attention timed the same way, ``write.step_write_us`` the
step's write alone.  ``write`` also reports quantize-write tokens/s on a
whole-cache fill, ``gather`` the dequantize-gather of the whole cache.
Fractions are against the 8 TB/s nominal and, as ``frac_of_measured_copy``,
against a 1 GiB device copy timed in the same run.  ``cpu_baseline`` times the oracle on a bounded sample.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402
import sub_byte_quantized_amd as kvq  # noqa: E402

HBM_PEAK_GBS = 8000.0
MALL_BYTES = 256 << 20
CSRC = os.path.join(ROOT, "sub_byte_quantized_amd", "csrc")
# sources that define the decode and prefill kernels (a counter summary is
# tied to them)
DECODE_SRC = [os.path.join(CSRC, f) for f in ("kvq_decode.hip", "kvq_device.h", "kvq_internal.h", "kvq_write_row.h")]
PREFILL_SRC = [os.path.join(CSRC, f) for f in ("kvq_prefill.hip", "kvq_device.h", "kvq_internal.h")]
GATHER_SRC = [os.path.join(CSRC, f) for f in ("kvq_gather.hip", "kvq_device.h", "kvq_internal.h")]
WRITE_SRC = [os.path.join(CSRC, f) for f in ("kvq_write.hip", "kvq_write_row.h", "kvq_device.h", "kvq_internal.h")]


def sha(paths):
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def decode_algo_bytes(spec, case, first=0):
    """Algorithmic bytes one decode launch over sequences first..B-1 reads and
    writes: codes + meta of every attended token (positions inside the
    window, in non-evicted blocks, below seq_len), the block-table entries
    walked, queries and outputs."""
    P = spec.D * {0: 8, 1: 4, 2: 2}[spec.mode] // 8
    M = 1 if spec.mode == 0 else 2
    row = 2 * (P + 4 * M)
    lens = case.seq_lens.cpu().numpy().astype(np.int64)
    win = None if case.window is None else case.window.cpu().numpy()
    bt = None if case.block_tables is None else case.block_tables.cpu().numpy()
    bth = None if case.block_tables_headwise is None else case.block_tables_headwise.cpu().numpy()
    tokens = 0
    entries = 0
    for b in range(first, spec.B):
        L = int(lens[b])
        for h in range(spec.Hkv):
            W = int(win[h]) if win is not None else 0
            start = L - W if (W > 0 and L > W) else 0
            row_ids = bth[b * spec.Hkv + h] if bth is not None else bt[b]
            if L <= 0:
                continue
            j0, j1 = start // spec.bs, (L - 1) // spec.bs
            ids = row_ids[j0:j1 + 1]
            entries += len(ids)
            pos = np.arange(j0 * spec.bs, (j1 + 1) * spec.bs)
            keep = (pos >= start) & (pos < L) & np.repeat(ids >= 0, spec.bs)
            tokens += int(keep.sum())
    nb = spec.B - first
    kv = tokens * row
    q = nb * spec.Hq * spec.D * 2
    out = nb * spec.Hq * spec.D * 4
    return kv + q + out + 4 * entries + 4 * nb, kv, tokens


def prefill_work(spec, case):
    """Useful work of the mixed step's chunked prefill: unmasked (query row,
    key) pairs over the first n_prefill sequences (query i of sequence b at
    p = L - n + i sees keys j <= p in present blocks and, for a windowed kv
    head, j >= p - W + 1), times the G q heads; flops = 4 D per pair (q.k and
    p.v); KV bytes = codes + meta of the positions any row of the chunk sees."""
    P = spec.D * {0: 8, 1: 4, 2: 2}[spec.mode] // 8
    M = 1 if spec.mode == 0 else 2
    row = 2 * (P + 4 * M)
    G = spec.Hq // spec.Hkv
    lens = case.seq_lens.cpu().numpy().astype(np.int64)
    cu = case.cu_seqlens_q.cpu().numpy().astype(np.int64)
    win = None if case.window is None else case.window.cpu().numpy()
    bt = None if case.block_tables is None else case.block_tables.cpu().numpy()
    bth = None if case.block_tables_headwise is None else case.block_tables_headwise.cpu().numpy()
    pairs = 0
    kv_pos = 0
    for b in range(spec.n_prefill):
        L, n = int(lens[b]), int(cu[b + 1] - cu[b])
        for h in range(spec.Hkv):
            ids = (bth[b * spec.Hkv + h] if bth is not None else bt[b])[:(L + spec.bs - 1) // spec.bs]
            present = np.repeat(ids >= 0, spec.bs)[:L].astype(np.int64)
            csum = np.concatenate([[0], np.cumsum(present)])       # csum[j] = present positions < j
            p = L - n + np.arange(n)
            W = int(win[h]) if win is not None else 0
            lo = np.maximum(p - W + 1, 0) if W > 0 else np.zeros_like(p)
            pairs += int((csum[p + 1] - csum[lo]).sum()) * G
            kv_pos += int(csum[L] - csum[lo[0]])
    return pairs, 4 * spec.D * pairs, kv_pos * row


def write_bytes_per_token(spec):
    P = spec.D * {0: 8, 1: 4, 2: 2}[spec.mode] // 8
    M = 1 if spec.mode == 0 else 2
    slot = 8 * (spec.Hkv if spec.headwise else 1)
    return spec.Hkv * 2 * (spec.D * 2 + P + 4 * M) + slot


def gather_bytes(spec, case, nseq=None):
    """Algorithmic bytes of a dequantize-gather of the first `nseq` sequences'
    whole contexts (all by default): per (position, kv head) row of K and of
    V, the packed codes and fp32 meta read (rows in present blocks) and the
    bf16 row written; plus the block-table entries and cu_seq_lens read."""
    P = spec.D * {0: 8, 1: 4, 2: 2}[spec.mode] // 8
    M = 1 if spec.mode == 0 else 2
    lens = case.seq_lens.cpu().numpy().astype(np.int64)[:nseq]
    present = 0
    entries = 0
    for b, L in enumerate(lens):
        nblk = -(-int(L) // spec.bs)
        for h in range(spec.Hkv):
            if case.block_tables_headwise is not None:
                row = case.tables.block_tables_headwise[b * spec.Hkv + h, :nblk]
            else:
                row = case.tables.block_tables[b, :nblk]
            pos_ok = np.repeat(row >= 0, spec.bs)[:L]
            present += int(pos_ok.sum())
            entries += nblk
    rows = int(lens.sum()) * spec.Hkv
    return 2 * present * (P + 4 * M) + 2 * rows * 2 * spec.D + 4 * entries + 4 * (len(lens) + 1)


def gather_cpu(spec, case, planes, lens, seconds):
    """The oracle's gather on the host cores: (sequence, kv head) pairs until
    ~`seconds` have passed, as bytes of the same accounting per second."""
    import oracle
    pl = [p.cpu().numpy() for p in planes]
    signs = None if case.rot_signs is None else case.rot_signs.cpu().numpy()
    bt = case.tables.block_tables
    bth = case.tables.block_tables_headwise
    P = spec.D * {0: 8, 1: 4, 2: 2}[spec.mode] // 8
    M = 1 if spec.mode == 0 else 2
    done, nbytes = 0, 0
    t0 = time.perf_counter()
    for b in range(spec.B):
        for h in range(spec.Hkv):
            oracle.gather_head(b, h, int(lens[b]), spec.mode, spec.D, spec.bs, spec.Hkv, *pl, signs=signs,
                               block_tables=bt, block_tables_headwise=bth)
            done += 1
            nbytes += 2 * int(lens[b]) * (P + 4 * M + 2 * spec.D)
            if time.perf_counter() - t0 > seconds:
                break
        if time.perf_counter() - t0 > seconds:
            break
    dt = time.perf_counter() - t0
    return {"GBps": round(nbytes / dt / 1e9, 4), "sample": f"{done} of {spec.B * spec.Hkv} (sequence, kv head) "
            f"pairs in {dt:.1f} s", "cores": int(torch.get_num_threads()), "kind": "oracle"}


def build_workload(spec, dev):
    case = synth.make_case(spec, dev)
    d = kvq.CacheDesc(spec.mode, spec.D, spec.Hkv, spec.bs, case.tables.num_blocks, case.rot_signs)
    planes = kvq.alloc_cache(d, dev, poison=True)
    kvq.kvq_reshape_and_cache(d, case.k, case.v, *planes, slot_mapping=case.slot_mapping,
                              slot_mapping_headwise=case.slot_mapping_headwise)
    # the step's new tokens: the last n_b positions of sequence b (one for a
    # decode sequence, the chunk for a prefill sequence)
    lens = case.seq_lens.cpu().numpy().astype(np.int64)
    n_new = synth.new_tokens_of(spec)
    ends = np.cumsum(lens)
    last = np.concatenate([np.arange(e - n, e) for e, n in zip(ends, n_new)])
    li = torch.as_tensor(last, device=dev)
    new = dict(k=case.k[li].contiguous(), v=case.v[li].contiguous(),
               sm=None if case.slot_mapping is None else case.slot_mapping[li].contiguous(),
               smh=None if case.slot_mapping_headwise is None else case.slot_mapping_headwise[li].contiguous())
    torch.cuda.synchronize()
    return case, d, planes, new


def measured_copy_gbs(dev, reps=5):
    """Device-copy rate: 2 x 1 GiB moved per copy_ (read + write), best of
    `reps` launches."""
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    ms = min(time_events(lambda i: dst.copy_(src), reps))
    del src, dst
    return 2 * n / (ms * 1e-3) / 1e9


def time_events(fn, reps):
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
    for i in range(reps):
        starts[i].record()
        fn(i)
        ends[i].record()
    torch.cuda.synchronize()
    return [s.elapsed_time(e) for s, e in zip(starts, ends)]


def time_span(fn, reps):
    """Mean duration of `reps` back-to-back calls: one HIP event before the
    first and one after the last, on the current stream (the kernels' own)."""
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(reps):
        fn(i)
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / reps


def cpu_baseline(spec, case, planes, seconds, min_seconds=10.0):
    """The oracle, as it stands, on a bounded sample of the same decode: as
    many (sequence, kv head) pairs as fit in ``seconds``; a workload whose
    pairs all finish sooner is passed over again until ``min_seconds``."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        cores = 1
    host_planes = [p.cpu().numpy() for p in planes]
    q = case.q.float().cpu().numpy()
    lens = case.seq_lens.cpu().numpy()
    bt = None if case.block_tables is None else case.block_tables.cpu().numpy()
    bth = None if case.block_tables_headwise is None else case.block_tables_headwise.cpu().numpy()
    win = None if case.window is None else case.window.cpu().numpy()
    signs = None if case.rot_signs is None else case.rot_signs.cpu().numpy()
    P = spec.D * {0: 8, 1: 4, 2: 2}[spec.mode] // 8
    M = 1 if spec.mode == 0 else 2
    r = np.random.default_rng(0)
    order = [(int(b), int(h)) for b, h in zip(r.permutation(np.repeat(np.arange(spec.B), spec.Hkv)),
                                                np.tile(np.arange(spec.Hkv), spec.B))]
    done, nbytes, passes = 0, 0, 0
    t0 = time.perf_counter()
    while True:
        for b, h in order:
            oracle.decode_attention(q, lens, spec.mode, spec.D, spec.bs, spec.Hkv, *host_planes,
                                    case.softmax_scale, signs=signs, block_tables=bt,
                                    block_tables_headwise=bth, window=win, pairs=[(b, h)])
            W = int(win[h]) if win is not None else 0
            L = int(lens[b])
            nbytes += (min(L, W) if W > 0 else L) * 2 * (P + 4 * M)
            done += 1
            if time.perf_counter() - t0 >= seconds:
                break
        passes += 1
        if time.perf_counter() - t0 >= min(seconds, min_seconds):
            break
    dt = time.perf_counter() - t0
    # oracle write on a token sample
    tw0 = time.perf_counter()
    nt = 2048
    k = case.k[:nt].float().cpu().numpy()
    v = case.v[:nt].float().cpu().numpy()
    for src in (k, v):
        oracle.encode_rows(src.reshape(-1, spec.D), spec.mode, signs)
    tw = time.perf_counter() - tw0
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{done} (sequence, kv head) decode pairs of {spec.B * spec.Hkv} ({passes} pass(es)) in {dt:.1f} s "
                      f"(float64 attention over the GPU's stored planes); write: {nt} tokens in {tw:.2f} s",
            "write_tokens_per_s": round(nt / tw, 1)}


def load_traffic(name, srcs=DECODE_SRC):
    """HBM bytes per launch from the committed counter summary, or None if it
    is missing or was taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        j = json.load(f)
    if j.get("kernel_source_sha") != sha(srcs):
        return None
    return j.get("hbm_bytes_per_launch")


def oracle_prefill_sample(spec, case, planes, seconds):
    """The oracle's chunked prefill on a bounded sample: rows of one
    (sequence, kv head) pair, counted as unmasked pairs x 4 D flops."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        cores = 1
    b, h = 0, spec.Hkv - 1          # a full-context head
    bth = case.block_tables_headwise.cpu().numpy() if case.block_tables_headwise is not None else None
    bt = case.block_tables.cpu().numpy() if case.block_tables is not None else None
    ids = oracle.table_row(b, h, spec.Hkv, bt, bth)
    ids = np.unique(ids[ids >= 0])
    idx = torch.as_tensor(ids, device=planes[0].device)
    small = [p[idx].cpu().numpy() for p in planes]
    remap = np.full(case.tables.num_blocks, -1, np.int64)
    remap[ids] = np.arange(len(ids))
    bth2 = None if bth is None else np.where(bth >= 0, remap[np.maximum(bth, 0)], -1)
    bt2 = None if bt is None else np.where(bt >= 0, remap[np.maximum(bt, 0)], -1)
    q = case.q_prefill.float().cpu().numpy()
    cu = case.cu_seqlens_q.cpu().numpy()
    lens = case.seq_lens.cpu().numpy()
    win = None if case.window is None else case.window.cpu().numpy()
    signs = None if case.rot_signs is None else case.rot_signs.cpu().numpy()
    n = int(cu[1] - cu[0])
    L = int(lens[0])
    G = spec.Hq // spec.Hkv
    rows, pairs, t0 = 0, 0, time.perf_counter()
    while rows < n and time.perf_counter() - t0 < seconds:
        r = np.arange(rows, min(n, rows + 8))
        oracle.prefill_attention(q, cu[:2], lens[:1], spec.mode, spec.D, spec.bs, spec.Hkv, *small,
                                 case.softmax_scale, signs=signs, block_tables=bt2, block_tables_headwise=bth2,
                                 window=win, pairs=[(b, h)], rows=r)
        pairs += int(sum(L - n + i + 1 for i in r)) * G
        rows = int(r[-1]) + 1
    dt = time.perf_counter() - t0
    return {"value": round(4 * spec.D * pairs / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(cores),
            "kind": "oracle",
            "sample": f"{rows} of {n} query rows of sequence {b}, kv head {h} ({G} q heads) of the chunked "
                      f"prefill in {dt:.1f} s (float64 attention over the GPU's stored planes)"}


def run_mixed(args, spec, dev):
    """The mixed step: quantize-write of every sequence's new tokens (the
    chunk of each prefill sequence, one token of each decode sequence),
    chunked-prefill attention of the prefill sequences, decode attention of
    the others.  Prefill is MFMA work, so its roofline is TFLOP/s against the
    dense bf16 peak; decode is reported as effective KV GB/s."""
    t_setup = time.perf_counter()
    case, d, planes, new = build_workload(spec, dev)
    npf = spec.n_prefill
    Hkv = spec.Hkv
    max_len = int(case.seq_lens.max().item())
    # decode part: sequences npf..B-1
    dq = case.q[npf:].contiguous()
    dsl = case.seq_lens[npf:].contiguous()
    dbt = None if case.block_tables is None else case.block_tables[npf:].contiguous()
    dbth = None if case.block_tables_headwise is None else case.block_tables_headwise[npf * Hkv:].contiguous()
    ws = kvq.alloc_workspace(kvq.kvq_decode_workspace_size(d, spec.B - npf, spec.Hq, max_len), dev)
    dout = torch.empty((spec.B - npf, spec.Hq, spec.D), dtype=torch.float32, device=dev)
    # prefill part: sequences 0..npf-1
    psl = case.seq_lens[:npf].contiguous()
    pbt = None if case.block_tables is None else case.block_tables[:npf].contiguous()
    pbth = None if case.block_tables_headwise is None else case.block_tables_headwise[:npf * Hkv].contiguous()
    pout = torch.empty(case.q_prefill.shape, dtype=torch.float32, device=dev)
    max_q = int(spec.prefill_new)
    d_algo, d_kv, d_tokens = decode_algo_bytes(spec, case, first=npf)
    pairs, flops, p_kv = prefill_work(spec, case)
    setup_s = time.perf_counter() - t_setup

    def write(i):
        kvq.kvq_reshape_and_cache(d, new["k"], new["v"], *planes, slot_mapping=new["sm"],
                                  slot_mapping_headwise=new["smh"])

    def prefill(i):
        kvq.kvq_paged_prefill_attention(d, case.q_prefill, case.cu_seqlens_q, max_q, *planes, psl, max_len,
                                        block_tables=pbt, block_tables_headwise=pbth, window=case.window,
                                        softmax_scale=case.softmax_scale, out=pout)

    def decode(i):
        kvq.kvq_paged_decode_attention(d, dq, *planes, dsl, max_len, block_tables=dbt,
                                       block_tables_headwise=dbth, window=case.window,
                                       softmax_scale=case.softmax_scale, out=dout, workspace=ws)

    for i in range(args.warmup):
        write(i)
        prefill(i)
        decode(i)
    torch.cuda.synchronize()
    # timed region: exactly `steps` steps, the three kernels back to back
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        write(i)
        prefill(i)
        decode(i)
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    # the kernels inside a step, bracketed by events
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for i in range(args.steps):
        ev[i][0].record()
        write(i)
        ev[i][1].record()
        prefill(i)
        ev[i][2].record()
        decode(i)
        ev[i][3].record()
    torch.cuda.synchronize()
    w_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    p_step_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
    d_step_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in ev]))
    # each kernel alone: back-to-back launches between two HIP events
    p_ms = time_span(prefill, args.steps)
    d_ms = time_span(decode, args.steps)
    T = int(new["k"].shape[0])
    wb = write_bytes_per_token(spec)
    p_tf = flops / (p_ms * 1e-3) / 1e12
    d_gbs = d_algo / (d_ms * 1e-3) / 1e9
    # the prefill fallback: dequantize-gather of the prefill sequences' whole
    # contexts (positions 0 .. L - 1, head-wise table, bf16 rows [T, Hkv, D])
    lens = psl.cpu().numpy().astype(np.int64)
    cu_np = np.concatenate([[0], np.cumsum(lens)])
    cu = torch.as_tensor(cu_np.astype(np.int32), device=dev)
    g_tot = int(cu_np[-1])
    g_out = [torch.empty((g_tot, spec.Hkv, spec.D), dtype=torch.bfloat16, device=dev) for _ in range(2)]

    def gather(i):
        kvq.kvq_gather_dequant(d, *planes, cu, max_len, g_tot, block_tables=pbt, block_tables_headwise=pbth,
                               key_out=g_out[0], value_out=g_out[1])

    gather(0)
    g_avg = float(np.mean(time_events(gather, 5)))
    g_bytes = gather_bytes(spec, case, npf)
    del g_out

    result = {
        "metric": "decode-attn effective KV GB/s (% HBM peak); quantize-write tokens/s",
        "value": round(d_gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int4 codes; int8 mfma (q.k), bf16 mfma (p.v), fp32 accumulate",
        "data": "synthetic (seeded)",
        "config": {"workload": spec.name, "batch": spec.B, "prefill_seqs": npf, "prefill_new_tokens": max_q,
                   "decode_seqs": spec.B - npf, "q_heads": spec.Hq, "kv_heads": spec.Hkv, "head_dim": spec.D,
                   "block_size": spec.bs, "mode": ["int8_sym", "int4_asym", "int2_asym"][spec.mode],
                   "rotation": spec.rotate, "window": list(spec.window or []), "headwise_table": spec.headwise,
                   "seq_len": max_len, "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "kernel": "prefill_kernel", "achieved": round(p_tf, 2),
                     "peak": 2500.0, "unit": "TFLOP/s", "frac": round(p_tf / 2500.0, 4),
                     "traffic": load_traffic(f"prefill_{spec.name}_counters.json", PREFILL_SRC),
                     "useful_pairs": pairs, "flops_per_launch": flops, "kv_bytes_per_launch": p_kv,
                     "avg_launch_us": round(p_ms * 1e3, 2), "launches": args.steps,
                     "in_step_launch_us": round(p_step_ms * 1e3, 2)},
        "decode": {"kernel": "decode_kernel", "achieved_GBps": round(d_gbs, 2),
                   "frac": round(d_gbs / HBM_PEAK_GBS, 4), "algorithmic_bytes_per_launch": int(d_algo),
                   "kv_tokens_attended": d_tokens, "avg_launch_us": round(d_ms * 1e3, 2),
                   "in_step_launch_us": round(d_step_ms * 1e3, 2)},
        "write": {"step_tokens": T, "step_write_us": round(w_ms * 1e3, 2),
                  "tokens_per_s": round(T / (w_ms * 1e-3), 1), "bytes_per_token": wb,
                  "GBps": round(T * wb / (w_ms * 1e-3) / 1e9, 2)},
        "gather": {"kernel": "gather_kernel (dequantize-gather of the prefill contexts, bf16 out)",
                   "rows": int(g_tot) * spec.Hkv * 2, "avg_launch_us": round(g_avg * 1e3, 2),
                   "algorithmic_bytes_per_launch": int(g_bytes),
                   "GBps": round(g_bytes / (g_avg * 1e-3) / 1e9, 2),
                   "frac": round(g_bytes / (g_avg * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
        "setup_s": round(setup_s, 1),
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = oracle_prefill_sample(spec, case, planes, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=2, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--replicas", type=int, default=0, help="cache replicas cycled (0 = enough for 1.2 GB)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true", help="replay the step from a HIP graph instead of launching it")
    ap.add_argument("--unfused", action="store_true", help="run the step as write then decode (two launches)")
    ap.add_argument("--mode", choices=["step", "copy"], default="step",
                    help="copy: time a plain 1 GiB device copy (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); this build measures the kernel "
              "on one GPU's share; see DESIGN.md for how the path shards.", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    kvq.load_library()

    if args.mode == "copy":
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        ms = time_events(lambda i: dst.copy_(src), max(1, args.steps))
        print(json.dumps({"mode": "copy", "bytes": n, "ms": ms, "GBps": [2 * n / (m * 1e6) for m in ms]}))
        return

    spec = synth.CONFIGS[args.config]
    if spec.n_prefill:
        return run_mixed(args, spec, dev)
    t_setup = time.perf_counter()
    case, d, planes, new = build_workload(spec, dev)
    cache_bytes = sum(p.numel() * p.element_size() for p in planes)
    R = args.replicas or max(1, min(16, math.ceil(max(1.2e9, 4 * MALL_BYTES) / cache_bytes)))
    replicas = [planes] + [tuple(p.clone() for p in planes) for _ in range(R - 1)]
    max_len = int(case.seq_lens.max().item())
    ws = kvq.alloc_workspace(kvq.kvq_decode_workspace_size(d, spec.B, spec.Hq, max_len), dev)
    out = torch.empty((spec.B, spec.Hq, spec.D), dtype=torch.float32, device=dev)
    algo, kv_bytes, tokens = decode_algo_bytes(spec, case)
    setup_s = time.perf_counter() - t_setup

    def write(i):
        rp = replicas[i % R]
        kvq.kvq_reshape_and_cache(d, new["k"], new["v"], *rp, slot_mapping=new["sm"],
                                  slot_mapping_headwise=new["smh"])

    def decode(i):
        rp = replicas[i % R]
        kvq.kvq_paged_decode_attention(d, case.q, *rp, case.seq_lens, max_len,
                                       block_tables=case.block_tables,
                                       block_tables_headwise=case.block_tables_headwise,
                                       window=case.window, softmax_scale=case.softmax_scale,
                                       out=out, workspace=ws)

    def fused(i):
        rp = replicas[i % R]
        kvq.kvq_decode_step(d, case.q, new["k"], new["v"], *rp, case.seq_lens, max_len,
                            slot_mapping=new["sm"], slot_mapping_headwise=new["smh"],
                            block_tables=case.block_tables, block_tables_headwise=case.block_tables_headwise,
                            window=case.window, softmax_scale=case.softmax_scale, out=out, workspace=ws)

    def two_calls(i):
        write(i)
        decode(i)

    one = two_calls if args.unfused else fused
    for i in range(args.warmup):
        one(i)
    torch.cuda.synchronize()

    # --graph: one HIP graph per cache replica holding the step, replayed
    # (measured slower than eager launches for the two-kernel step)
    graphs = None
    if args.graph:
        graphs = []
        for k in range(R):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                one(k)
            graphs.append(g)
        for i in range(args.warmup):
            graphs[i % R].replay()
        torch.cuda.synchronize()

    def step(i):
        if graphs is not None:
            graphs[i % R].replay()
        else:
            one(i)

    # timed region: exactly `steps` steps
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    # the step's kernel alone (the fused write + decode; with --unfused the
    # decode): `steps` back-to-back launches over the replicas between two
    # HIP events on the stream it runs on (the host stays ahead of the GPU,
    # so the span is the kernels and the gaps between them)
    step_kernel = decode if args.unfused else fused
    dec_avg = time_span(step_kernel, args.steps)
    # for reference: decode alone and the step's write alone, same way
    dec_only_avg = time_span(decode, args.steps)
    step_write_avg = time_span(write, args.steps)
    wb = write_bytes_per_token(spec)
    step_write_bytes = spec.B * wb
    k_algo = algo if args.unfused else algo + step_write_bytes

    # measured device-copy bandwidth (1 GiB read + 1 GiB written), the
    # practical ceiling the fractions are also quoted against
    copy_gbs = measured_copy_gbs(dev)

    # quantize-write throughput: whole-cache fill into a scratch replica
    T = case.k.shape[0]
    scratch = replicas[-1]

    def fill(i):
        kvq.kvq_reshape_and_cache(d, case.k, case.v, *scratch, slot_mapping=case.slot_mapping,
                                  slot_mapping_headwise=case.slot_mapping_headwise)

    fill(0)
    fill_ms = time_events(fill, 5)
    fill_avg = float(np.mean(fill_ms))

    # dequantize-gather of the whole cache (every sequence, positions 0 ..
    # L - 1, bf16 rows [T, Hkv, D] for K and for V), cycling the replicas
    lens = case.seq_lens.cpu().numpy().astype(np.int64)
    cu_np = np.concatenate([[0], np.cumsum(lens)])
    cu = torch.as_tensor(cu_np.astype(np.int32), device=dev)
    g_tot = int(cu_np[-1])
    g_out = [torch.empty((g_tot, spec.Hkv, spec.D), dtype=torch.bfloat16, device=dev) for _ in range(2)]

    def gather(i):
        kvq.kvq_gather_dequant(d, *replicas[i % R], cu, max_len, g_tot, block_tables=case.block_tables,
                               block_tables_headwise=case.block_tables_headwise,
                               key_out=g_out[0], value_out=g_out[1])

    gather(0)
    g_ms = time_events(gather, 5)
    g_avg = float(np.mean(g_ms))
    g_bytes = gather_bytes(spec, case)
    g_cpu = None if args.no_cpu_baseline else gather_cpu(spec, case, planes, lens, 3.0)
    del g_out

    result = {
        "metric": "decode-attn effective KV GB/s (% HBM peak); quantize-write tokens/s",
        "value": round(algo / (ms_step * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {0: "int8 codes, bf16 mfma, fp32 accumulate", 1: "int4 codes, bf16 mfma, fp32 accumulate",
                  2: "int2 codes, bf16 mfma, fp32 accumulate"}[spec.mode],
        "data": "synthetic (seeded)",
        "config": {"workload": spec.name, "batch": spec.B, "q_heads": spec.Hq, "kv_heads": spec.Hkv,
                   "head_dim": spec.D, "block_size": spec.bs, "mode": ["int8_sym", "int4_asym", "int2_asym"][spec.mode],
                   "rotation": spec.rotate, "tokens_cached": int(T), "kv_tokens_attended": tokens,
                   "cache_replicas": R, "parallelism": "single GPU",
                   "step": "write + decode, two launches" if args.unfused else "fused write + decode, one launch",
                   "step_launch": "eager" if graphs is None else "hip graph per replica"},
        "hbm_frac_of_step": round(algo / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "roofline": {"bound": "hbm", "kernel": "decode_kernel" + ("" if args.unfused else " (fused step: new-token write + decode)"),
                     "achieved": round(k_algo / (dec_avg * 1e-3) / 1e9, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(k_algo / (dec_avg * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "traffic": load_traffic(f"decode_{spec.name}_counters.json"),
                     "algorithmic_bytes_per_launch": int(k_algo), "kv_bytes_per_launch": int(kv_bytes),
                     "avg_launch_us": round(dec_avg * 1e3, 3), "launches": args.steps,
                     "measured_copy_GBps": round(copy_gbs, 1),
                     "frac_of_measured_copy": round(k_algo / (dec_avg * 1e-3) / 1e9 / copy_gbs, 4)},
        "decode_only": {"avg_launch_us": round(dec_only_avg * 1e3, 3),
                        "achieved": round(algo / (dec_only_avg * 1e-3) / 1e9, 2),
                        "algorithmic_bytes_per_launch": int(algo)},
        "write": {"step_write_us": round(step_write_avg * 1e3, 3), "step_tokens": spec.B,
                  "fill_tokens": int(T), "fill_us": round(fill_avg * 1e3, 2),
                  "tokens_per_s": round(T / (fill_avg * 1e-3), 1),
                  "bytes_per_token": wb, "GBps": round(T * wb / (fill_avg * 1e-3) / 1e9, 2),
                  "frac": round(T * wb / (fill_avg * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                  "frac_of_measured_copy": round(T * wb / (fill_avg * 1e-3) / 1e9 / copy_gbs, 4),
                  "traffic": load_traffic(f"write_{spec.name}_counters.json", WRITE_SRC)},
        "gather": {"kernel": "gather_kernel (dequantize-gather, bf16 out)", "rows": int(g_tot) * spec.Hkv * 2,
                   "avg_launch_us": round(g_avg * 1e3, 2), "algorithmic_bytes_per_launch": int(g_bytes),
                   "GBps": round(g_bytes / (g_avg * 1e-3) / 1e9, 2),
                   "frac": round(g_bytes / (g_avg * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                   "frac_of_measured_copy": round(g_bytes / (g_avg * 1e-3) / 1e9 / copy_gbs, 4),
                   "traffic": load_traffic(f"gather_{spec.name}_counters.json", GATHER_SRC),
                   "cpu_oracle": g_cpu},
        "setup_s": round(setup_s, 1),
    }
    if spec.layers > 1:
        # the workload is `layers` layers' caches run back to back; one layer's
        # buffers (cycled over the replicas) are timed, the step scales by layers
        result["config"]["layers"] = spec.layers
        result["config"]["timed"] = "one layer's cache per step"
        result["ms_per_step_all_layers"] = round(ms_step * spec.layers, 4)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(spec, case, planes, args.cpu_seconds)
        if spec.layers > 1:
            result["cpu_baseline"]["sample"] += f"; one layer (x{spec.layers} for all layers)"
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
