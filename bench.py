#!/usr/bin/env python3
"""Benchmark of the quantized paged KV cache on one MI355X.

The headline workload (default, ``--config 4``) is the largest one: INT2
asymmetric + Hadamard decode, batch 4 x 131 072 positions, 32 q / 8 kv
heads, head_dim 128, block 64, with 48 layers' caches held as separate
buffers.  A step is one decode step of the whole model: for every layer in
turn, one launch of kvq_decode_step (quantize-on-write of each sequence's
new token, then paged decode attention over the layer's cache), 48 launches
back to back.  ``--config 2`` / ``3`` time one-layer workloads whose step is
one launch, cycling cache replicas (>= 1.2 GB in all) so that steps stream
from HBM rather than the 256 MB Infinity Cache; ``--config 5`` is the mixed
step (write, chunked prefill, decode).  With the default config the INT8,
INT4 and mixed-step workloads, and the INT8 workload's shapes held as FP8
E4M3 and as per-channel INT8 ("2:fp8", "2:chan"), and the INT4 workload in
the inline layout ("3:inline"), are measured in the same run and reported as
sub-objects under ``configs``.

Prints ONE JSON line.  Timing: after ``warmup`` untimed steps, ``repeats``
(>= 5) timed regions of exactly ``steps`` steps, each bracketed by
synchronize + wall clock and by two HIP events on the stream the kernels
run on; ``ms_per_step`` and ``value`` come from the median region.
``value`` is decode effective KV GB/s of the whole step: the algorithmic
bytes decode reads (packed codes + fp32 scale/zero of attended tokens, plus
queries, outputs and block-table entries; all layers) over the step time.
``roofline`` is the step's kernel: its average launch time is the median
region's event span divided by the launches in it, so it can never exceed
the step time; its algorithmic bytes add the new tokens' write.  ``write``
reports quantize-write tokens/s on a whole-cache fill of one layer,
``gather`` the dequantize-gather of one layer's cache.  Fractions are
against the 8 TB/s nominal and against a 1 GiB device copy and a 4 GiB
streaming read (a read-only HIP kernel, libkvq_bench.so) timed in the same
run.  ``cpu_baseline`` times the oracle on a
bounded sample, with all host threads and with one, median of 3 each.
"""
from __future__ import annotations

import argparse
import ctypes
import dataclasses
import hashlib
import json
import math
import os
import statistics
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402
import sub_byte_quantized_amd as kvq  # noqa: E402

METRIC = "decode-attn effective KV GB/s (% HBM peak); quantize-write tokens/s"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFS = 2500.0
MALL_BYTES = 256 << 20
CSRC = os.path.join(ROOT, "sub_byte_quantized_amd", "csrc")
# sources that define each kernel (a counter summary is tied to them)
DECODE_SRC = [os.path.join(CSRC, f) for f in ("kvq_decode.hip", "kvq_device.h", "kvq_internal.h", "kvq_write_row.h")]
PREFILL_SRC = [os.path.join(CSRC, f) for f in ("kvq_prefill.hip", "kvq_device.h", "kvq_internal.h")]
GATHER_SRC = [os.path.join(CSRC, f) for f in ("kvq_gather.hip", "kvq_device.h", "kvq_internal.h")]
WRITE_SRC = [os.path.join(CSRC, f) for f in ("kvq_write.hip", "kvq_write_row.h", "kvq_device.h", "kvq_internal.h")]
MODE_NAMES = ["int8_sym", "int4_asym", "int2_asym", "int8_channel", "fp8_e4m3", "int4_inline"]


def gather_kernel_name(spec):
    """The gather kernel a cache format runs: the rotated integer formats
    un-rotate on the matrix cores (gather_rot_kernel), the rest stream
    through gather_kernel."""
    return "gather_rot_kernel" if spec.rotate and spec.mode != 4 else "gather_kernel"


# per-mode decode contraction types
MODE_DTYPES = {0: "int8 codes; int8 mfma (q.k), bf16 mfma (p.v), fp32 accumulate",
               1: "int4 codes; int8 mfma (q.k), bf16 mfma (p.v), fp32 accumulate",
               2: "int2 codes; int8 mfma (q.k), bf16 mfma (p.v), fp32 accumulate",
               3: "int8 codes (per-channel scales); int8 mfma (q.k), bf16 mfma (p.v), fp32 accumulate",
               4: "fp8 e4m3 codes; bf16 mfma (q.k, p.v), fp32 accumulate",
               5: "int4 codes (inline rows, zero point in the scale); int8 mfma (q.k), bf16 mfma (p.v), "
                  "fp32 accumulate"}
# workload variants a sub-object may name as "<config>:<variant>": the
# config's shapes and inputs with another cache mode
VARIANTS = {"fp8": dict(mode=4, rotate=False, suffix="fp8-e4m3"),
            "chan": dict(mode=3, rotate=False, suffix="int8-channel"),
            "inline": dict(mode=5, rotate=True, suffix="inline")}


def spec_of(key):
    """synth.CONFIGS[c] for "c"; for "c:variant" the same workload with the
    variant's cache mode (one-layer workloads only)."""
    c, _, var = str(key).partition(":")
    spec = synth.CONFIGS[int(c)]
    if not var:
        return spec
    v = VARIANTS[var]
    if spec.layers > 1 or spec.n_prefill:
        raise SystemExit(f"variant {var} is for one-layer decode workloads")
    return dataclasses.replace(spec, name=f"{spec.name}-{v['suffix']}", mode=v["mode"], rotate=v["rotate"])


def sha(paths):
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def row_layout(spec):
    """(packed code bytes, fp32 meta floats) of one (token, kv head) row:
    INT8 8 bits + scale, INT4 4 bits + scale and zero, INT2 2 bits + scale
    and zero, per-channel INT8 8 bits and no meta, FP8 8 bits + scale,
    inline INT4 4 bits + the 4-byte stored scale in the row."""
    if spec.mode == 5:
        return spec.D // 2 + 4, 0
    bits = {0: 8, 1: 4, 2: 2, 3: 8, 4: 8}[spec.mode]
    return spec.D * bits // 8, {0: 1, 1: 2, 2: 2, 3: 0, 4: 1}[spec.mode]


def decode_algo_bytes(spec, case, first=0):
    """Algorithmic bytes one decode launch over sequences first..B-1 reads and
    writes: codes + meta of every attended token (positions inside the
    window, in non-evicted blocks, below seq_len), the block-table entries
    walked, queries and outputs."""
    P, M = row_layout(spec)
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
    chs = 2 * spec.Hkv * spec.D * 4 if spec.mode == 3 else 0   # per-channel scales
    return kv + q + out + 4 * entries + 4 * nb + chs, kv, tokens


def prefill_work(spec, case):
    """Useful work of the mixed step's chunked prefill: unmasked (query row,
    key) pairs over the first n_prefill sequences (query i of sequence b at
    p = L - n + i sees keys j <= p in present blocks and, for a windowed kv
    head, j >= p - W + 1), times the G q heads; flops = 4 D per pair (q.k and
    p.v); KV bytes = codes + meta of the positions any row of the chunk sees."""
    P, M = row_layout(spec)
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
    P, M = row_layout(spec)
    slot = 8 * (spec.Hkv if spec.headwise else 1)
    return spec.Hkv * 2 * (spec.D * 2 + P + 4 * M) + slot


def gather_bytes(spec, case, nseq=None):
    """Algorithmic bytes of a dequantize-gather of the first `nseq` sequences'
    whole contexts (all by default): per (position, kv head) row of K and of
    V, the packed codes and fp32 meta read (rows in present blocks) and the
    bf16 row written; plus the block-table entries and cu_seq_lens read."""
    P, M = row_layout(spec)
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


# ---------------------------------------------------------------- timing ---
def timed_regions(step, steps, launches, repeats):
    """`repeats` timed regions of exactly `steps` calls of step(i), each
    bracketed by synchronize + wall clock and by two HIP events on the
    current stream (the kernels' own).  Returns per region (ms per step by
    the wall clock, us per launch by the events); the event span lies inside
    the wall-clock span, so launch time x launches <= step time."""
    walls, launch_us = [], []
    for _ in range(repeats):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record()
        for i in range(steps):
            step(i)
        e1.record()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        walls.append((t1 - t0) * 1e3 / steps)
        launch_us.append(e0.elapsed_time(e1) * 1e3 / (steps * launches))
    return walls, launch_us


def median_region(walls, launch_us):
    """Index of the median region by wall time."""
    order = sorted(range(len(walls)), key=lambda i: walls[i])
    return order[len(order) // 2]


def spread(x):
    return [round(min(x), 4), round(max(x), 4)]


def time_events(fn, reps):
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
    for i in range(reps):
        starts[i].record()
        fn(i)
        ends[i].record()
    torch.cuda.synchronize()
    return [s.elapsed_time(e) for s, e in zip(starts, ends)]


def stream_read_lib():
    """The benchmark's read-ceiling kernel (libkvq_bench.so, built beside
    libkvq.so)."""
    path = os.path.join(ROOT, "sub_byte_quantized_amd", "libkvq_bench.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build first (python __graft_entry__.py)")
    lib = ctypes.CDLL(path)
    lib.kvq_bench_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_uint32, ctypes.c_void_p,
                                          ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.kvq_bench_stream_read.restype = ctypes.c_int
    return lib


# (waves per CU, loads in flight per lane) tried for the read ceiling
READ_SHAPES = ((4, 8), (8, 4), (12, 2), (16, 1), (32, 1))


def measured_ceilings(dev, reps=5):
    """Practical HBM ceilings timed in this run: a 1 GiB device copy (2 x 1
    GiB moved per copy_) and a 4 GiB streaming read by a read-only HIP kernel
    (best launch shape of READ_SHAPES), best of `reps` each, GB/s."""
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    copy_ms = min(time_events(lambda i: dst.copy_(src), reps))
    del src, dst
    lib = stream_read_lib()
    nb = 4 << 30
    big = torch.empty(nb, dtype=torch.uint8, device=dev).fill_(1)   # XOR of every 16-byte load is 0
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    best = float("inf")
    for wpc, unroll in READ_SHAPES:
        blocks = cus * wpc // 4

        def rd(i, blocks=blocks, unroll=unroll):
            rc = lib.kvq_bench_stream_read(big.data_ptr(), nb, 0x12345678, sink.data_ptr(), blocks, unroll, stream)
            if rc != 0:
                raise RuntimeError(f"kvq_bench_stream_read failed ({rc})")
        rd(0)
        best = min(best, min(time_events(rd, reps)))
    torch.cuda.synchronize()
    assert int(sink.item()) == 0
    del big, sink
    torch.cuda.empty_cache()
    return 2 * n / (copy_ms * 1e-3) / 1e9, nb / (best * 1e-3) / 1e9


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


# ------------------------------------------------------------- workloads ---
def new_token_index(spec, case):
    """Token rows (into case.k / case.v) of each sequence's step tokens: the
    last n_b positions of sequence b."""
    lens = case.seq_lens.cpu().numpy().astype(np.int64)
    n_new = synth.new_tokens_of(spec)
    ends = np.cumsum(lens)
    return np.concatenate([np.arange(e - n, e) for e, n in zip(ends, n_new)])


def build_buffers(spec, dev, n_bufs, layers):
    """The workload's caches.  layers: `n_bufs` layers, each written from its
    own seeded K/V draws with its own queries; otherwise `n_bufs` replicas
    (device copies) of one cache sharing one batch of queries.  Returns
    (case of layer 0, desc, [dict(planes, q, new)])."""
    case = synth.make_case(spec, dev)
    d = kvq.CacheDesc(spec.mode, spec.D, spec.Hkv, spec.bs, case.tables.num_blocks, case.rot_signs)
    if spec.mode == 3:
        # per-channel INT8: scales from the layer's first K/V, here the whole
        # cached context (one layer; the step's new tokens saturate if beyond)
        assert not layers or n_bufs == 1
        d.channel_scales = kvq.kvq_calibrate_channel_scales(d, case.k, case.v)
    li = torch.as_tensor(new_token_index(spec, case), device=dev)
    T = int(case.k.shape[0])

    def new_of(k, v):
        return dict(k=k[li].contiguous(), v=v[li].contiguous(),
                    sm=None if case.slot_mapping is None else case.slot_mapping[li].contiguous(),
                    smh=None if case.slot_mapping_headwise is None else case.slot_mapping_headwise[li].contiguous())

    bufs = []
    for l in range(n_bufs):
        if l == 0 or not layers:
            k, v, q = case.k, case.v, case.q
        else:
            k = synth.kv_values(spec, T, synth.S_K, dev, layer=l)
            v = synth.kv_values(spec, T, synth.S_V, dev, layer=l)
            q = synth.bf16_normal((spec.B, spec.Hq, spec.D), spec.cfg, synth.S_Q + 100 * l, dev)
        if l == 0 or layers:
            planes = kvq.alloc_cache(d, dev, poison=True)
            kvq.kvq_reshape_and_cache(d, k, v, *planes, slot_mapping=case.slot_mapping,
                                      slot_mapping_headwise=case.slot_mapping_headwise)
        else:
            planes = tuple(None if p is None else p.clone() for p in bufs[0]["planes"])
        bufs.append(dict(planes=planes, q=q, new=new_of(k, v) if (l == 0 or layers) else bufs[0]["new"]))
        if l > 0 and layers:
            del k, v
    torch.cuda.synchronize()
    return case, d, bufs


def cpu_baseline(spec, case, planes, seconds):
    """The oracle, as it stands, on a bounded sample of the same decode:
    (sequence, kv head) pairs in a seeded order until `seconds` have passed,
    as algorithmic KV bytes per second.  Run three times with every host
    thread the BLAS may use and three times with one; the medians are
    reported."""
    import oracle
    from threadpoolctl import threadpool_info, threadpool_limits
    host_planes = [None if p is None else p.cpu().numpy() for p in planes]
    q = case.q.float().cpu().numpy()
    lens = case.seq_lens.cpu().numpy()
    bt = None if case.block_tables is None else case.block_tables.cpu().numpy()
    bth = None if case.block_tables_headwise is None else case.block_tables_headwise.cpu().numpy()
    win = None if case.window is None else case.window.cpu().numpy()
    signs = None if case.rot_signs is None else case.rot_signs.cpu().numpy()
    P, M = row_layout(spec)
    r = np.random.default_rng(0)
    order = [(int(b), int(h)) for b, h in zip(r.permutation(np.repeat(np.arange(spec.B), spec.Hkv)),
                                                np.tile(np.arange(spec.Hkv), spec.B))]

    def one_run():
        done, nbytes = 0, 0
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < seconds:
            b, h = order[done % len(order)]
            oracle.decode_attention(q, lens, spec.mode, spec.D, spec.bs, spec.Hkv, *host_planes,
                                    case.softmax_scale, signs=signs, block_tables=bt,
                                    block_tables_headwise=bth, window=win, pairs=[(b, h)])
            W = int(win[h]) if win is not None else 0
            L = int(lens[b])
            nbytes += (min(L, W) if W > 0 else L) * 2 * (P + 4 * M)
            done += 1
        return nbytes / (time.perf_counter() - t0) / 1e9, done

    all_threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    runs_all = [one_run() for _ in range(3)]
    with threadpool_limits(limits=1):
        runs_one = [one_run() for _ in range(3)]
    med_all = statistics.median(v for v, _ in runs_all)
    med_one = statistics.median(v for v, _ in runs_one)
    # write: the oracle's encode of a token sample
    nt = min(2048, int(case.k.shape[0]))
    k = case.k[:nt].float().cpu().numpy()
    v = case.v[:nt].float().cpu().numpy()
    tw0 = time.perf_counter()
    for src in (k, v):
        oracle.encode_rows(src.reshape(-1, spec.D), spec.mode, signs)
    tw = time.perf_counter() - tw0
    pairs = [n for _, n in runs_all]
    return {"value": round(med_all, 4), "unit": "GB/s", "cores": int(all_threads), "kind": "oracle",
            "affinity_cores": len(os.sched_getaffinity(0)),
            "sample": f"(sequence, kv head) decode pairs of one layer's cache, {seconds:.0f} s per run "
                      f"({min(pairs)}-{max(pairs)} pairs of {spec.B * spec.Hkv}), float64 attention over the "
                      f"GPU's stored planes; median of 3 runs",
            "one_core": {"value": round(med_one, 4), "unit": "GB/s", "cores": 1},
            "write_tokens_per_s": round(nt / tw, 1)}


def run_decode(args, spec, dev, ceilings, headline):
    """A decode workload: the step is kvq_decode_step over every layer
    (multi-layer workloads) or over one cache replica (one-layer ones)."""
    t_setup = time.perf_counter()
    layered = spec.layers > 1
    case, d, bufs = build_buffers(spec, dev, spec.layers if layered else 1, layered)
    n_bufs = len(bufs)
    if not layered:
        cache_bytes = sum(p.numel() * p.element_size() for p in bufs[0]["planes"] if p is not None)
        R = args.replicas or max(1, min(16, math.ceil(max(1.2e9, 4 * MALL_BYTES) / cache_bytes)))
        for _ in range(R - 1):
            bufs.append(dict(planes=tuple(None if p is None else p.clone() for p in bufs[0]["planes"]),
                             q=bufs[0]["q"], new=bufs[0]["new"]))
        n_bufs = R
    max_len = int(case.seq_lens.max().item())
    ws = kvq.alloc_workspace(kvq.kvq_decode_workspace_size(d, spec.B, spec.Hq, max_len), dev)
    out = torch.empty((spec.B, spec.Hq, spec.D), dtype=torch.float32, device=dev)
    algo, kv_bytes, tokens = decode_algo_bytes(spec, case)
    wb = write_bytes_per_token(spec)
    step_write_bytes = spec.B * wb
    setup_s = time.perf_counter() - t_setup

    def fused(buf):
        kvq.kvq_decode_step(d, buf["q"], buf["new"]["k"], buf["new"]["v"], *buf["planes"], case.seq_lens, max_len,
                            slot_mapping=buf["new"]["sm"], slot_mapping_headwise=buf["new"]["smh"],
                            block_tables=case.block_tables, block_tables_headwise=case.block_tables_headwise,
                            window=case.window, softmax_scale=case.softmax_scale, out=out, workspace=ws)

    def decode_only(buf):
        kvq.kvq_paged_decode_attention(d, buf["q"], *buf["planes"], case.seq_lens, max_len,
                                       block_tables=case.block_tables,
                                       block_tables_headwise=case.block_tables_headwise,
                                       window=case.window, softmax_scale=case.softmax_scale, out=out, workspace=ws)

    if layered:
        def step(i):
            for b in bufs:
                fused(b)
        launches = n_bufs
    else:
        def step(i):
            fused(bufs[i % n_bufs])
        launches = 1

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    walls, lus = timed_regions(step, args.steps, launches, args.repeats)
    mi = median_region(walls, lus)
    ms_step, launch_us = walls[mi], lus[mi]
    step_algo = algo * launches                     # decode bytes of the whole step
    k_algo = algo + step_write_bytes                # one launch of the fused kernel
    k_gbs = k_algo / (launch_us * 1e-6) / 1e9
    copy_gbs, read_gbs = ceilings

    skip = set(args.skip.split(",")) if args.skip else set()
    # decode alone (no new-token write), same regions over the same buffers
    if layered:
        def dstep(i):
            for b in bufs:
                decode_only(b)
    else:
        def dstep(i):
            decode_only(bufs[i % n_bufs])
    d_us = float("nan")
    if "decode_only" not in skip:
        dw, dl = timed_regions(dstep, max(5, args.steps // 2), launches, 3)
        d_us = dl[median_region(dw, dl)]

    # quantize-write throughput: whole-cache fill of one layer into fresh planes
    T = int(case.k.shape[0])
    scratch = kvq.alloc_cache(d, dev)
    fill = lambda i: kvq.kvq_reshape_and_cache(d, case.k, case.v, *scratch, slot_mapping=case.slot_mapping,
                                               slot_mapping_headwise=case.slot_mapping_headwise)
    fill_ms = float("nan")
    if "fill" not in skip:
        fill(0)
        fill_ms = statistics.median(time_events(fill, 5))
    del scratch

    # dequantize-gather of one layer's whole cache (bf16 rows [T, Hkv, D])
    lens = case.seq_lens.cpu().numpy().astype(np.int64)
    cu_np = np.concatenate([[0], np.cumsum(lens)])
    cu = torch.as_tensor(cu_np.astype(np.int32), device=dev)
    g_tot = int(cu_np[-1])
    g_out = [torch.empty((g_tot, spec.Hkv, spec.D), dtype=torch.bfloat16, device=dev) for _ in range(2)]
    gather = lambda i: kvq.kvq_gather_dequant(d, *bufs[i % n_bufs]["planes"], cu, max_len, g_tot,
                                              block_tables=case.block_tables,
                                              block_tables_headwise=case.block_tables_headwise,
                                              key_out=g_out[0], value_out=g_out[1])
    g_ms = float("nan")
    if "gather" not in skip:
        gather(0)
        g_ms = statistics.median(time_events(gather, 5))
    g_bytes = gather_bytes(spec, case)
    del g_out

    gbs = lambda nbytes, ms: nbytes / (ms * 1e-3) / 1e9
    res = {
        "metric": METRIC,
        "value": round(gbs(step_algo, ms_step), 2),
        "unit": "GB/s",
        "ms_per_step": round(ms_step, 5),
        "dtype": MODE_DTYPES[spec.mode],
        "config": {"workload": spec.name, "batch": spec.B, "q_heads": spec.Hq, "kv_heads": spec.Hkv,
                   "head_dim": spec.D, "block_size": spec.bs, "mode": MODE_NAMES[spec.mode],
                   "rotation": spec.rotate, "seq_len_max": max_len, "tokens_cached_per_layer": T,
                   "kv_tokens_attended_per_layer": tokens,
                   "layers": spec.layers if layered else 1,
                   "cache_buffers": n_bufs,
                   "buffers": "separate per layer, each written from its own K/V draws" if layered
                   else "device copies of one cache, cycled (>= 1.2 GB in all)",
                   "step": f"kvq_decode_step (new-token write + decode, one launch) x {launches}",
                   "parallelism": "single GPU"},
        "repeats": {"n": args.repeats, "ms_per_step": [round(w, 4) for w in walls],
                    "launch_us": [round(x, 3) for x in lus]},
        "hbm_frac_of_step": round(gbs(step_algo, ms_step) / HBM_PEAK_GBS, 4),
        "roofline": {"bound": "hbm", "kernel": "decode_kernel (fused step: new-token write + decode)",
                     "achieved": round(k_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(k_gbs / HBM_PEAK_GBS, 4),
                     "traffic": load_traffic(f"decode_{spec.name}_counters.json"),
                     "algorithmic_bytes_per_launch": int(k_algo), "kv_bytes_per_launch": int(kv_bytes),
                     "avg_launch_us": round(launch_us, 3), "launch_us_spread": spread(lus),
                     "launches": args.steps * launches,
                     "measured_copy_GBps": round(copy_gbs, 1), "measured_read_GBps": round(read_gbs, 1),
                     "frac_of_measured_copy": round(k_gbs / copy_gbs, 4),
                     "frac_of_measured_read": round(k_gbs / read_gbs, 4)},
        "decode_only": {"avg_launch_us": round(d_us, 3), "achieved": round(gbs(algo, d_us * 1e-3), 2),
                        "frac": round(gbs(algo, d_us * 1e-3) / HBM_PEAK_GBS, 4),
                        "algorithmic_bytes_per_launch": int(algo)},
        "write": {"kernel": "write_kernel (whole-cache fill of one layer)", "fill_tokens": T,
                  "fill_us": round(fill_ms * 1e3, 2), "tokens_per_s": round(T / (fill_ms * 1e-3), 1),
                  "bytes_per_token": wb, "GBps": round(gbs(T * wb, fill_ms), 2),
                  "frac": round(gbs(T * wb, fill_ms) / HBM_PEAK_GBS, 4),
                  "frac_of_measured_copy": round(gbs(T * wb, fill_ms) / copy_gbs, 4),
                  "traffic": load_traffic(f"write_{spec.name}_counters.json", WRITE_SRC)},
        "gather": {"kernel": gather_kernel_name(spec) + " (dequantize-gather of one layer, bf16 out)", "rows": g_tot * spec.Hkv * 2,
                   "avg_launch_us": round(g_ms * 1e3, 2), "algorithmic_bytes_per_launch": int(g_bytes),
                   "GBps": round(gbs(g_bytes, g_ms), 2), "frac": round(gbs(g_bytes, g_ms) / HBM_PEAK_GBS, 4),
                   "frac_of_measured_copy": round(gbs(g_bytes, g_ms) / copy_gbs, 4),
                   "traffic": load_traffic(f"gather_{spec.name}_counters.json", GATHER_SRC)},
        "setup_s": round(setup_s, 1),
    }
    if headline and not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(spec, case, bufs[0]["planes"], args.cpu_seconds)
        if layered:
            res["cpu_baseline"]["sample"] += f" (one layer of {spec.layers}; the rate is per byte, so it holds for all)"
    del bufs, ws
    torch.cuda.empty_cache()
    return res


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


def run_mixed(args, spec, dev, ceilings, headline):
    """The mixed step: quantize-write of every sequence's new tokens (the
    chunk of each prefill sequence, one token of each decode sequence),
    chunked-prefill attention of the prefill sequences, decode attention of
    the others, three launches.  Prefill is MFMA work, so its roofline is
    TFLOP/s against the dense bf16 peak; decode is effective KV GB/s."""
    t_setup = time.perf_counter()
    case, d, bufs = build_buffers(spec, dev, 1, False)
    planes, new = bufs[0]["planes"], bufs[0]["new"]
    npf = spec.n_prefill
    Hkv = spec.Hkv
    max_len = int(case.seq_lens.max().item())
    dq = case.q[npf:].contiguous()
    dsl = case.seq_lens[npf:].contiguous()
    dbt = None if case.block_tables is None else case.block_tables[npf:].contiguous()
    dbth = None if case.block_tables_headwise is None else case.block_tables_headwise[npf * Hkv:].contiguous()
    ws = kvq.alloc_workspace(kvq.kvq_decode_workspace_size(d, spec.B - npf, spec.Hq, max_len), dev)
    dout = torch.empty((spec.B - npf, spec.Hq, spec.D), dtype=torch.float32, device=dev)
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

    def step(i):
        write(i)
        prefill(i)
        decode(i)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    n = max(5, args.steps // 2)
    walls, _ = timed_regions(step, n, 3, args.repeats)
    ms_step = statistics.median(walls)
    # each kernel alone: median of regions of back-to-back launches
    pw, pl = timed_regions(prefill, n, 1, args.repeats)
    p_us = pl[median_region(pw, pl)]
    dw, dl = timed_regions(decode, n, 1, args.repeats)
    d_us = dl[median_region(dw, dl)]
    ww, wl = timed_regions(write, n, 1, args.repeats)
    w_us = wl[median_region(ww, wl)]
    T = int(new["k"].shape[0])
    wb = write_bytes_per_token(spec)
    p_tf = flops / (p_us * 1e-6) / 1e12
    d_gbs = d_algo / (d_us * 1e-6) / 1e9

    # the prefill fallback: dequantize-gather of the prefill sequences' whole
    # contexts (positions 0 .. L - 1, head-wise table, bf16 rows [T, Hkv, D])
    lens = psl.cpu().numpy().astype(np.int64)
    cu_np = np.concatenate([[0], np.cumsum(lens)])
    cu = torch.as_tensor(cu_np.astype(np.int32), device=dev)
    g_tot = int(cu_np[-1])
    g_out = [torch.empty((g_tot, spec.Hkv, spec.D), dtype=torch.bfloat16, device=dev) for _ in range(2)]
    gather = lambda i: kvq.kvq_gather_dequant(d, *planes, cu, max_len, g_tot, block_tables=pbt,
                                              block_tables_headwise=pbth, key_out=g_out[0], value_out=g_out[1])
    gather(0)
    g_ms = statistics.median(time_events(gather, 5))
    g_bytes = gather_bytes(spec, case, npf)
    del g_out

    res = {
        "metric": METRIC,
        "value": round(d_gbs, 2),
        "unit": "GB/s",
        "ms_per_step": round(ms_step, 5),
        "dtype": "int4 codes; int8 mfma (q.k), bf16 mfma (p.v), fp32 accumulate",
        "config": {"workload": spec.name, "batch": spec.B, "prefill_seqs": npf, "prefill_new_tokens": max_q,
                   "decode_seqs": spec.B - npf, "q_heads": spec.Hq, "kv_heads": spec.Hkv, "head_dim": spec.D,
                   "block_size": spec.bs, "mode": MODE_NAMES[spec.mode], "rotation": spec.rotate,
                   "window": list(spec.window or []), "headwise_table": spec.headwise, "seq_len": max_len,
                   "step": "write + prefill + decode, three launches", "parallelism": "single GPU"},
        "repeats": {"n": args.repeats, "ms_per_step": [round(w, 4) for w in walls]},
        "roofline": {"bound": "mfma", "kernel": "prefill_kernel", "achieved": round(p_tf, 2),
                     "peak": BF16_PEAK_TFS, "unit": "TFLOP/s", "frac": round(p_tf / BF16_PEAK_TFS, 4),
                     "traffic": load_traffic(f"prefill_{spec.name}_counters.json", PREFILL_SRC),
                     "useful_pairs": pairs, "flops_per_launch": flops, "kv_bytes_per_launch": p_kv,
                     "avg_launch_us": round(p_us, 2), "launch_us_spread": spread(pl), "launches": n * args.repeats},
        "decode": {"kernel": "decode_kernel", "achieved_GBps": round(d_gbs, 2),
                   "frac": round(d_gbs / HBM_PEAK_GBS, 4), "algorithmic_bytes_per_launch": int(d_algo),
                   "kv_tokens_attended": d_tokens, "avg_launch_us": round(d_us, 2),
                   "traffic": load_traffic(f"decode_{spec.name}_counters.json")},
        "write": {"step_tokens": T, "step_write_us": round(w_us, 2), "tokens_per_s": round(T / (w_us * 1e-6), 1),
                  "bytes_per_token": wb, "GBps": round(T * wb / (w_us * 1e-6) / 1e9, 2)},
        "gather": {"kernel": gather_kernel_name(spec) + " (dequantize-gather of the prefill contexts, bf16 out)",
                   "rows": g_tot * spec.Hkv * 2, "avg_launch_us": round(g_ms * 1e3, 2),
                   "algorithmic_bytes_per_launch": int(g_bytes),
                   "GBps": round(g_bytes / (g_ms * 1e-3) / 1e9, 2),
                   "frac": round(g_bytes / (g_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                   "traffic": load_traffic(f"gather_{spec.name}_counters.json", GATHER_SRC)},
        "setup_s": round(setup_s, 1),
    }
    if headline and not args.no_cpu_baseline:
        res["cpu_baseline"] = oracle_prefill_sample(spec, case, planes, args.cpu_seconds)
    del bufs, planes, ws
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--repeats", type=int, default=5, help="timed regions of `steps` steps (median reported)")
    ap.add_argument("--config", default="4",
                    help="workload: 1..5, or config:variant (variants: fp8, chan, inline; one-layer decode configs)")
    ap.add_argument("--subs", default=None,
                    help="comma-separated workloads reported as sub-objects, a config or config:variant "
                         "(variants: fp8, chan, inline); default 2,3,5,2:fp8,2:chan,3:inline with --config 4; "
                         "'none' for none")
    ap.add_argument("--replicas", type=int, default=0, help="cache replicas of a one-layer workload (0 = >= 1.2 GB)")
    ap.add_argument("--cpu-seconds", type=float, default=4.0, help="seconds of each of the oracle's six runs")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--skip", default="", help="comma-separated parts not to run: decode_only, fill, gather "
                    "(for profiling one kernel)")
    ap.add_argument("--mode", choices=["step", "copy"], default="step",
                    help="copy: time a plain 1 GiB device copy (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): it measures each kernel on one GPU's "
              "share; DESIGN.md describes how the path would shard.", file=sys.stderr)
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

    if args.subs is None:
        subs = ["2", "3", "5", "2:fp8", "2:chan", "3:inline"] if args.config == "4" else []
    elif args.subs in ("", "none"):
        subs = []
    else:
        subs = args.subs.split(",")
    ceilings = measured_ceilings(dev)

    def run(key, headline):
        spec = spec_of(key)
        return (run_mixed if spec.n_prefill else run_decode)(args, spec, dev, ceilings, headline)

    result = run(args.config, True)
    head = {"metric": result.pop("metric"), "value": result.pop("value"), "unit": result.pop("unit"),
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": result.pop("ms_per_step"),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": result.pop("dtype"),
            "data": "synthetic (seeded)", "config": result.pop("config")}
    line = dict(head)
    line["roofline"] = result.pop("roofline")
    if "cpu_baseline" in result:
        line["cpu_baseline"] = result.pop("cpu_baseline")
    line.update(result)
    if subs:
        line["configs"] = {}
        for c in subs:
            sub = run(c, False)
            line["configs"][sub["config"]["workload"]] = sub
            print(f"[bench] {sub['config']['workload']}: {sub['value']} GB/s, roofline "
                  f"{sub['roofline']['frac']}", file=sys.stderr, flush=True)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
