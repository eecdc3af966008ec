"""The algorithmic byte and flop counts every roofline figure of bench.py
divides by, recounted here by brute force on small seeded workloads (CPU
only): each (sequence, kv head) row's allowed positions come from the
oracle's own gather (its per-position block presence) and the window and
causal rules written out position by position, and the per-row byte sizes
from the library's layout query."""
import ctypes

import numpy as np
import pytest

import bench
import oracle
import synth
from sub_byte_quantized_amd import _lib


def _row_sizes(spec):
    """(P, M) of the spec's mode from the C library's layout query."""
    lib = _lib.load()
    d = _lib.CacheDesc(spec.mode, spec.D, spec.Hkv, spec.bs, 4, None)
    out = _lib.Layout()
    assert lib.kvq_query_layout(ctypes.byref(d), ctypes.byref(out)) == 0
    return int(out.row_code_bytes), int(out.row_meta_floats)


def _case(spec):
    return synth.make_case(spec, "cpu", with_kv=False)


def _present(spec, case, b, h, n):
    """Per position j < n of (b, h): its block is present, from the oracle's
    gather over a tiny all-zero cache of the case's table."""
    nb = case.tables.num_blocks
    cs, ms = oracle.plane_shapes(spec.mode, spec.D, spec.Hkv, spec.bs, nb)
    z = [np.zeros(cs, np.uint8), np.zeros(ms, np.float32), np.zeros(cs, np.uint8), np.zeros(ms, np.float32)]
    bt = None if case.block_tables is None else case.block_tables.numpy()
    bth = None if case.block_tables_headwise is None else case.block_tables_headwise.numpy()
    _, _, present = oracle.gather_head(b, h, n, spec.mode, spec.D, spec.bs, spec.Hkv, *z,
                                       block_tables=bt, block_tables_headwise=bth)
    return present


SPECS = [
    synth.small_spec(name="acct-int8", cfg=900, mode=0, rotate=False, B=4, Hkv=2, Hq=8, lens=[1, 64, 130, 700]),
    synth.small_spec(name="acct-swa", cfg=901, mode=1, rotate=True, B=3, Hkv=4, Hq=16, lens=[300, 1000, 129],
                     window=[100, 64, 0, 0], headwise=True, evict_outside_window=True),
    synth.small_spec(name="acct-int2", cfg=902, mode=2, rotate=True, B=2, Hkv=2, Hq=4, D=64, bs=16, lens=[37, 100]),
]


@pytest.mark.parametrize("spec", SPECS, ids=lambda s: s.name)
def test_decode_bytes_bruteforce(spec):
    case = _case(spec)
    P, M = _row_sizes(spec)
    lens = case.seq_lens.numpy()
    win = None if case.window is None else case.window.numpy()
    tokens, entries = 0, 0
    for b in range(spec.B):
        L = int(lens[b])
        for h in range(spec.Hkv):
            if L == 0:
                continue
            W = int(win[h]) if win is not None else 0
            pres = _present(spec, case, b, h, L)
            for j in range(L):
                if pres[j] and (W <= 0 or j >= L - W):
                    tokens += 1
            first = (L - W if (W > 0 and L > W) else 0) // spec.bs
            entries += (L - 1) // spec.bs - first + 1
    expect = tokens * 2 * (P + 4 * M) + spec.B * spec.Hq * spec.D * (2 + 4) + 4 * entries + 4 * spec.B
    total, kv, tok = bench.decode_algo_bytes(spec, case)
    assert tok == tokens and kv == tokens * 2 * (P + 4 * M) and total == expect


@pytest.mark.parametrize("spec", SPECS, ids=lambda s: s.name)
def test_gather_bytes_bruteforce(spec):
    case = _case(spec)
    P, M = _row_sizes(spec)
    lens = case.seq_lens.numpy()
    present_rows = sum(int(_present(spec, case, b, h, int(lens[b])).sum())
                       for b in range(spec.B) for h in range(spec.Hkv))
    rows = int(lens.sum()) * spec.Hkv
    entries = sum(-(-int(L) // spec.bs) for L in lens) * spec.Hkv
    expect = 2 * present_rows * (P + 4 * M) + 2 * rows * 2 * spec.D + 4 * entries + 4 * (spec.B + 1)
    assert bench.gather_bytes(spec, case) == expect


@pytest.mark.parametrize("spec", SPECS, ids=lambda s: s.name)
def test_write_bytes_per_token(spec):
    P, M = _row_sizes(spec)
    slot = 8 * (spec.Hkv if spec.headwise else 1)
    # a token: K and V bf16 rows read, codes and meta written, for every kv head
    assert bench.write_bytes_per_token(spec) == spec.Hkv * 2 * (2 * spec.D + P + 4 * M) + slot


def test_prefill_work_bruteforce():
    spec = synth.small_spec(name="acct-prefill", cfg=903, mode=1, rotate=True, B=3, Hkv=2, Hq=6, lens=[200, 90, 300],
                            window=[50, 0], headwise=True, evict_outside_window=True, n_prefill=2,
                            prefill_new=40)
    case = _case(spec)
    P, M = _row_sizes(spec)
    G = spec.Hq // spec.Hkv
    lens = case.seq_lens.numpy()
    cu = case.cu_seqlens_q.numpy()
    win = case.window.numpy()
    pairs, seen = 0, 0
    for b in range(spec.n_prefill):
        L, n = int(lens[b]), int(cu[b + 1] - cu[b])
        for h in range(spec.Hkv):
            W = int(win[h])
            pres = _present(spec, case, b, h, L)
            for i in range(n):
                p = L - n + i
                ok = np.array([pres[j] and j <= p and (W <= 0 or j >= p - W + 1) for j in range(L)])
                pairs += int(ok.sum()) * G
            # the KV bytes count every present position from the first row's window start on
            lo = max(L - n - W + 1, 0) if W > 0 else 0
            seen += int(sum(pres[j] for j in range(lo, L)))
    got_pairs, flops, kv = bench.prefill_work(spec, case)
    assert got_pairs == pairs and flops == 4 * spec.D * pairs and kv == seen * 2 * (P + 4 * M)
