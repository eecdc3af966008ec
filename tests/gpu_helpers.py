"""Shared helpers for the GPU parity tests: build a workload, write it with
the HIP path into a poisoned cache, and run the oracle on the GPU's stored
planes (so attention parity does not depend on write parity)."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import synth
import sub_byte_quantized_amd as kvq

# Attention acceptance on float32 output (max-abs, mean-abs).
ATOL_MAX = 2e-3
ATOL_MEAN = 2e-4


def dev():
    return torch.device("cuda:0")


def desc_of(spec, case, num_blocks=None):
    return kvq.CacheDesc(spec.mode, spec.D, spec.Hkv, spec.bs,
                         num_blocks or case.tables.num_blocks, case.rot_signs)


def build(spec, device=None, write=True, case=None):
    """Case on the device, poisoned planes, every position written by the HIP
    write kernel.  Returns (case, desc, planes)."""
    device = device or dev()
    case = case or synth.make_case(spec, device)
    d = desc_of(spec, case)
    planes = kvq.alloc_cache(d, device, poison=True)
    if write:
        kvq.kvq_reshape_and_cache(d, case.k, case.v, *planes, slot_mapping=case.slot_mapping,
                                  slot_mapping_headwise=case.slot_mapping_headwise)
    torch.cuda.synchronize()
    return case, d, planes


def host(t):
    return None if t is None else t.detach().cpu().numpy()


def host_planes(planes):
    return [host(p) for p in planes]


def f32(t):
    return t.detach().float().cpu().numpy()


def oracle_decode(spec, case, planes_np, pairs=None):
    return oracle.decode_attention(
        f32(case.q), host(case.seq_lens), spec.mode, spec.D, spec.bs, spec.Hkv,
        *planes_np, case.softmax_scale, signs=host(case.rot_signs),
        block_tables=host(case.block_tables), block_tables_headwise=host(case.block_tables_headwise),
        window=host(case.window), pairs=pairs)


def gpu_decode(spec, case, d, planes, **kw):
    return kvq.kvq_paged_decode_attention(
        d, case.q, *planes, case.seq_lens, int(case.seq_lens.max().item()),
        block_tables=case.block_tables, block_tables_headwise=case.block_tables_headwise,
        window=case.window, softmax_scale=case.softmax_scale, **kw)


def assert_close(got, ref, what=""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    mask = ~np.isnan(ref)
    assert mask.any()
    assert np.all(np.isfinite(got[mask])), f"{what}: non-finite output"
    err = np.abs(got[mask] - ref[mask])
    mx, mean = float(err.max()), float(err.mean())
    print(f"[parity] {what}: max-abs {mx:.3e} mean-abs {mean:.3e} over {mask.sum()} values")
    assert mx <= ATOL_MAX and mean <= ATOL_MEAN, f"{what}: max-abs {mx:.3e} mean-abs {mean:.3e}"


def code_ordinals(packed, mode, D):
    """Codes as integers in value order: the codes themselves, or for FP8 the
    E4M3 byte's magnitude bits with its sign (adjacent E4M3 values differ by
    one; +0 and -0 are both 0)."""
    if mode == oracle.FP8_E4M3:
        c = np.asarray(packed, np.int64)
        return np.where(c & 0x80, -(c & 0x7F), c & 0x7F)
    return oracle.unpack_codes(packed, mode, D).astype(np.int64)


def compare_codes(spec, got_codes, ref_codes, rotated, what=""):
    """Packed codes: bit-exact without rotation; with rotation at most 0.01 %
    of elements may differ, each by one step."""
    if not rotated:
        assert np.array_equal(got_codes, ref_codes), f"{what}: codes differ"
        return
    g = code_ordinals(got_codes, spec.mode, spec.D)
    r = code_ordinals(ref_codes, spec.mode, spec.D)
    diff = np.abs(g - r)
    n_bad = int((diff > 0).sum())
    print(f"[parity] {what}: {n_bad} of {diff.size} codes differ (max step {int(diff.max())})")
    assert diff.max() <= 1 and n_bad <= 1e-4 * diff.size, f"{what}: {n_bad} codes differ"


def compare_meta(got, ref, what=""):
    """Scales and zero points within 1e-6 relative (absolute floor 1e-30)."""
    err = np.abs(got.astype(np.float64) - ref.astype(np.float64))
    tol = 1e-6 * np.abs(ref.astype(np.float64)) + 1e-30
    bad = err > tol
    assert not bad.any(), f"{what}: {int(bad.sum())} meta values differ; worst {err.max():.3e}"


def prefill_inputs(spec, n_new, device=None, stream=60):
    """Seeded prefill queries for sequences 0..len(n_new)-1: q [sum n_new,
    Hq, D] bf16 and cu_seqlens_q [len(n_new)+1] int32."""
    device = device or dev()
    n_new = np.asarray(n_new, np.int64)
    q = synth.bf16_normal((int(n_new.sum()), spec.Hq, spec.D), spec.cfg, stream, device)
    cu = torch.as_tensor(np.concatenate([[0], np.cumsum(n_new)]).astype(np.int32), device=device)
    return q, cu


def prefill_tables(case, nseq):
    """Tables, seq_lens of the first nseq sequences (row slices)."""
    spec = case.spec
    bt = None if case.block_tables is None else case.block_tables[:nseq].contiguous()
    bth = None if case.block_tables_headwise is None else case.block_tables_headwise[:nseq * spec.Hkv].contiguous()
    return bt, bth, case.seq_lens[:nseq].contiguous()


def gpu_prefill(spec, case, d, planes, q, cu, max_q_len=None, **kw):
    nseq = int(cu.shape[0]) - 1
    bt, bth, sl = prefill_tables(case, nseq)
    if max_q_len is None:
        max_q_len = int((cu[1:] - cu[:-1]).max().item()) if nseq else 0
    return kvq.kvq_paged_prefill_attention(
        d, q, cu, max_q_len, *planes, sl, int(case.seq_lens.max().item()),
        block_tables=bt, block_tables_headwise=bth, window=case.window,
        softmax_scale=case.softmax_scale, **kw)


def oracle_prefill(spec, case, planes_np, q, cu, pairs=None, rows=None):
    nseq = int(cu.shape[0]) - 1
    bt, bth, sl = prefill_tables(case, nseq)
    return oracle.prefill_attention(
        f32(q), host(cu), host(sl), spec.mode, spec.D, spec.bs, spec.Hkv, *planes_np,
        case.softmax_scale, signs=host(case.rot_signs), block_tables=host(bt),
        block_tables_headwise=host(bth), window=host(case.window), pairs=pairs, rows=rows)
