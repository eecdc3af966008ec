"""Dequantize-gather (the cache-fetch-and-dequantize operator of FastDeploy PR
5173's review thread; the gather-and-dequantize of the paged cache that
prefill uses in the vllm-ascend-quantized-kv-cache package, 运行机制): the HIP
path against the oracle's gather_dequant on the GPU's stored planes.

Tolerance, per output row (a float32 evaluation of an exact definition):
dequantization rounds c*s and the sum with z (each within 2^-24 relative),
the rotation back adds log2(D) butterfly stages on partial sums bounded by
sum|x_hat|, and the two final products round once more.  With ||x_hat||_2 =
||out||_2 (R is orthogonal) and |z| <= max|x_hat| (the row minimum gets code
0), every element is within 2^-24 (log2 D + 4 + sqrt D) ||out_row||_2; the
test allows twice that.  bf16 outputs may further differ by one bf16 rounding
(2^-8 relative).  Evicted positions must be exactly zero.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
import sub_byte_quantized_amd as kvq
from tests import gpu_helpers as gh

pytestmark = pytest.mark.gpu


def _row_tol(ref, D):
    norm = np.sqrt((ref.astype(np.float64) ** 2).sum(axis=-1, keepdims=True))
    return 2.0 * 2.0 ** -24 * (math.log2(D) + 4 + math.sqrt(D)) * norm


def check_gather(got, ref, D, bf16, what):
    got = np.asarray(got, np.float64)
    tol = _row_tol(ref, D)
    if bf16:
        tol = tol + 2.0 ** -8 * np.abs(ref)
    err = np.abs(got - ref)
    print(f"[parity] gather {what}: max-abs {err.max() if err.size else 0:.3e} over {err.size} values", flush=True)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    bad = err > tol
    assert not bad.any(), f"{what}: {int(bad.sum())} values out of tolerance; worst {err.max():.3e}"
    zero = np.all(ref == 0, axis=-1)
    assert np.all(got[zero] == 0), f"{what}: evicted rows not zero"


def run_gather(spec, case, d, planes, cu, max_len, total, out_dtype):
    return kvq.kvq_gather_dequant(d, *planes, cu, max_len, total,
                                  block_tables=case.block_tables,
                                  block_tables_headwise=case.block_tables_headwise,
                                  out_dtype=out_dtype)


def oracle_gather(spec, case, planes_np, cu):
    return oracle.gather_dequant(gh.host(cu), spec.mode, spec.D, spec.bs, spec.Hkv, *planes_np,
                                 signs=gh.host(case.rot_signs), block_tables=gh.host(case.block_tables),
                                 block_tables_headwise=gh.host(case.block_tables_headwise))


SPECS = []
for mode in (0, 1, 2, 4):
    for D in (64, 128):
        for rot in (False, True):
            SPECS.append(synth.small_spec(name=f"m{mode}-d{D}-r{int(rot)}", cfg=700 + 10 * mode + D // 64 + 5 * rot,
                                          mode=mode, D=D, rotate=rot, bs=16 if D == 64 else 64,
                                          lens=[1, 37, 300, 1000], B=4, Hkv=2, Hq=8))


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("spec", SPECS, ids=lambda s: s.name)
def test_gather_matches_oracle(spec, out_dtype):
    print(f"[case] gather {spec.name} {out_dtype}", flush=True)
    case, d, planes = gh.build(spec)
    lens = case.seq_lens.cpu().numpy().astype(np.int64)
    cu = torch.as_tensor(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32), device=gh.dev())
    K, V = run_gather(spec, case, d, planes, cu, int(lens.max()), int(lens.sum()), out_dtype)
    torch.cuda.synchronize()
    Kr, Vr = oracle_gather(spec, case, gh.host_planes(planes), cu)
    bf = out_dtype == torch.bfloat16
    check_gather(K.float().cpu().numpy(), Kr, spec.D, bf, f"{spec.name} K")
    check_gather(V.float().cpu().numpy(), Vr, spec.D, bf, f"{spec.name} V")


def test_gather_headwise_evicted_and_partial():
    """Head-wise table with -1 entries (windowed heads), a zero-length
    sequence, and a gather of fewer positions than cached (n_b < seq_len)."""
    spec = synth.small_spec(name="gather-swa-headwise", cfg=760, mode=1, rotate=True, B=3, Hkv=4, Hq=16,
                            lens=[300, 1000, 129], window=[100, 64, 0, 0], headwise=True,
                            evict_outside_window=True)
    print(f"[case] gather {spec.name}", flush=True)
    case, d, planes = gh.build(spec)
    bt = case.block_tables_headwise.cpu().numpy()
    assert (bt == -1).any()
    n = np.array([300, 0, 77], np.int64)
    cu = torch.as_tensor(np.concatenate([[0], np.cumsum(n)]).astype(np.int32), device=gh.dev())
    K, V = run_gather(spec, case, d, planes, cu, 1000, int(n.sum()), torch.float32)
    torch.cuda.synchronize()
    Kr, Vr = oracle_gather(spec, case, gh.host_planes(planes), cu)
    assert np.any(np.all(Kr == 0, axis=-1))
    check_gather(K.cpu().numpy(), Kr, spec.D, False, "headwise K")
    check_gather(V.cpu().numpy(), Vr, spec.D, False, "headwise V")


def test_gather_total_tokens_bounds_rows():
    """Rows at or past total_tokens are never written (the outputs are views
    into larger buffers whose tail keeps its sentinel); an empty call writes
    nothing."""
    spec = SPECS[3]
    print(f"[case] gather bounds {spec.name}", flush=True)
    case, d, planes = gh.build(spec)
    lens = case.seq_lens.cpu().numpy().astype(np.int64)
    cu = torch.as_tensor(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32), device=gh.dev())
    total = int(lens.sum()) - 50
    shape = (total + 64, spec.Hkv, spec.D)
    kb = torch.full(shape, 7.0, device=gh.dev())
    vb = torch.full(shape, 7.0, device=gh.dev())
    kvq.kvq_gather_dequant(d, *planes, cu, int(lens.max()), total, block_tables=case.block_tables,
                           key_out=kb[:total], value_out=vb[:total], out_dtype=torch.float32)
    kvq.kvq_gather_dequant(d, *planes, cu[:1], 0, 0, block_tables=case.block_tables,
                           key_out=kb[:0], value_out=vb[:0], out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.all(kb[total:] == 7.0) and torch.all(vb[total:] == 7.0)
    Kr, Vr = oracle_gather(spec, case, gh.host_planes(planes), cu)
    check_gather(kb[:total].cpu().numpy(), Kr[:total], spec.D, False, "bounded K")
    check_gather(vb[:total].cpu().numpy(), Vr[:total], spec.D, False, "bounded V")


@pytest.mark.parametrize("idx", [2, 3], ids=["streaming", "rotated"])
def test_gather_positions_past_max_seq_len_untouched(idx):
    """max_seq_len below some sequences' n_b: their positions at or past it
    keep the outputs' sentinel (the grid covers max_seq_len positions), the
    others are the oracle's rows; both gather kernels."""
    spec = SPECS[idx]
    print(f"[case] gather max_seq_len cap {spec.name}", flush=True)
    case, d, planes = gh.build(spec)
    lens = case.seq_lens.cpu().numpy().astype(np.int64)
    cu = torch.as_tensor(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32), device=gh.dev())
    total, cap = int(lens.sum()), 200
    assert lens.max() > cap
    kb = torch.full((total, spec.Hkv, spec.D), 7.0, device=gh.dev())
    vb = torch.full((total, spec.Hkv, spec.D), 7.0, device=gh.dev())
    kvq.kvq_gather_dequant(d, *planes, cu, cap, total, block_tables=case.block_tables,
                           key_out=kb, value_out=vb, out_dtype=torch.float32)
    torch.cuda.synchronize()
    Kr, Vr = oracle_gather(spec, case, gh.host_planes(planes), cu)
    pos = np.concatenate([np.arange(n) for n in lens])
    keep = pos < cap
    K, V = kb.cpu().numpy(), vb.cpu().numpy()
    assert np.all(K[~keep] == 7.0) and np.all(V[~keep] == 7.0)
    check_gather(K[keep], Kr[keep], spec.D, False, "capped K")
    check_gather(V[keep], Vr[keep], spec.D, False, "capped V")


def test_gather_repeatable():
    spec = SPECS[9]
    case, d, planes = gh.build(spec)
    lens = case.seq_lens.cpu().numpy().astype(np.int64)
    cu = torch.as_tensor(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32), device=gh.dev())
    a = run_gather(spec, case, d, planes, cu, int(lens.max()), int(lens.sum()), torch.bfloat16)
    b = run_gather(spec, case, d, planes, cu, int(lens.max()), int(lens.sum()), torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_gather_full_config_sampled(cfg):
    """The whole cache of the INT8 (batch 32), INT4 + rotation (batch 96) and
    INT2 + rotation (4 x 131072) workloads, and the 16 prefill contexts of the
    mixed step (head-wise table with -1 entries), gathered in one bf16 call
    each, as the bench times them; sampled (sequence, kv head) pairs checked
    against the oracle."""
    spec = synth.CONFIGS[cfg]
    print(f"[case] gather full {spec.name}", flush=True)
    case, d, planes = gh.build(spec)
    nseq = spec.n_prefill or spec.B
    lens = case.seq_lens.cpu().numpy().astype(np.int64)[:nseq]
    cu_np = np.concatenate([[0], np.cumsum(lens)])
    cu = torch.as_tensor(cu_np.astype(np.int32), device=gh.dev())
    bt = None if case.block_tables is None else case.block_tables[:nseq].contiguous()
    bth = None if case.block_tables_headwise is None else case.block_tables_headwise[:nseq * spec.Hkv].contiguous()
    K, V = kvq.kvq_gather_dequant(d, *planes, cu, int(lens.max()), int(lens.sum()), block_tables=bt,
                                  block_tables_headwise=bth, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    pl = gh.host_planes(planes)
    r = np.random.default_rng(cfg)
    for b in r.choice(nseq, 3, replace=False):
        h = int(r.integers(spec.Hkv))
        Kr, Vr, _ = oracle.gather_head(int(b), h, int(lens[b]), spec.mode, spec.D, spec.bs, spec.Hkv, *pl,
                                       signs=gh.host(case.rot_signs), block_tables=gh.host(bt),
                                       block_tables_headwise=gh.host(bth))
        rows = slice(int(cu_np[b]), int(cu_np[b + 1]))
        check_gather(K[rows, h].float().cpu().numpy(), Kr, spec.D, True, f"{spec.name} b{b} h{h} K")
        check_gather(V[rows, h].float().cpu().numpy(), Vr, spec.D, True, f"{spec.name} b{b} h{h} V")
