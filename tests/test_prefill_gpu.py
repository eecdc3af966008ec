"""Chunked-prefill attention: HIP path vs the oracle run on the GPU's stored
planes, element by element (float32 output within max-abs 2e-3 and mean-abs
2e-4): every mode, head size and rotation; GQA groups that leave ragged
query tiles; fresh and continued prefill; per-head windows with head-wise
tables and -1 entries (FastDeploy PR 7718 correctness gates); bf16 output;
empty chunks and a sampled check at the mixed-step size."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests import gpu_helpers as gh

pytestmark = pytest.mark.gpu


def run_and_check(spec, n_new, what=None, **kw):
    what = what or spec.name
    print(f"[case] prefill {what} n_new={list(n_new)}", flush=True)
    case, d, planes = gh.build(spec)
    q, cu = gh.prefill_inputs(spec, n_new)
    out = gh.gpu_prefill(spec, case, d, planes, q, cu, **kw)
    torch.cuda.synchronize()
    ref = gh.oracle_prefill(spec, case, gh.host_planes(planes), q, cu)
    gh.assert_close(out.float().cpu().numpy(), ref, what)
    return case, d, planes, q, cu, out


SPECS = []
for mode in (0, 1, 2):
    for D in (64, 128):
        for rot in (False, True):
            SPECS.append(synth.small_spec(name=f"pf-m{mode}-d{D}-r{int(rot)}", cfg=500 + 10 * mode + D // 64 + 5 * rot,
                                          mode=mode, D=D, rotate=rot, bs=16 if D == 64 else 64,
                                          lens=[1, 130, 301, 700], B=4, Hkv=2, Hq=8))


@pytest.mark.parametrize("spec", SPECS, ids=lambda s: s.name)
def test_prefill_matches_oracle(spec):
    # fresh prefill (n == L) for the first two, continued prefill for the others
    run_and_check(spec, [1, 130, 57, 200])


@pytest.mark.parametrize("G", [1, 3, 5, 8, 16])
def test_prefill_gqa_groups(G):
    spec = synth.small_spec(name=f"pf-gqa{G}", cfg=550 + G, mode=1, rotate=True, Hkv=2, Hq=2 * G,
                            lens=[200, 333], B=2)
    run_and_check(spec, [200, 97])


def test_prefill_window_headwise_evicted():
    spec = synth.small_spec(name="pf-swa-headwise", cfg=560, mode=1, rotate=True, B=3, Hkv=4, Hq=16,
                            lens=[1000, 700, 129], window=[100, 64, 0, 0], headwise=True,
                            evict_outside_window=True)
    run_and_check(spec, [300, 64, 129])


def test_prefill_window_uniform_table():
    spec = synth.small_spec(name="pf-swa-uniform", cfg=561, mode=0, rotate=False, B=2, Hkv=2, Hq=4,
                            lens=[650, 90], window=[50, 0])
    run_and_check(spec, [200, 90])


def test_prefill_bf16_output():
    spec = synth.small_spec(name="pf-bf16", cfg=562, mode=1, rotate=True, lens=[77, 600], B=2)
    case, d, planes = gh.build(spec)
    q, cu = gh.prefill_inputs(spec, [77, 150])
    out32 = gh.gpu_prefill(spec, case, d, planes, q, cu)
    out16 = gh.gpu_prefill(spec, case, d, planes, q, cu, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    a = out16.float().cpu().numpy()
    b = out32.to(torch.bfloat16).float().cpu().numpy()
    assert np.all(np.abs(a - b) <= np.abs(b) * 2.0 ** -7 + 1e-30)


def test_prefill_repeatable_and_headwise_equals_uniform():
    spec = synth.small_spec(name="pf-hw-eq", cfg=563, mode=2, rotate=True, lens=[300, 1000, 5], B=3, Hkv=4, Hq=8)
    case, d, planes = gh.build(spec)
    q, cu = gh.prefill_inputs(spec, [300, 130, 5])
    out_u = gh.gpu_prefill(spec, case, d, planes, q, cu)
    out_u2 = gh.gpu_prefill(spec, case, d, planes, q, cu)
    case.block_tables, case.block_tables_headwise = None, case.block_tables.repeat_interleave(spec.Hkv, dim=0).contiguous()
    out_h = gh.gpu_prefill(spec, case, d, planes, q, cu)
    torch.cuda.synchronize()
    assert torch.equal(out_u, out_u2)
    assert torch.equal(out_u, out_h)


def test_prefill_all_evicted_and_empty_chunks():
    spec = synth.small_spec(name="pf-empty", cfg=564, mode=1, rotate=True, lens=[300, 100, 64], B=3, Hkv=2, Hq=4)
    case, d, planes = gh.build(spec)
    # kv head 0 of sequence 0 keeps nothing; sequence 1 appends no token
    hw = case.block_tables.repeat_interleave(spec.Hkv, dim=0).contiguous()
    hw[0] = -1
    case.block_tables, case.block_tables_headwise = None, hw
    q, cu = gh.prefill_inputs(spec, [40, 0, 64])
    out = gh.gpu_prefill(spec, case, d, planes, q, cu, max_q_len=200)   # generous grid bound
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    assert np.all(o[0:40, 0:2] == 0)
    ref = gh.oracle_prefill(spec, case, gh.host_planes(planes), q, cu)
    gh.assert_close(o, ref, "all-evicted / empty chunk")


def test_prefill_single_token_equals_decode():
    """A one-token chunk at the end of the context is a decode step."""
    spec = synth.small_spec(name="pf-vs-dec", cfg=565, mode=1, rotate=True, lens=[333, 1000], B=2, Hkv=2, Hq=8)
    case, d, planes = gh.build(spec)
    cu = torch.tensor([0, 1, 2], dtype=torch.int32, device=gh.dev())
    out_p = gh.gpu_prefill(spec, case, d, planes, case.q.reshape(2, spec.Hq, spec.D).contiguous(), cu)
    out_d = gh.gpu_decode(spec, case, d, planes)
    torch.cuda.synchronize()
    gh.assert_close(out_p.cpu().numpy(), out_d.cpu().numpy().astype(np.float64), "prefill-1 vs decode")


def test_prefill_mixed_step_sampled():
    """The mixed-step workload (16 sequences x 512 new tokens at 32768
    positions, SWA heads with -1 blocks): sampled (sequence, kv head) pairs and
    rows against the oracle."""
    spec = synth.CONFIGS[5]
    print(f"[case] prefill full config 5 {spec.name}", flush=True)
    case, d, planes = gh.build(spec)
    out = gh.gpu_prefill(spec, case, d, planes, case.q_prefill, case.cu_seqlens_q)
    torch.cuda.synchronize()
    r = np.random.default_rng([5, 97])
    pairs = sorted({(int(b), int(h)) for b, h in zip(r.integers(0, spec.n_prefill, 6),
                                                    r.integers(0, spec.Hkv, 6))} | {(0, 0), (1, 3)})
    rows = np.unique(np.concatenate([[0, 1, 63, 64, 511], r.integers(0, spec.prefill_new, 8)]))
    bt, bth, sl = gh.prefill_tables(case, spec.n_prefill)
    bth_np = gh.host(bth)
    ids = np.unique(np.concatenate([oracle.table_row(b, h, spec.Hkv, None, bth_np) for b, h in pairs]))
    ids = ids[ids >= 0]
    idx = torch.as_tensor(ids, device=planes[0].device)
    small = [p[idx].cpu().numpy() for p in planes]
    remap = np.full(case.tables.num_blocks, -1, np.int64)
    remap[ids] = np.arange(len(ids))
    bth2 = np.where(bth_np >= 0, remap[np.maximum(bth_np, 0)], -1)
    ref = oracle.prefill_attention(gh.f32(case.q_prefill), gh.host(case.cu_seqlens_q), gh.host(sl), spec.mode,
                                   spec.D, spec.bs, spec.Hkv, *small, case.softmax_scale,
                                   signs=gh.host(case.rot_signs), block_tables_headwise=bth2,
                                   window=gh.host(case.window), pairs=pairs, rows=rows)
    gh.assert_close(out.cpu().numpy(), ref, f"config 5 prefill, {len(pairs)} pairs x {len(rows)} rows")
    del planes, case
    torch.cuda.empty_cache()
