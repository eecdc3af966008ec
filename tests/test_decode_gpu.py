"""Paged decode attention: HIP path vs the oracle run on the GPU's stored
planes, element by element (float32 output within max-abs 2e-3 and mean-abs
2e-4), plus invariances that must hold bit for bit: block-id permutation,
head-wise rows equal to the uniform row (FastDeploy PR 7718 correctness
gates), repeated calls; and ones that hold within tolerance: split count,
-1 entries for blocks outside the window."""
import numpy as np
import pytest
import torch

import oracle
import synth
import sub_byte_quantized_amd as kvq
from tests import gpu_helpers as gh

pytestmark = pytest.mark.gpu


def run_and_check(spec, what=None, pairs=None, **kw):
    what = what or spec.name
    print(f"[case] decode {what}", flush=True)
    case, d, planes = gh.build(spec)
    out = gh.gpu_decode(spec, case, d, planes, **kw)
    torch.cuda.synchronize()
    ref = gh.oracle_decode(spec, case, gh.host_planes(planes), pairs=pairs)
    gh.assert_close(out.float().cpu().numpy(), ref, what)
    return case, d, planes, out


SPECS = []
for mode in (0, 1, 2, 4):
    for D in (64, 128):
        for rot in (False, True):
            SPECS.append(synth.small_spec(name=f"m{mode}-d{D}-r{int(rot)}", cfg=400 + 10 * mode + D // 64 + 5 * rot,
                                          mode=mode, D=D, rotate=rot, bs=16 if D == 64 else 64,
                                          lens=[1, 37, 300, 1000], B=4, Hkv=2, Hq=8))


@pytest.mark.parametrize("spec", SPECS, ids=lambda s: s.name)
def test_decode_matches_oracle(spec):
    run_and_check(spec)


@pytest.mark.parametrize("G", [1, 2, 3, 5, 8, 16])
def test_decode_gqa_groups(G):
    spec = synth.small_spec(name=f"gqa{G}", cfg=450 + G, mode=1, rotate=True, Hkv=2, Hq=2 * G,
                            lens=[65, 513], B=2)
    run_and_check(spec)


def test_decode_config1_full():
    run_and_check(synth.CONFIGS[1])


def test_decode_window_and_headwise():
    spec = synth.small_spec(name="swa-headwise", cfg=460, mode=1, rotate=True, B=3, Hkv=4, Hq=16,
                            lens=[300, 1000, 129], window=[100, 64, 0, 0], headwise=True,
                            evict_outside_window=True)
    run_and_check(spec)


def test_decode_window_uniform_table():
    spec = synth.small_spec(name="swa-uniform", cfg=461, mode=0, rotate=False, B=3, Hkv=2, Hq=4,
                            lens=[300, 1000, 33], window=[50, 0])
    run_and_check(spec)


def test_decode_bf16_output():
    spec = synth.small_spec(name="bf16-out", cfg=462, mode=1, rotate=True, lens=[77, 600], B=2)
    case, d, planes = gh.build(spec)
    out32 = gh.gpu_decode(spec, case, d, planes)
    out16 = gh.gpu_decode(spec, case, d, planes, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    # bf16 output = the float32 result rounded to bf16 (within one bf16 ulp)
    a = out16.float().cpu().numpy()
    b = out32.to(torch.bfloat16).float().cpu().numpy()
    ulp = np.abs(b) * 2.0 ** -7 + 1e-30
    assert np.all(np.abs(a - b) <= ulp)


@pytest.mark.parametrize("mode", [2, 5], ids=["int2", "inline"])
def test_decode_repeatable_and_split_invariant(mode):
    """The inline layout numbers its pairs head-major, so its cut pairs and
    merges follow another order than the planes layouts'."""
    spec = synth.small_spec(name=f"splits-m{mode}", cfg=463, mode=mode, rotate=True, lens=[2000, 45, 700], B=3)
    print(f"[case] decode {spec.name}", flush=True)
    case, d, planes = gh.build(spec)
    outs = []
    # workgroup counts: one share per pair or fewer, shares cutting pairs at
    # odd places, more workgroups than tiles (the partition then shrinks)
    for nwg in (1, 3, 7, 1000):
        o1 = gh.gpu_decode(spec, case, d, planes, num_workgroups=nwg)
        o2 = gh.gpu_decode(spec, case, d, planes, num_workgroups=nwg)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2), f"repeat differs at {nwg} workgroups"
        outs.append(o1.cpu().numpy())
    ref = gh.oracle_decode(spec, case, gh.host_planes(planes))
    for o in outs:
        gh.assert_close(o, ref, "split-count")


def test_decode_block_permutation_bitexact():
    """The same logical cache under two block-id permutations gives the same
    output bit for bit."""
    spec_a = synth.small_spec(name="perm-a", cfg=464, mode=1, rotate=True, lens=[300, 1000], B=2)
    case, d, planes = gh.build(spec_a)
    out_a = gh.gpu_decode(spec_a, case, d, planes)
    # move every block to a new id: new = perm[old]
    nb = case.tables.num_blocks
    perm = torch.as_tensor(np.random.default_rng(5).permutation(nb), device=planes[0].device)
    moved = [torch.empty_like(p) for p in planes]
    for m, p in zip(moved, planes):
        m[perm] = p
    bt = case.block_tables.clone()
    live = bt >= 0
    bt[live] = perm[bt[live].long()].to(torch.int32)
    case.block_tables = bt
    out_b = gh.gpu_decode(spec_a, case, d, moved)
    torch.cuda.synchronize()
    assert torch.equal(out_a, out_b)


def test_decode_headwise_equals_uniform_bitexact():
    spec = synth.small_spec(name="hw-eq", cfg=465, mode=0, rotate=False, lens=[300, 1000, 5], B=3, Hkv=4, Hq=8)
    case, d, planes = gh.build(spec)
    out_u = gh.gpu_decode(spec, case, d, planes)
    hw = case.block_tables.repeat_interleave(spec.Hkv, dim=0).contiguous()
    case.block_tables, case.block_tables_headwise = None, hw
    out_h = gh.gpu_decode(spec, case, d, planes)
    torch.cuda.synchronize()
    assert torch.equal(out_u, out_h)


def test_decode_evicted_outside_window_matches_window_only():
    spec = synth.small_spec(name="evict", cfg=466, mode=1, rotate=True, lens=[1000, 700], B=2, Hkv=2, Hq=4,
                            window=[200, 0])
    case, d, planes = gh.build(spec)
    out_w = gh.gpu_decode(spec, case, d, planes)
    hw = case.block_tables.repeat_interleave(spec.Hkv, dim=0).contiguous()
    lens = gh.host(case.seq_lens)
    for b, L in enumerate(lens):
        start = L - 200
        for j in range(hw.shape[1]):
            if (j + 1) * spec.bs <= start:
                hw[b * spec.Hkv + 0, j] = -1
    case.block_tables, case.block_tables_headwise = None, hw
    out_e = gh.gpu_decode(spec, case, d, planes)
    torch.cuda.synchronize()
    gh.assert_close(out_e.cpu().numpy(), out_w.cpu().numpy().astype(np.float64), "evict-vs-window")


def test_decode_all_evicted_gives_zero():
    spec = synth.small_spec(name="all-evicted", cfg=467, mode=1, rotate=True, lens=[300, 100], B=2, Hkv=2, Hq=4)
    case, d, planes = gh.build(spec)
    hw = torch.full((2 * spec.Hkv, case.block_tables.shape[1]), -1, dtype=torch.int32, device=planes[0].device)
    hw[1] = case.block_tables[0]          # seq 0 kv head 1 keeps its blocks
    case.block_tables, case.block_tables_headwise = None, hw
    out = gh.gpu_decode(spec, case, d, planes)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    assert np.all(o[0, :2] == 0) and np.all(o[1] == 0)
    ref = gh.oracle_decode(spec, case, gh.host_planes(planes))
    gh.assert_close(o, ref, "all-evicted")


def test_decode_zero_length_sequence():
    spec = synth.small_spec(name="zero-len", cfg=468, mode=1, rotate=True, lens=[0, 50], B=2)
    case, d, planes = gh.build(spec)
    out = gh.gpu_decode(spec, case, d, planes)
    torch.cuda.synchronize()
    assert torch.all(out[0] == 0)
    ref = gh.oracle_decode(spec, case, gh.host_planes(planes))
    gh.assert_close(out.cpu().numpy(), ref, "zero-len")


def _sampled(cfg, n_pairs=12):
    spec = synth.CONFIGS[cfg]
    print(f"[case] decode full config {cfg} {spec.name}", flush=True)
    case, d, planes = gh.build(spec)
    out = gh.gpu_decode(spec, case, d, planes)
    torch.cuda.synchronize()
    r = np.random.default_rng([cfg, 98])
    pairs = sorted({(int(b), int(h)) for b, h in zip(r.integers(0, spec.B, n_pairs),
                                                    r.integers(0, spec.Hkv, n_pairs))})
    # host copies of only the blocks those pairs read
    tabs = gh.host(case.block_tables if case.block_tables is not None else case.block_tables_headwise)
    ids = np.unique(np.concatenate([oracle.table_row(b, h, spec.Hkv, gh.host(case.block_tables),
                                                     gh.host(case.block_tables_headwise)) for b, h in pairs]))
    ids = ids[ids >= 0]
    sub = {}
    idx = torch.as_tensor(ids, device=planes[0].device)
    small = [p[idx].cpu().numpy() for p in planes]
    remap = np.full(case.tables.num_blocks, -1, np.int64)
    remap[ids] = np.arange(len(ids))
    bt = gh.host(case.block_tables)
    bth = gh.host(case.block_tables_headwise)
    bt2 = None if bt is None else np.where(bt >= 0, remap[np.maximum(bt, 0)], -1)
    bth2 = None if bth is None else np.where(bth >= 0, remap[np.maximum(bth, 0)], -1)
    ref = oracle.decode_attention(gh.f32(case.q), gh.host(case.seq_lens), spec.mode, spec.D, spec.bs, spec.Hkv,
                                  *small, case.softmax_scale, signs=gh.host(case.rot_signs),
                                  block_tables=bt2, block_tables_headwise=bth2, window=gh.host(case.window),
                                  pairs=pairs)
    gh.assert_close(out.cpu().numpy(), ref, f"config {cfg} sampled {len(pairs)} pairs")
    del planes, case
    torch.cuda.empty_cache()


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_decode_full_config_sampled(cfg):
    _sampled(cfg)


def _many_pair_lens(seed, n):
    """Lengths for a batch with more (sequence, kv head) pairs than one LDS
    scan chunk holds: some empty, most short, a fifth long enough that a few
    segments fill the per-batch block-id table (block 16)."""
    r = np.random.default_rng([seed, 7])
    kind = r.random(n)
    return [0 if k < 0.1 else int(r.integers(1, 201)) if k < 0.8 else int(r.integers(2000, 3001)) for k in kind]


@pytest.mark.parametrize("mode,bs", [(1, 16), (0, 64), (2, 64), (5, 16)])
def test_decode_many_pairs_chunks_and_batches(mode, bs):
    """1200 pairs (several prefix chunks), shares holding hundreds of
    segments (many segment batches, some cut short by the block-id table),
    empty sequences in between; default grid and a 7-workgroup grid."""
    spec = synth.small_spec(name=f"many-m{mode}-b{bs}", cfg=470 + mode, mode=mode, rotate=mode != 0, bs=bs,
                            B=300, Hkv=4, Hq=8, lens=_many_pair_lens(470 + mode, 300))
    print(f"[case] decode {spec.name}", flush=True)
    case, d, planes = gh.build(spec)
    ref = gh.oracle_decode(spec, case, gh.host_planes(planes))
    for nwg in (0, 7):
        o1 = gh.gpu_decode(spec, case, d, planes, num_workgroups=nwg)
        o2 = gh.gpu_decode(spec, case, d, planes, num_workgroups=nwg)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2), f"repeat differs ({nwg} workgroups)"
        o = o1.cpu().numpy()
        lens = np.asarray(spec.lens)
        assert np.all(o[lens == 0] == 0)
        gh.assert_close(o, ref, f"{spec.name} wgs={nwg}")
