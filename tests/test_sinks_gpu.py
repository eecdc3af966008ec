"""Attention sinks (FastDeploy PR 7718, Modifications: a sink_size parameter of
the attention op): a windowed kv head attends its window and the first
sink_size positions.  Decode and chunked prefill on the HIP path against the
oracle (max-abs 2e-3 / mean-abs 2e-4), with uniform and head-wise tables
(-1 for the blocks between the sinks and the window), block sizes 16 and 64,
and sink_size 0 equal to the window-only result bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests import gpu_helpers as gh

pytestmark = pytest.mark.gpu


def _evict_gap(case, spec, sink):
    """Head-wise table with -1 for the blocks of windowed heads that lie
    wholly between the sinks and the window start."""
    bt = gh.host(case.block_tables)
    hw = np.repeat(bt, spec.Hkv, axis=0)
    lens = gh.host(case.seq_lens)
    for b, L in enumerate(lens):
        for h, W in enumerate(spec.window):
            if W <= 0:
                continue
            start = max(0, L - W)
            for j in range(hw.shape[1]):
                lo, hi = j * spec.bs, (j + 1) * spec.bs
                if lo >= sink and hi <= start:
                    hw[b * spec.Hkv + h, j] = -1
    return torch.as_tensor(hw, device=case.seq_lens.device)


@pytest.mark.parametrize("mode,bs,D,headwise", [(1, 64, 128, False), (1, 16, 64, True), (0, 64, 128, True),
                                                (2, 16, 128, False)])
def test_sinks_decode_and_prefill(mode, bs, D, headwise):
    spec = synth.small_spec(name=f"sinks-m{mode}-b{bs}", cfg=780 + mode + bs, mode=mode, rotate=mode != 0, bs=bs,
                            D=D, B=3, Hkv=2, Hq=8, lens=[700, 90, 1500], window=[200, 0])
    print(f"[case] sinks {spec.name} headwise {headwise}", flush=True)
    case, d, planes = gh.build(spec)
    hp = gh.host_planes(planes)
    for sink in (4, 37, 130):
        if headwise:
            case.block_tables_headwise = _evict_gap(case, spec, sink)
            bt_keep, case.block_tables = case.block_tables, None
        out = gh.gpu_decode(spec, case, d, planes, sink_size=sink)
        torch.cuda.synchronize()
        ref = oracle.decode_attention(gh.f32(case.q), gh.host(case.seq_lens), spec.mode, spec.D, spec.bs, spec.Hkv,
                                      *hp, case.softmax_scale, signs=gh.host(case.rot_signs),
                                      block_tables=gh.host(case.block_tables),
                                      block_tables_headwise=gh.host(case.block_tables_headwise),
                                      window=gh.host(case.window), sink_size=sink)
        gh.assert_close(out.cpu().numpy(), ref, f"{spec.name} decode sink {sink}")
        n_new = [40, 90, 77]
        q, cu = gh.prefill_inputs(spec, n_new, stream=63)
        outp = gh.gpu_prefill(spec, case, d, planes, q, cu, sink_size=sink)
        torch.cuda.synchronize()
        bt, bth, sl = gh.prefill_tables(case, 3)
        refp = oracle.prefill_attention(gh.f32(q), gh.host(cu), gh.host(sl), spec.mode, spec.D, spec.bs, spec.Hkv,
                                        *hp, case.softmax_scale, signs=gh.host(case.rot_signs),
                                        block_tables=gh.host(bt), block_tables_headwise=gh.host(bth),
                                        window=gh.host(case.window), sink_size=sink)
        gh.assert_close(outp.cpu().numpy(), refp, f"{spec.name} prefill sink {sink}")
        if headwise:
            case.block_tables, case.block_tables_headwise = bt_keep, None


def test_sink_zero_is_window_only_bitexact():
    spec = synth.small_spec(name="sink0", cfg=790, mode=1, rotate=True, B=2, Hkv=2, Hq=4, lens=[900, 300],
                            window=[100, 0])
    case, d, planes = gh.build(spec)
    a = gh.gpu_decode(spec, case, d, planes)
    b = gh.gpu_decode(spec, case, d, planes, sink_size=0)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    # sinks past the window start make the window head see everything: equal
    # (within tolerance) to no window at all
    c = gh.gpu_decode(spec, case, d, planes, sink_size=10 ** 6)
    case.window = None
    e = gh.gpu_decode(spec, case, d, planes)
    torch.cuda.synchronize()
    gh.assert_close(c.cpu().numpy(), e.cpu().numpy().astype(np.float64), "sink >= L")


def test_sinks_overlapping_window_starts_in_prefill():
    """Chunks whose rows' window starts straddle the sink range: the earliest
    row's window starts inside [0, sink) or at 0, and later rows' starts move
    past it, so positions between a row's window start and the sink end are
    seen only as sinks (two query tiles per sequence; windows 256 and 128)."""
    spec = synth.small_spec(name="sinks-straddle", cfg=795, mode=1, rotate=True, B=3, Hkv=4, Hq=16,
                            lens=[300, 330, 160], window=[256, 0, 128, 300])
    case, d, planes = gh.build(spec)
    hp = gh.host_planes(planes)
    q, cu = gh.prefill_inputs(spec, [40, 64, 50], stream=68)
    for sink in (16, 40, 100):
        outp = gh.gpu_prefill(spec, case, d, planes, q, cu, sink_size=sink)
        torch.cuda.synchronize()
        bt, bth, sl = gh.prefill_tables(case, 3)
        refp = oracle.prefill_attention(gh.f32(q), gh.host(cu), gh.host(sl), spec.mode, spec.D, spec.bs, spec.Hkv,
                                        *hp, case.softmax_scale, signs=gh.host(case.rot_signs),
                                        block_tables=gh.host(bt), window=gh.host(case.window), sink_size=sink)
        gh.assert_close(outp.cpu().numpy(), refp, f"straddling sinks {sink}")
