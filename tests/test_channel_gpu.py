"""Dynamic per-channel INT8 (the vllm-ascend-quantized-kv-cache package,
运行机制: K and V scales per (kv head, channel) from the first K/V a layer
receives, then fixed) on the HIP path against the oracle: calibration and
codes bit for bit (later rows beyond the calibrated range saturate),
decode / prefill within max-abs 2e-3 and mean-abs 2e-4, the gather within
float32 rounding, the fused step bit-equal to write-then-decode."""
import numpy as np
import pytest
import torch

import oracle
import synth
import sub_byte_quantized_amd as kvq
from tests import gpu_helpers as gh

pytestmark = pytest.mark.gpu


def build_channel(spec, first_frac=0.5, boost=5.0):
    """Case, descriptor with GPU-calibrated scales, planes written by the HIP
    kernel.  The scales come from the first `first_frac` of every sequence's
    tokens (the layer's first K/V); some later tokens are scaled by `boost` so
    that they exceed the calibrated range and saturate."""
    dev = gh.dev()
    case = synth.make_case(spec, dev)
    lens = gh.host(case.seq_lens)
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]])
    first = np.concatenate([np.arange(s0, s0 + max(1, int(L * first_frac))) for s0, L in zip(starts, lens) if L])
    later = np.setdiff1d(np.arange(int(lens.sum())), first)
    r = np.random.default_rng(spec.cfg)
    boosted = r.choice(later, size=min(len(later), 5), replace=False) if len(later) else np.zeros(0, np.int64)
    bi = torch.as_tensor(boosted, device=dev)
    case.k[bi] = (case.k[bi].float() * boost).to(torch.bfloat16)
    case.v[bi] = (case.v[bi].float() * boost).to(torch.bfloat16)
    d = kvq.CacheDesc(spec.mode, spec.D, spec.Hkv, spec.bs, case.tables.num_blocks)
    fi = torch.as_tensor(first, device=dev)
    scales = kvq.kvq_calibrate_channel_scales(d, case.k[fi].contiguous(), case.v[fi].contiguous())
    d.channel_scales = scales
    planes = kvq.alloc_cache(d, dev, poison=True)
    kvq.kvq_reshape_and_cache(d, case.k, case.v, *planes, slot_mapping=case.slot_mapping,
                              slot_mapping_headwise=case.slot_mapping_headwise)
    torch.cuda.synchronize()
    return case, d, planes, first


def _ref_scales(case, first):
    k = gh.f32(case.k)[first]
    v = gh.f32(case.v)[first]
    return np.stack([oracle.calibrate_channel_scales(k), oracle.calibrate_channel_scales(v)])


SPECS = [synth.small_spec(name=f"chan-d{D}-g{G}-b{bs}", cfg=800 + D + G + bs, mode=3, rotate=False, D=D, bs=bs,
                          B=3, Hkv=2, Hq=2 * G, lens=[300, 45, 1100]) for D, G, bs in
         ((128, 4, 64), (64, 1, 16), (128, 8, 16), (64, 5, 64))]


@pytest.mark.parametrize("spec", SPECS, ids=lambda s: s.name)
def test_channel_write_decode_prefill_gather(spec):
    print(f"[case] per-channel {spec.name}", flush=True)
    case, d, planes, first = build_channel(spec)
    sc = d.channel_scales.cpu().numpy()
    ref_sc = _ref_scales(case, first)
    assert np.array_equal(sc.view(np.uint32), ref_sc.view(np.uint32)), "calibrated scales differ"
    got = gh.host_planes(planes)
    cs, ms = oracle.plane_shapes(3, spec.D, spec.Hkv, spec.bs, case.tables.num_blocks)
    ref = [np.full(cs, 0xFF, np.uint8), np.zeros(ms, np.float32), np.full(cs, 0xFF, np.uint8),
           np.zeros(ms, np.float32)]
    oracle.write_cache(gh.f32(case.k), gh.f32(case.v), 3, spec.bs, *ref, slot_mapping=gh.host(case.slot_mapping),
                       channel_scales=ref_sc)
    assert np.array_equal(got[0], ref[0]) and np.array_equal(got[2], ref[2]), "codes differ"
    codes = oracle.unpack_codes(got[0], 3, spec.D)
    assert (np.abs(codes) == 127).any(), "no saturated code: the test does not reach saturation"
    # decode
    out = gh.gpu_decode(spec, case, d, planes)
    torch.cuda.synchronize()
    refd = oracle.decode_attention(gh.f32(case.q), gh.host(case.seq_lens), 3, spec.D, spec.bs, spec.Hkv, *got,
                                   case.softmax_scale, block_tables=gh.host(case.block_tables),
                                   channel_scales=ref_sc)
    gh.assert_close(out.cpu().numpy(), refd, f"{spec.name} decode")
    # prefill of the last 50 positions of every sequence (fewer for short ones)
    n_new = [min(50, int(L)) for L in gh.host(case.seq_lens)]
    q, cu = gh.prefill_inputs(spec, n_new, stream=64)
    outp = gh.gpu_prefill(spec, case, d, planes, q, cu)
    torch.cuda.synchronize()
    refp = oracle.prefill_attention(gh.f32(q), gh.host(cu), gh.host(case.seq_lens), 3, spec.D, spec.bs, spec.Hkv,
                                    *got, case.softmax_scale, block_tables=gh.host(case.block_tables),
                                    channel_scales=ref_sc)
    gh.assert_close(outp.cpu().numpy(), refp, f"{spec.name} prefill")
    # gather: x_hat = c * s_d in float32, against float64 within one rounding
    lens = gh.host(case.seq_lens)
    cu_g = torch.as_tensor(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32), device=planes[0].device)
    kg, vg = kvq.kvq_gather_dequant(d, *planes, cu_g, int(lens.max()), int(lens.sum()),
                                    block_tables=case.block_tables, out_dtype=torch.float32)
    torch.cuda.synchronize()
    Kr, Vr = oracle.gather_dequant(gh.host(cu_g), 3, spec.D, spec.bs, spec.Hkv, *got,
                                   block_tables=gh.host(case.block_tables), channel_scales=ref_sc)
    for g_, r_ in ((kg.cpu().numpy(), Kr), (vg.cpu().numpy(), Vr)):
        assert np.all(np.abs(g_ - r_) <= 2.0 ** -23 * np.abs(r_)), "gather differs beyond float32 rounding"


def test_channel_fused_step_matches_write_then_decode():
    spec = synth.small_spec(name="chan-step", cfg=820, mode=3, rotate=False, B=3, Hkv=2, Hq=8, lens=[300, 64, 901])
    case, d, planes, first = build_channel(spec)
    dev = planes[0].device
    lens = gh.host(case.seq_lens)
    last = torch.as_tensor(np.cumsum(lens) - 1, device=dev)
    k_new, v_new = case.k[last].contiguous(), case.v[last].contiguous()
    sm = case.slot_mapping[last].contiguous()
    a = [p.clone() for p in planes]
    b = [p.clone() for p in planes]
    max_len = int(lens.max())
    kvq.kvq_reshape_and_cache(d, k_new, v_new, *a, slot_mapping=sm)
    out_a = kvq.kvq_paged_decode_attention(d, case.q, *a, case.seq_lens, max_len, block_tables=case.block_tables)
    out_b = kvq.kvq_decode_step(d, case.q, k_new, v_new, *b, case.seq_lens, max_len, slot_mapping=sm,
                                block_tables=case.block_tables)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[2], b[2])
    assert torch.equal(out_a, out_b)


def test_channel_zero_channel_and_empty_calibration():
    """A channel that is zero in the first batch has scale 0 and codes 0
    afterwards; calibrating on zero tokens gives all-zero scales."""
    spec = synth.small_spec(name="chan-zero", cfg=821, mode=3, rotate=False, B=1, Hkv=2, Hq=4, lens=[80], D=64,
                            bs=16)
    dev = gh.dev()
    case = synth.make_case(spec, dev)
    case.k[:40, 1, 7] = 0
    d = kvq.CacheDesc(3, spec.D, spec.Hkv, spec.bs, case.tables.num_blocks)
    sc = kvq.kvq_calibrate_channel_scales(d, case.k[:40].contiguous(), case.v[:40].contiguous())
    empty = kvq.kvq_calibrate_channel_scales(d, case.k[:0].contiguous(), case.v[:0].contiguous())
    torch.cuda.synchronize()
    assert float(sc[0, 1, 7]) == 0.0
    assert bool((empty == 0).all())
    d.channel_scales = sc
    planes = kvq.alloc_cache(d, dev, poison=True)
    kvq.kvq_reshape_and_cache(d, case.k, case.v, *planes, slot_mapping=case.slot_mapping)
    torch.cuda.synchronize()
    codes = oracle.unpack_codes(planes[0].cpu().numpy(), 3, spec.D)
    bt = gh.host(case.block_tables)[0]
    rows = codes[bt[np.arange(80) // 16], 1, np.arange(80) % 16]
    assert np.all(rows[:, 7] == 0)
