"""INT4 in the inline layout with the zero point in the stored scale's low 4
bits (vLLM PR 40835 summary, 关键源码片段 and 评论区精华) on the HIP path
against the oracle: the written tensor byte for byte without rotation (with
rotation at most 0.01 % of codes one step off and stored scales within 1e-6
relative), rows no slot names untouched; decode and the fused step within
max-abs 2e-3 / mean-abs 2e-4 over tables, windows, head-wise rows and
evicted blocks, and chunked prefill likewise; the gather within float32
rounding."""
import numpy as np
import pytest
import torch

import oracle
import synth
import sub_byte_quantized_amd as kvq
from tests import gpu_helpers as gh
from tests.test_gather_gpu import check_gather

pytestmark = pytest.mark.gpu


def oracle_cache(spec, case):
    cache = np.full(oracle.inline_cache_shape(spec.D, spec.Hkv, spec.bs, case.tables.num_blocks), 0xFF, np.uint8)
    oracle.write_cache(gh.f32(case.k), gh.f32(case.v), oracle.INT4_INLINE, spec.bs, cache, None, None, None,
                       slot_mapping=gh.host(case.slot_mapping),
                       slot_mapping_headwise=gh.host(case.slot_mapping_headwise), signs=gh.host(case.rot_signs))
    return cache


def check_cache(spec, got, ref, what):
    P = spec.D // 2
    written = ~np.all(ref == 0xFF, axis=-1)
    assert np.array_equal(got[~written], ref[~written]), f"{what}: unwritten rows changed"
    if not spec.rotate:
        assert np.array_equal(got, ref), f"{what}: inline cache differs"
        return
    gc, rc = got[written][:, :P], ref[written][:, :P]
    gh.compare_codes(spec, gc, rc, True, f"{what} codes")
    gs = np.ascontiguousarray(got[written][:, P:]).view("<f4")[:, 0]
    rs = np.ascontiguousarray(ref[written][:, P:]).view("<f4")[:, 0]
    gh.compare_meta(gs, rs, f"{what} stored scales")


SPECS = []
for D in (64, 128):
    for rot in (False, True):
        for bs in (16, 64):
            SPECS.append(synth.small_spec(name=f"inl-d{D}-r{int(rot)}-b{bs}", cfg=860 + D // 64 + 2 * rot + bs // 16,
                                          mode=5, D=D, rotate=rot, bs=bs, lens=[1, 37, 300, 1000], B=4, Hkv=2,
                                          Hq=8))


@pytest.mark.parametrize("spec", SPECS, ids=lambda s: s.name)
def test_inline_write_decode_gather(spec):
    print(f"[case] inline {spec.name}", flush=True)
    case, d, planes = gh.build(spec)
    assert planes[1] is None and planes[2] is None and planes[3] is None
    got = planes[0].cpu().numpy()
    ref = oracle_cache(spec, case)
    check_cache(spec, got, ref, spec.name)
    out = gh.gpu_decode(spec, case, d, planes)
    torch.cuda.synchronize()
    gh.assert_close(out.cpu().numpy(), gh.oracle_decode(spec, case, [got, None, None, None]), f"{spec.name} decode")
    lens = gh.host(case.seq_lens)
    cu = torch.as_tensor(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32), device=planes[0].device)
    kg, vg = kvq.kvq_gather_dequant(d, *planes, cu, int(lens.max()), int(lens.sum()),
                                    block_tables=case.block_tables, out_dtype=torch.float32)
    torch.cuda.synchronize()
    Kr, Vr = oracle.gather_dequant(gh.host(cu), 5, spec.D, spec.bs, spec.Hkv, got, None, None, None,
                                   signs=gh.host(case.rot_signs), block_tables=gh.host(case.block_tables))
    check_gather(kg.cpu().numpy(), Kr, spec.D, False, f"{spec.name} K")
    check_gather(vg.cpu().numpy(), Vr, spec.D, False, f"{spec.name} V")


@pytest.mark.parametrize("G", [1, 2, 5, 16])
def test_inline_gqa_windows_headwise_evicted(G):
    """Every phase packing (G 1 .. 16), a head-wise table with windowed heads
    whose out-of-window blocks are evicted (-1), and the sinks of windowed
    heads."""
    spec = synth.small_spec(name=f"inl-swa-g{G}", cfg=870 + G, mode=5, rotate=True, B=3, Hkv=4, Hq=4 * G,
                            lens=[300, 1000, 129], window=[128, 0, 256, 0], headwise=True,
                            evict_outside_window=True)
    print(f"[case] inline {spec.name}", flush=True)
    case, d, planes = gh.build(spec)
    got = planes[0].cpu().numpy()
    for sink in (0, 16):
        out = gh.gpu_decode(spec, case, d, planes, sink_size=sink)
        torch.cuda.synchronize()
        ref = oracle.decode_attention(gh.f32(case.q), gh.host(case.seq_lens), 5, spec.D, spec.bs, spec.Hkv, got,
                                      None, None, None, case.softmax_scale, signs=gh.host(case.rot_signs),
                                      block_tables_headwise=gh.host(case.block_tables_headwise),
                                      window=gh.host(case.window), sink_size=sink)
        gh.assert_close(out.cpu().numpy(), ref, f"{spec.name} sink {sink}")


def test_inline_fused_step_matches_write_then_decode():
    spec = synth.small_spec(name="inl-step", cfg=880, mode=5, rotate=True, B=4, Hkv=2, Hq=8,
                            lens=[1, 64, 300, 1000])
    case, d, planes = gh.build(spec)
    lens = gh.host(case.seq_lens)
    dev = planes[0].device
    last = torch.as_tensor(np.cumsum(lens) - 1, device=dev)
    k_new, v_new = case.k[last].contiguous(), case.v[last].contiguous()
    sm = case.slot_mapping[last].contiguous()
    a = planes[0].clone()
    b = planes[0].clone()
    max_len = int(lens.max())
    kvq.kvq_reshape_and_cache(d, k_new, v_new, a, None, None, None, slot_mapping=sm)
    out_a = kvq.kvq_paged_decode_attention(d, case.q, a, None, None, None, case.seq_lens, max_len,
                                           block_tables=case.block_tables)
    out_b = kvq.kvq_decode_step(d, case.q, k_new, v_new, b, None, None, None, case.seq_lens, max_len,
                                slot_mapping=sm, block_tables=case.block_tables)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert torch.equal(out_a, out_b)
    ref = gh.oracle_decode(spec, case, [b.cpu().numpy(), None, None, None])
    gh.assert_close(out_b.cpu().numpy(), ref, "inline fused step")


def test_inline_degenerate_rows():
    """Zero rows store st = 0 and codes 0; one-signed rows get zp 0 or 15;
    the HIP bytes equal the oracle's."""
    spec = synth.small_spec(name="inl-degenerate", cfg=890, mode=5, rotate=False, D=64, bs=16, B=1, Hkv=2,
                            Hq=4, lens=[48])
    case = synth.make_case(spec, gh.dev())
    case.k[0:4] = 0
    case.k[4:8] = case.k[4:8].abs() + 1
    case.v[8:12] = -(case.v[8:12].abs() + 1)
    case, d, planes = gh.build(spec, case=case)
    got = planes[0].cpu().numpy()
    ref = oracle_cache(spec, case)
    assert np.array_equal(got, ref)
    slots = gh.host(case.slot_mapping)
    P = spec.D // 2
    for t, kv, want in ((0, 0, 0), (5, 0, 0), (9, 1, 15)):
        blk, off = divmod(int(slots[t]), spec.bs)
        st = np.ascontiguousarray(got[blk, kv, off, :, P:]).view("<u4")[:, 0]
        if t == 0:
            assert np.all(st == 0) and not got[blk, kv, off, :, :P].any()
        else:
            assert np.all(st & 0xF == want), (t, kv, st)


PREFILL = [synth.small_spec(name=f"inl-pre-d{D}-r{int(rot)}-b{bs}-g{G}", cfg=895 + D // 64 + 2 * rot + G, mode=5,
                            D=D, rotate=rot, bs=bs, B=3, Hkv=2, Hq=2 * G, lens=[300, 45, 1000])
           for D, rot, bs, G in ((128, True, 64, 4), (64, False, 16, 1), (128, False, 16, 5), (64, True, 64, 16))]


@pytest.mark.parametrize("spec", PREFILL, ids=lambda s: s.name)
def test_inline_prefill(spec):
    """Chunked prefill over the inline cache: the last 50 positions of every
    sequence (fewer for short ones) against the oracle."""
    print(f"[case] inline prefill {spec.name}", flush=True)
    case, d, planes = gh.build(spec)
    got = planes[0].cpu().numpy()
    n_new = [min(50, int(L)) for L in gh.host(case.seq_lens)]
    q, cu = gh.prefill_inputs(spec, n_new, stream=66)
    out = gh.gpu_prefill(spec, case, d, planes, q, cu)
    torch.cuda.synchronize()
    ref = gh.oracle_prefill(spec, case, [got, None, None, None], q, cu)
    gh.assert_close(out.cpu().numpy(), ref, f"{spec.name} prefill")


def test_inline_prefill_windows_headwise():
    spec = synth.small_spec(name="inl-pre-swa", cfg=899, mode=5, rotate=True, B=3, Hkv=4, Hq=16,
                            lens=[300, 1000, 129], window=[128, 0, 256, 0], headwise=True,
                            evict_outside_window=True)
    case, d, planes = gh.build(spec)
    got = planes[0].cpu().numpy()
    q, cu = gh.prefill_inputs(spec, [40, 64, 1], stream=67)
    for sink in (0, 16):
        out = gh.gpu_prefill(spec, case, d, planes, q, cu, sink_size=sink)
        torch.cuda.synchronize()
        bt, bth, sl = gh.prefill_tables(case, 3)
        ref = oracle.prefill_attention(gh.f32(q), gh.host(cu), gh.host(sl), 5, spec.D, spec.bs, spec.Hkv, got, None,
                                       None, None, case.softmax_scale, signs=gh.host(case.rot_signs),
                                       block_tables_headwise=gh.host(bth), window=gh.host(case.window),
                                       sink_size=sink)
        gh.assert_close(out.cpu().numpy(), ref, f"inline prefill windows sink {sink}")
