"""kvq_paged_decode_attention_noalloc (the decode call that allocates
nothing: its workspace is the library's device scratch) against
kvq_paged_decode_attention with a caller workspace, through the C ABI: two
calls in a row, the second with a smaller input, each bit-equal to the
existing entry point and within max-abs 2e-3 / mean-abs 2e-4 of the oracle."""
import numpy as np
import pytest
import torch

import synth
import sub_byte_quantized_amd as kvq
from tests import gpu_helpers as gh

pytestmark = pytest.mark.gpu


def _sub_case(case, spec, nseq):
    """The first nseq sequences of a case (tables, lengths, queries)."""
    sub = synth.dataclasses.replace(spec, B=nseq, lens=list(spec.lens[:nseq]))
    c = synth.dataclasses.replace(case)
    c.q = case.q[:nseq].contiguous()
    c.seq_lens = case.seq_lens[:nseq].contiguous()
    c.block_tables = None if case.block_tables is None else case.block_tables[:nseq].contiguous()
    c.block_tables_headwise = None if case.block_tables_headwise is None else \
        case.block_tables_headwise[:nseq * spec.Hkv].contiguous()
    return sub, c


@pytest.mark.parametrize("mode,rotate,headwise", [(1, True, False), (0, False, True), (2, True, False),
                                                   (4, True, False), (5, True, True)])
def test_noalloc_matches_decode_twice(mode, rotate, headwise):
    spec = synth.small_spec(name=f"noalloc-m{mode}", cfg=760 + mode, mode=mode, rotate=rotate, B=5, Hkv=2, Hq=8,
                            lens=[700, 1, 2100, 64, 333], headwise=headwise)
    print(f"[case] noalloc mode {mode} headwise {headwise}", flush=True)
    case, d, planes = gh.build(spec)
    hp = gh.host_planes(planes)
    for nseq in (5, 2):            # the second call is smaller
        sub, c = _sub_case(case, spec, nseq)
        max_len = int(c.seq_lens.max().item())
        ref_gpu = kvq.kvq_paged_decode_attention(d, c.q, *planes, c.seq_lens, max_len,
                                                 block_tables=c.block_tables,
                                                 block_tables_headwise=c.block_tables_headwise,
                                                 window=c.window, softmax_scale=c.softmax_scale)
        out = torch.full_like(ref_gpu, float("nan"))
        kvq.kvq_paged_decode_attention_noalloc(d, c.q, *planes, c.seq_lens, max_len,
                                               block_tables=c.block_tables,
                                               block_tables_headwise=c.block_tables_headwise,
                                               window=c.window, softmax_scale=c.softmax_scale, out=out)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_gpu), f"{nseq} sequences: differs from kvq_paged_decode_attention"
        gh.assert_close(out.cpu().numpy(), gh.oracle_decode(sub, c, hp), f"noalloc {nseq} seqs")


def test_noalloc_repeated_calls_stay_correct():
    """Many calls in a row (counters cleared each time) and a bf16 output."""
    spec = synth.small_spec(name="noalloc-rep", cfg=765, mode=1, rotate=True, B=3, Hkv=2, Hq=8,
                            lens=[1500, 40, 900])
    case, d, planes = gh.build(spec)
    max_len = int(case.seq_lens.max().item())
    ref = gh.gpu_decode(spec, case, d, planes)
    outs = [kvq.kvq_paged_decode_attention_noalloc(d, case.q, *planes, case.seq_lens, max_len,
                                                   block_tables=case.block_tables,
                                                   softmax_scale=case.softmax_scale) for _ in range(5)]
    o16 = kvq.kvq_paged_decode_attention_noalloc(d, case.q, *planes, case.seq_lens, max_len,
                                                 block_tables=case.block_tables, softmax_scale=case.softmax_scale,
                                                 out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    for o in outs:
        assert torch.equal(o, ref)
    assert torch.equal(o16, ref.to(torch.bfloat16)) or \
        float((o16.float() - ref).abs().max()) <= float(ref.abs().max()) * 2.0 ** -7
