"""The fused decode step (kvq_decode_step: write each sequence's new token,
then attend, in one launch) against the two-call path (kvq_reshape_and_cache
then kvq_paged_decode_attention): cache planes and output bit for bit, and
the output against the oracle on the written planes."""
import numpy as np
import pytest
import torch

import synth
import sub_byte_quantized_amd as kvq
from tests import gpu_helpers as gh

pytestmark = pytest.mark.gpu


def _new_tokens(spec, case, seed):
    """Fresh bf16 K/V for every sequence's last position, with that
    position's slot (table slot of seq_len - 1); a tenth of the tokens (or
    heads) skipped with slot -1, and -1 for empty sequences."""
    dev = case.q.device
    B, H, D = spec.B, spec.Hkv, spec.D
    g = torch.Generator(device=dev).manual_seed(seed)
    k = torch.randn((B, H, D), generator=g, device=dev).to(torch.bfloat16)
    v = torch.randn((B, H, D), generator=g, device=dev).to(torch.bfloat16)
    lens = case.seq_lens.long()
    last = torch.clamp(torch.cumsum(lens, 0) - 1, min=0)
    r = np.random.default_rng([seed, 3])
    if case.slot_mapping_headwise is not None:
        s = case.slot_mapping_headwise[last].clone()
        skip = torch.as_tensor(r.random((B, H)) < 0.1, device=dev)
        s[skip] = -1
        s[lens == 0] = -1
        return k, v, None, s.contiguous()
    s = case.slot_mapping[last].clone()
    skip = torch.as_tensor(r.random(B) < 0.1, device=dev)
    s[skip] = -1
    s[lens == 0] = -1
    return k, v, s.contiguous(), None


CASES = [
    dict(name="m0-b64", mode=0, rotate=False, bs=64, D=128, lens=[1, 64, 65, 300, 1000, 2049], B=6, Hkv=2, Hq=8),
    dict(name="m1-b16-rot", mode=1, rotate=True, bs=16, D=128, lens=[0, 17, 129, 700, 1500], B=5, Hkv=2, Hq=10),
    dict(name="m2-b64-rot", mode=2, rotate=True, bs=64, D=128, lens=[5, 4000, 63, 128], B=4, Hkv=4, Hq=16),
    dict(name="m1-d64-rot", mode=1, rotate=True, bs=16, D=64, lens=[3, 200, 1000], B=3, Hkv=2, Hq=4),
    dict(name="m4-b16-rot", mode=4, rotate=True, bs=16, D=128, lens=[1, 64, 300, 1000], B=4, Hkv=2, Hq=8),
    dict(name="m1-headwise-window", mode=1, rotate=True, bs=64, D=128, lens=[300, 1000, 129], B=3, Hkv=4, Hq=16,
         window=[100, 64, 0, 0], headwise=True, evict_outside_window=True),
]


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c["name"])
def test_decode_step_equals_write_then_decode(cfg):
    kw = dict(cfg)
    name = kw.pop("name")
    spec = synth.small_spec(name=f"step-{name}", cfg=490 + len(CASES), **kw)
    print(f"[case] decode step {name}", flush=True)
    case, d, planes = gh.build(spec)
    k, v, sm, smh = _new_tokens(spec, case, seed=500 + spec.mode)
    max_len = int(case.seq_lens.max().item())
    dev = planes[0].device
    a = [p.clone() for p in planes]
    b = [p.clone() for p in planes]
    kvq.kvq_reshape_and_cache(d, k, v, *a, slot_mapping=sm, slot_mapping_headwise=smh)
    out_a = gh.gpu_decode(spec, case, d, a)
    ws = kvq.alloc_workspace(kvq.kvq_decode_workspace_size(d, spec.B, spec.Hq, max_len), dev)
    out_b = kvq.kvq_decode_step(d, case.q, k, v, *b, case.seq_lens, max_len, slot_mapping=sm,
                                slot_mapping_headwise=smh, block_tables=case.block_tables,
                                block_tables_headwise=case.block_tables_headwise, window=case.window,
                                softmax_scale=case.softmax_scale, workspace=ws)
    torch.cuda.synchronize()
    for pa, pb, n in zip(a, b, ("k_codes", "k_meta", "v_codes", "v_meta")):
        assert torch.equal(pa.view(torch.uint8), pb.view(torch.uint8)), f"{n} differs"
    assert torch.equal(out_a, out_b), "fused output differs from write-then-decode"
    ref = gh.oracle_decode(spec, case, gh.host_planes(b))
    gh.assert_close(out_b.cpu().numpy(), ref, f"step {name}")
