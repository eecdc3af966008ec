"""The decode step (quantize-on-write, then decode) captured once in a HIP
graph and replayed: every replay, with eager work and synchronizations in
between, must give the eager result bit for bit (the decode workspace's
counters are left at zero by every call, so a replay starts clean)."""
import pytest
import torch

import synth
import sub_byte_quantized_amd as kvq
from tests import gpu_helpers as gh

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("mode", [0, 1, 2, 4, 5])
def test_step_graph_replays_match_eager(mode):
    spec = synth.small_spec(name=f"graph-m{mode}", cfg=480 + mode, mode=mode, rotate=mode != 0, B=6, Hkv=2, Hq=8,
                            lens=[1, 70, 300, 1000, 2049, 4000])
    print(f"[case] graph {spec.name}", flush=True)
    case, d, planes = gh.build(spec)
    dev = planes[0].device
    max_len = int(case.seq_lens.max().item())
    ws = kvq.alloc_workspace(kvq.kvq_decode_workspace_size(d, spec.B, spec.Hq, max_len), dev)
    out = torch.empty((spec.B, spec.Hq, spec.D), dtype=torch.float32, device=dev)
    # the step's new token of every sequence: its last position
    last = (torch.cumsum(case.seq_lens.long(), 0) - 1)
    k_new, v_new = case.k[last].contiguous(), case.v[last].contiguous()
    sm = None if case.slot_mapping is None else case.slot_mapping[last].contiguous()
    smh = None if case.slot_mapping_headwise is None else case.slot_mapping_headwise[last].contiguous()

    def step():
        kvq.kvq_reshape_and_cache(d, k_new, v_new, *planes, slot_mapping=sm, slot_mapping_headwise=smh)
        kvq.kvq_paged_decode_attention(d, case.q, *planes, case.seq_lens, max_len,
                                       block_tables=case.block_tables,
                                       block_tables_headwise=case.block_tables_headwise, window=case.window,
                                       softmax_scale=case.softmax_scale, out=out, workspace=ws)

    step()
    torch.cuda.synchronize()
    eager = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep} differs from the eager step"
        step()            # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(out, eager)
