"""FP8 (OCP E4M3) per-token-head mode (the INT8/FP8 per-token-head schemes of
the vLLM PR 40835 summary, 功能与动机) on the HIP path: rounding of the codes
at exact midpoints and in the subnormal range against bytes fixed by the
E4M3 definition and against the oracle, and the chunked-prefill refusal.
The decode, gather, fused-step and write sweeps over modes include FP8 in
their own files."""
import numpy as np
import pytest
import torch

import oracle
import synth
import sub_byte_quantized_amd as kvq
from tests import gpu_helpers as gh

pytestmark = pytest.mark.gpu

# (t, E4M3 byte of t): t = y / s with s = max|y| / 448 a power of two, so t is
# exact and the byte follows from the format alone (bias 7, 3 mantissa bits,
# subnormal step 2^-9, ties to even mantissa).
PINNED = [
    (448.0, 0x7E), (-448.0, 0xFE), (1.0, 0x38), (1.0625, 0x38), (1.1875, 0x3A), (-1.1875, 0xBA),
    (2.0 ** -6, 0x08), (2.0 ** -9, 0x01), (2.0 ** -10, 0x00), (3 * 2.0 ** -10, 0x02), (5 * 2.0 ** -10, 0x02),
    (7 * 2.0 ** -10, 0x04), (-(2.0 ** -10), 0x80), (15 * 2.0 ** -10, 0x08), (240.0, 0x77), (232.0, 0x76),
    (248.0, 0x78), (0.0, 0x00), (13.0, 0x55), (-13.5, 0xD6), (0.3125, 0x2A), (0.34375, 0x2B),
]


@pytest.mark.parametrize("D", [64, 128])
def test_fp8_codes_at_midpoints_and_subnormals(D):
    print(f"[case] fp8 midpoints D {D}", flush=True)
    spec = synth.small_spec(name=f"fp8-mid-d{D}", cfg=840 + D, mode=4, rotate=False, D=D, bs=16, B=1, Hkv=2,
                            Hq=4, lens=[40])
    dev = gh.dev()
    case = synth.make_case(spec, dev)
    T = case.k.shape[0]
    rows = np.zeros((T, spec.Hkv, D), np.float32)
    r = np.random.default_rng(841)
    ts = np.array([t for t, _ in PINNED])
    for i in range(T):
        for h in range(spec.Hkv):
            scale = 2.0 ** int(r.integers(-8, 4))          # s = scale, a power of two
            perm = r.permutation(D)[:len(ts)]
            rows[i, h, perm] = ts * scale
            if i == 3:
                rows[i, h] = 0.0                           # zero row: s = 0, codes 0
    k = torch.as_tensor(rows, dtype=torch.bfloat16, device=dev)
    assert np.array_equal(k.float().cpu().numpy(), rows), "pinned values must be exact in bf16"
    case.k = k
    case.v = (-k).contiguous()
    case, d, planes = gh.build(spec, case=case)
    got = gh.host_planes(planes)
    cs, ms = oracle.plane_shapes(4, D, spec.Hkv, spec.bs, case.tables.num_blocks)
    ref = [np.full(cs, 0xFF, np.uint8), np.full(ms, np.nan, np.float32), np.full(cs, 0xFF, np.uint8),
           np.full(ms, np.nan, np.float32)]
    oracle.write_cache(gh.f32(case.k), gh.f32(case.v), 4, spec.bs, *ref, slot_mapping=gh.host(case.slot_mapping))
    assert np.array_equal(got[0], ref[0]) and np.array_equal(got[2], ref[2]), "codes differ from the oracle"
    ok = ~np.isnan(ref[1])
    assert np.array_equal(got[1][ok].view(np.uint32), ref[1][ok].view(np.uint32)), "K scales differ"
    assert np.array_equal(got[3][ok].view(np.uint32), ref[3][ok].view(np.uint32)), "V scales differ"
    # bytes fixed by the format: row (token i, head h) at its slot
    slots = gh.host(case.slot_mapping)
    want = {t: b for t, b in PINNED}
    for i in range(T):
        blk, off = divmod(int(slots[i]), spec.bs)
        for h in range(spec.Hkv):
            kc, vc = got[0][blk, h, off], got[2][blk, h, off]
            if i == 3:
                assert not kc.any() and got[1][blk, h, off, 0] == 0.0
                continue
            s = float(got[1][blk, h, off, 0])
            assert s == float(np.max(np.abs(rows[i, h]))) / 448.0
            for dd in np.flatnonzero(rows[i, h]):
                t = float(rows[i, h, dd]) / s
                assert kc[dd] == want[t], (i, h, dd, t, hex(kc[dd]))
                assert vc[dd] == want[t] ^ 0x80 or (t == 0.0), (i, h, dd, t, hex(vc[dd]))


def test_fp8_prefill_is_refused():
    spec = synth.small_spec(name="fp8-prefill", cfg=850, mode=4, rotate=True, B=2, Hkv=2, Hq=4, lens=[70, 9])
    case, d, planes = gh.build(spec)
    q, cu = gh.prefill_inputs(spec, [5, 9])
    with pytest.raises(kvq.KvqError) as e:
        gh.gpu_prefill(spec, case, d, planes, q, cu)
    assert "FP8" in str(e.value)
