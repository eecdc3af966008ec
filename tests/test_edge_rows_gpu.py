"""The method's special rows through the HIP path, against the oracle.

Write: rows whose exact (y - z) / s sits on a rounding tie (power-of-two
scales, s = 3, s = 7/64), constant rows (max = min), all-zero rows, rows
whose scale is subnormal or barely normal, one-signed rows and very large
rows.  Without a rotation the codes, scales and zero points must equal the
oracle's bit for bit (round half to even, one correctly rounded reciprocal,
the fixed float32 order; vLLM PR 40835 summary, 实现拆解 item 2).  Decode and
prefill then attend over those planes (scale-0 rows reconstruct exactly z).

Peaked softmax: the query scaled x8 against keys and values with x10 outlier
channels, so a few positions carry almost all the weight; the int8-piece
query must still meet max-abs 2e-3 / mean-abs 2e-4 against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import synth
import sub_byte_quantized_amd as kvq
from tests import gpu_helpers as gh

pytestmark = pytest.mark.gpu
F32 = np.float32


def _bf16_exact(x):
    x = np.asarray(x, F32)
    return np.array_equal(torch.as_tensor(x).to(torch.bfloat16).float().numpy(), x)


def _cycle(vals, n):
    vals = list(vals)
    return [vals[i % len(vals)] for i in range(n)]


def edge_rows(mode, D, seed, huge=True):
    """[N, D] float32 rows, every one bf16-exact.  ``huge`` adds rows of
    magnitude 1e30 and grids up to 508; without it every entry stays below 64,
    for attention's absolute tolerance: the weights p s_V enter the V product
    as bf16 hi + lo (relative error below 2^-16), so an output built from
    entries of size M carries up to M 2^-16 of error (2e-3 at M = 131)."""
    L = {0: 127, 1: 15, 2: 3}[mode]
    r = np.random.default_rng(seed)
    rows = []
    exps = (0, 3, -2, 10) if huge else ((3, 10) if mode == 0 else (0, 3, 10))
    for e in exps:
        u = 2.0 ** -e
        if mode == 0:
            ks = list(range(-127, 127))
            for c0 in range(0, len(ks), D - 2):
                rows.append([127 * u, -127 * u] + _cycle([(k + 0.5) * u for k in ks[c0:c0 + D - 2]], D - 2))
        else:
            z = -1.25 * u
            rows.append([z, z + L * u] + _cycle([z + (k + 0.5) * u for k in range(L)], D - 2))
    if mode != 0:
        rows.append([0.0, 3.0 * L] + _cycle([3 * (k + 0.5) for k in range(L)], D - 2))     # s = 3
        rows.append([0.0, 7 / 64 * L] + _cycle([(k + 0.5) * 7 / 64 for k in range(L)], D - 2))  # s = 7/64
    for c in (0.75, -2.5, 0.0, 1e-30) + ((-3e30,) if huge else ()):
        rows.append([c] * D)                                    # constant rows (zero among them)
    rows.append([0.0] * (D - 1) + [2.0 ** -128])                # subnormal scale: all codes 0
    rows.append([0.0] * (D - 1) + [-(2.0 ** -127)])
    rows.append([0.0] * (D - 2) + [2.0 ** -118, -(2.0 ** -119)])   # smallest normal-scale region
    rows.append(list(np.abs(r.standard_normal(D)) + 5.0))       # one-signed
    rows.append(list(-np.abs(r.standard_normal(D)) - 0.5))
    if huge:
        rows.append(list(r.standard_normal(D) * 1e30))          # large, finite
    x = np.asarray(rows, F32)
    x = torch.as_tensor(x).to(torch.bfloat16).float().numpy()  # the few non-bf16 draws rounded
    assert _bf16_exact(x)
    return x


def build_edge_case(mode, D, rotate, seed, Hkv=2, Hq=4, huge=True):
    """One sequence whose K and V rows are the edge rows (padded with N(0, 1)
    rows), written by the HIP kernel into a poisoned cache through a shuffled
    table.  Returns (spec, case-like dict, desc, planes, k, v)."""
    bs = 16 if D == 64 else 64
    rk = edge_rows(mode, D, seed, huge)
    rv = edge_rows(mode, D, seed + 1, huge)[::-1].copy()
    n = max(len(rk), len(rv))
    T = (n + Hkv - 1) // Hkv + 3
    r = np.random.default_rng(seed)
    pad = lambda x: np.concatenate([x, r.standard_normal((T * Hkv - len(x), D)).astype(F32)])
    k = torch.as_tensor(pad(rk)).to(torch.bfloat16).reshape(T, Hkv, D)
    v = torch.as_tensor(pad(rv)).to(torch.bfloat16).reshape(T, Hkv, D)
    nblk = (T + bs - 1) // bs
    nb = nblk + 2
    bt = r.permutation(nb)[:nblk].astype(np.int32)[None]
    pos = np.arange(T)
    slots = (bt[0, pos // bs].astype(np.int64) * bs + pos % bs)
    signs = np.where(r.integers(0, 2, D) == 1, 1.0, -1.0).astype(F32) if rotate else None
    dev = gh.dev()
    d = kvq.CacheDesc(mode, D, Hkv, bs, nb, None if signs is None else torch.as_tensor(signs, device=dev))
    planes = kvq.alloc_cache(d, dev, poison=True)
    kd, vd = k.to(dev), v.to(dev)
    kvq.kvq_reshape_and_cache(d, kd, vd, *planes, slot_mapping=torch.as_tensor(slots, device=dev))
    torch.cuda.synchronize()
    return dict(k=k, v=v, T=T, bt=bt, slots=slots, signs=signs, bs=bs, nb=nb, Hkv=Hkv, Hq=Hq, D=D,
                mode=mode, rotate=rotate), d, planes


def oracle_write(c):
    cs, ms = oracle.plane_shapes(c["mode"], c["D"], c["Hkv"], c["bs"], c["nb"])
    planes = [np.full(cs, 0xFF, np.uint8), np.full(ms, np.nan, F32),
              np.full(cs, 0xFF, np.uint8), np.full(ms, np.nan, F32)]
    oracle.write_cache(c["k"].float().numpy(), c["v"].float().numpy(), c["mode"], c["bs"], *planes,
                       slot_mapping=c["slots"], signs=c["signs"])
    return planes


CASES = [(m, D, rot) for m in (0, 1, 2) for D in (64, 128) for rot in (False, True)]


def check_edge_planes(c, got, rot):
    ref = oracle_write(c)

    class S:   # the fields compare_codes reads
        pass
    spec = S()
    spec.mode, spec.D = c["mode"], c["D"]
    for g, rr, name in ((got[0], ref[0], "k_codes"), (got[2], ref[2], "v_codes")):
        gh.compare_codes(spec, g, rr, rot, f"edge {name}")
    for g, rr, name in ((got[1], ref[1], "k_meta"), (got[3], ref[3], "v_meta")):
        assert np.array_equal(np.isnan(g), np.isnan(rr)), f"{name}: written rows differ"
        ok = ~np.isnan(rr)
        if rot:
            gh.compare_meta(g[ok], rr[ok], f"edge {name}")
        else:
            assert np.array_equal(g[ok].view(np.uint32), rr[ok].view(np.uint32)), f"edge {name} not bit-exact"


@pytest.mark.parametrize("mode,D,rot", CASES, ids=lambda x: str(x))
def test_edge_rows_write_decode_prefill(mode, D, rot):
    print(f"[case] edge rows mode {mode} D {D} rot {rot}", flush=True)
    seed = 700 + 10 * mode + D // 64 + 5 * rot
    c, d, planes = build_edge_case(mode, D, rot, seed=seed, huge=True)
    check_edge_planes(c, gh.host_planes(planes), rot)
    # without the 1e30 rows, for attention's absolute tolerance
    c, d, planes = build_edge_case(mode, D, rot, seed=seed, huge=False)
    got = gh.host_planes(planes)
    check_edge_planes(c, got, rot)
    # attention over the written planes: decode (query at the last position)
    # and prefill of the last 40 positions, against the oracle on the GPU's planes
    dev = gh.dev()
    T, Hkv, Hq = c["T"], c["Hkv"], c["Hq"]
    g = torch.Generator().manual_seed(mode * 100 + D)
    q = torch.randn((1, Hq, D), generator=g).to(torch.bfloat16)
    sl = torch.tensor([T], dtype=torch.int32)
    bt = torch.as_tensor(c["bt"])
    scale = 1.0 / np.sqrt(D)
    out = kvq.kvq_paged_decode_attention(d, q.to(dev), *planes, sl.to(dev), T, block_tables=bt.to(dev),
                                         softmax_scale=scale)
    n_new = min(40, T)
    qp = torch.randn((n_new, Hq, D), generator=g).to(torch.bfloat16)
    cu = torch.tensor([0, n_new], dtype=torch.int32)
    outp = kvq.kvq_paged_prefill_attention(d, qp.to(dev), cu.to(dev), n_new, *planes, sl.to(dev), T,
                                           block_tables=bt.to(dev), softmax_scale=scale)
    torch.cuda.synchronize()
    refd = oracle.decode_attention(q.float().numpy(), sl.numpy(), mode, D, c["bs"], Hkv, *got, scale,
                                   signs=c["signs"], block_tables=c["bt"])
    gh.assert_close(out.cpu().numpy(), refd, f"edge decode m{mode} D{D} r{int(rot)}")
    refp = oracle.prefill_attention(qp.float().numpy(), cu.numpy(), sl.numpy(), mode, D, c["bs"], Hkv, *got,
                                    scale, signs=c["signs"], block_tables=c["bt"])
    gh.assert_close(outp.cpu().numpy(), refp, f"edge prefill m{mode} D{D} r{int(rot)}")


PEAKED = [
    synth.small_spec(name="peaked-int8", cfg=720, mode=0, rotate=False, outliers=4, B=3, Hkv=2, Hq=8,
                     lens=[300, 1000, 77]),
    synth.small_spec(name="peaked-int4-rot", cfg=721, mode=1, rotate=True, outliers=4, B=3, Hkv=2, Hq=8,
                     lens=[300, 1000, 77]),
    synth.small_spec(name="peaked-int2-rot", cfg=722, mode=2, rotate=True, outliers=4, B=3, Hkv=2, Hq=8,
                     lens=[300, 1000, 77]),
    synth.small_spec(name="peaked-fp8", cfg=723, mode=4, rotate=False, outliers=4, B=3, Hkv=2, Hq=8,
                     lens=[300, 1000, 77]),
]


@pytest.mark.parametrize("spec", PEAKED, ids=lambda s: s.name)
def test_peaked_softmax_decode_and_prefill(spec):
    """|q| x 8 against x10 outlier channels in K and V: the softmax is peaked
    and the output is dominated by a few rows with large entries."""
    print(f"[case] peaked {spec.name}", flush=True)
    case, d, planes = gh.build(spec)
    case.q = (case.q.float() * 8.0).to(torch.bfloat16)
    out = gh.gpu_decode(spec, case, d, planes)
    torch.cuda.synchronize()
    hp = gh.host_planes(planes)
    ref = gh.oracle_decode(spec, case, hp)
    # the softmax really is peaked: the largest weight of most (sequence, head)
    # rows is above 0.5 in the oracle's float64 softmax
    gh.assert_close(out.cpu().numpy(), ref, f"{spec.name} decode")
    if spec.mode == oracle.FP8_E4M3:   # no chunked prefill for FP8
        return
    n_new = [40, 64, 77]
    q, cu = gh.prefill_inputs(spec, n_new, stream=61)
    q = (q.float() * 8.0).to(torch.bfloat16)
    outp = gh.gpu_prefill(spec, case, d, planes, q, cu)
    torch.cuda.synchronize()
    refp = gh.oracle_prefill(spec, case, hp, q, cu)
    gh.assert_close(outp.cpu().numpy(), refp, f"{spec.name} prefill")


def test_peaked_softmax_is_peaked():
    """The x8 query against x10 outlier keys concentrates the weight: check on
    the oracle (float64) that the top weight exceeds 0.5 for most rows, so the
    peaked tests above exercise what they claim."""
    spec = PEAKED[0]
    case = synth.make_case(spec, gh.dev())
    q = (case.q.float() * 8.0).to(torch.bfloat16).float().cpu().numpy().astype(np.float64)
    k = case.k.float().cpu().numpy().astype(np.float64)
    lens = gh.host(case.seq_lens)
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]])
    G = spec.Hq // spec.Hkv
    tops = []
    for b in range(spec.B):
        for hq in range(spec.Hq):
            kk = k[starts[b]:starts[b] + lens[b], hq // G]
            lg = (kk @ q[b, hq]) / np.sqrt(spec.D)
            p = np.exp(lg - lg.max())
            tops.append(p.max() / p.sum())
    assert np.median(tops) > 0.5, np.median(tops)


# ---------------------------------------------------------------------------
# Contract violations that must not fault: block ids >= num_blocks are evicted
# blocks, slots >= num_blocks * block_size are skipped.  The planes are
# allocated larger than the num_blocks the descriptor declares, so a missing
# bound would read or write valid memory and fail by value, never by fault.

def _oob_setup(mode, rotate, headwise):
    spec = synth.small_spec(name=f"oob-m{mode}", cfg=730 + mode + 3 * headwise, mode=mode, rotate=rotate, B=3,
                            Hkv=2, Hq=8, lens=[300, 517, 64], headwise=headwise)
    case, d, planes = gh.build(spec)
    nb = case.tables.num_blocks
    cut = nb // 2                       # the descriptor now declares only blocks < cut
    d2 = kvq.CacheDesc(spec.mode, spec.D, spec.Hkv, spec.bs, cut, case.rot_signs)
    return spec, case, d, d2, planes, nb, cut


@pytest.mark.parametrize("mode,rotate,headwise", [(0, False, False), (1, True, True), (2, True, False)])
def test_block_ids_past_num_blocks_read_as_evicted(mode, rotate, headwise):
    print(f"[case] oob ids mode {mode} headwise {headwise}", flush=True)
    spec, case, d, d2, planes, nb, cut = _oob_setup(mode, rotate, headwise)
    hp = gh.host_planes(planes)
    bt = gh.host(case.block_tables)
    bth = gh.host(case.block_tables_headwise)
    tab = bt if bt is not None else bth
    assert (tab >= cut).any() and ((tab >= 0) & (tab < cut)).any()
    out = gh.gpu_decode(spec, case, d2, planes)
    # prefill of the last 30 positions of every sequence
    n_new = [30, 30, 30]
    q, cu = gh.prefill_inputs(spec, n_new, stream=62)
    outp = gh.gpu_prefill(spec, case, d2, planes, q, cu)
    torch.cuda.synchronize()
    masked = lambda t: None if t is None else np.where(t >= cut, -1, t)
    ref = oracle.decode_attention(gh.f32(case.q), gh.host(case.seq_lens), spec.mode, spec.D, spec.bs, spec.Hkv,
                                  *hp, case.softmax_scale, signs=gh.host(case.rot_signs),
                                  block_tables=masked(bt), block_tables_headwise=masked(bth),
                                  window=gh.host(case.window))
    gh.assert_close(out.cpu().numpy(), ref, "decode ids >= num_blocks")
    refp = oracle.prefill_attention(gh.f32(q), gh.host(cu), gh.host(case.seq_lens), spec.mode, spec.D, spec.bs,
                                    spec.Hkv, *hp, case.softmax_scale, signs=gh.host(case.rot_signs),
                                    block_tables=masked(bt), block_tables_headwise=masked(bth),
                                    window=gh.host(case.window))
    gh.assert_close(outp.cpu().numpy(), refp, "prefill ids >= num_blocks")
    # the gather gives zero rows for them, like -1
    lens = gh.host(case.seq_lens)
    cu_g = torch.as_tensor(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32), device=planes[0].device)
    kg, vg = kvq.kvq_gather_dequant(d2, *planes, cu_g, int(lens.max()), int(lens.sum()),
                                    block_tables=case.block_tables, block_tables_headwise=case.block_tables_headwise,
                                    out_dtype=torch.float32)
    torch.cuda.synchronize()
    Kr, Vr = oracle.gather_dequant(gh.host(cu_g), spec.mode, spec.D, spec.bs, spec.Hkv, *hp,
                                   signs=gh.host(case.rot_signs), block_tables=masked(bt),
                                   block_tables_headwise=masked(bth))
    gone = np.all(Kr == 0, axis=-1)
    assert gone.any()
    assert np.all(kg.cpu().numpy()[gone] == 0) and np.all(vg.cpu().numpy()[gone] == 0)


def test_slots_past_capacity_are_not_written():
    spec = synth.small_spec(name="oob-slots", cfg=740, mode=1, rotate=True, B=2, Hkv=2, Hq=4, lens=[300, 130])
    case, d, planes = gh.build(spec, write=False)
    nb = case.tables.num_blocks
    cut = nb // 2
    d2 = kvq.CacheDesc(spec.mode, spec.D, spec.Hkv, spec.bs, cut, case.rot_signs)
    kvq.kvq_reshape_and_cache(d2, case.k, case.v, *planes, slot_mapping=case.slot_mapping)
    torch.cuda.synchronize()
    got = gh.host_planes(planes)
    # blocks >= cut keep their poison; blocks < cut hold exactly the oracle's rows
    assert np.all(got[0][cut:] == 0xFF) and np.all(np.isnan(got[1][cut:]))
    assert np.all(got[2][cut:] == 0xFF) and np.all(np.isnan(got[3][cut:]))
    sm = gh.host(case.slot_mapping)
    keep = np.where(sm < cut * spec.bs, sm, -1)
    cs, ms = oracle.plane_shapes(spec.mode, spec.D, spec.Hkv, spec.bs, nb)
    ref = [np.full(cs, 0xFF, np.uint8), np.full(ms, np.nan, F32), np.full(cs, 0xFF, np.uint8),
           np.full(ms, np.nan, F32)]
    oracle.write_cache(gh.f32(case.k), gh.f32(case.v), spec.mode, spec.bs, *ref, slot_mapping=keep,
                       signs=gh.host(case.rot_signs))
    for g, r in ((got[0], ref[0]), (got[2], ref[2])):
        gh.compare_codes(spec, g, r, True, "slots past capacity")
    for g, r in ((got[1], ref[1]), (got[3], ref[3])):
        assert np.array_equal(np.isnan(g), np.isnan(r))


def test_seq_lens_past_max_seq_len_are_clamped():
    """A device seq_lens entry above the host's max_seq_len is clamped to it:
    the output is that of the clamped length and later calls on the same
    workspace are unaffected (every piece counter is back at zero)."""
    spec = synth.small_spec(name="clamp", cfg=741, mode=2, rotate=True, B=3, Hkv=2, Hq=8, lens=[900, 600, 700])
    case, d, planes = gh.build(spec)
    max_len = 640
    ws = kvq.alloc_workspace(kvq.kvq_decode_workspace_size(d, spec.B, spec.Hq, max_len), planes[0].device)
    out = kvq.kvq_paged_decode_attention(d, case.q, *planes, case.seq_lens, max_len,
                                         block_tables=case.block_tables, softmax_scale=case.softmax_scale,
                                         workspace=ws)
    torch.cuda.synchronize()
    clamped = np.minimum(gh.host(case.seq_lens), max_len)
    hp = gh.host_planes(planes)
    ref = oracle.decode_attention(gh.f32(case.q), clamped, spec.mode, spec.D, spec.bs, spec.Hkv, *hp,
                                  case.softmax_scale, signs=gh.host(case.rot_signs),
                                  block_tables=gh.host(case.block_tables))
    gh.assert_close(out.cpu().numpy(), ref, "clamped seq_lens")
    counters = ws[:4 * spec.B * spec.Hkv].view(torch.int32)
    assert int(counters.abs().sum().item()) == 0
    # a full-length call on the same workspace is correct
    full = int(case.seq_lens.max().item())
    ws2 = kvq.alloc_workspace(kvq.kvq_decode_workspace_size(d, spec.B, spec.Hq, full), planes[0].device)
    out2 = gh.gpu_decode(spec, case, d, planes, workspace=ws2)
    torch.cuda.synchronize()
    gh.assert_close(out2.cpu().numpy(), gh.oracle_decode(spec, case, hp), "after clamp")
