"""The C-ABI library on a machine without a GPU: it loads, exports every
symbol include/kvq.h declares, and rejects invalid arguments before any HIP
call (FastDeploy PR 7718 Modifications: checks report instead of asserting;
FastDeploy PR 7757 修复: sizes come from the layout query)."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from sub_byte_quantized_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvq.h")


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(kvq_\w+)\s*\(", src, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def desc(mode=1, D=128, H=4, bs=64, nb=10, signs=None):
    return _lib.CacheDesc(mode, D, H, bs, nb, signs, None)


def test_header_lists_entry_points():
    names = header_functions()
    for n in ("kvq_query_layout", "kvq_reshape_and_cache", "kvq_paged_decode_attention",
              "kvq_decode_workspace_size", "kvq_workspace_init", "kvq_paged_prefill_attention",
              "kvq_decode_step", "kvq_gather_dequant", "kvq_last_error", "kvq_prefill_workspace_size"):
        assert n in names


def test_exports_every_header_symbol(lib):
    for name in header_functions():
        assert hasattr(lib, name), name
        assert name in _lib.SIGNATURES, f"binding lacks {name}"


@pytest.mark.parametrize("mode", [0, 1, 2, 3, 4])
@pytest.mark.parametrize("D", [64, 128])
def test_layout_matches_formula(lib, mode, D):
    d = desc(mode, D, H=3, bs=32, nb=7)
    out = _lib.Layout()
    assert lib.kvq_query_layout(ctypes.byref(d), ctypes.byref(out)) == 0
    cshape, mshape = oracle.plane_shapes(mode, D, 3, 32, 7)
    assert out.row_code_bytes == cshape[-1] == D * {0: 8, 1: 4, 2: 2, 3: 8, 4: 8}[mode] // 8
    assert out.row_meta_floats == mshape[-1]
    assert out.code_bytes == 7 * 3 * 32 * cshape[-1]
    assert out.meta_bytes == 7 * 3 * 32 * mshape[-1] * 4


@pytest.mark.parametrize("kw,status", [
    (dict(mode=6), _lib.KVQ_EINVAL), (dict(mode=-1), _lib.KVQ_EINVAL),
    (dict(mode=3, signs=4096), _lib.KVQ_EUNSUPPORTED),
    (dict(D=96), _lib.KVQ_EINVAL), (dict(D=256), _lib.KVQ_EUNSUPPORTED), (dict(D=0), _lib.KVQ_EINVAL),
    (dict(H=0), _lib.KVQ_EINVAL), (dict(bs=8), _lib.KVQ_EINVAL), (dict(bs=40), _lib.KVQ_EINVAL), (dict(bs=48), _lib.KVQ_EINVAL),
    (dict(nb=0), _lib.KVQ_EINVAL)])
def test_layout_rejects(lib, kw, status):
    out = _lib.Layout()
    d = desc(**kw)
    assert lib.kvq_query_layout(ctypes.byref(d), ctypes.byref(out)) == status
    assert lib.kvq_last_error().decode()
    assert lib.kvq_query_layout(None, ctypes.byref(out)) == _lib.KVQ_EINVAL


def test_channel_mode_validation(lib):
    """KVQ_INT8_CHANNEL: no rotation, channel scales required by calls that
    read or write codes, meta planes optional; calibration only in that mode."""
    P = ctypes.c_void_p(4096)
    d = _lib.CacheDesc(3, 128, 4, 64, 10, None, None)
    # write without channel scales
    assert lib.kvq_reshape_and_cache(ctypes.byref(d), P, P, 512, 512, P, None, 4, P, None, P, None, None) \
        == _lib.KVQ_EINVAL
    assert "channel_scales" in lib.kvq_last_error().decode()
    # misaligned scales
    d2 = _lib.CacheDesc(3, 128, 4, 64, 10, None, 4100)
    assert lib.kvq_reshape_and_cache(ctypes.byref(d2), P, P, 512, 512, P, None, 4, P, None, P, None, None) \
        == _lib.KVQ_EINVAL
    # calibration: wrong mode, null output, bad stride
    d0 = _lib.CacheDesc(0, 128, 4, 64, 10, None, None)
    assert lib.kvq_calibrate_channel_scales(ctypes.byref(d0), P, P, 512, 512, 8, P, None) == _lib.KVQ_EINVAL
    assert lib.kvq_calibrate_channel_scales(ctypes.byref(d), P, P, 512, 512, 8, None, None) == _lib.KVQ_EINVAL
    assert lib.kvq_calibrate_channel_scales(ctypes.byref(d), P, P, 100, 512, 8, P, None) == _lib.KVQ_EINVAL
    assert lib.kvq_calibrate_channel_scales(ctypes.byref(d), P, P, 512, 512, -1, P, None) == _lib.KVQ_EINVAL


def test_write_validation(lib):
    d = desc()
    P = ctypes.c_void_p(4096)   # never dereferenced: validation fails first
    # neither / both slot mappings
    assert lib.kvq_reshape_and_cache(ctypes.byref(d), P, P, 512, 512, None, None, 4, P, P, P, P, None) == _lib.KVQ_EINVAL
    assert lib.kvq_reshape_and_cache(ctypes.byref(d), P, P, 512, 512, P, P, 4, P, P, P, P, None) == _lib.KVQ_EINVAL
    # null plane
    assert lib.kvq_reshape_and_cache(ctypes.byref(d), P, P, 512, 512, P, None, 4, None, P, P, P, None) == _lib.KVQ_EINVAL
    # stride below Hkv*D
    assert lib.kvq_reshape_and_cache(ctypes.byref(d), P, P, 100, 512, P, None, 4, P, P, P, P, None) == _lib.KVQ_EINVAL
    assert "stride" in lib.kvq_last_error().decode()
    # negative token count
    assert lib.kvq_reshape_and_cache(ctypes.byref(d), P, P, 512, 512, P, None, -1, P, P, P, P, None) == _lib.KVQ_EINVAL
    # zero tokens: OK and nothing launched
    assert lib.kvq_reshape_and_cache(ctypes.byref(d), P, P, 512, 512, P, None, 0, P, P, P, P, None) == _lib.KVQ_OK


def _decode(lib, d, **kw):
    P = ctypes.c_void_p(4096)
    a = dict(out=P, odt=0, q=P, B=2, Hq=8, kc=P, km=P, vc=P, vm=P, bt=P, bth=None, mb=4, sl=P, msl=200,
             win=None, scale=0.125, opt=None, ws=P, wsb=1 << 20)
    a.update(kw)
    return lib.kvq_paged_decode_attention(ctypes.byref(d), a["out"], a["odt"], a["q"], a["B"], a["Hq"],
                                          a["kc"], a["km"], a["vc"], a["vm"], a["bt"], a["bth"], a["mb"],
                                          a["sl"], a["msl"], a["win"], 0, a["scale"], a["opt"], a["ws"], a["wsb"],
                                          None)


def test_inline_layout_and_planes(lib):
    """KVQ_INT4_INLINE: one tensor [nb, 2, bs, Hkv, D/2 + 4] passed as k_codes;
    k_meta, v_codes and v_meta must be NULL; no chunked prefill; rows of the
    tensor stay below 2^31."""
    d = desc(mode=5, D=128, H=4, bs=32, nb=7)
    out = _lib.Layout()
    assert lib.kvq_query_layout(ctypes.byref(d), ctypes.byref(out)) == 0
    assert out.row_code_bytes == 68 and out.row_meta_floats == 0 and out.meta_bytes == 0
    assert out.code_bytes == int(np.prod(oracle.inline_cache_shape(128, 4, 32, 7)))
    P = ctypes.c_void_p(4096)
    assert _decode(lib, d, km=P, vc=None, vm=None, msl=4 * 32) == _lib.KVQ_EINVAL
    assert "must be NULL" in lib.kvq_last_error().decode()
    assert _decode(lib, d, km=None, vc=P, vm=None, msl=4 * 32) == _lib.KVQ_EINVAL
    assert _decode(lib, d, kc=None, km=None, vc=None, vm=None, msl=4 * 32) == _lib.KVQ_EINVAL
    assert lib.kvq_reshape_and_cache(ctypes.byref(d), P, P, 512, 512, P, None, 4, P, None, P, None, None) \
        == _lib.KVQ_EINVAL
    assert _prefill(lib, d, km=P, vc=None, vm=None, msl=4 * 32) == _lib.KVQ_EINVAL
    big = desc(mode=5, D=128, H=8, bs=1024, nb=1 << 17)   # 2^30 rows per half: 2^31 in the tensor
    assert lib.kvq_query_layout(ctypes.byref(big), ctypes.byref(out)) == _lib.KVQ_EUNSUPPORTED
    half = desc(mode=1, D=128, H=8, bs=1024, nb=1 << 17)  # the same rows in separate planes fit
    assert lib.kvq_query_layout(ctypes.byref(half), ctypes.byref(out)) == _lib.KVQ_OK


def test_decode_validation(lib):
    d = desc(H=4, bs=64)
    P = ctypes.c_void_p(4096)
    assert _decode(lib, d, Hq=6) == _lib.KVQ_EINVAL                 # GQA divisibility
    assert "multiple" in lib.kvq_last_error().decode()
    assert _decode(lib, d, Hq=4 * 17) == _lib.KVQ_EUNSUPPORTED      # group > 16
    assert _decode(lib, d, bt=None, bth=None) == _lib.KVQ_EINVAL    # no table
    assert _decode(lib, d, bt=P, bth=P) == _lib.KVQ_EINVAL          # both tables
    assert _decode(lib, d, msl=4 * 64 + 1) == _lib.KVQ_EINVAL       # beyond the table
    assert _decode(lib, d, odt=5) == _lib.KVQ_EINVAL
    assert _decode(lib, d, scale=float("nan")) == _lib.KVQ_EINVAL
    assert _decode(lib, d, q=None) == _lib.KVQ_EINVAL
    assert _decode(lib, d, B=-1) == _lib.KVQ_EINVAL
    assert _decode(lib, d, kc=None) == _lib.KVQ_EINVAL
    assert _decode(lib, d, out=ctypes.c_void_p(4098)) == _lib.KVQ_EINVAL   # misaligned
    assert _decode(lib, d, B=0) == _lib.KVQ_OK                      # nothing to do
    need = ctypes.c_size_t()
    assert lib.kvq_decode_workspace_size(ctypes.byref(d), 2, 8, 200, None, ctypes.byref(need)) == 0
    if need.value:
        assert _decode(lib, d, wsb=need.value - 1) == _lib.KVQ_ENOSPACE
        assert _decode(lib, d, ws=None) == _lib.KVQ_EINVAL
    # options: a negative workgroup count is rejected; an explicit count
    # changes the workspace size, and the decode call checks it with its own
    bad = _lib.DecodeOptions(-1)
    assert _decode(lib, d, opt=ctypes.byref(bad)) == _lib.KVQ_EINVAL
    assert lib.kvq_decode_workspace_size(ctypes.byref(d), 2, 8, 200, ctypes.byref(bad), ctypes.byref(need)) \
        == _lib.KVQ_EINVAL
    big = _lib.DecodeOptions(5000)
    n_big = ctypes.c_size_t()
    assert lib.kvq_decode_workspace_size(ctypes.byref(d), 2, 8, 200, ctypes.byref(big), ctypes.byref(n_big)) == 0
    n_def = ctypes.c_size_t()
    assert lib.kvq_decode_workspace_size(ctypes.byref(d), 2, 8, 200, None, ctypes.byref(n_def)) == 0
    assert n_big.value > n_def.value
    assert _decode(lib, d, opt=ctypes.byref(big), wsb=n_def.value) == _lib.KVQ_ENOSPACE


def _step(lib, d, **kw):
    P = ctypes.c_void_p(4096)
    a = dict(out=P, odt=0, q=P, B=2, Hq=8, key=P, value=P, ks=512, vs=512, sm=P, smh=None, kc=P, km=P, vc=P,
             vm=P, bt=P, bth=None, mb=4, sl=P, msl=200, win=None, scale=0.125, opt=None, ws=P, wsb=1 << 20)
    a.update(kw)
    return lib.kvq_decode_step(ctypes.byref(d), a["out"], a["odt"], a["q"], a["B"], a["Hq"], a["key"], a["value"],
                               a["ks"], a["vs"], a["sm"], a["smh"], a["kc"], a["km"], a["vc"], a["vm"], a["bt"],
                               a["bth"], a["mb"], a["sl"], a["msl"], a["win"], 0, a["scale"], a["opt"], a["ws"],
                               a["wsb"], None)


def test_noalloc_rejects_oversize_and_validates(lib):
    """The allocation-free decode validates like the decode call and refuses
    a plan larger than its device scratch before touching the GPU."""
    d = desc(H=8, bs=64)
    P = ctypes.c_void_p(4096)

    def call(**kw):
        a = dict(out=P, odt=0, q=P, B=2, Hq=32, kc=P, km=P, vc=P, vm=P, bt=P, bth=None, mb=4, sl=P, msl=200,
                 win=None, scale=0.125)
        a.update(kw)
        return lib.kvq_paged_decode_attention_noalloc(ctypes.byref(d), a["out"], a["odt"], a["q"], a["B"], a["Hq"],
                                                      a["kc"], a["km"], a["vc"], a["vm"], a["bt"], a["bth"],
                                                      a["mb"], a["sl"], a["msl"], a["win"], 0, a["scale"], None)
    need = ctypes.c_size_t()
    assert lib.kvq_decode_workspace_size(ctypes.byref(d), 4096, 128, 64, None, ctypes.byref(need)) == 0
    assert need.value > 8 << 20
    assert call(B=4096, Hq=128, msl=64, mb=1) == _lib.KVQ_ENOSPACE
    assert "allocation-free" in lib.kvq_last_error().decode()
    assert call(Hq=12) == _lib.KVQ_EINVAL                 # GQA divisibility
    assert call(bt=None) == _lib.KVQ_EINVAL               # no table
    assert call(B=0) == _lib.KVQ_OK                       # nothing to do


def test_decode_step_validation(lib):
    d = desc(H=4, bs=64)                                           # D 128: token stride >= 512
    P = ctypes.c_void_p(4096)
    assert _step(lib, d, sm=None, smh=None) == _lib.KVQ_EINVAL      # no slot mapping
    assert "slot_mapping" in lib.kvq_last_error().decode()
    assert _step(lib, d, sm=P, smh=P) == _lib.KVQ_EINVAL            # both slot mappings
    assert _step(lib, d, key=None) == _lib.KVQ_EINVAL
    assert _step(lib, d, ks=100) == _lib.KVQ_EINVAL                 # stride below Hkv*D
    assert "stride" in lib.kvq_last_error().decode()
    assert _step(lib, d, vs=516) == _lib.KVQ_EINVAL                 # stride not a multiple of 8
    assert _step(lib, d, value=ctypes.c_void_p(4098)) == _lib.KVQ_EINVAL   # misaligned
    assert _step(lib, d, Hq=6) == _lib.KVQ_EINVAL                   # decode checks apply too
    assert _step(lib, d, bt=None, bth=None) == _lib.KVQ_EINVAL
    assert _step(lib, d, kc=None) == _lib.KVQ_EINVAL
    assert _step(lib, d, wsb=16) == _lib.KVQ_ENOSPACE
    assert _step(lib, d, B=0, sm=None, key=None) == _lib.KVQ_OK     # nothing to do


def _prefill(lib, d, **kw):
    P = ctypes.c_void_p(4096)
    a = dict(out=P, odt=0, q=P, cu=P, B=2, Hq=8, mq=64, kc=P, km=P, vc=P, vm=P, bt=P, bth=None, mb=4, sl=P,
             msl=200, win=None, scale=0.125, ws=None, wsb=0)
    a.update(kw)
    return lib.kvq_paged_prefill_attention(ctypes.byref(d), a["out"], a["odt"], a["q"], a["cu"], a["B"], a["Hq"],
                                           a["mq"], a["kc"], a["km"], a["vc"], a["vm"], a["bt"], a["bth"],
                                           a["mb"], a["sl"], a["msl"], a["win"], 0, a["scale"], a["ws"], a["wsb"],
                                           None)


def test_prefill_validation(lib):
    d = desc(H=4, bs=64)
    P = ctypes.c_void_p(4096)
    assert _prefill(lib, d, Hq=6) == _lib.KVQ_EINVAL                 # GQA divisibility
    assert "multiple" in lib.kvq_last_error().decode()
    assert _prefill(lib, d, Hq=4 * 129) == _lib.KVQ_EUNSUPPORTED     # group > 128
    assert _prefill(lib, d, bt=None, bth=None) == _lib.KVQ_EINVAL    # no table
    assert _prefill(lib, d, bt=P, bth=P) == _lib.KVQ_EINVAL          # both tables
    assert _prefill(lib, d, msl=4 * 64 + 1) == _lib.KVQ_EINVAL       # beyond the table
    assert _prefill(lib, d, odt=7) == _lib.KVQ_EINVAL
    assert _prefill(lib, d, scale=float("inf")) == _lib.KVQ_EINVAL
    assert _prefill(lib, d, mq=-1) == _lib.KVQ_EINVAL
    assert _prefill(lib, d, cu=None) == _lib.KVQ_EINVAL
    assert _prefill(lib, d, vm=None) == _lib.KVQ_EINVAL
    assert _prefill(lib, d, B=-3) == _lib.KVQ_EINVAL
    assert _prefill(lib, d, B=0) == _lib.KVQ_OK                      # nothing to do
    assert _prefill(lib, d, mq=0) == _lib.KVQ_OK
    assert _prefill(lib, desc(D=96)) == _lib.KVQ_EINVAL
    assert _prefill(lib, desc(mode=4, H=4, bs=64)) == _lib.KVQ_EUNSUPPORTED   # no FP8 prefill
    assert "FP8" in lib.kvq_last_error().decode()


def test_prefill_workspace_size(lib):
    d = desc(H=4, bs=64)
    n = ctypes.c_size_t(123)
    assert lib.kvq_prefill_workspace_size(ctypes.byref(d), 16, 16, 512, 32768, ctypes.byref(n)) == _lib.KVQ_OK
    assert n.value == 0
    # the same size checks as the prefill call
    assert lib.kvq_prefill_workspace_size(ctypes.byref(d), 16, 6, 512, 32768, ctypes.byref(n)) == _lib.KVQ_EINVAL
    assert lib.kvq_prefill_workspace_size(ctypes.byref(d), -1, 16, 512, 32768, ctypes.byref(n)) == _lib.KVQ_EINVAL
    assert lib.kvq_prefill_workspace_size(ctypes.byref(d), 16, 16, -2, 32768, ctypes.byref(n)) == _lib.KVQ_EINVAL
    assert lib.kvq_prefill_workspace_size(ctypes.byref(d), 16, 16, 512, 32768, None) == _lib.KVQ_EINVAL
    assert lib.kvq_prefill_workspace_size(None, 16, 16, 512, 32768, ctypes.byref(n)) == _lib.KVQ_EINVAL
    d4 = desc(mode=4, H=4, bs=64)
    assert lib.kvq_prefill_workspace_size(ctypes.byref(d4), 16, 16, 512, 32768, ctypes.byref(n)) \
        == _lib.KVQ_EUNSUPPORTED


def test_workspace_size_grows_with_work(lib):
    d = desc(H=8, bs=64)
    sizes = []
    for msl in (64, 4096, 131072):
        n = ctypes.c_size_t()
        assert lib.kvq_decode_workspace_size(ctypes.byref(d), 4, 32, msl, None, ctypes.byref(n)) == 0
        sizes.append(n.value)
        assert n.value % 16 == 0
    assert sizes[0] <= sizes[1] <= sizes[2]


def test_workspace_init_validation(lib):
    assert lib.kvq_workspace_init(None, 0, None) == _lib.KVQ_OK
    assert lib.kvq_workspace_init(None, 256, None) == _lib.KVQ_EINVAL
    assert lib.kvq_workspace_init(ctypes.c_void_p(4096 + 16), 256, None) == _lib.KVQ_EINVAL


def test_version(lib):
    assert lib.kvq_version() >= 100


def _gather(lib, d, **kw):
    P = ctypes.c_void_p(4096)
    a = dict(ko=P, vo=P, odt=1, kc=P, km=P, vc=P, vm=P, bt=P, bth=None, mb=4, cu=P, B=2, tot=300, msl=200)
    a.update(kw)
    return lib.kvq_gather_dequant(ctypes.byref(d), a["ko"], a["vo"], a["odt"], a["kc"], a["km"], a["vc"], a["vm"],
                                  a["bt"], a["bth"], a["mb"], a["cu"], a["B"], a["tot"], a["msl"], None)


def test_gather_validation(lib):
    d = desc(H=4, bs=64)
    P = ctypes.c_void_p(4096)
    assert _gather(lib, d, bt=None, bth=None) == _lib.KVQ_EINVAL     # no table
    assert "exactly one" in lib.kvq_last_error().decode()
    assert _gather(lib, d, bt=P, bth=P) == _lib.KVQ_EINVAL           # both tables
    assert _gather(lib, d, msl=4 * 64 + 1) == _lib.KVQ_EINVAL        # beyond the table
    assert _gather(lib, d, odt=3) == _lib.KVQ_EINVAL
    assert _gather(lib, d, ko=None) == _lib.KVQ_EINVAL
    assert _gather(lib, d, cu=None) == _lib.KVQ_EINVAL
    assert _gather(lib, d, km=None) == _lib.KVQ_EINVAL
    assert _gather(lib, d, vo=ctypes.c_void_p(4100)) == _lib.KVQ_EINVAL   # misaligned
    assert _gather(lib, d, B=-1) == _lib.KVQ_EINVAL
    assert _gather(lib, d, B=70000) == _lib.KVQ_EUNSUPPORTED
    assert _gather(lib, d, tot=-5) == _lib.KVQ_EINVAL
    assert _gather(lib, d, mb=0) == _lib.KVQ_EINVAL
    assert _gather(lib, desc(D=96)) == _lib.KVQ_EINVAL
    # nothing to do: OK, nothing launched (no GPU here)
    assert _gather(lib, d, B=0) == _lib.KVQ_OK
    assert _gather(lib, d, tot=0, ko=None, vo=None) == _lib.KVQ_OK
    assert _gather(lib, d, msl=0) == _lib.KVQ_OK
