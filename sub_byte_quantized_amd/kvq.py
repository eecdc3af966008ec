"""Python binding of libkvq with the C ABI's names.

Argument marshalling only: tensors are checked for dtype, device and
contiguity, their data pointers and the current HIP stream are passed to the
library, and a non-OK status raises KvqError with the library's message.
Every step of the computation runs in the library's HIP kernels.  PyTorch is
used for device memory and streams.
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
from typing import Optional

import torch

from . import _lib
from ._lib import (KVQ_FP8_E4M3, KVQ_INT2_ASYM, KVQ_INT4_ASYM, KVQ_INT4_INLINE, KVQ_INT8_CHANNEL,  # noqa: F401
                   KVQ_INT8_SYM,
                   KVQ_OUT_BF16, KVQ_OUT_F32)


class KvqError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_lib.STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


def _check(status: int) -> None:
    if status != _lib.KVQ_OK:
        raise KvqError(status, _lib.load().kvq_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t, name, dtype, device=None, contiguous=True):
    if t is None:
        return
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _opts(num_workgroups: int):
    """kvq_decode_options for a workgroup count (0 = the library's choice)."""
    return ctypes.byref(_lib.DecodeOptions(int(num_workgroups))) if num_workgroups else None


def _check_planes(desc, k_codes, k_meta, v_codes, v_meta):
    """The four planes: dtype, device, contiguity, and at least the bytes the
    layout query gives for ``desc`` (a larger allocation is allowed: the
    kernels address only the first num_blocks blocks).  KVQ_INT4_INLINE: the
    one cache tensor as k_codes, the other three None."""
    lay = kvq_query_layout(desc)
    dev = k_codes.device
    if desc.mode == KVQ_INT4_INLINE:
        if k_meta is not None or v_codes is not None or v_meta is not None:
            raise ValueError("KVQ_INT4_INLINE takes the cache as k_codes; k_meta, v_codes, v_meta must be None")
        _need(k_codes, "k_codes", torch.uint8, dev)
        if k_codes.numel() < lay["code_bytes"]:
            raise ValueError(f"k_codes holds {k_codes.numel()} bytes, the layout needs {lay['code_bytes']}")
        return dev
    for t, n, dt, need in ((k_codes, "k_codes", torch.uint8, lay["code_bytes"]),
                           (v_codes, "v_codes", torch.uint8, lay["code_bytes"]),
                           (k_meta, "k_meta", torch.float32, lay["meta_bytes"]),
                           (v_meta, "v_meta", torch.float32, lay["meta_bytes"])):
        if t is None:
            raise ValueError(f"{n} is None")
        _need(t, n, dt, dev)
        if t.numel() * t.element_size() < need:
            raise ValueError(f"{n} holds {t.numel() * t.element_size()} bytes, the layout needs {need}")
    return dev


def _check_tables(desc, B, block_tables, block_tables_headwise, dev):
    """Exactly one table, int32 on the device, B (uniform) or B*Hkv
    (head-wise) rows; returns its row length."""
    if (block_tables is None) == (block_tables_headwise is None):
        raise ValueError("exactly one of block_tables and block_tables_headwise must be given")
    tab = block_tables if block_tables is not None else block_tables_headwise
    name = "block_tables" if block_tables is not None else "block_tables_headwise"
    _need(tab, name, torch.int32, dev)
    rows = B if block_tables is not None else B * desc.num_kv_heads
    if tab.dim() != 2 or tab.shape[0] < rows:
        raise ValueError(f"{name} must be [>= {rows}, max_blocks], got {tuple(tab.shape)}")
    return int(tab.shape[1])


def _check_lens_window(desc, B, seq_lens, window, dev):
    _need(seq_lens, "seq_lens", torch.int32, dev)
    if seq_lens is None or seq_lens.dim() != 1 or seq_lens.shape[0] < B:
        raise ValueError(f"seq_lens must be int32 [>= {B}]")
    _need(window, "window", torch.int32, dev)
    if window is not None and (window.dim() != 1 or window.shape[0] < desc.num_kv_heads):
        raise ValueError(f"window must be int32 [>= {desc.num_kv_heads}]")


def _check_query(desc, query, name="query"):
    dev = query.device
    _need(query, name, torch.bfloat16, dev)
    if query.dim() != 3 or query.shape[2] != desc.head_dim:
        raise ValueError(f"{name} must be [N, Hq, {desc.head_dim}], got {tuple(query.shape)}")
    return dev


def _out_for(out, shape, out_dtype, dev):
    if out is None:
        out = torch.empty(shape, dtype=out_dtype, device=dev)
    if out.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError(f"out must be float32 or bfloat16, got {out.dtype}")
    _need(out, "out", out.dtype, dev)
    if tuple(out.shape) != tuple(shape):
        raise ValueError(f"out must be {tuple(shape)}, got {tuple(out.shape)}")
    return out, {torch.float32: KVQ_OUT_F32, torch.bfloat16: KVQ_OUT_BF16}[out.dtype]


def _stream(device) -> ctypes.c_void_p:
    if device.type != "cuda":
        raise ValueError(f"tensors must be on a HIP device, got {device}")
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


@dataclasses.dataclass
class CacheDesc:
    mode: int
    head_dim: int
    num_kv_heads: int
    block_size: int
    num_blocks: int
    rot_signs: Optional[torch.Tensor] = None   # float32 [head_dim] of +-1, on the device
    # KVQ_INT8_CHANNEL: float32 [2, Hkv, D] per-channel scales (K then V)
    channel_scales: Optional[torch.Tensor] = None

    def c(self) -> _lib.CacheDesc:
        if self.rot_signs is not None:
            _need(self.rot_signs, "rot_signs", torch.float32)
        if self.channel_scales is not None:
            _need(self.channel_scales, "channel_scales", torch.float32)
            if tuple(self.channel_scales.shape) != (2, self.num_kv_heads, self.head_dim):
                raise ValueError(f"channel_scales must be [2, {self.num_kv_heads}, {self.head_dim}]")
        return _lib.CacheDesc(int(self.mode), int(self.head_dim), int(self.num_kv_heads),
                              int(self.block_size), int(self.num_blocks),
                              None if self.rot_signs is None else self.rot_signs.data_ptr(),
                              None if self.channel_scales is None else self.channel_scales.data_ptr())


def kvq_query_layout(desc: CacheDesc) -> dict:
    out = _lib.Layout()
    d = desc.c()
    _check(_lib.load().kvq_query_layout(ctypes.byref(d), ctypes.byref(out)))
    return dict(code_bytes=out.code_bytes, meta_bytes=out.meta_bytes,
                row_code_bytes=out.row_code_bytes, row_meta_floats=out.row_meta_floats)


def alloc_cache(desc: CacheDesc, device, poison: bool = False):
    """Allocate (k_codes, k_meta, v_codes, v_meta) at the sizes
    kvq_query_layout reports: uint8 [nb, Hkv, bs, P] and float32
    [nb, Hkv, bs, M].  ``poison`` fills codes with 0xFF and meta with NaN.
    KVQ_INT4_INLINE: (cache, None, None, None), cache uint8 [nb, 2, bs, Hkv,
    D/2 + 4]."""
    lay = kvq_query_layout(desc)
    P, M = lay["row_code_bytes"], lay["row_meta_floats"]
    if desc.mode == KVQ_INT4_INLINE:
        c = torch.empty((desc.num_blocks, 2, desc.block_size, desc.num_kv_heads, P), dtype=torch.uint8,
                        device=device)
        assert c.numel() == lay["code_bytes"]
        if poison:
            c.fill_(0xFF)
        return c, None, None, None
    shape_c = (desc.num_blocks, desc.num_kv_heads, desc.block_size, P)
    shape_m = (desc.num_blocks, desc.num_kv_heads, desc.block_size, M)
    planes = []
    for _ in range(2):
        c = torch.empty(shape_c, dtype=torch.uint8, device=device)
        m = torch.empty(shape_m, dtype=torch.float32, device=device)
        assert c.numel() == lay["code_bytes"] and m.numel() * 4 == lay["meta_bytes"]
        if poison:
            c.fill_(0xFF)
            m.fill_(float("nan"))
        planes += [c, m]
    return tuple(planes)


def kvq_reshape_and_cache(desc: CacheDesc, key: torch.Tensor, value: torch.Tensor,
                          k_codes: torch.Tensor, k_meta: torch.Tensor,
                          v_codes: torch.Tensor, v_meta: torch.Tensor,
                          slot_mapping: Optional[torch.Tensor] = None,
                          slot_mapping_headwise: Optional[torch.Tensor] = None) -> None:
    """Quantize bf16 key/value [T, Hkv, D] into the paged cache."""
    dev = k_codes.device
    for t, n in ((key, "key"), (value, "value")):
        _need(t, n, torch.bfloat16, dev, contiguous=False)
        if t.dim() != 3 or t.stride(2) != 1 or t.stride(1) != desc.head_dim:
            raise ValueError(f"{n} must be [T, Hkv, D] with heads and D contiguous")
    if key.shape != value.shape:
        raise ValueError("key and value shapes differ")
    _check_planes(desc, k_codes, k_meta, v_codes, v_meta)
    T = int(key.shape[0])
    if key.shape[1] != desc.num_kv_heads or key.shape[2] != desc.head_dim:
        raise ValueError(f"key must be [T, {desc.num_kv_heads}, {desc.head_dim}], got {tuple(key.shape)}")
    _need(slot_mapping, "slot_mapping", torch.int64, dev)
    _need(slot_mapping_headwise, "slot_mapping_headwise", torch.int64, dev)
    if slot_mapping is not None and tuple(slot_mapping.shape) != (T,):
        raise ValueError(f"slot_mapping must be [{T}], got {tuple(slot_mapping.shape)}")
    if slot_mapping_headwise is not None and tuple(slot_mapping_headwise.shape) != (T, desc.num_kv_heads):
        raise ValueError(f"slot_mapping_headwise must be [{T}, {desc.num_kv_heads}], "
                         f"got {tuple(slot_mapping_headwise.shape)}")
    d = desc.c()
    _check(_lib.load().kvq_reshape_and_cache(
        ctypes.byref(d), _ptr(key), _ptr(value), key.stride(0), value.stride(0),
        _ptr(slot_mapping), _ptr(slot_mapping_headwise), int(key.shape[0]),
        _ptr(k_codes), _ptr(k_meta), _ptr(v_codes), _ptr(v_meta), _stream(dev)))


def kvq_calibrate_channel_scales(desc: CacheDesc, key: torch.Tensor, value: torch.Tensor,
                                 out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Per-channel INT8 scales [2, Hkv, D] (K then V) of a layer's first
    K/V, key/value bf16 [T, Hkv, D]: max over tokens of |x| / 127."""
    dev = key.device
    for t, n in ((key, "key"), (value, "value")):
        _need(t, n, torch.bfloat16, dev, contiguous=False)
        if t.dim() != 3 or tuple(t.shape[1:]) != (desc.num_kv_heads, desc.head_dim) or t.stride(2) != 1 \
                or t.stride(1) != desc.head_dim:
            raise ValueError(f"{n} must be [T, {desc.num_kv_heads}, {desc.head_dim}] with heads and D contiguous")
    if key.shape != value.shape:
        raise ValueError("key and value shapes differ")
    if out is None:
        out = torch.empty((2, desc.num_kv_heads, desc.head_dim), dtype=torch.float32, device=dev)
    _need(out, "out", torch.float32, dev)
    if tuple(out.shape) != (2, desc.num_kv_heads, desc.head_dim):
        raise ValueError(f"out must be [2, {desc.num_kv_heads}, {desc.head_dim}]")
    d = desc.c()
    _check(_lib.load().kvq_calibrate_channel_scales(ctypes.byref(d), _ptr(key), _ptr(value), key.stride(0),
                                                    value.stride(0), int(key.shape[0]), _ptr(out), _stream(dev)))
    return out


def kvq_decode_workspace_size(desc: CacheDesc, num_seqs: int, num_q_heads: int,
                              max_seq_len: int, num_workgroups: int = 0) -> int:
    """Workspace bytes of a decode call with these sizes; ``num_workgroups``
    (0 = the library's choice) must match the decode call's."""
    n = ctypes.c_size_t(0)
    d = desc.c()
    _check(_lib.load().kvq_decode_workspace_size(ctypes.byref(d), int(num_seqs), int(num_q_heads),
                                                 int(max_seq_len), _opts(num_workgroups), ctypes.byref(n)))
    return int(n.value)


def kvq_prefill_workspace_size(desc: CacheDesc, num_seqs: int, num_q_heads: int, max_q_len: int,
                               max_seq_len: int) -> int:
    n = ctypes.c_size_t(0)
    d = desc.c()
    _check(_lib.load().kvq_prefill_workspace_size(ctypes.byref(d), int(num_seqs), int(num_q_heads),
                                                  int(max_q_len), int(max_seq_len), ctypes.byref(n)))
    return int(n.value)


def kvq_workspace_init(workspace: torch.Tensor) -> None:
    _need(workspace, "workspace", torch.uint8)
    _check(_lib.load().kvq_workspace_init(_ptr(workspace), workspace.numel(), _stream(workspace.device)))


def alloc_workspace(nbytes: int, device) -> torch.Tensor:
    """A device workspace of at least ``nbytes`` (rounded to 256), zeroed by
    kvq_workspace_init."""
    n = max(256, (int(nbytes) + 255) // 256 * 256)
    ws = torch.empty(n, dtype=torch.uint8, device=device)
    kvq_workspace_init(ws)
    return ws


def kvq_paged_decode_attention(desc: CacheDesc, query: torch.Tensor,
                               k_codes: torch.Tensor, k_meta: torch.Tensor,
                               v_codes: torch.Tensor, v_meta: torch.Tensor,
                               seq_lens: torch.Tensor, max_seq_len: int,
                               block_tables: Optional[torch.Tensor] = None,
                               block_tables_headwise: Optional[torch.Tensor] = None,
                               window: Optional[torch.Tensor] = None,
                               softmax_scale: Optional[float] = None,
                               out: Optional[torch.Tensor] = None,
                               out_dtype: torch.dtype = torch.float32,
                               workspace: Optional[torch.Tensor] = None,
                               num_workgroups: int = 0, sink_size: int = 0) -> torch.Tensor:
    """Decode attention for query [B, Hq, D] (bf16); returns out [B, Hq, D]."""
    dev = _check_query(desc, query)
    B, Hq, D = query.shape
    _check_planes(desc, k_codes, k_meta, v_codes, v_meta)
    max_blocks = _check_tables(desc, B, block_tables, block_tables_headwise, dev)
    _check_lens_window(desc, B, seq_lens, window, dev)
    out, odt = _out_for(out, (B, Hq, D), out_dtype, dev)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    if workspace is None:
        workspace = alloc_workspace(kvq_decode_workspace_size(desc, B, Hq, max_seq_len, num_workgroups), dev)
    _need(workspace, "workspace", torch.uint8, dev)
    d = desc.c()
    _check(_lib.load().kvq_paged_decode_attention(
        ctypes.byref(d), _ptr(out), odt, _ptr(query), int(B), int(Hq),
        _ptr(k_codes), _ptr(k_meta), _ptr(v_codes), _ptr(v_meta),
        _ptr(block_tables), _ptr(block_tables_headwise), max_blocks,
        _ptr(seq_lens), int(max_seq_len), _ptr(window), int(sink_size), float(softmax_scale), _opts(num_workgroups),
        _ptr(workspace), workspace.numel(), _stream(dev)))
    return out


def kvq_paged_decode_attention_noalloc(desc: CacheDesc, query: torch.Tensor,
                                       k_codes: torch.Tensor, k_meta: torch.Tensor,
                                       v_codes: torch.Tensor, v_meta: torch.Tensor,
                                       seq_lens: torch.Tensor, max_seq_len: int,
                                       block_tables: Optional[torch.Tensor] = None,
                                       block_tables_headwise: Optional[torch.Tensor] = None,
                                       window: Optional[torch.Tensor] = None,
                                       softmax_scale: Optional[float] = None,
                                       out: Optional[torch.Tensor] = None,
                                       out_dtype: torch.dtype = torch.float32,
                                       sink_size: int = 0) -> torch.Tensor:
    """Decode attention with the library's device scratch as workspace (no
    workspace argument; nothing is allocated when ``out`` is given)."""
    dev = _check_query(desc, query)
    B, Hq, D = query.shape
    _check_planes(desc, k_codes, k_meta, v_codes, v_meta)
    max_blocks = _check_tables(desc, B, block_tables, block_tables_headwise, dev)
    _check_lens_window(desc, B, seq_lens, window, dev)
    out, odt = _out_for(out, (B, Hq, D), out_dtype, dev)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    d = desc.c()
    with torch.cuda.device(dev):
        _check(_lib.load().kvq_paged_decode_attention_noalloc(
            ctypes.byref(d), _ptr(out), odt, _ptr(query), int(B), int(Hq),
            _ptr(k_codes), _ptr(k_meta), _ptr(v_codes), _ptr(v_meta),
            _ptr(block_tables), _ptr(block_tables_headwise), max_blocks,
            _ptr(seq_lens), int(max_seq_len), _ptr(window), int(sink_size), float(softmax_scale), _stream(dev)))
    return out


def kvq_decode_step(desc: CacheDesc, query: torch.Tensor, key: torch.Tensor, value: torch.Tensor,
                    k_codes: torch.Tensor, k_meta: torch.Tensor,
                    v_codes: torch.Tensor, v_meta: torch.Tensor,
                    seq_lens: torch.Tensor, max_seq_len: int,
                    slot_mapping: Optional[torch.Tensor] = None,
                    slot_mapping_headwise: Optional[torch.Tensor] = None,
                    block_tables: Optional[torch.Tensor] = None,
                    block_tables_headwise: Optional[torch.Tensor] = None,
                    window: Optional[torch.Tensor] = None,
                    softmax_scale: Optional[float] = None,
                    out: Optional[torch.Tensor] = None,
                    out_dtype: torch.dtype = torch.float32,
                    workspace: Optional[torch.Tensor] = None,
                    num_workgroups: int = 0, sink_size: int = 0) -> torch.Tensor:
    """One decode step in one launch: quantize-on-write of each sequence's
    new token (key/value [B, Hkv, D] bf16, token b at slot_mapping[b], which
    must be position seq_lens[b] - 1 of sequence b's table), then decode
    attention of query [B, Hq, D]; returns out [B, Hq, D]."""
    dev = _check_query(desc, query)
    B, Hq, D = query.shape
    for t, n in ((key, "key"), (value, "value")):
        _need(t, n, torch.bfloat16, dev, contiguous=False)
        if t.dim() != 3 or tuple(t.shape) != (B, desc.num_kv_heads, D) or t.stride(2) != 1 \
                or t.stride(1) != desc.head_dim:
            raise ValueError(f"{n} must be [{B}, {desc.num_kv_heads}, {D}] with heads and D contiguous")
    _need(slot_mapping, "slot_mapping", torch.int64, dev)
    _need(slot_mapping_headwise, "slot_mapping_headwise", torch.int64, dev)
    if slot_mapping is not None and tuple(slot_mapping.shape) != (B,):
        raise ValueError(f"slot_mapping must be [{B}]")
    if slot_mapping_headwise is not None and tuple(slot_mapping_headwise.shape) != (B, desc.num_kv_heads):
        raise ValueError(f"slot_mapping_headwise must be [{B}, {desc.num_kv_heads}]")
    _check_planes(desc, k_codes, k_meta, v_codes, v_meta)
    max_blocks = _check_tables(desc, B, block_tables, block_tables_headwise, dev)
    _check_lens_window(desc, B, seq_lens, window, dev)
    out, odt = _out_for(out, (B, Hq, D), out_dtype, dev)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    if workspace is None:
        workspace = alloc_workspace(kvq_decode_workspace_size(desc, B, Hq, max_seq_len, num_workgroups), dev)
    _need(workspace, "workspace", torch.uint8, dev)
    d = desc.c()
    _check(_lib.load().kvq_decode_step(
        ctypes.byref(d), _ptr(out), odt, _ptr(query), int(B), int(Hq),
        _ptr(key), _ptr(value), key.stride(0), value.stride(0),
        _ptr(slot_mapping), _ptr(slot_mapping_headwise),
        _ptr(k_codes), _ptr(k_meta), _ptr(v_codes), _ptr(v_meta),
        _ptr(block_tables), _ptr(block_tables_headwise), max_blocks,
        _ptr(seq_lens), int(max_seq_len), _ptr(window), int(sink_size), float(softmax_scale), _opts(num_workgroups),
        _ptr(workspace), workspace.numel(), _stream(dev)))
    return out


def kvq_paged_prefill_attention(desc: CacheDesc, query: torch.Tensor, cu_seqlens_q: torch.Tensor,
                                max_q_len: int,
                                k_codes: torch.Tensor, k_meta: torch.Tensor,
                                v_codes: torch.Tensor, v_meta: torch.Tensor,
                                seq_lens: torch.Tensor, max_seq_len: int,
                                block_tables: Optional[torch.Tensor] = None,
                                block_tables_headwise: Optional[torch.Tensor] = None,
                                window: Optional[torch.Tensor] = None,
                                softmax_scale: Optional[float] = None,
                                out: Optional[torch.Tensor] = None,
                                out_dtype: torch.dtype = torch.float32,
                                workspace: Optional[torch.Tensor] = None, sink_size: int = 0) -> torch.Tensor:
    """Chunked-prefill attention for query [total_q, Hq, D] (bf16) with
    sequence b owning rows cu_seqlens_q[b]..cu_seqlens_q[b+1]-1; returns out
    [total_q, Hq, D]."""
    dev = _check_query(desc, query)
    Tq, Hq, D = query.shape
    _need(cu_seqlens_q, "cu_seqlens_q", torch.int32, dev)
    B = int(seq_lens.shape[0])
    if cu_seqlens_q.shape[0] != B + 1:
        raise KvqError(1, f"cu_seqlens_q has {cu_seqlens_q.shape[0]} entries, {B + 1} expected")
    _check_planes(desc, k_codes, k_meta, v_codes, v_meta)
    max_blocks = _check_tables(desc, B, block_tables, block_tables_headwise, dev)
    _check_lens_window(desc, B, seq_lens, window, dev)
    out, odt = _out_for(out, (Tq, Hq, D), out_dtype, dev)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    need = kvq_prefill_workspace_size(desc, B, Hq, max_q_len, max_seq_len)
    if workspace is None and need:
        workspace = alloc_workspace(need, dev)
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8, dev)
    d = desc.c()
    _check(_lib.load().kvq_paged_prefill_attention(
        ctypes.byref(d), _ptr(out), odt, _ptr(query), _ptr(cu_seqlens_q), B, int(Hq), int(max_q_len),
        _ptr(k_codes), _ptr(k_meta), _ptr(v_codes), _ptr(v_meta),
        _ptr(block_tables), _ptr(block_tables_headwise), max_blocks,
        _ptr(seq_lens), int(max_seq_len), _ptr(window), int(sink_size), float(softmax_scale),
        _ptr(workspace), 0 if workspace is None else workspace.numel(), _stream(dev)))
    return out


def kvq_gather_dequant(desc: CacheDesc, k_codes: torch.Tensor, k_meta: torch.Tensor,
                       v_codes: torch.Tensor, v_meta: torch.Tensor,
                       cu_seq_lens: torch.Tensor, max_seq_len: int, total_tokens: int,
                       block_tables: Optional[torch.Tensor] = None,
                       block_tables_headwise: Optional[torch.Tensor] = None,
                       key_out: Optional[torch.Tensor] = None,
                       value_out: Optional[torch.Tensor] = None,
                       out_dtype: torch.dtype = torch.bfloat16):
    """Dequantized, un-rotated K and V [total_tokens, Hkv, D] of the
    sequences' positions 0 .. n_b - 1 (n_b = cu_seq_lens[b+1] -
    cu_seq_lens[b]) at rows cu_seq_lens[b] ..; evicted positions are zero.
    Returns (key_out, value_out)."""
    dev = _check_planes(desc, k_codes, k_meta, v_codes, v_meta)
    _need(cu_seq_lens, "cu_seq_lens", torch.int32, dev)
    _check_tables(desc, int(cu_seq_lens.shape[0]) - 1, block_tables, block_tables_headwise, dev)
    shape = (int(total_tokens), desc.num_kv_heads, desc.head_dim)
    if key_out is None:
        key_out = torch.empty(shape, dtype=out_dtype, device=dev)
    if value_out is None:
        value_out = torch.empty(shape, dtype=key_out.dtype, device=dev)
    for t, n in ((key_out, "key_out"), (value_out, "value_out")):
        _need(t, n, key_out.dtype, dev)
        if tuple(t.shape) != shape:
            raise ValueError(f"{n} must be {shape}, got {tuple(t.shape)}")
    odt = {torch.float32: KVQ_OUT_F32, torch.bfloat16: KVQ_OUT_BF16}[key_out.dtype]
    tab = block_tables if block_tables is not None else block_tables_headwise
    max_blocks = int(tab.shape[1]) if tab is not None else 0
    B = int(cu_seq_lens.shape[0]) - 1
    d = desc.c()
    _check(_lib.load().kvq_gather_dequant(
        ctypes.byref(d), _ptr(key_out), _ptr(value_out), odt,
        _ptr(k_codes), _ptr(k_meta), _ptr(v_codes), _ptr(v_meta),
        _ptr(block_tables), _ptr(block_tables_headwise), max_blocks,
        _ptr(cu_seq_lens), B, int(total_tokens), int(max_seq_len), _stream(dev)))
    return key_out, value_out
