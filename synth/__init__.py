"""Seeded synthetic workloads for the quantized paged KV cache.

This module only draws inputs: K/V/Q values, sequence lengths, block tables,
slot mappings, rotation signs and poison.  It holds none of the method's
arithmetic (no rotation, quantization, packing or attention), so both the HIP
path and the CPU oracle can consume the same tensors.

Workloads (the shapes and value distributions of the pages' serving setups,
drawn synthetically because the pages' models and datasets are not used):

  1  tiny INT4 + rotation: B=2, Hq/Hkv=4/2, D=64, block 16, L={37,100}
  2  INT8 symmetric: B=32, 32/8, D=128, block 64, L~U[1024,8192], 4 outlier
     channels per kv head (separately for K and V) scaled x10
  3  INT4 + rotation: B=96, 20/4, D=128, block 64, L~U[8192,32768],
     per-(kv head, channel) offsets ~N(0, 0.5) (separately for K and V)
  4  INT2 + rotation: B=4, L=131072, 32/8, D=128, block 64, 48 layer buffers
  5  INT4 + rotation mixed step: 16 prefill sequences x 512 new tokens
     (context 32768 at the end of the step) + 80 decode sequences
     (context 32768), 16/4, D=128, block 64; kv heads 0,1 use a 4096 window
     and a head-wise block table whose blocks wholly before the earliest window
     start are -1; kv heads 2,3 see the full context.

Random streams: small host-side draws use numpy ``default_rng([cfg, stream])``
with streams 0 lens, 1 K, 2 V, 3 Q, 4 signs, 5 block permutation, 6 outlier
picks, 7 offsets.  K/V/Q values are drawn with ``torch.Generator`` seeded from
(cfg, stream) on the device that will hold them; fp32 draws are rounded to
bf16 (round-to-nearest-even).
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional

import numpy as np
import torch

INT8_SYM, INT4_ASYM, INT2_ASYM = 0, 1, 2
INT8_CHANNEL = 3
FP8_E4M3 = 4
INT4_INLINE = 5
_BITS = {INT8_SYM: 8, INT4_ASYM: 4, INT2_ASYM: 2, INT8_CHANNEL: 8, FP8_E4M3: 8, INT4_INLINE: 4}
_META = {INT8_SYM: 1, INT4_ASYM: 2, INT2_ASYM: 2, INT8_CHANNEL: 0, FP8_E4M3: 1, INT4_INLINE: 0}

S_LENS, S_K, S_V, S_Q, S_SIGNS, S_PERM, S_OUTLIER, S_OFFSET = range(8)


@dataclasses.dataclass
class Spec:
    name: str
    cfg: int                      # seed namespace
    B: int
    Hq: int
    Hkv: int
    D: int
    bs: int
    mode: int
    rotate: bool
    lens: Optional[List[int]] = None        # explicit lengths, or
    len_range: Optional[tuple] = None       # inclusive uniform integer range
    outliers: int = 0                       # outlier channels per kv head (x10)
    offset_sigma: float = 0.0               # per-(head, channel) offset std
    window: Optional[List[int]] = None      # per kv head, <=0 = full
    headwise: bool = False                  # head-wise block table + slot map
    evict_outside_window: bool = False      # -1 for blocks wholly before window
    spare_frac: float = 0.10
    min_spare: int = 2
    layers: int = 1
    # mixed step (prefill part): number of prefill sequences among the B and
    # their new-token count; the remaining B - n_prefill sequences decode.
    n_prefill: int = 0
    prefill_new: int = 0


CONFIGS = {
    1: Spec("tiny-int4-rht", 1, B=2, Hq=4, Hkv=2, D=64, bs=16, mode=INT4_ASYM,
            rotate=True, lens=[37, 100]),
    2: Spec("int8-sym-b32", 2, B=32, Hq=32, Hkv=8, D=128, bs=64, mode=INT8_SYM,
            rotate=False, len_range=(1024, 8192), outliers=4),
    3: Spec("int4-rht-b96", 3, B=96, Hq=20, Hkv=4, D=128, bs=64, mode=INT4_ASYM,
            rotate=True, len_range=(8192, 32768), offset_sigma=0.5),
    4: Spec("int2-rht-131k", 4, B=4, Hq=32, Hkv=8, D=128, bs=64, mode=INT2_ASYM,
            rotate=True, lens=[131072] * 4, layers=48),
    5: Spec("int4-mixed-step", 5, B=96, Hq=16, Hkv=4, D=128, bs=64, mode=INT4_ASYM,
            rotate=True, lens=[32768] * 96, window=[4096, 4096, 0, 0],
            headwise=True, evict_outside_window=True, n_prefill=16, prefill_new=512),
}


def rng(cfg: int, stream: int) -> np.random.Generator:
    return np.random.default_rng([cfg, stream])


def torch_gen(cfg: int, stream: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(cfg) * 1000003 + int(stream) * 7919 + 12345)
    return g


def seq_lens_of(spec: Spec) -> np.ndarray:
    if spec.lens is not None:
        assert len(spec.lens) == spec.B
        return np.asarray(spec.lens, np.int64)
    lo, hi = spec.len_range
    return rng(spec.cfg, S_LENS).integers(lo, hi + 1, size=spec.B).astype(np.int64)


def new_tokens_of(spec: Spec) -> np.ndarray:
    """Tokens each sequence appends in the step: prefill_new for the first
    n_prefill sequences, 1 for the others (decode)."""
    n = np.ones(spec.B, np.int64)
    n[:spec.n_prefill] = spec.prefill_new
    return n


def rot_signs(spec: Spec) -> Optional[np.ndarray]:
    if not spec.rotate:
        return None
    return np.where(rng(spec.cfg, S_SIGNS).integers(0, 2, size=spec.D) == 1, 1.0, -1.0).astype(np.float32)


def window_of(spec: Spec) -> Optional[np.ndarray]:
    if spec.window is None:
        return None
    return np.asarray(spec.window, np.int32)


def _first_kept_block(spec: Spec, h: int, L: int, n_new: int) -> int:
    """Blocks wholly before the earliest window start of (seq, head) get -1.
    The earliest query of the step sits at position L - n_new; its window
    starts at L - n_new - W + 1."""
    if not spec.evict_outside_window or spec.window is None or spec.window[h] <= 0:
        return 0
    start = max(0, L - n_new - spec.window[h] + 1)
    return start // spec.bs


@dataclasses.dataclass
class Tables:
    num_blocks: int
    max_blocks: int
    block_tables: Optional[np.ndarray]            # int32 [B, max_blocks]
    block_tables_headwise: Optional[np.ndarray]   # int32 [B*Hkv, max_blocks]
    used: np.ndarray                              # bool [num_blocks, Hkv]


def make_tables(spec: Spec, seq_lens: np.ndarray) -> Tables:
    """Random block-id permutation.  Uniform table: one id per (seq, logical
    block), shared by all kv heads.  Head-wise table: each kv head draws its
    own permutation over the same id range; evicted blocks are -1.  Physical
    blocks = needed + max(spare_frac, min_spare) spares (never referenced)."""
    r = rng(spec.cfg, S_PERM)
    nblk = [(int(L) + spec.bs - 1) // spec.bs for L in seq_lens]
    max_blocks = max(1, max(nblk))
    n_new = new_tokens_of(spec)
    if not spec.headwise:
        need = sum(nblk)
        nb = need + max(int(math.ceil(need * spec.spare_frac)), spec.min_spare)
        perm = r.permutation(nb)[:need]
        bt = np.full((spec.B, max_blocks), -1, np.int32)
        used = np.zeros((nb, spec.Hkv), bool)
        k = 0
        for b, n in enumerate(nblk):
            bt[b, :n] = perm[k:k + n]
            k += n
        used[perm, :] = True
        return Tables(nb, max_blocks, bt, None, used)
    kept = np.zeros((spec.B, spec.Hkv), np.int64)
    first = np.zeros((spec.B, spec.Hkv), np.int64)
    for b, n in enumerate(nblk):
        for h in range(spec.Hkv):
            f = min(_first_kept_block(spec, h, int(seq_lens[b]), int(n_new[b])), n)
            first[b, h] = f
            kept[b, h] = n - f
    need = int(kept.sum(axis=0).max())
    nb = need + max(int(math.ceil(need * spec.spare_frac)), spec.min_spare)
    bth = np.full((spec.B * spec.Hkv, max_blocks), -1, np.int32)
    used = np.zeros((nb, spec.Hkv), bool)
    for h in range(spec.Hkv):
        perm = r.permutation(nb)
        k = 0
        for b, n in enumerate(nblk):
            f = int(first[b, h])
            cnt = n - f
            bth[b * spec.Hkv + h, f:n] = perm[k:k + cnt]
            used[perm[k:k + cnt], h] = True
            k += cnt
    return Tables(nb, max_blocks, None, bth, used)


def slots_for(spec: Spec, tables: Tables, seq_idx: np.ndarray, pos: np.ndarray):
    """Slot of each (token, kv head): block id of the token's logical block
    times block size plus its offset; -1 where the block is evicted.  Returns
    (slot_mapping [T] or None, slot_mapping_headwise [T, Hkv] or None)."""
    lb = pos // spec.bs
    off = pos % spec.bs
    if tables.block_tables is not None:
        ids = tables.block_tables[seq_idx, lb].astype(np.int64)
        return np.where(ids >= 0, ids * spec.bs + off, -1).astype(np.int64), None
    rows = seq_idx[:, None] * spec.Hkv + np.arange(spec.Hkv)[None, :]
    ids = tables.block_tables_headwise[rows, lb[:, None]].astype(np.int64)
    return None, np.where(ids >= 0, ids * spec.bs + off[:, None], -1).astype(np.int64)


def bf16_normal(shape, cfg: int, stream: int, device, mean=0.0, std=1.0) -> torch.Tensor:
    g = torch_gen(cfg, stream, device)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    if mean != 0.0:
        x.add_(mean)
    return x.to(torch.bfloat16)


def kv_values(spec: Spec, T: int, which: int, device, layer: int = 0) -> torch.Tensor:
    """bf16 [T, Hkv, D] values of K (which=S_K) or V (which=S_V): N(0,1), plus
    the workload's outlier channels (x10) or per-channel offsets.  ``layer``
    selects an independent draw for multi-layer buffers."""
    g = torch_gen(spec.cfg, which + 100 * layer, device)
    x = torch.randn((T, spec.Hkv, spec.D), generator=g, device=device, dtype=torch.float32)
    if spec.outliers:
        r = rng(spec.cfg, S_OUTLIER)
        picks = np.stack([r.choice(spec.D, size=spec.outliers, replace=False)
                          for _ in range(2 * spec.Hkv)]).reshape(2, spec.Hkv, spec.outliers)
        mult = torch.ones((spec.Hkv, spec.D), device=device)
        for h in range(spec.Hkv):
            mult[h, torch.as_tensor(picks[which - S_K, h], device=device)] = 10.0
        x.mul_(mult)
    if spec.offset_sigma:
        r = rng(spec.cfg, S_OFFSET)
        offs = r.normal(0.0, spec.offset_sigma, size=(2, spec.Hkv, spec.D)).astype(np.float32)
        x.add_(torch.as_tensor(offs[which - S_K], device=device))
    return x.to(torch.bfloat16)


@dataclasses.dataclass
class Case:
    """Everything one workload needs, as torch tensors on ``device``.

    ``k``, ``v`` [T, Hkv, D] hold every cached token of every sequence
    (positions 0..L_b-1, sequence-major), with ``tok_seq`` / ``tok_pos`` and
    their slots; ``q`` [B, Hq, D] is one decode query per sequence; for the
    mixed step, ``q_prefill`` [sum n_new, Hq, D] with ``cu_seqlens_q``.
    """
    spec: Spec
    seq_lens: torch.Tensor
    tables: Tables
    block_tables: Optional[torch.Tensor]
    block_tables_headwise: Optional[torch.Tensor]
    window: Optional[torch.Tensor]
    rot_signs: Optional[torch.Tensor]
    k: torch.Tensor
    v: torch.Tensor
    tok_seq: np.ndarray
    tok_pos: np.ndarray
    slot_mapping: Optional[torch.Tensor]
    slot_mapping_headwise: Optional[torch.Tensor]
    q: torch.Tensor
    softmax_scale: float
    q_prefill: Optional[torch.Tensor] = None
    cu_seqlens_q: Optional[torch.Tensor] = None


def make_case(spec: Spec, device="cpu", *, with_kv: bool = True, layer: int = 0) -> Case:
    """Build a workload.  K/V of every cached position are drawn (with_kv);
    the caller writes them into a poisoned cache and then attends."""
    lens = seq_lens_of(spec)
    tables = make_tables(spec, lens)
    tok_seq = np.repeat(np.arange(spec.B), lens)
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]])
    tok_pos = np.arange(int(lens.sum())) - np.repeat(starts, lens)
    sm, smh = slots_for(spec, tables, tok_seq, tok_pos)
    T = int(lens.sum())
    dev = torch.device(device)
    k = kv_values(spec, T, S_K, dev, layer=layer) if with_kv else None
    v = kv_values(spec, T, S_V, dev, layer=layer) if with_kv else None
    q = bf16_normal((spec.B, spec.Hq, spec.D), spec.cfg, S_Q + 100 * layer, dev)
    signs = rot_signs(spec)
    win = window_of(spec)
    n_new = new_tokens_of(spec)
    qp = cu = None
    if spec.n_prefill:
        nq = int(n_new[:spec.n_prefill].sum())
        qp = bf16_normal((nq, spec.Hq, spec.D), spec.cfg, S_Q + 50, dev)
        cu = torch.as_tensor(np.concatenate([[0], np.cumsum(n_new[:spec.n_prefill])]).astype(np.int32),
                             device=dev)
    return Case(
        spec=spec,
        seq_lens=torch.as_tensor(lens.astype(np.int32), device=dev),
        tables=tables,
        block_tables=None if tables.block_tables is None else torch.as_tensor(tables.block_tables, device=dev),
        block_tables_headwise=None if tables.block_tables_headwise is None
        else torch.as_tensor(tables.block_tables_headwise, device=dev),
        window=None if win is None else torch.as_tensor(win, device=dev),
        rot_signs=None if signs is None else torch.as_tensor(signs, device=dev),
        k=k, v=v, tok_seq=tok_seq, tok_pos=tok_pos,
        slot_mapping=None if sm is None else torch.as_tensor(sm, device=dev),
        slot_mapping_headwise=None if smh is None else torch.as_tensor(smh, device=dev),
        q=q, softmax_scale=1.0 / math.sqrt(spec.D), q_prefill=qp, cu_seqlens_q=cu)


def poison_(codes: torch.Tensor, meta: torch.Tensor) -> None:
    """Fill a cache plane pair with poison: 0xFF code bytes, NaN metadata."""
    codes.fill_(0xFF)
    meta.fill_(float("nan"))


def small_spec(**kw) -> Spec:
    """A parity-size workload: defaults are a few tiles with a ragged tail."""
    base = dict(name="small", cfg=100, B=3, Hq=8, Hkv=2, D=128, bs=64, mode=INT4_ASYM,
                rotate=True, lens=[1, 130, 301])
    if "len_range" in kw and "lens" not in kw:
        base["lens"] = None
    base.update(kw)
    return Spec(**base)
