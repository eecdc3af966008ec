"""CPU oracle for the dynamically quantized paged KV cache and the attention
that reads it.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module. The HIP library
(``sub_byte_quantized_amd``) never imports, links or calls anything here, and
nothing here imports it.

Plain numpy. The quantize-on-write steps are an *encoding*, so they are written
as the method's steps in order, in float32 (the precision the codes are decided
in on both sides). Attention has a plain definition (softmax attention over the
dequantized, un-rotated keys and values), so it is that definition written out
in float64.

Sources (web pages; cited by title and section):

* [P1] FastDeploy PR 5173, "[Feature] support dynamic int2 quantization cache
  kv" -- sections "Motivation" and the pull-request overview: a 2-bit KV cache
  whose scales are computed at run time, written by an encoder/decoder cache
  write kernel and read by an attention kernel.
* [P2] prhub summary of vLLM PR 40835, "INT4 per-token-head KV cache
  quantization for the Triton backend" -- sections 功能与动机 (motivation:
  two 4-bit values per byte, randomized Hadamard transform, asymmetric
  quantization with a zero point), 实现拆解 (implementation: the write kernel
  applies the RHT, computes one scale and zero point per token and head, and
  packs nibbles; the read kernel unpacks, dequantizes and attends), 关键源码片段
  (the cache shape snippet).
* [P3] FastDeploy PR 7718, "Optimize AppendAttention for discrete head-wise
  block_idx" -- sections Motivation (head-wise block table, logical
  [batch, kv_head, block], physical [batch*kv_heads, max_blocks]) and
  Modifications / correctness gates (-1 marks an evicted sliding-window block;
  such rows are skipped before any K/V pointer is formed).
* [P4] vllm-ascend-quantized-kv-cache 0.2.0rc2 package description, section
  运行机制 (decode dequantizes inside attention; prefill gathers and
  dequantizes the paged cache).
* [P5] FastDeploy PR 7757, "fix cache_manager_v1 allocating kv cache with wrong
  dtype" -- section 修复: every quantized cache is stored as uint8.

Readings where the pages are silent (each also listed in the design doc):

* INT4/INT2 codes are unsigned in [0, L], L = 2^b - 1; the zero point is the
  real-valued row minimum, x_hat = c*s + z.  INT8 is symmetric, s = absmax/127,
  codes in [-127, 127] stored as two's complement bytes.
* Rounding is round-half-to-even (np.rint); s and 1/s are correctly rounded
  float32 divisions; (y - z) and the product by 1/s are separate float32 ops.
* A row whose scale is zero, subnormal or NaN gets all-zero codes.
* The rotation is y = (1/sqrt(D)) * H_D * (d (.) x), H_D the Sylvester Hadamard
  matrix in natural order, d the caller's +-1 signs; K and V are both rotated,
  and the attention output is rotated back once.
* Element 2j of a row goes to the low nibble of byte j; for INT2 element 4j+k
  goes to bits 2k..2k+1 of byte j.
* A token position p of sequence b attends (decode) to positions j < L_b that
  lie in a non-evicted block and, for a windowed kv head, j >= L_b - W.
  kv head = q head // (Hq/Hkv).  An empty allowed set gives output 0.
* Dynamic per-channel INT8 ([P4] 运行机制: the INT8 scales are computed along
  the token axis the first time a layer receives K/V, symmetric, per channel,
  separately for K and V): s[h, d] = max_t |x[t, h, d]| / 127 over that first
  batch, in float32; every row written later is quantized with those fixed
  scales, c = clamp(rint(x * fl(1/s_d)), -127, 127) (values beyond the
  calibrated range saturate), a channel with a zero or subnormal scale gets
  code 0, and x_hat = c * s_d.  No rotation and no per-token metadata.
* FP8 per-token-head ([P2] 功能与动机: the INT8/FP8 per-token-head schemes the
  INT4 mode extends): OCP E4M3 codes (1 sign, 4 exponent bits with bias 7, 3
  mantissa bits, no infinities, largest finite 448, subnormal step 2^-9),
  symmetric per (token, kv head): s = max|y| / 448, t = clamp(y * fl(1/s),
  -448, 448) in float32, code = t rounded to the nearest E4M3 value, ties to
  even; x_hat = E4M3(code) * s.  The same optional rotation as INT4/INT2.
* Attention sinks ([P3] Modifications: a sink_size parameter threaded into the
  attention op, semantics unstated): a windowed kv head also attends the
  first sink_size positions of the sequence (when present in the table), as
  in sliding-window attention with sink tokens; heads without a window see
  everything anyway.
* INT4 inline layout ([P2] 关键源码片段: the cache shape (num_blocks, 2,
  block_size, num_kv_heads, head_size // 2 + scale_pad) with the float32
  scale in the last 4 bytes of each row; 评论区精华: the 4-bit zero point is
  kept in the scale's low 4 bits).  One uint8 tensor [nb, 2, bs, Hkv, D/2 +
  4], index 1 = 0 for K and 1 for V; row = D/2 nibble bytes (INT4 order)
  then the 4 little-endian bytes of the stored scale st.  The zero point is
  an integer zp in [0, 15] (the textbook asymmetric scheme, zero exactly
  representable): mn = min(min y, 0), mx = max(max y, 0) in float32, s =
  (mx - mn) / 15, zp = clamp(rint(-mn / s), 0, 15), st = the float32 whose
  bits are those of s with the low 4 replaced by zp (|st - s| <= 15 ulp(s),
  so st is the scale a reader that ignores the zero point still gets), then
  c = clamp(rint(y * fl(1/st)) + zp, 0, 15) and x_hat = (c - zp) * st.  A
  row whose s is zero, subnormal or NaN stores st = 0 and codes 0.  The
  same optional rotation as INT4.
"""
from __future__ import annotations

import math

import numpy as np

INT8_SYM = 0
INT4_ASYM = 1
INT2_ASYM = 2
INT8_CHANNEL = 3
FP8_E4M3 = 4
INT4_INLINE = 5
MODES = (INT8_SYM, INT4_ASYM, INT2_ASYM)          # the integer per-token-head modes
BITS = {INT8_SYM: 8, INT4_ASYM: 4, INT2_ASYM: 2, INT8_CHANNEL: 8, FP8_E4M3: 8, INT4_INLINE: 4}
# number of quantization steps: codes span [0, L] (asymmetric) or [-L, L]
LEVELS = {INT8_SYM: 127, INT4_ASYM: 15, INT2_ASYM: 3, INT8_CHANNEL: 127}
# meta floats in a separate plane (the inline layout keeps its scale in the row)
META_FLOATS = {INT8_SYM: 1, INT4_ASYM: 2, INT2_ASYM: 2, INT8_CHANNEL: 0, FP8_E4M3: 1, INT4_INLINE: 0}
INLINE_LEVELS = 15
E4M3_MAX = 448.0

_F32 = np.float32
_FLT_MIN = _F32(2.0 ** -126)


# --------------------------------------------------------------------------
# Layout  ([P2] 关键源码片段: the packed row holds head_size*b/8 code bytes;
#          [P5] 修复: storage dtype is uint8 for every quantized mode)
# --------------------------------------------------------------------------
def row_code_bytes(mode: int, head_dim: int) -> int:
    """Packed code bytes of one (token, kv head) row: head_dim * b / 8."""
    return head_dim * BITS[mode] // 8


def plane_shapes(mode: int, head_dim: int, num_kv_heads: int, block_size: int,
                 num_blocks: int):
    """Shapes of one code plane and one meta plane (K and V each have both).

    codes: uint8 [num_blocks, Hkv, block_size, P]
    meta : float32 [num_blocks, Hkv, block_size, M], M = 1 (s) or 2 (s, z)
    """
    if mode == INT4_INLINE:
        raise ValueError("the inline layout is one tensor: inline_cache_shape")
    P = row_code_bytes(mode, head_dim)
    M = META_FLOATS[mode]
    return ((num_blocks, num_kv_heads, block_size, P),
            (num_blocks, num_kv_heads, block_size, M))


def inline_cache_shape(head_dim: int, num_kv_heads: int, block_size: int, num_blocks: int):
    """The INT4 inline cache: uint8 [num_blocks, 2 (K, V), block_size, Hkv,
    D/2 + 4] ([P2] 关键源码片段: head_size // 2 + scale_pad, scale_pad = 4
    bytes of float32 scale)."""
    return (num_blocks, 2, block_size, num_kv_heads, head_dim // 2 + 4)


# --------------------------------------------------------------------------
# Hadamard rotation ([P2] 功能与动机 / 实现拆解: RHT before quantization)
# --------------------------------------------------------------------------
def sylvester_hadamard(n: int) -> np.ndarray:
    """H[i, j] = (-1)^popcount(i & j): the Sylvester matrix in natural order."""
    assert n > 0 and n & (n - 1) == 0
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    bits = i & j
    pop = np.zeros_like(bits)
    while np.any(bits):
        pop += bits & 1
        bits >>= 1
    return np.where(pop % 2 == 0, 1, -1).astype(np.int64)


def fwht(x: np.ndarray) -> np.ndarray:
    """Unnormalized fast Walsh-Hadamard transform along the last axis.

    Stages h = 1, 2, 4, ..., D/2; each stage maps the pair (i, i+h), i with bit
    h clear, to (x_i + x_{i+h}, x_i - x_{i+h}).  Arithmetic stays in x's dtype
    (float32 for the stored-code path, float64 for checks), so the float32
    result is fully specified by this stage order.
    """
    x = np.array(x, copy=True)
    D = x.shape[-1]
    assert D & (D - 1) == 0
    lead = x.shape[:-1]
    h = 1
    while h < D:
        y = x.reshape(lead + (D // (2 * h), 2, h))
        a = y[..., 0, :]
        b = y[..., 1, :]
        x = np.stack([a + b, a - b], axis=-2).reshape(lead + (D,))
        h *= 2
    return x


def inv_sqrt_f32(D: int) -> np.float32:
    """float32 rounding of 1/sqrt(D)."""
    return _F32(1.0 / math.sqrt(D))


def rotate_f32(x: np.ndarray, signs: np.ndarray) -> np.ndarray:
    """y = fl32( FWHT32(d (.) x) * fl32(1/sqrt(D)) ), rows along the last axis.

    The sign flip is exact; the FWHT is the float32 stage sequence of fwht();
    the normalization is one float32 multiply per element.
    """
    x = np.asarray(x, dtype=_F32)
    d = np.asarray(signs, dtype=_F32)
    y = fwht(x * d)
    return (y * inv_sqrt_f32(x.shape[-1])).astype(_F32)


def rotate_dense_f64(x: np.ndarray, signs: np.ndarray) -> np.ndarray:
    """Check path: (1/sqrt(D)) * H @ (d (.) x) with a dense float64 H."""
    D = x.shape[-1]
    H = sylvester_hadamard(D).astype(np.float64)
    xd = np.asarray(x, np.float64) * np.asarray(signs, np.float64)
    return (xd @ H.T) / math.sqrt(D)


def unrotate_f64(x: np.ndarray, signs: np.ndarray) -> np.ndarray:
    """R^T x with R = (1/sqrt(D)) H diag(d):  (1/sqrt(D)) * d (.) (H x), float64."""
    x = np.asarray(x, np.float64)
    D = x.shape[-1]
    return fwht(x) * np.asarray(signs, np.float64) / math.sqrt(D)


# --------------------------------------------------------------------------
# Per-token-head quantization ([P2] 功能与动机 / 实现拆解: one scale and zero
# point per (token, head); [P1] Motivation: 2-bit codes, scales at run time)
# --------------------------------------------------------------------------
def quantize_rows(y: np.ndarray, mode: int):
    """Quantize float32 rows y [R, D] -> (codes int32 [R, D], s f32 [R], z f32 [R]).

    INT8 (symmetric): a = max|y|, s = a / 127, z = 0,
      c = clamp(rint(y * inv), -127, 127) with inv = 1/s.
    INT4 / INT2 (asymmetric): mn = min y, mx = max y, s = (mx - mn) / L,
      z = mn, c = clamp(rint((y - mn) * inv), 0, L).
    Rows with s == 0, subnormal s or NaN s get all-zero codes.
    """
    y = np.asarray(y, dtype=_F32)
    L = _F32(LEVELS[mode])
    if mode == INT8_SYM:
        a = np.max(np.abs(y), axis=-1)
        s = (a / L).astype(_F32)
        z = np.zeros_like(s)
        base = y
        lo, hi = -LEVELS[mode], LEVELS[mode]
    else:
        mn = np.min(y, axis=-1)
        mx = np.max(y, axis=-1)
        s = ((mx - mn) / L).astype(_F32)
        z = mn.astype(_F32)
        base = (y - mn[..., None]).astype(_F32)
        lo, hi = 0, LEVELS[mode]
    ok = s >= _FLT_MIN  # False for 0, subnormal and NaN
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        inv = np.where(ok, _F32(1.0) / np.where(ok, s, _F32(1.0)), _F32(0.0)).astype(_F32)
        t = (base * inv[..., None]).astype(_F32)
    c = np.clip(np.rint(t), lo, hi)
    c = np.where(ok[..., None], c, 0).astype(np.int32)
    return c, s, z


def dequant_rows_f64(codes: np.ndarray, s: np.ndarray, z: np.ndarray) -> np.ndarray:
    """x_hat = c * s + z in float64 (z = 0 for INT8)."""
    return (np.asarray(codes, np.float64) * np.asarray(s, np.float64)[..., None]
            + np.asarray(z, np.float64)[..., None])


# --------------------------------------------------------------------------
# Packing ([P2] 实现拆解: pack/unpack of 4-bit values, two per byte;
#          [P1]: 2-bit codes, four per byte)
# --------------------------------------------------------------------------
def pack_codes(codes: np.ndarray, mode: int) -> np.ndarray:
    """codes [..., D] -> uint8 [..., D*b/8]."""
    c = np.asarray(codes, np.int64)
    if BITS[mode] == 8:
        return (c & 0xFF).astype(np.uint8)
    b = BITS[mode]
    per = 8 // b
    D = c.shape[-1]
    g = (c & ((1 << b) - 1)).reshape(c.shape[:-1] + (D // per, per))
    out = np.zeros(g.shape[:-1], dtype=np.int64)
    for k in range(per):
        out |= g[..., k] << (b * k)
    return out.astype(np.uint8)


def unpack_codes(packed: np.ndarray, mode: int, head_dim: int) -> np.ndarray:
    """uint8 [..., D*b/8] -> int32 codes [..., D] (INT8 sign-extended)."""
    p = np.asarray(packed, np.uint8).astype(np.int64)
    if BITS[mode] == 8:
        return np.where(p >= 128, p - 256, p).astype(np.int32)
    b = BITS[mode]
    per = 8 // b
    parts = [(p >> (b * k)) & ((1 << b) - 1) for k in range(per)]
    out = np.stack(parts, axis=-1).reshape(p.shape[:-1] + (p.shape[-1] * per,))
    assert out.shape[-1] == head_dim
    return out.astype(np.int32)


# --------------------------------------------------------------------------
# FP8 (OCP E4M3) per-token-head ([P2] 功能与动机: INT8/FP8 per-token-head)
# --------------------------------------------------------------------------
def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """Value of each E4M3 byte (float64): exponent field e, mantissa m, sign s;
    e > 0: (-1)^s 2^(e-7) (1 + m/8); e = 0: (-1)^s 2^-6 m/8; 0x7F / 0xFF: NaN."""
    c = np.asarray(codes, np.int64)
    sgn = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    v = np.where(e > 0, np.ldexp(1.0 + m / 8.0, e - 7), np.ldexp(m / 8.0, -6))
    v = sgn * v
    return np.where((c & 0x7F) == 0x7F, np.nan, v)


def e4m3_encode(t: np.ndarray) -> np.ndarray:
    """Nearest E4M3 byte to each finite |t| <= 448 (ties to even mantissa;
    -0 keeps its sign bit).  Below 2^-6 the grid is 2^-9 (subnormals);
    above, 8 steps per binade.  Computed in float64, where every step here is
    exact."""
    t = np.asarray(t, np.float64)
    assert np.all(np.isfinite(t)) and np.all(np.abs(t) <= E4M3_MAX)
    a = np.abs(t)
    sub = a < 2.0 ** -6
    q_sub = np.rint(a / 2.0 ** -9)                     # 0 .. 8 (8 is the first normal)
    e = np.floor(np.log2(np.where(sub, 1.0, a)))
    # log2 may be off by one ulp at exact powers of two: fix e so 2^e <= a < 2^(e+1)
    e = np.where(np.ldexp(1.0, e.astype(np.int64)) > a, e - 1, e)
    e = np.where(np.ldexp(1.0, (e + 1).astype(np.int64)) <= a, e + 1, e)
    q = np.rint(a / np.ldexp(1.0, (e - 3).astype(np.int64)))   # 8 .. 16
    e = np.where(q == 16, e + 1, e)
    q = np.where(q == 16, 8, q)
    normal = ((e + 7).astype(np.int64) << 3) | (q.astype(np.int64) - 8)
    code = np.where(sub, q_sub.astype(np.int64), normal)
    code = np.where(np.signbit(t), code | 0x80, code)
    return code.astype(np.uint8)


def quantize_rows_fp8(y: np.ndarray):
    """FP8 rows y [R, D] float32 -> (codes uint8 [R, D], s f32 [R]):
    s = max|y| / 448, t = clamp(y * fl(1/s), -448, 448) in float32, codes
    the nearest E4M3 values; rows with a zero, subnormal or NaN scale get
    code 0."""
    y = np.asarray(y, _F32)
    a = np.max(np.abs(y), axis=-1)
    s = (a / _F32(E4M3_MAX)).astype(_F32)
    ok = s >= _FLT_MIN
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        inv = np.where(ok, _F32(1.0) / np.where(ok, s, _F32(1.0)), _F32(0.0)).astype(_F32)
        t = (y * inv[..., None]).astype(_F32)
    t = np.clip(np.where(ok[..., None], t, _F32(0.0)), -E4M3_MAX, E4M3_MAX)
    codes = e4m3_encode(t)
    return np.where(ok[..., None], codes, np.uint8(0)).astype(np.uint8), s


# --------------------------------------------------------------------------
# Dynamic per-channel INT8 ([P4] 运行机制: scales from the first K/V a layer
# receives, along the token axis, symmetric, per channel, K and V separately)
# --------------------------------------------------------------------------
def calibrate_channel_scales(x: np.ndarray) -> np.ndarray:
    """Scales of one of K or V from the first batch x [T, Hkv, D] (float32
    images of bf16): s[h, d] = max_t |x[t, h, d]| / 127, one correctly rounded
    float32 division."""
    a = np.max(np.abs(np.asarray(x, _F32)), axis=0)
    return (a / _F32(127.0)).astype(_F32)


def quantize_rows_channel(y: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Codes of rows y [R, D] against fixed per-channel scales [D] (or [R, D]):
    c = clamp(rint(y * fl(1/s)), -127, 127) in float32; a channel whose scale
    is zero, subnormal or NaN gets code 0."""
    y = np.asarray(y, _F32)
    s = np.broadcast_to(np.asarray(scales, _F32), y.shape)
    ok = s >= _FLT_MIN
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        inv = np.where(ok, _F32(1.0) / np.where(ok, s, _F32(1.0)), _F32(0.0)).astype(_F32)
        t = (y * inv).astype(_F32)
    c = np.clip(np.rint(t), -127, 127)
    return np.where(ok, c, 0).astype(np.int32)


# --------------------------------------------------------------------------
# INT4 with the zero point in the scale's low bits ([P2] 关键源码片段 and
# 评论区精华: 4-bit zero point hidden in the low 4 bits of the float32 scale)
# --------------------------------------------------------------------------
def embed_zero(s: np.ndarray, zp: np.ndarray) -> np.ndarray:
    """float32 whose bits are those of s with the low 4 replaced by zp."""
    bits = np.asarray(s, _F32).view(np.uint32)
    return ((bits & np.uint32(0xFFFFFFF0)) | np.asarray(zp, np.uint32)).astype(np.uint32).view(_F32)


def hidden_zero(st: np.ndarray) -> np.ndarray:
    """The zero point kept in a stored scale: its low 4 bits."""
    return (np.asarray(st, _F32).view(np.uint32) & np.uint32(0xF)).astype(np.int32)


def quantize_rows_inline(y: np.ndarray):
    """float32 rows y [R, D] -> (codes int32 [R, D] in [0, 15], st f32 [R]).

    mn = min(min y, 0), mx = max(max y, 0); s = (mx - mn) / 15; zp =
    clamp(rint(-mn / s), 0, 15); st = s with zp in its low 4 bits; c =
    clamp(rint(y * fl(1/st)) + zp, 0, 15).  Rows with a zero, subnormal or
    NaN s store st = 0 and codes 0."""
    y = np.asarray(y, dtype=_F32)
    mn = np.minimum(np.min(y, axis=-1), _F32(0.0)).astype(_F32)
    mx = np.maximum(np.max(y, axis=-1), _F32(0.0)).astype(_F32)
    s = ((mx - mn) / _F32(INLINE_LEVELS)).astype(_F32)
    ok = s >= _FLT_MIN
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        s1 = np.where(ok, s, _F32(1.0)).astype(_F32)
        zp = np.clip(np.rint((-mn / s1).astype(_F32)), 0, INLINE_LEVELS).astype(np.int64)
        zp = np.where(ok, zp, 0)
        st = np.where(ok, embed_zero(s1, zp), _F32(0.0)).astype(_F32)
        inv = (_F32(1.0) / np.where(ok, st, _F32(1.0))).astype(_F32)
        t = (y * inv[..., None]).astype(_F32)
    c = np.clip(np.rint(t) + zp[..., None], 0, INLINE_LEVELS)
    c = np.where(ok[..., None], c, 0).astype(np.int32)
    return c, st


def inline_rows(packed: np.ndarray, st: np.ndarray) -> np.ndarray:
    """Stored rows: the packed nibbles [R, D/2] then st's 4 little-endian bytes."""
    tail = np.asarray(st, '<f4').reshape(-1, 1).view(np.uint8)
    return np.concatenate([np.asarray(packed, np.uint8).reshape(len(tail), -1), tail], axis=1)


def dequant_inline_rows_f64(rows: np.ndarray, head_dim: int) -> np.ndarray:
    """x_hat = (c - zp) * st in float64 from stored inline rows [R, D/2 + 4]."""
    rows = np.asarray(rows, np.uint8)
    P = head_dim // 2
    codes = unpack_codes(rows[:, :P], INT4_ASYM, head_dim).astype(np.float64)
    st = np.ascontiguousarray(rows[:, P:P + 4]).view('<f4')[:, 0].astype(_F32)
    zp = hidden_zero(st).astype(np.float64)
    return (codes - zp[:, None]) * st.astype(np.float64)[:, None]


# --------------------------------------------------------------------------
# Quantize-on-write into the paged layout  ([P2] 实现拆解 item 2: RHT, then
# scale and zero per token and head, then pack and store; [P3] Motivation:
# per-head block rows)
# --------------------------------------------------------------------------
def encode_rows(x_bf16_as_f32: np.ndarray, mode: int, signs=None):
    """Steps O1-O5 on rows [R, D]: rotation (optional), stats, codes, packing.

    Returns (packed uint8 [R, P], s f32 [R], z f32 [R], codes int32 [R, D]).
    """
    x = np.asarray(x_bf16_as_f32, dtype=_F32)
    y = rotate_f32(x, signs) if signs is not None else x
    if mode == FP8_E4M3:
        codes, s = quantize_rows_fp8(y)
        return codes, s, np.zeros_like(s), codes
    if mode == INT4_INLINE:
        codes, st = quantize_rows_inline(y)
        return pack_codes(codes, INT4_ASYM), st, np.zeros_like(st), codes
    codes, s, z = quantize_rows(y, mode)
    return pack_codes(codes, mode), s, z, codes


def write_cache(k: np.ndarray, v: np.ndarray, mode: int, block_size: int,
                k_codes: np.ndarray, k_meta: np.ndarray,
                v_codes: np.ndarray, v_meta: np.ndarray,
                slot_mapping=None, slot_mapping_headwise=None, signs=None, channel_scales=None):
    """Quantize the rows of k, v [T, Hkv, D] (float32 images of bf16) and store
    them at their slots (step O6).

    slot_mapping [T] (the same slot for every kv head) or slot_mapping_headwise
    [T, Hkv]; slot = block * block_size + offset; a negative slot skips the row.
    Planes are modified in place.  INT8_CHANNEL takes channel_scales [2, Hkv, D]
    (K then V) and writes no metadata.  INT4_INLINE takes its one cache tensor
    (inline_cache_shape) as k_codes; the other three are None.
    """
    T, Hkv, D = k.shape
    if (slot_mapping is None) == (slot_mapping_headwise is None):
        raise ValueError("exactly one slot mapping")
    if slot_mapping_headwise is None:
        slots = np.repeat(np.asarray(slot_mapping, np.int64)[:, None], Hkv, axis=1)
    else:
        slots = np.asarray(slot_mapping_headwise, np.int64).reshape(T, Hkv)
    tt, hh = np.nonzero(slots >= 0)           # rows written: token tt, kv head hh
    sl = slots[tt, hh]
    blk, off = sl // block_size, sl % block_size
    for kv, (src, codes_pl, meta_pl) in enumerate(((k, k_codes, k_meta), (v, v_codes, v_meta))):
        if mode == INT8_CHANNEL:
            sc = np.asarray(channel_scales, _F32)[kv]                         # [Hkv, D]
            packed = pack_codes(quantize_rows_channel(np.asarray(src, _F32), sc[None]), mode)
            codes_pl[blk, hh, off, :] = packed[tt, hh]
            continue
        packed, s, z, _ = encode_rows(np.asarray(src, _F32).reshape(T * Hkv, D), mode, signs)
        if mode == INT4_INLINE:
            rows = inline_rows(packed, s).reshape(T, Hkv, -1)
            k_codes[blk, kv, off, hh, :] = rows[tt, hh]
            continue
        packed = packed.reshape(T, Hkv, -1)
        s = s.reshape(T, Hkv)
        z = z.reshape(T, Hkv)
        codes_pl[blk, hh, off, :] = packed[tt, hh]
        meta_pl[blk, hh, off, 0] = s[tt, hh]
        if META_FLOATS[mode] == 2:
            meta_pl[blk, hh, off, 1] = z[tt, hh]


# --------------------------------------------------------------------------
# Reading the cache back ([P4] 运行机制: gather and dequantize the paged cache;
# [P3] correctness gates: -1 rows are skipped, never dereferenced)
# --------------------------------------------------------------------------
def table_row(b: int, h: int, num_kv_heads: int, block_tables=None,
              block_tables_headwise=None) -> np.ndarray:
    """Block-id row walked by (sequence b, kv head h): the uniform row b, or the
    head-wise row b*Hkv + h."""
    if block_tables_headwise is not None:
        return np.asarray(block_tables_headwise)[b * num_kv_heads + h]
    return np.asarray(block_tables)[b]


def gather_head(b: int, h: int, n_pos: int, mode: int, head_dim: int,
                block_size: int, num_kv_heads: int,
                k_codes, k_meta, v_codes, v_meta, signs=None,
                block_tables=None, block_tables_headwise=None, channel_scales=None):
    """Dequantized, un-rotated K and V (float64 [n_pos, D]) of positions
    0..n_pos-1 of (b, h), plus a bool [n_pos] that is False for positions in an
    evicted (-1) block.  Evicted rows are returned as zeros and never read."""
    row = table_row(b, h, num_kv_heads, block_tables, block_tables_headwise)
    pos = np.arange(n_pos)
    ids = np.asarray(row, np.int64)[pos // block_size] if n_pos else np.zeros(0, np.int64)
    present = ids >= 0
    K = np.zeros((n_pos, head_dim))
    V = np.zeros((n_pos, head_dim))
    if np.any(present):
        bi = ids[present]
        off = pos[present] % block_size
        for kv, (pl_c, pl_m, out) in enumerate(((k_codes, k_meta, K), (v_codes, v_meta, V))):
            if mode == INT4_INLINE:   # one tensor, passed as k_codes
                xhat = dequant_inline_rows_f64(k_codes[bi, kv, off, h, :], head_dim)
                out[present] = unrotate_f64(xhat, signs) if signs is not None else xhat
                continue
            if mode == FP8_E4M3:
                xhat = e4m3_decode(pl_c[bi, h, off, :]) * np.asarray(pl_m[bi, h, off, 0], np.float64)[:, None]
                out[present] = unrotate_f64(xhat, signs) if signs is not None else xhat
                continue
            codes = unpack_codes(pl_c[bi, h, off, :], mode, head_dim)
            if mode == INT8_CHANNEL:
                out[present] = codes * np.asarray(channel_scales, np.float64)[kv, h][None, :]
                continue
            s = pl_m[bi, h, off, 0]
            z = pl_m[bi, h, off, 1] if mode != INT8_SYM else np.zeros_like(s)
            xhat = dequant_rows_f64(codes, s, z)
            out[present] = unrotate_f64(xhat, signs) if signs is not None else xhat
    return K, V, present


def gather_dequant(cu_seq_lens, mode: int, head_dim: int, block_size: int,
                   num_kv_heads: int, k_codes, k_meta, v_codes, v_meta, signs=None,
                   block_tables=None, block_tables_headwise=None, channel_scales=None):
    """Dequantize-gather: the custom op that fetches K/V out of the quantized
    cache and dequantizes them ([P1] review thread, the cache-fetch operator
    with its composed-op test version; [P4] 运行机制: prefill gathers and
    dequantizes the paged cache when it needs dense K/V).

    Sequence b's positions 0 .. n_b - 1, n_b = cu_seq_lens[b+1] -
    cu_seq_lens[b], become rows cu_seq_lens[b] .. cu_seq_lens[b+1] - 1 of the
    float64 outputs K, V [cu_seq_lens[-1], Hkv, D], dequantized and
    un-rotated.  Positions in an evicted (-1) block are zero rows."""
    cu = np.asarray(cu_seq_lens, np.int64)
    n_tok = int(cu[-1])
    K = np.zeros((n_tok, num_kv_heads, head_dim))
    V = np.zeros((n_tok, num_kv_heads, head_dim))
    for b in range(len(cu) - 1):
        n = int(cu[b + 1] - cu[b])
        for h in range(num_kv_heads):
            Kb, Vb, _ = gather_head(b, h, n, mode, head_dim, block_size, num_kv_heads,
                                    k_codes, k_meta, v_codes, v_meta, signs,
                                    block_tables, block_tables_headwise, channel_scales)
            K[cu[b]:cu[b + 1], h] = Kb
            V[cu[b]:cu[b + 1], h] = Vb
    return K, V


def _attend(qs: np.ndarray, K: np.ndarray, V: np.ndarray, allowed: np.ndarray,
            scale: float) -> np.ndarray:
    """Plain softmax attention in float64.  qs [n, D]; allowed [n, Lk] bool.
    Rows with no allowed key give 0."""
    out = np.zeros((qs.shape[0], V.shape[1]))
    if K.shape[0] == 0:
        return out
    logits = scale * (np.asarray(qs, np.float64) @ K.T)
    logits = np.where(allowed, logits, -np.inf)
    m = np.max(logits, axis=1, keepdims=True)
    has = np.isfinite(m[:, 0])
    m = np.where(np.isfinite(m), m, 0.0)
    p = np.where(allowed, np.exp(logits - m), 0.0)
    l = p.sum(axis=1, keepdims=True)
    out[has] = (p[has] @ V) / l[has]
    return out


def decode_attention(q, seq_lens, mode: int, head_dim: int, block_size: int,
                     num_kv_heads: int, k_codes, k_meta, v_codes, v_meta,
                     softmax_scale: float, signs=None, block_tables=None,
                     block_tables_headwise=None, window=None, pairs=None, sink_size=0,
                     channel_scales=None):
    """Step O9: one query token per sequence, q [B, Hq, D] (float images of
    bf16).  Returns float64 [B, Hq, D].

    If ``pairs`` is given (list of (b, kv_head)), only those are computed and
    the rest of the output stays NaN.  ``sink_size``: a windowed head also
    attends positions j < sink_size.
    """
    q = np.asarray(q, np.float64)
    B, Hq, D = q.shape
    G = Hq // num_kv_heads
    out = np.full((B, Hq, D), np.nan)
    todo = pairs if pairs is not None else [(b, h) for b in range(B) for h in range(num_kv_heads)]
    for b, h in todo:
        L = int(seq_lens[b])
        K, V, present = gather_head(b, h, L, mode, head_dim, block_size, num_kv_heads,
                                    k_codes, k_meta, v_codes, v_meta, signs,
                                    block_tables, block_tables_headwise, channel_scales)
        allowed = present.copy()
        W = int(window[h]) if window is not None else 0
        if W > 0:
            j = np.arange(L)
            allowed &= (j >= L - W) | (j < sink_size)
        qs = q[b, h * G:(h + 1) * G]
        out[b, h * G:(h + 1) * G] = _attend(qs, K, V, np.broadcast_to(allowed, (G, L)),
                                             softmax_scale)
    return out


def prefill_attention(q, cu_seqlens_q, seq_lens, mode: int, head_dim: int,
                      block_size: int, num_kv_heads: int, k_codes, k_meta, v_codes,
                      v_meta, softmax_scale: float, signs=None, block_tables=None,
                      block_tables_headwise=None, window=None, pairs=None,
                      rows=None, sink_size=0, channel_scales=None):
    """Step O10: chunked prefill.  q [Tq, Hq, D]; sequence b owns query rows
    cu[b]..cu[b+1]-1, which sit at positions L_b - n_b + i (n_b = new tokens).
    Query at position p attends to keys j <= p that are present and, for a
    windowed kv head, j >= p - W + 1.  Returns float64 [Tq, Hq, D].

    ``pairs`` restricts the (b, kv_head) pairs computed; ``rows`` (an int array
    of query indices within each sequence) restricts the query rows;
    ``sink_size``: a windowed head also attends positions j < sink_size.
    """
    q = np.asarray(q, np.float64)
    Tq, Hq, D = q.shape
    G = Hq // num_kv_heads
    out = np.full((Tq, Hq, D), np.nan)
    B = len(seq_lens)
    todo = pairs if pairs is not None else [(b, h) for b in range(B) for h in range(num_kv_heads)]
    for b, h in todo:
        L = int(seq_lens[b])
        q0, q1 = int(cu_seqlens_q[b]), int(cu_seqlens_q[b + 1])
        n = q1 - q0
        if n == 0:
            continue
        K, V, present = gather_head(b, h, L, mode, head_dim, block_size, num_kv_heads,
                                    k_codes, k_meta, v_codes, v_meta, signs,
                                    block_tables, block_tables_headwise, channel_scales)
        idx = np.arange(n) if rows is None else np.asarray([r for r in rows if r < n], np.int64)
        if idx.size == 0:
            continue
        pos = (L - n + idx)[:, None]
        j = np.arange(L)[None, :]
        allowed = (j <= pos) & present[None, :]
        W = int(window[h]) if window is not None else 0
        if W > 0:
            allowed &= (j >= pos - W + 1) | (j < sink_size)
        for g in range(G):
            hq = h * G + g
            out[q0 + idx, hq] = _attend(q[q0 + idx, hq], K, V, allowed, softmax_scale)
    return out
