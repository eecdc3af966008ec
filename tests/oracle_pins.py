"""Pins for the CPU oracle: each ``check_*(o)`` takes an oracle module and
raises AssertionError when the oracle disagrees with something fixed outside
it (a closed form, a library routine, an invariant, brute force, or a fact the
pages state).  ``test_oracle_pins.py`` runs them on the oracle; the mutation
tests run them on copies of the oracle with a planted mistake and require that
at least one pin fails.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import scipy.linalg
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
F32 = np.float32
MODES = (0, 1, 2)


def _bf16_rows(shape, seed, scale=1.0, offset=0.0):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(shape, generator=g) * scale + offset
    return x.to(torch.bfloat16).float().numpy()


# ---------------------------------------------------------------- packing ---
def check_pack_exhaustive(o):
    """Every byte value survives unpack -> pack, for each mode (INT4: two
    codes per byte, INT2: four, INT8: one signed code)."""
    allb = np.arange(256, dtype=np.uint8)
    for mode, D in ((1, 2), (2, 4), (0, 1)):
        rows = allb.reshape(256, 1)
        codes = o.unpack_codes(rows, mode, D)
        assert codes.shape == (256, D)
        back = o.pack_codes(codes, mode)
        assert np.array_equal(back, rows), f"mode {mode} byte round trip"
    # INT8: two's complement value of every byte
    c = o.unpack_codes(allb.reshape(256, 1), 0, 1)[:, 0]
    assert np.array_equal(c, np.where(allb >= 128, allb.astype(int) - 256, allb))


def check_pack_positions(o):
    """Element 2j -> low nibble of byte j; element 4j+k -> bits 2k..2k+1."""
    for j in range(8):
        c = np.zeros(8, int); c[j] = 15
        p = o.pack_codes(c[None], 1)[0]
        exp = np.zeros(4, int); exp[j // 2] = 0x0F if j % 2 == 0 else 0xF0
        assert np.array_equal(p, exp), f"INT4 element {j}"
        c = np.zeros(16, int); c[j] = 3
        p = o.pack_codes(c[None], 2)[0]
        exp = np.zeros(4, int); exp[j // 4] = 3 << (2 * (j % 4))
        assert np.array_equal(p, exp), f"INT2 element {j}"


def check_pack_random_roundtrip(o):
    r = np.random.default_rng(7)
    for mode, lo, hi in ((0, -127, 127), (1, 0, 15), (2, 0, 3)):
        c = r.integers(lo, hi + 1, size=(50, 128))
        assert np.array_equal(o.unpack_codes(o.pack_codes(c, mode), mode, 128), c)


# --------------------------------------------------------------- hadamard ---
def check_hadamard_matrix(o):
    for n in (2, 8, 64, 128):
        H = o.sylvester_hadamard(n)
        assert np.array_equal(H @ H.T, n * np.eye(n, dtype=np.int64)), f"H H^T = nI, n={n}"
        assert np.array_equal(H, scipy.linalg.hadamard(n)), f"Sylvester order, n={n}"


def check_fwht_is_hadamard(o):
    """FWHT of each basis vector is the matching column of scipy's H."""
    for n in (4, 64, 128):
        E = np.eye(n)
        assert np.array_equal(o.fwht(E), scipy.linalg.hadamard(n).T.astype(float))


def check_fwht_involution(o):
    r = np.random.default_rng(3)
    x = r.standard_normal((20, 128))
    assert np.allclose(o.fwht(o.fwht(x)), 128 * x, rtol=0, atol=1e-10)


def check_rotation_orthogonal(o):
    r = np.random.default_rng(4)
    for n in (64, 128):
        d = np.where(r.integers(0, 2, n) == 1, 1.0, -1.0)
        R = scipy.linalg.hadamard(n) * d[None, :] / math.sqrt(n)   # H diag(d) / sqrt(n)
        assert np.allclose(R.T @ R, np.eye(n), atol=1e-12)
        x = r.standard_normal((5, n))
        # rotate (dense check path) and unrotate agree with R and R^T
        assert np.allclose(o.rotate_dense_f64(x, d), x @ R.T, atol=1e-12)
        assert np.allclose(o.unrotate_f64(x @ R.T, d), x, atol=1e-12)


def check_rotate_f32_accuracy(o):
    """The float32 FWHT path is within its rounding bound of the exact
    rotation: log2(D) * sqrt(D) * 2^-24 * max|x| + 2^-24 |y|."""
    r = np.random.default_rng(5)
    u = 2.0 ** -24
    for n in (64, 128):
        d = np.where(r.integers(0, 2, n) == 1, 1.0, -1.0).astype(F32)
        x = _bf16_rows((64, n), 11 + n, scale=3.0)
        y32 = o.rotate_f32(x, d).astype(np.float64)
        R = scipy.linalg.hadamard(n) * d.astype(float)[None, :] / math.sqrt(n)
        y = x.astype(np.float64) @ R.T
        bound = math.log2(n) * math.sqrt(n) * u * np.abs(x).max(axis=1, keepdims=True) + u * np.abs(y)
        assert np.all(np.abs(y32 - y) <= 1.01 * bound)
        assert y32.dtype == np.float64 and o.rotate_f32(x, d).dtype == F32


# ---------------------------------------------------------- quantization ---
def check_quant_ranges_and_error(o):
    """Codes lie in [0, L] / [-127, 127]; reconstruction error <= s/2 (plus
    the float32 slack of 1/s and the product)."""
    for mode in MODES:
        for seed, (sc, off) in enumerate(((1.0, 0.0), (10.0, 3.0), (1e-3, -5.0))):
            y = _bf16_rows((200, 128), 100 + seed, scale=sc, offset=off)
            c, s, z = o.quantize_rows(y, mode)
            L = o.LEVELS[mode]
            lo = -L if mode == 0 else 0
            assert c.min() >= lo and c.max() <= L
            if mode == 0:
                assert np.all(z == 0)
                assert np.array_equal(s, (np.abs(y).max(axis=1) / F32(127)).astype(F32))
            else:
                assert np.array_equal(z, y.min(axis=1))
                assert np.array_equal(s, ((y.max(axis=1) - y.min(axis=1)) / F32(L)).astype(F32))
            xh = o.dequant_rows_f64(c, s, z)
            err = np.abs(xh - y.astype(np.float64))
            assert np.all(err <= s[:, None].astype(np.float64) * (0.5 + 1e-5)), mode


def check_quant_nearest(o):
    """Each code is the nearest grid point to the exact value (y-z)/s, up to
    float32 ties: |t - c| <= 0.5 + 1e-5."""
    for mode in MODES:
        y = _bf16_rows((300, 64), 200 + mode, scale=2.0)
        c, s, z = o.quantize_rows(y, mode)
        t = (y.astype(np.float64) - z[:, None]) / s[:, None].astype(np.float64)
        L = o.LEVELS[mode]
        lo = -L if mode == 0 else 0
        assert np.all(np.abs(np.clip(t, lo, L) - c) <= 0.5 + 1e-5)


def check_quant_grid_rows(o):
    """Rows on an exact power-of-two grid reconstruct exactly: s = 2^-e,
    codes = the grid indices, x_hat = y."""
    r = np.random.default_rng(9)
    for mode in MODES:
        L = o.LEVELS[mode]
        for e in (-3, 0, 4):
            if mode == 0:
                k = r.integers(-L, L + 1, size=(40, 128))
                k[:, 0] = L * np.where(r.integers(0, 2, 40) == 1, 1, -1)
                y = (k * 2.0 ** -e).astype(F32)
            else:
                k = r.integers(0, L + 1, size=(40, 128))
                k[:, 0], k[:, 1] = 0, L
                m = r.integers(-1000, 1001, size=(40, 1))     # grid offset, a multiple of 2^-e
                y = ((m + k) * 2.0 ** -e).astype(F32)
            c, s, z = o.quantize_rows(y, mode)
            assert np.all(s == F32(2.0 ** -e)), (mode, e)
            assert np.array_equal(c, k), (mode, e)
            assert np.array_equal(o.dequant_rows_f64(c, s, z), y.astype(np.float64))


def check_quant_degenerate(o):
    for mode in MODES:
        y = np.full((3, 64), F32(0.75), F32)
        y[1] = 0.0
        y[2] = F32(-2.5)
        c, s, z = o.quantize_rows(y, mode)
        if mode == 0:
            # only the zero row is degenerate for absmax; a constant row maps to +-127
            assert s[1] == 0 and np.all(c[1] == 0)
            assert np.all(c[0] == 127) and np.all(c[2] == -127)
        else:
            assert np.all(c == 0)
            assert np.all(s == 0) and np.array_equal(z, y[:, 0])
            assert np.array_equal(o.dequant_rows_f64(c, s, z), y.astype(np.float64))
        tiny = np.zeros((1, 64), F32); tiny[0, 0] = F32(2.0 ** -140)
        c, s, z = o.quantize_rows(tiny, mode)
        assert np.all(c == 0)


# ------------------------------------------- exact model of the fp32 steps ---
# The write's codes are decided by a fixed sequence of float32 operations
# (s = fl(fl(max - min) / L), inv = fl(1 / s), base = fl(y - z), t = fl(base * inv),
# c = round-half-even(t), clamped).  The pins below model that sequence with
# exact rationals and an explicit round-to-nearest-even onto the 24-bit
# float32 significand, independent of numpy's float32 arithmetic, and feed it
# rows built to sit on or next to rounding ties, where any other reading
# (round half up or away, a float64 t, a division instead of the reciprocal,
# an unrounded subtraction) gives a different code.
from fractions import Fraction as _Fr


def _f32r(x):
    """Round a rational to the nearest float32 (ties to even), normal range."""
    x = _Fr(x)
    if x == 0:
        return _Fr(0)
    sgn = -1 if x < 0 else 1
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if _Fr(2) ** e > a:
        e -= 1
    assert _Fr(2) ** e <= a < _Fr(2) ** (e + 1)
    assert -126 <= e <= 127, "outside the normal float32 range"
    ulp = _Fr(2) ** (e - 23)
    n = _rne_int(a / ulp)
    return sgn * n * ulp


def _rne_int(t):
    """Nearest integer to a rational, ties to even."""
    t = _Fr(t)
    f = t.numerator // t.denominator
    r = t - f
    if r > _Fr(1, 2) or (r == _Fr(1, 2) and f % 2 == 1):
        return f + 1
    return f


def _model_codes(row, mode):
    """Codes, s, z of one float32 row by the exact model of the steps."""
    L = {0: 127, 1: 15, 2: 3}[mode]
    y = [_Fr(float(v)) for v in row]
    if mode == 0:
        s = _f32r(max(abs(v) for v in y) / L)
        z = _Fr(0)
        base = y
        lo = -L
    else:
        mn, mx = min(y), max(y)
        s = _f32r(_f32r(mx - mn) / L)
        z = mn
        base = [_f32r(v - mn) for v in y]
        lo = 0
    if s < _Fr(2) ** -126:
        return [0] * len(y), s, z
    inv = _f32r(1 / s)
    return [min(max(_rne_int(_f32r(b * inv)), lo), L) for b in base], s, z


def _tie_rows():
    """Rows (mode, float32 row) whose exact (y - z) / s lands on or beside
    k + 1/2:
      * s = 2^-e: every code step is exact, t = k + 1/2 exactly;
      * INT4 s = 3 (z = 0, max 45): fl(1/3) = (2^25 + 1) / (3 2^25), so
        (k + 1/2) fl(1/3) lies within half an ulp of k + 1/2 and rounds back
        onto the tie;
      * INT4 s = 7/64 (max 105/64): fl(64/7) exceeds 64/7 by 4.5e-8
        relative, so (k + 1/2) fl(64/7) rounds up past the tie for k = 6,
        12, 14, where the exact quotient would round to the even neighbour;
      * float32 rows with a non-dyadic z and scale, y placed a few ulps either
        side of fl((k + 1/2) s + z), where the rounding of y - z decides."""
    rows = []
    for e in (0, 3, -2):
        u = 2.0 ** -e
        rows.append((0, np.array([127 * u, -127 * u] + [(k + 0.5) * u for k in range(-127, 127)], F32)))
        for mode, L in ((1, 15), (2, 3)):
            z = -1.25 * u
            rows.append((mode, np.array([z, z + L * u] + [z + (k + 0.5) * u for k in range(L)] * 4, F32)))
    rows.append((1, np.array([0.0, 45.0] + [3 * (k + 0.5) for k in range(15)], F32)))
    rows.append((1, np.array([0.0, 105 / 64] + [(k + 0.5) * 7 / 64 for k in range(15)], F32)))
    r = np.random.default_rng(17)
    for mode, L in ((1, 15), (2, 3), (1, 15)):
        for _ in range(6):
            s = F32(int(r.integers(1, 1 << 12)) * 2.0 ** -12)
            z = F32(-int(r.integers(1, 1 << 20)) * 2.0 ** -24)
            ys = [z, F32(z + F32(L) * s)]
            for k in range(L):
                c = F32(F32(k + 0.5) * s + z)
                for d in (-2, -1, 0, 1, 2):
                    v = c
                    for _ in range(abs(d)):
                        v = np.nextafter(v, F32(np.inf) if d > 0 else F32(-np.inf))
                    ys.append(F32(v))
            rows.append((mode, np.array(ys, F32)))
    return rows


def check_quant_exact_model_ties(o):
    """Codes, scales and zero points of rows on and beside rounding ties equal
    the exact model of the float32 steps (round half to even; one correctly
    rounded reciprocal; rounded subtraction; rounded product)."""
    for mode, row in _tie_rows():
        c, s, z = o.quantize_rows(row[None, :], mode)
        mc, ms, mz = _model_codes(row, mode)
        assert _Fr(float(s[0])) == ms and _Fr(float(z[0])) == mz, (mode, row[:4])
        assert [int(v) for v in c[0]] == mc, (mode, row[:4], [int(v) for v in c[0]], mc)


def check_quant_ties_to_even(o):
    """On a power-of-two grid every t is exactly k + 1/2: the codes are the
    even neighbours (0.5 -> 0, 1.5 -> 2, -0.5 -> 0, -1.5 -> -2)."""
    for mode, L in ((0, 127), (1, 15), (2, 3)):
        if mode == 0:
            ks = np.arange(-127, 127)
            row = np.concatenate([[127.0, -127.0], ks + 0.5]).astype(F32)
            exp = np.where(ks % 2 == 0, ks, ks + 1)
        else:
            ks = np.arange(L)
            row = np.concatenate([[0.0, float(L)], ks + 0.5]).astype(F32)
            exp = np.where(ks % 2 == 0, ks, ks + 1)
        c, s, z = o.quantize_rows(row[None, :], mode)
        assert s[0] == 1.0
        assert np.array_equal(c[0, 2:], exp), mode


# ------------------------------------------------------------------ layout ---
def check_layout_facts(o):
    with open(os.path.join(HERE, "golden", "layout_facts.json")) as f:
        g = json.load(f)
    assert o.row_code_bytes(1, g["int4_data_head_size"]["head_size"]) == g["int4_data_head_size"]["data_head_size"]
    assert o.row_code_bytes(0, g["int8_data_head_size"]["head_size"]) == g["int8_data_head_size"]["data_head_size"]
    assert o.META_FLOATS[0] * 4 == g["scale_bytes_per_token_head"]["value"]
    assert o.row_code_bytes(1, 128) / o.row_code_bytes(0, 128) == g["int4_over_int8_code_bytes"]["value"]
    assert 128 // o.row_code_bytes(2, 128) == g["int2_codes_per_byte"]["value"]


def _tiny_cache(o, mode, D=64, bs=16, Hkv=2, lens=(37, 100), seed=0, rotate=True):
    r = np.random.default_rng(seed)
    nblk = [(L + bs - 1) // bs for L in lens]
    nb = sum(nblk) + 3
    perm = r.permutation(nb)
    bt = np.full((len(lens), max(nblk)), -1, np.int64)
    k0 = 0
    for b, n in enumerate(nblk):
        bt[b, :n] = perm[k0:k0 + n]
        k0 += n
    T = sum(lens)
    tok_seq = np.repeat(np.arange(len(lens)), lens)
    tok_pos = np.concatenate([np.arange(L) for L in lens])
    slots = bt[tok_seq, tok_pos // bs] * bs + tok_pos % bs
    k = _bf16_rows((T, Hkv, D), 1000 + seed)
    v = _bf16_rows((T, Hkv, D), 2000 + seed, offset=0.5)
    signs = np.where(r.integers(0, 2, D) == 1, 1.0, -1.0).astype(F32) if rotate else None
    cs, ms = o.plane_shapes(mode, D, Hkv, bs, nb)
    planes = [np.full(cs, 0xFF, np.uint8), np.full(ms, np.nan, F32),
              np.full(cs, 0xFF, np.uint8), np.full(ms, np.nan, F32)]
    o.write_cache(k, v, mode, bs, *planes, slot_mapping=slots, signs=signs)
    return dict(k=k, v=v, bt=bt, slots=slots, planes=planes, signs=signs, lens=np.array(lens),
                D=D, bs=bs, Hkv=Hkv, nb=nb, used=perm[:k0], tok_seq=tok_seq, tok_pos=tok_pos)


def check_paged_roundtrip(o):
    """Writing through a shuffled block table and reading back through it
    gives the rows encoded densely; unused blocks keep their poison."""
    for mode in MODES:
        t = _tiny_cache(o, mode)
        kc, km, vc, vm = t["planes"]
        for src, pc, pm in ((t["k"], kc, km), (t["v"], vc, vm)):
            T, Hkv, D = src.shape
            packed, s, z, _ = o.encode_rows(src.reshape(T * Hkv, D), mode, t["signs"])
            blk, off = t["slots"] // t["bs"], t["slots"] % t["bs"]
            for h in range(Hkv):
                assert np.array_equal(pc[blk, h, off], packed.reshape(T, Hkv, -1)[:, h])
                assert np.array_equal(pm[blk, h, off, 0], s.reshape(T, Hkv)[:, h])
                if mode != 0:
                    assert np.array_equal(pm[blk, h, off, 1], z.reshape(T, Hkv)[:, h])
        unused = np.setdiff1d(np.arange(t["nb"]), t["used"])
        assert np.all(kc[unused] == 0xFF) and np.all(np.isnan(km[unused]))


def check_write_headwise_slot_map(o):
    """A head-wise slot map [T, Hkv] sends row (t, h) to its own slot: with
    independent per-head block permutations, the (block, h) slice named by
    slot_hw[t, h] holds the encoding of k[t, h] and v[t, h] and nothing else
    changes; reading each head back through its own head-wise table row gives
    the tokens in order."""
    D, bs, Hkv, T = 64, 4, 3, 10          # T != Hkv, so a transposed map reads wrong slots
    nblk = (T + bs - 1) // bs
    nb = nblk + 2
    r = np.random.default_rng(21)
    bth = np.full((Hkv, nblk), -1, np.int64)
    for h in range(Hkv):
        bth[h] = r.permutation(nb)[:nblk]
    pos = np.arange(T)
    slot_hw = np.stack([bth[h, pos // bs] * bs + pos % bs for h in range(Hkv)], axis=1)   # [T, Hkv]
    assert not np.array_equal(slot_hw[:, 0], slot_hw[:, 1])
    k = _bf16_rows((T, Hkv, D), 61)
    v = _bf16_rows((T, Hkv, D), 62, offset=0.25)
    for mode in MODES:
        cs, ms = o.plane_shapes(mode, D, Hkv, bs, nb)
        planes = [np.full(cs, 0xFF, np.uint8), np.full(ms, np.nan, F32),
                  np.full(cs, 0xFF, np.uint8), np.full(ms, np.nan, F32)]
        o.write_cache(k, v, mode, bs, *planes, slot_mapping_headwise=slot_hw)
        touched = np.zeros((nb, Hkv, bs), bool)
        for src, pc, pm in ((k, planes[0], planes[1]), (v, planes[2], planes[3])):
            for t in range(T):
                for h in range(Hkv):
                    packed, sc, z, _ = o.encode_rows(src[t, h][None], mode)
                    blk, off = divmod(int(slot_hw[t, h]), bs)
                    touched[blk, h, off] = True
                    assert np.array_equal(pc[blk, h, off], packed[0]), (mode, t, h)
                    assert pm[blk, h, off, 0] == sc[0]
                    if mode != 0:
                        assert pm[blk, h, off, 1] == z[0]
            assert np.all(pc[~touched] == 0xFF) and np.all(np.isnan(pm[~touched]))
        table = np.repeat(bth[None], 1, axis=0).reshape(Hkv, nblk)   # rows b*Hkv + h with b = 0
        for h in range(Hkv):
            K, V, pres = o.gather_head(0, h, T, mode, D, bs, Hkv, *planes, block_tables_headwise=table)
            assert pres.all()
            ck, sk, zk = o.quantize_rows(k[:, h], mode)
            assert np.array_equal(K, o.dequant_rows_f64(ck, sk, zk)), (mode, h)


def check_gather_matches_dense(o):
    """gather_head through the table equals dequantize(unrotate(encode(row)))
    computed row by row with the dense float64 R^T."""
    t = _tiny_cache(o, 1)
    kc, km, vc, vm = t["planes"]
    D, bs, Hkv = t["D"], t["bs"], t["Hkv"]
    R = scipy.linalg.hadamard(D) * t["signs"].astype(float)[None, :] / math.sqrt(D)
    for b, L in enumerate(t["lens"]):
        for h in range(Hkv):
            K, V, pres = o.gather_head(b, h, int(L), 1, D, bs, Hkv, kc, km, vc, vm,
                                       t["signs"], block_tables=t["bt"])
            assert pres.all()
            rows = np.nonzero(t["tok_seq"] == b)[0]
            for src, got in ((t["k"], K), (t["v"], V)):
                packed, s, z, codes = o.encode_rows(src[rows, h], 1, t["signs"])
                xh = codes * s[:, None].astype(float) + z[:, None].astype(float)
                assert np.allclose(got, xh @ R, atol=1e-12)


def _grid_rows(mode, n, D, seed):
    """Rows x = c*s + z whose quantization is exact: s a power of two, z
    bf16-exact, codes drawn in [lo, L] with both ends present in every row, so
    the row's min/max (or absmax) give back s and z, 1/s is exact, and every
    code and x_hat = c*s + z come back without rounding.  Returns (x float32
    [n, D], codes int [n, D])."""
    r = np.random.default_rng(seed)
    L = {0: 127, 1: 15, 2: 3}[mode]
    lo = -L if mode == 0 else 0
    c = r.integers(lo, L + 1, (n, D))
    c[:, 0] = L
    c[:, 1] = lo
    s = 2.0 ** -r.integers(2, 6, (n, 1))
    z = 0.0 if mode == 0 else r.choice([-1.5, -0.75, 0.25, 1.0], (n, 1))
    return (c * s + z).astype(F32), c


def check_gather_dequant_grid(o):
    """Dequantize-gather of rows whose quantization is exact returns them bit
    for bit at rows cu[b] + j (shuffled table, a zero-length sequence, every
    mode); an evicted block gives zero rows and leaves the rest; with a
    rotation the result is the dense float64 R^T of the rotated-space gather."""
    D, bs, Hkv = 64, 16, 3
    lens = np.array([21, 0, 40])
    cu = np.concatenate([[0], np.cumsum(lens)])
    nblk = [(L + bs - 1) // bs for L in lens]
    nb = sum(nblk) + 2
    perm = np.random.default_rng(11).permutation(nb)
    bt = np.full((len(lens), max(nblk)), -1, np.int64)
    k0 = 0
    for b, n in enumerate(nblk):
        bt[b, :n] = perm[k0:k0 + n]
        k0 += n
    tok_seq = np.repeat(np.arange(len(lens)), lens)
    tok_pos = np.concatenate([np.arange(L) for L in lens])
    slots = bt[tok_seq, tok_pos // bs] * bs + tok_pos % bs
    T = int(lens.sum())
    for mode in MODES:
        xk, _ = _grid_rows(mode, T * Hkv, D, 20 + mode)
        xv, _ = _grid_rows(mode, T * Hkv, D, 30 + mode)
        k, v = xk.reshape(T, Hkv, D), xv.reshape(T, Hkv, D)
        cs, ms = o.plane_shapes(mode, D, Hkv, bs, nb)
        planes = [np.full(cs, 0xFF, np.uint8), np.full(ms, np.nan, F32),
                  np.full(cs, 0xFF, np.uint8), np.full(ms, np.nan, F32)]
        o.write_cache(k, v, mode, bs, *planes, slot_mapping=slots)
        K, V = o.gather_dequant(cu, mode, D, bs, Hkv, *planes, block_tables=bt)
        assert K.shape == (T, Hkv, D)
        assert np.array_equal(K, k.astype(np.float64)) and np.array_equal(V, v.astype(np.float64)), mode
        # evict block 1 of sequence 2: its 16 positions read as zero rows
        ev = bt.copy()
        ev[2, 1] = -1
        Ke, Ve = o.gather_dequant(cu, mode, D, bs, Hkv, *planes, block_tables=ev)
        gone = np.zeros(T, bool)
        gone[cu[2] + bs:cu[2] + 2 * bs] = True
        assert np.all(Ke[gone] == 0) and np.all(Ve[gone] == 0)
        assert np.array_equal(Ke[~gone], K[~gone]) and np.array_equal(Ve[~gone], V[~gone])
        # head-wise rows equal to the uniform row: same result
        Kh, _ = o.gather_dequant(cu, mode, D, bs, Hkv, *planes, block_tables_headwise=np.repeat(bt, Hkv, axis=0))
        assert np.array_equal(Kh, K)
    signs = np.where(np.random.default_rng(12).integers(0, 2, D) == 1, 1.0, -1.0).astype(F32)
    R = scipy.linalg.hadamard(D) * signs.astype(float)[None, :] / math.sqrt(D)
    Kr, Vr = o.gather_dequant(cu, mode, D, bs, Hkv, *planes, signs=signs, block_tables=bt)
    assert np.allclose(Kr, K @ R, atol=1e-12) and np.allclose(Vr, V @ R, atol=1e-12)


# --------------------------------------------------------------- attention ---
def _sdpa64(q, K, V, mask, scale):
    qt = torch.as_tensor(q, dtype=torch.float64)[None, None]
    kt = torch.as_tensor(K, dtype=torch.float64)[None, None]
    vt = torch.as_tensor(V, dtype=torch.float64)[None, None]
    m = torch.as_tensor(mask)[None, None]
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, scale=scale)[0, 0].numpy()


def check_decode_vs_sdpa(o):
    """Decode equals torch's float64 scaled_dot_product_attention over the
    gathered K/V, with the window mask, for every mode."""
    for mode in MODES:
        t = _tiny_cache(o, mode, seed=mode)
        kc, km, vc, vm = t["planes"]
        D, bs, Hkv = t["D"], t["bs"], t["Hkv"]
        Hq = 4
        q = _bf16_rows((2, Hq, D), 77 + mode)
        win = np.array([0, 20], np.int32)
        out = o.decode_attention(q, t["lens"], mode, D, bs, Hkv, kc, km, vc, vm, 0.125,
                                 signs=t["signs"], block_tables=t["bt"], window=win)
        for b, L in enumerate(t["lens"]):
            for hq in range(Hq):
                h = hq // (Hq // Hkv)
                K, V, _ = o.gather_head(b, h, int(L), mode, D, bs, Hkv, kc, km, vc, vm,
                                        t["signs"], block_tables=t["bt"])
                mask = np.ones((1, L), bool)
                if win[h] > 0:
                    mask[0, :L - win[h]] = False
                ref = _sdpa64(q[b, hq][None], K, V, mask, 0.125)[0]
                assert np.allclose(out[b, hq], ref, atol=1e-12, rtol=1e-12), (mode, b, hq)


def check_decode_closed_forms(o):
    """All keys equal -> output = mean of the values; L = 1 -> output = v_0;
    q = 0 -> mean of the values; identical q within a GQA group -> identical
    outputs; different q heads of one group see the same keys."""
    D, bs, Hkv, Hq = 64, 16, 2, 4
    nb = 6
    cs, ms = o.plane_shapes(1, D, Hkv, bs, nb)
    kc = np.zeros(cs, np.uint8); vc = np.zeros(cs, np.uint8)
    km = np.zeros(ms, F32); vm = np.zeros(ms, F32)
    r = np.random.default_rng(1)
    L = 40
    T = L
    k = np.tile(_bf16_rows((1, Hkv, D), 5), (T, 1, 1))         # all keys equal
    v = _bf16_rows((T, Hkv, D), 6)
    bt = np.array([[4, 0, 2], [5, 1, 3]], np.int64)
    slots = bt[0, np.arange(T) // bs] * bs + np.arange(T) % bs
    o.write_cache(k, v, 1, bs, kc, km, vc, vm, slot_mapping=slots, signs=None)
    q = _bf16_rows((1, Hq, D), 8)
    q[0, 1] = q[0, 0]
    out = o.decode_attention(q, np.array([L]), 1, D, bs, Hkv, kc, km, vc, vm, 0.125,
                             block_tables=bt[:1])
    for hq in range(Hq):
        h = hq // 2
        _, V, _ = o.gather_head(0, h, L, 1, D, bs, Hkv, kc, km, vc, vm, None, block_tables=bt[:1])
        assert np.allclose(out[0, hq], V.mean(axis=0), atol=1e-12)
    assert np.array_equal(out[0, 0], out[0, 1])
    # q = 0 with distinct keys -> mean
    k2 = _bf16_rows((T, Hkv, D), 9)
    o.write_cache(k2, v, 1, bs, kc, km, vc, vm, slot_mapping=slots)
    out0 = o.decode_attention(np.zeros((1, Hq, D)), np.array([L]), 1, D, bs, Hkv, kc, km, vc, vm,
                              0.125, block_tables=bt[:1])
    _, V0, _ = o.gather_head(0, 0, L, 1, D, bs, Hkv, kc, km, vc, vm, None, block_tables=bt[:1])
    assert np.allclose(out0[0, 0], V0.mean(axis=0), atol=1e-12)
    # L = 1 -> v_0 exactly (dequantized)
    out1 = o.decode_attention(q, np.array([1]), 1, D, bs, Hkv, kc, km, vc, vm, 0.125,
                              block_tables=bt[:1])
    v_first = o.gather_head(0, 1, 1, 1, D, bs, Hkv, kc, km, vc, vm, None, block_tables=bt[:1])[1][0]
    assert np.allclose(out1[0, 3], v_first, atol=1e-14)
    # empty allowed set -> 0
    outE = o.decode_attention(q, np.array([0]), 1, D, bs, Hkv, kc, km, vc, vm, 0.125,
                              block_tables=bt[:1])
    assert np.all(outE == 0)


def check_rotation_identity(o):
    """Attending in rotated space with a pre-rotated query and rotating the
    output back equals the oracle's un-rotate-then-attend path."""
    t = _tiny_cache(o, 1, seed=3)
    kc, km, vc, vm = t["planes"]
    D, bs, Hkv = t["D"], t["bs"], t["Hkv"]
    d = t["signs"].astype(float)
    R = scipy.linalg.hadamard(D) * d[None, :] / math.sqrt(D)
    q = _bf16_rows((2, 4, D), 31)
    out = o.decode_attention(q, t["lens"], 1, D, bs, Hkv, kc, km, vc, vm, 0.125,
                             signs=t["signs"], block_tables=t["bt"])
    for b, L in enumerate(t["lens"]):
        for hq in range(4):
            h = hq // 2
            Kr, Vr, _ = o.gather_head(b, h, int(L), 1, D, bs, Hkv, kc, km, vc, vm, None,
                                      block_tables=t["bt"])   # rotated-space x_hat
            qr = R @ q[b, hq].astype(float)
            lg = 0.125 * (Kr @ qr)
            p = np.exp(lg - lg.max()); p /= p.sum()
            o_rot = p @ Vr
            assert np.allclose(R.T @ o_rot, out[b, hq], atol=1e-12)


def check_headwise_equivalence(o):
    """A head-wise table whose rows all equal the uniform row gives the same
    output; -1 only on blocks wholly outside the window equals the window mask
    alone."""
    t = _tiny_cache(o, 2, seed=5)
    kc, km, vc, vm = t["planes"]
    D, bs, Hkv = t["D"], t["bs"], t["Hkv"]
    q = _bf16_rows((2, 4, D), 41)
    win = np.array([24, 0], np.int32)
    base = o.decode_attention(q, t["lens"], 2, D, bs, Hkv, kc, km, vc, vm, 0.125,
                              signs=t["signs"], block_tables=t["bt"], window=win)
    hw = np.repeat(t["bt"], Hkv, axis=0)
    same = o.decode_attention(q, t["lens"], 2, D, bs, Hkv, kc, km, vc, vm, 0.125,
                              signs=t["signs"], block_tables_headwise=hw, window=win)
    assert np.array_equal(base, same)
    hw2 = hw.copy()
    for b, L in enumerate(t["lens"]):
        start = L - win[0]
        for j in range(hw2.shape[1]):
            if (j + 1) * bs <= start:
                hw2[b * Hkv + 0, j] = -1
    ev = o.decode_attention(q, t["lens"], 2, D, bs, Hkv, kc, km, vc, vm, 0.125,
                            signs=t["signs"], block_tables_headwise=hw2, window=win)
    assert np.allclose(ev, base, atol=1e-13)
    # evicting a block inside the window removes exactly its tokens
    hw3 = hw.copy()
    hw3[1 * Hkv + 1, 2] = -1      # seq 1, kv head 1 (full), block 2
    ev3 = o.decode_attention(q, t["lens"], 2, D, bs, Hkv, kc, km, vc, vm, 0.125,
                             signs=t["signs"], block_tables_headwise=hw3, window=win)
    L1 = int(t["lens"][1])
    K, V, _ = o.gather_head(1, 1, L1, 2, D, bs, Hkv, kc, km, vc, vm, t["signs"], block_tables=t["bt"])
    mask = np.ones((1, L1), bool)
    mask[0, 2 * bs:3 * bs] = False
    for hq in (2, 3):
        ref = _sdpa64(q[1, hq][None], K, V, mask, 0.125)[0]
        assert np.allclose(ev3[1, hq], ref, atol=1e-12)


def check_prefill_vs_bruteforce(o):
    """Chunked prefill equals a per-query loop of SDPA with the causal and
    window masks; its last row equals decode with the same query."""
    t = _tiny_cache(o, 1, seed=6)
    kc, km, vc, vm = t["planes"]
    D, bs, Hkv = t["D"], t["bs"], t["Hkv"]
    lens = t["lens"]
    n_new = np.array([5, 17])
    cu = np.concatenate([[0], np.cumsum(n_new)])
    q = _bf16_rows((int(cu[-1]), 4, D), 51)
    win = np.array([0, 30], np.int32)
    out = o.prefill_attention(q, cu, lens, 1, D, bs, Hkv, kc, km, vc, vm, 0.125,
                              signs=t["signs"], block_tables=t["bt"], window=win)
    for b, L in enumerate(lens):
        for h in range(Hkv):
            K, V, _ = o.gather_head(b, h, int(L), 1, D, bs, Hkv, kc, km, vc, vm, t["signs"],
                                    block_tables=t["bt"])
            for i in range(n_new[b]):
                p = L - n_new[b] + i
                mask = np.zeros((1, L), bool)
                mask[0, :p + 1] = True
                if win[h] > 0:
                    mask[0, :max(0, p - win[h] + 1)] = False
                for g in range(2):
                    hq = 2 * h + g
                    ref = _sdpa64(q[cu[b] + i, hq][None], K, V, mask, 0.125)[0]
                    assert np.allclose(out[cu[b] + i, hq], ref, atol=1e-12)
    last = q[cu[1:] - 1]
    dec = o.decode_attention(last, lens, 1, D, bs, Hkv, kc, km, vc, vm, 0.125,
                             signs=t["signs"], block_tables=t["bt"], window=win)
    assert np.allclose(dec, out[cu[1:] - 1], atol=1e-13)


def check_sinks(o):
    """Attention sinks: a windowed head attends the window and the first
    sink_size positions, checked against float64 SDPA with that union mask
    for decode and (per query row) for prefill; sink_size 0 is the window
    alone; sink_size >= L is the whole context."""
    t = _tiny_cache(o, 1, seed=8)
    kc, km, vc, vm = t["planes"]
    D, bs, Hkv = t["D"], t["bs"], t["Hkv"]
    q = _bf16_rows((2, 4, D), 81)
    win = np.array([20, 0], np.int32)
    for sink in (0, 3, 17):
        out = o.decode_attention(q, t["lens"], 1, D, bs, Hkv, kc, km, vc, vm, 0.125, signs=t["signs"],
                                 block_tables=t["bt"], window=win, sink_size=sink)
        for b, L in enumerate(t["lens"]):
            for hq in range(4):
                h = hq // 2
                K, V, _ = o.gather_head(b, h, int(L), 1, D, bs, Hkv, kc, km, vc, vm, t["signs"],
                                        block_tables=t["bt"])
                mask = np.ones((1, L), bool)
                if win[h] > 0:
                    mask[0, :L - win[h]] = False
                    mask[0, :min(sink, L)] = True
                ref = _sdpa64(q[b, hq][None], K, V, mask, 0.125)[0]
                assert np.allclose(out[b, hq], ref, atol=1e-12), (sink, b, hq)
    base = o.decode_attention(q, t["lens"], 1, D, bs, Hkv, kc, km, vc, vm, 0.125, signs=t["signs"],
                              block_tables=t["bt"])
    allsink = o.decode_attention(q, t["lens"], 1, D, bs, Hkv, kc, km, vc, vm, 0.125, signs=t["signs"],
                                 block_tables=t["bt"], window=win, sink_size=1000)
    assert np.allclose(base, allsink, atol=1e-13)
    # prefill: row i at position p sees j <= p with j >= p - W + 1 or j < sink
    n_new = np.array([9, 30])
    cu = np.concatenate([[0], np.cumsum(n_new)])
    qp = _bf16_rows((int(cu[-1]), 4, D), 82)
    sink = 5
    outp = o.prefill_attention(qp, cu, t["lens"], 1, D, bs, Hkv, kc, km, vc, vm, 0.125, signs=t["signs"],
                               block_tables=t["bt"], window=win, sink_size=sink)
    for b, L in enumerate(t["lens"]):
        K, V, _ = o.gather_head(b, 0, int(L), 1, D, bs, Hkv, kc, km, vc, vm, t["signs"], block_tables=t["bt"])
        for i in range(n_new[b]):
            pos = L - n_new[b] + i
            mask = np.zeros((1, L), bool)
            mask[0, max(0, pos - win[0] + 1):pos + 1] = True
            mask[0, :min(sink, pos + 1)] = True
            ref = _sdpa64(qp[cu[b] + i, 0][None], K, V, mask, 0.125)[0]
            assert np.allclose(outp[cu[b] + i, 0], ref, atol=1e-12), (b, i)


# ------------------------------------------------------------- FP8 E4M3 ----
def _e4m3_probe_inputs():
    """Every bf16 value with |x| <= 448, the midpoints between consecutive
    E4M3 values and their float32 neighbours."""
    b = np.arange(0, 1 << 16, dtype=np.uint32) << 16
    x = b.view(np.float32)
    x = x[np.isfinite(x) & (np.abs(x) <= 448.0)]
    fin = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    fin = np.sort(np.unique(fin[np.isfinite(fin)]))
    mids = ((fin[:-1].astype(np.float64) + fin[1:]) / 2).astype(F32)
    return np.concatenate([x, mids, np.nextafter(mids, F32(np.inf)), np.nextafter(mids, F32(-np.inf))]).astype(F32)


def check_e4m3_codec(o):
    """The E4M3 codec equals torch's float8_e4m3fn (a library routine): the
    value of every byte, and the nearest-even encoding of every bf16 value in
    [-448, 448] and of every midpoint between neighbouring E4M3 values (and
    one float32 step either side of it); encode(decode(c)) = c."""
    c = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(c).view(torch.float8_e4m3fn).float().numpy()
    v = o.e4m3_decode(c)
    fin = np.isfinite(ref)
    assert np.array_equal(v[fin], ref[fin]) and np.all(np.isnan(v[~fin]))
    assert np.array_equal(np.signbit(v[fin]), np.signbit(ref[fin]))
    x = _e4m3_probe_inputs()
    assert np.array_equal(o.e4m3_encode(x), torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy())
    assert np.array_equal(o.e4m3_encode(v[fin]), c[fin])


def check_fp8_quantize(o):
    """FP8 rows: on a grid y = v 2^-e with v E4M3 values and +-448 present,
    s = 2^-e, the codes are the E4M3 bytes of v and x_hat = y exactly;
    otherwise |y - x_hat| <= max(|y| 2^-4, s 2^-10) (half a step of three
    mantissa bits, or of the subnormal grid); a zero row has scale 0 and
    codes 0."""
    r = np.random.default_rng(41)
    fin = o.e4m3_decode(np.arange(256, dtype=np.uint8))
    fin = fin[np.isfinite(fin)]
    for e in (0, 3, -5):
        v = r.choice(fin, size=(30, 128))
        v[:, 0] = np.where(r.integers(0, 2, 30) == 1, 448.0, -448.0)
        y = (v * 2.0 ** -e).astype(F32)
        packed, s, z, codes = o.encode_rows(y, o.FP8_E4M3)
        assert np.all(s == F32(2.0 ** -e)) and np.all(z == 0)
        assert np.array_equal(codes, o.e4m3_encode(v.astype(F32)))
        assert np.array_equal(o.e4m3_decode(codes) * s[:, None].astype(np.float64), y.astype(np.float64))
    y = _bf16_rows((200, 64), 42, scale=3.0)
    packed, s, z, codes = o.encode_rows(y, o.FP8_E4M3)
    xh = o.e4m3_decode(codes) * s[:, None].astype(np.float64)
    bound = np.maximum(np.abs(y) * 2.0 ** -4, s[:, None] * 2.0 ** -10) * (1 + 1e-6)
    assert np.all(np.abs(xh - y) <= bound)
    assert np.all(np.abs(o.e4m3_decode(codes)) <= 448.0)
    zero = np.zeros((1, 64), F32)
    _, s0, _, c0 = o.encode_rows(zero, o.FP8_E4M3)
    assert s0[0] == 0 and np.all(c0 == 0)


def check_fp8_attention(o):
    """FP8 decode through a shuffled table (with rotation) equals float64 SDPA
    over the gathered, un-rotated rows."""
    t = _tiny_cache(o, o.FP8_E4M3, seed=9)
    kc, km, vc, vm = t["planes"]
    D, bs, Hkv = t["D"], t["bs"], t["Hkv"]
    q = _bf16_rows((2, 4, D), 93)
    out = o.decode_attention(q, t["lens"], o.FP8_E4M3, D, bs, Hkv, kc, km, vc, vm, 0.125, signs=t["signs"],
                             block_tables=t["bt"])
    R = scipy.linalg.hadamard(D) * t["signs"].astype(float)[None, :] / math.sqrt(D)
    for b, L in enumerate(t["lens"]):
        for hq in range(4):
            h = hq // 2
            rows = np.nonzero(t["tok_seq"] == b)[0]
            K = o.e4m3_decode(o.encode_rows(t["k"][rows, h], o.FP8_E4M3, t["signs"])[3]) * \
                o.encode_rows(t["k"][rows, h], o.FP8_E4M3, t["signs"])[1][:, None].astype(np.float64)
            V = o.e4m3_decode(o.encode_rows(t["v"][rows, h], o.FP8_E4M3, t["signs"])[3]) * \
                o.encode_rows(t["v"][rows, h], o.FP8_E4M3, t["signs"])[1][:, None].astype(np.float64)
            ref = _sdpa64(q[b, hq][None], K @ R, V @ R, np.ones((1, L), bool), 0.125)[0]
            assert np.allclose(out[b, hq], ref, atol=1e-12), (b, hq)


# --------------------------------------------------- per-channel INT8 ------
def _channel_batch(r, T, Hkv, D, exps):
    """[T, Hkv, D] rows whose per-(head, channel) absolute maximum over tokens
    is exactly 127 * 2^-e (e from `exps`), other entries k * 2^-e with |k| <=
    127 integer, so the scales are 2^-e exactly and every code is k."""
    e = r.choice(exps, size=(Hkv, D))
    k = r.integers(-127, 128, size=(T, Hkv, D))
    k[0] = np.where(r.integers(0, 2, size=(Hkv, D)) == 1, 127, -127)   # the maximum
    return (k * 2.0 ** -e[None]).astype(F32), k, (2.0 ** -e).astype(F32)


def check_channel_calibration_and_codes(o):
    """Per-channel INT8: the calibrated scale of each (head, channel) is its
    maximum |x| over the first batch / 127 (2^-e exactly on power-of-two
    grids); rows on the grid quantize to their integers; later values beyond
    the calibrated range saturate at +-127; an all-zero channel has scale 0
    and codes 0; exact .5 steps round half to even."""
    r = np.random.default_rng(31)
    T, Hkv, D = 9, 3, 64
    x, k, sexp = _channel_batch(r, T, Hkv, D, [0, 3, 7])
    x[:, 1, 5] = 0.0
    k[:, 1, 5] = 0
    sexp[1, 5] = 0.0
    sc = o.calibrate_channel_scales(x)
    assert sc.shape == (Hkv, D) and sc.dtype == F32
    assert np.array_equal(sc, sexp)
    c = o.quantize_rows_channel(x, sc[None])
    assert np.array_equal(c, k)
    # saturation of later tokens beyond the calibrated maximum
    big = (np.array([300.0, -1000.0, 128.0, -127.6]) * sexp[0, :4]).astype(F32)
    cb = o.quantize_rows_channel(big[None], sc[0, :4][None])
    assert np.array_equal(cb[0], [127, -127, 127, -127])
    # ties: t = k + 1/2 exactly on the grid -> even neighbour
    ks = np.arange(-10, 10)
    ties = ((ks + 0.5) * sexp[2, 0]).astype(F32)
    ct = o.quantize_rows_channel(ties[:, None], np.full((len(ks), 1), sc[2, 0], F32))[:, 0]
    assert np.array_equal(ct, np.where(ks % 2 == 0, ks, ks + 1))
    # a zero-scale channel gives code 0 whatever the later value
    assert o.quantize_rows_channel(np.array([[5.0]], F32), np.array([[0.0]], F32))[0, 0] == 0


def check_channel_write_gather_and_attention(o):
    """Per-channel INT8 through the paged layout: grid rows written with their
    own calibrated scales come back exactly from the gather (shuffled table,
    K and V scales distinct); decode equals float64 SDPA over those rows."""
    r = np.random.default_rng(32)
    D, bs, Hkv, L = 64, 16, 2, 40
    k, _, _ = _channel_batch(r, L, Hkv, D, [1, 4])
    v, _, _ = _channel_batch(r, L, Hkv, D, [0, 2, 5])
    sc = np.stack([o.calibrate_channel_scales(k), o.calibrate_channel_scales(v)])
    assert not np.array_equal(sc[0], sc[1])
    nblk = (L + bs - 1) // bs
    nb = nblk + 2
    bt = r.permutation(nb)[:nblk][None].astype(np.int64)
    pos = np.arange(L)
    slots = bt[0, pos // bs] * bs + pos % bs
    cs, ms = o.plane_shapes(o.INT8_CHANNEL, D, Hkv, bs, nb)
    assert ms[-1] == 0 and cs[-1] == D
    kc = np.full(cs, 0xFF, np.uint8)
    vc = np.full(cs, 0xFF, np.uint8)
    km = np.zeros(ms, F32)
    vm = np.zeros(ms, F32)
    o.write_cache(k, v, o.INT8_CHANNEL, bs, kc, km, vc, vm, slot_mapping=slots, channel_scales=sc)
    K, V = o.gather_dequant(np.array([0, L]), o.INT8_CHANNEL, D, bs, Hkv, kc, km, vc, vm, block_tables=bt,
                            channel_scales=sc)
    assert np.array_equal(K, k.astype(np.float64)) and np.array_equal(V, v.astype(np.float64))
    q = _bf16_rows((1, 4, D), 91)
    out = o.decode_attention(q, np.array([L]), o.INT8_CHANNEL, D, bs, Hkv, kc, km, vc, vm, 0.125,
                             block_tables=bt, channel_scales=sc)
    for hq in range(4):
        h = hq // 2
        ref = _sdpa64(q[0, hq][None], k[:, h].astype(np.float64), v[:, h].astype(np.float64),
                      np.ones((1, L), bool), 0.125)[0]
        assert np.allclose(out[0, hq], ref, atol=1e-12), hq


# ------------------------------------- INT4 with the zero in the scale -----
def _f32_bits(x):
    """Bits of a float32-representable rational."""
    return int(np.array([float(x)], F32).view(np.uint32)[0])


def _inline_model(row):
    """Codes and stored-scale bits of one float32 row by the exact model of
    the inline INT4 steps: zero-including range, s = (mx - mn) / 15 (two
    float32 roundings), zp = rint(-mn / s) clamped to [0, 15], st = s with zp
    in its low 4 bits, c = clamp(rint(fl(y fl(1/st))) + zp, 0, 15)."""
    y = [_Fr(float(v)) for v in row]
    mn, mx = min(min(y), _Fr(0)), max(max(y), _Fr(0))
    s = _f32r(_f32r(mx - mn) / 15)
    if s < _Fr(2) ** -126:
        return [0] * len(y), 0
    zp = min(max(_rne_int(_f32r(-mn / s)), 0), 15)
    bits = (_f32_bits(s) & ~0xF) | zp
    st = _Fr(float(np.array([bits], np.uint32).view(F32)[0]))
    inv = _f32r(1 / st)
    return [min(max(_rne_int(_f32r(v * inv)) + zp, 0), 15) for v in y], bits


def _inline_rows_for_pins():
    """Float32 rows: grids (c - zp) 2^-e, exact ties with zp = 0 and with odd
    zp, values half a step from the grid with zp = 15, one-signed rows, and
    random rows."""
    rows = []
    r = np.random.default_rng(51)
    for zp, e in ((0, 4), (3, 0), (5, 7), (15, 2)):
        c = r.permutation(np.tile(np.arange(16), 2))
        c[:2] = (0, 15)
        rows.append(((c - zp) * 2.0 ** -e).astype(F32))
    # zp = 0, s = 2^-4 exactly: ties at t = k + 1/2 go to the even code
    tie = np.zeros(32, F32)
    tie[:2] = (0.0, 15 / 16)
    tie[2:12] = (np.arange(10) + 0.5) / 16
    rows.append(tie)
    # zp = 1 (st = 2^-4 (1 + 2^-23)): y near 2.5 st whose product with
    # fl(1/st) rounds to exactly 2.5 (an odd zero point then decides the
    # order of the rounding and the zero's addition)
    st1 = np.array([0x3D800001], np.uint32).view(F32)[0]
    inv1 = F32(1.0) / st1
    cand = [F32(2.5 / 16) + F32(k) * F32(2.0 ** -26) for k in range(-8, 9)]
    hit = [v for v in cand if F32(v * inv1) == F32(2.5)]
    assert hit, "no exact tie found"
    odd = np.zeros(32, F32)
    odd[:3] = (-1 / 16, 14 / 16, hit[0])
    rows.append(odd)
    # zp = 15 (largest perturbation of the scale): y = fl((k + 1/2) st)
    st15 = np.array([0x3D80000F], np.uint32).view(F32)[0]
    half = np.zeros(32, F32)
    half[:2] = (-15 / 16, 0.0)
    half[2:16] = (-(np.arange(14) + 0.5) * np.float64(st15)).astype(F32)
    rows.append(half)
    rows.append(np.abs(_bf16_rows((32,), 52)) + F32(1.0))     # all positive: zp = 0
    rows.append(-np.abs(_bf16_rows((32,), 53)) - F32(1.0))    # all negative: zp = 15
    rows.extend(_bf16_rows((40, 32), 54, scale=2.0, offset=0.3))
    return np.stack(rows).astype(F32)


def check_inline_exact_model(o):
    """Inline INT4 codes and stored scales equal the exact rational model of
    the steps on grid rows, exact ties (zp = 0 and odd zp), half-step values
    under the largest scale perturbation, one-signed and random rows."""
    y = _inline_rows_for_pins()
    codes, st = o.quantize_rows_inline(y)
    bits = st.view(np.uint32)
    for i, row in enumerate(y):
        mc, mb = _inline_model(row)
        assert list(codes[i]) == mc, (i, list(codes[i]), mc)
        assert int(bits[i]) == mb, (i, hex(int(bits[i])), hex(mb))
    # the grid rows: zp and codes as built, st = 2^-e with zp in the low bits
    r = np.random.default_rng(51)
    for i, (zp, e) in enumerate(((0, 4), (3, 0), (5, 7), (15, 2))):
        c = r.permutation(np.tile(np.arange(16), 2))
        c[:2] = (0, 15)
        assert np.array_equal(codes[i], c)
        assert int(bits[i]) == (_f32_bits(_Fr(2) ** -e) | zp)
    assert list(codes[4][2:12]) == [0, 2, 2, 4, 4, 6, 6, 8, 8, 10]   # ties to even, zp = 0
    assert codes[5][2] == 3                                          # rint(2.5) = 2, plus zp = 1
    assert o.hidden_zero(st[7:8])[0] == 0 and o.hidden_zero(st[8:9])[0] == 15


def check_inline_bounds_and_degenerate(o):
    """|x_hat - y| <= st/2 (plus float32 rounding of the product) on random
    and one-signed rows; st within 15 ulp of the unperturbed scale, same
    upper 28 bits; zero and subnormal-range rows store st = 0 and codes 0,
    and dequantize to 0."""
    y = np.concatenate([_bf16_rows((300, 64), 55, scale=3.0, offset=-0.7),
                        np.abs(_bf16_rows((20, 64), 56)) + F32(0.5)]).astype(F32)
    codes, st = o.quantize_rows_inline(y)
    rows = o.inline_rows(o.pack_codes(codes, o.INT4_ASYM), st)
    xh = o.dequant_inline_rows_f64(rows, 64)
    mn = np.minimum(y.min(1), 0).astype(F32)
    mx = np.maximum(y.max(1), 0).astype(F32)
    s = ((mx - mn) / F32(15)).astype(F32)
    assert np.all((st.view(np.uint32) >> 4) == (s.view(np.uint32) >> 4))
    assert np.all(np.abs(st.astype(np.float64) - s) <= 15 * 2.0 ** -23 * s)
    bound = 0.5 * st.astype(np.float64)[:, None] * (1 + 2.0 ** -16) + 2.0 ** -22 * np.abs(y)
    assert np.all(np.abs(xh - y) <= bound)
    for row in (np.zeros((1, 64), F32), np.full((1, 64), F32(1e-40))):
        c0, s0 = o.quantize_rows_inline(row)
        assert s0.view(np.uint32)[0] == 0 and not c0.any()
        r0 = o.inline_rows(o.pack_codes(c0, o.INT4_ASYM), s0)
        assert not o.dequant_inline_rows_f64(r0, 64).any()


def check_inline_layout_write_gather_attention(o):
    """The inline cache: shape (nb, 2, bs, Hkv, D/2 + 4); a written row holds
    the nibbles (element 2j low) then the little-endian float32 stored
    scale, K at index 0 and V at index 1 of the second axis; unwritten rows
    keep their bytes; gather through a shuffled table (with rotation) is the
    un-rotated (c - zp) st, and decode equals float64 SDPA over it."""
    D, bs, Hkv, lens = 64, 16, 2, (37, 100)
    assert o.inline_cache_shape(128, 4, 16, 3) == (3, 2, 16, 4, 68)
    r = np.random.default_rng(57)
    nblk = [(L + bs - 1) // bs for L in lens]
    nb = sum(nblk) + 3
    perm = r.permutation(nb)
    bt = np.full((2, max(nblk)), -1, np.int64)
    bt[0, :nblk[0]] = perm[:nblk[0]]
    bt[1, :nblk[1]] = perm[nblk[0]:sum(nblk)]
    tok_seq = np.repeat([0, 1], lens)
    tok_pos = np.concatenate([np.arange(L) for L in lens])
    slots = bt[tok_seq, tok_pos // bs] * bs + tok_pos % bs
    T = sum(lens)
    k = _bf16_rows((T, Hkv, D), 58)
    v = _bf16_rows((T, Hkv, D), 59, offset=0.5)
    signs = np.where(r.integers(0, 2, D) == 1, 1.0, -1.0).astype(F32)
    for sg in (None, signs):
        cache = np.full(o.inline_cache_shape(D, Hkv, bs, nb), 0xFF, np.uint8)
        o.write_cache(k, v, o.INT4_INLINE, bs, cache, None, None, None, slot_mapping=slots, signs=sg)
        written = np.zeros(cache.shape[:4], bool)
        for t in range(T):
            blk, off = divmod(int(slots[t]), bs)
            for h in range(Hkv):
                for kv, src in ((0, k), (1, v)):
                    written[blk, kv, off, h] = True
                    if sg is not None:
                        continue
                    c, bits = _inline_model(src[t, h])
                    row = cache[blk, kv, off, h]
                    nib = [int(row[j // 2]) >> (4 * (j % 2)) & 15 for j in range(D)]
                    assert nib == c, (t, h, kv)
                    assert bytes(row[D // 2:]) == int(bits).to_bytes(4, "little"), (t, h, kv)
        assert np.all(cache[~written] == 0xFF)
        K, V = o.gather_dequant(np.array([0, lens[0], T]), o.INT4_INLINE, D, bs, Hkv, cache, None, None, None,
                                signs=sg, block_tables=bt)
        R = np.eye(D) if sg is None else scipy.linalg.hadamard(D) * sg.astype(float)[None, :] / math.sqrt(D)
        for src, G_ in ((k, K), (v, V)):
            y = src.reshape(T * Hkv, D) if sg is None else o.rotate_f32(src.reshape(T * Hkv, D), sg)
            c, st = o.quantize_rows_inline(y)
            xh = (c - o.hidden_zero(st)[:, None]) * st.astype(np.float64)[:, None]
            assert np.allclose(G_.reshape(T * Hkv, D), xh @ R, atol=1e-12)
        q = _bf16_rows((2, 4, D), 60)
        out = o.decode_attention(q, np.array(lens), o.INT4_INLINE, D, bs, Hkv, cache, None, None, None, 0.125,
                                 signs=sg, block_tables=bt)
        for b, L in enumerate(lens):
            rows = np.nonzero(tok_seq == b)[0]
            for hq in range(4):
                h = hq // 2
                ref = _sdpa64(q[b, hq][None], K[rows, h], V[rows, h], np.ones((1, L), bool), 0.125)[0]
                assert np.allclose(out[b, hq], ref, atol=1e-12), (b, hq)


ALL = [v for k, v in sorted(globals().items()) if k.startswith("check_")]
