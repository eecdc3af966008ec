"""Plant a plausible mistake in a copy of the oracle (CPU only) and require
that at least one pin fails: the pins are strong enough to catch a dropped
term, a wrong sign or index, or a transposed operand."""
import os
import types

import pytest

from tests import oracle_pins as pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "oracle", "kvq_oracle.py")

MUTATIONS = {
    "fwht_sign": ("np.stack([a + b, a - b], axis=-2)", "np.stack([a + b, b - a], axis=-2)"),
    "fwht_pairing": ("y = x.reshape(lead + (D // (2 * h), 2, h))", "y = x.reshape(lead + (D // (2 * h), h, 2)).swapaxes(-1, -2)"),
    "no_normalization": ("return (y * inv_sqrt_f32(x.shape[-1])).astype(_F32)", "return y.astype(_F32)"),
    "unrotate_no_signs": ("return fwht(x) * np.asarray(signs, np.float64) / math.sqrt(D)", "return fwht(x) / math.sqrt(D)"),
    "floor_not_rint": ("c = np.clip(np.rint(t), lo, hi)", "c = np.clip(np.floor(t), lo, hi)"),
    "zero_is_max": ("z = mn.astype(_F32)", "z = mx.astype(_F32)"),
    "int4_levels_16": ("LEVELS = {INT8_SYM: 127, INT4_ASYM: 15, INT2_ASYM: 3, INT8_CHANNEL: 127}",
                       "LEVELS = {INT8_SYM: 127, INT4_ASYM: 16, INT2_ASYM: 3, INT8_CHANNEL: 127}"),
    "int8_levels_128": ("LEVELS = {INT8_SYM: 127, INT4_ASYM: 15, INT2_ASYM: 3, INT8_CHANNEL: 127}",
                        "LEVELS = {INT8_SYM: 128, INT4_ASYM: 15, INT2_ASYM: 3, INT8_CHANNEL: 127}"),
    "nibble_order": ("out |= g[..., k] << (b * k)", "out |= g[..., k] << (b * (per - 1 - k))"),
    "int8_no_sign_extend": ("return np.where(p >= 128, p - 256, p).astype(np.int32)", "return p.astype(np.int32)"),
    "dequant_wrong": ("return (np.asarray(codes, np.float64) * np.asarray(s, np.float64)[..., None]\n            + np.asarray(z, np.float64)[..., None])",
                      "return ((np.asarray(codes, np.float64) + np.asarray(z, np.float64)[..., None])\n            * np.asarray(s, np.float64)[..., None])"),
    "gqa_map": ("qs = q[b, h * G:(h + 1) * G]", "qs = q[b, h::num_kv_heads]"),
    "window_off_by_one": ("allowed &= (j >= L - W) | (j < sink_size)", "allowed &= (j > L - W) | (j < sink_size)"),
    "causal_strict": ("allowed = (j <= pos) & present[None, :]", "allowed = (j < pos) & present[None, :]"),
    "prefill_window_off_by_one": ("allowed &= (j >= pos - W + 1) | (j < sink_size)",
                                  "allowed &= (j >= pos - W) | (j < sink_size)"),
    "evicted_read": ("present = ids >= 0", "present = ids >= -1"),
    "headwise_row": ("return np.asarray(block_tables_headwise)[b * num_kv_heads + h]", "return np.asarray(block_tables_headwise)[h * num_kv_heads + b]"),
    "scale_dropped": ("logits = scale * (np.asarray(qs, np.float64) @ K.T)", "logits = np.asarray(qs, np.float64) @ K.T"),
    "gather_head_index": ("K[cu[b]:cu[b + 1], h] = Kb", "K[cu[b]:cu[b + 1], num_kv_heads - 1 - h] = Kb"),
    "gather_row_offset": ("n = int(cu[b + 1] - cu[b])", "n = int(cu[b + 1] - cu[b]) - (b > 0)"),
    "slot_offset": ("blk, off = sl // block_size, sl % block_size", "blk, off = sl // block_size, (sl + 1) % block_size"),
    # rounding and the float32 operation order of the code decision
    "round_half_up": ("c = np.clip(np.rint(t), lo, hi)", "c = np.clip(np.floor(t + 0.5), lo, hi)"),
    "round_half_away": ("c = np.clip(np.rint(t), lo, hi)", "c = np.clip(np.sign(t) * np.floor(np.abs(t) + 0.5), lo, hi)"),
    "t_float64": ("t = (base * inv[..., None]).astype(_F32)", "t = base.astype(np.float64) * inv[..., None].astype(np.float64)"),
    "t_divide": ("t = (base * inv[..., None]).astype(_F32)", "t = (base / np.where(ok, s, _F32(1.0))[..., None]).astype(_F32)"),
    "sub_unrounded": ("base = (y - mn[..., None]).astype(_F32)", "base = y.astype(np.float64) - mn[..., None].astype(np.float64)"),
    "range_unrounded": ("s = ((mx - mn) / L).astype(_F32)", "s = ((mx.astype(np.float64) - mn) / L).astype(_F32)"),
    "sink_off_by_one": ("allowed &= (j >= L - W) | (j < sink_size)", "allowed &= (j >= L - W) | (j <= sink_size)"),
    "prefill_sink_dropped": ("allowed &= (j >= pos - W + 1) | (j < sink_size)", "allowed &= (j >= pos - W + 1)"),
    "channel_axis": ("a = np.max(np.abs(np.asarray(x, _F32)), axis=0)", "a = np.max(np.abs(np.asarray(x, _F32)), axis=1)"),
    "channel_no_saturation": ("c = np.clip(np.rint(t), -127, 127)", "c = np.rint(t)"),
    "channel_kv_swapped": ("out[present] = codes * np.asarray(channel_scales, np.float64)[kv, h][None, :]",
                           "out[present] = codes * np.asarray(channel_scales, np.float64)[1 - kv, h][None, :]"),
    "channel_scale_head": ("out[present] = codes * np.asarray(channel_scales, np.float64)[kv, h][None, :]",
                           "out[present] = codes * np.asarray(channel_scales, np.float64)[kv, 0][None, :]"),
    "fp8_bias": ("v = np.where(e > 0, np.ldexp(1.0 + m / 8.0, e - 7), np.ldexp(m / 8.0, -6))",
                 "v = np.where(e > 0, np.ldexp(1.0 + m / 8.0, e - 8), np.ldexp(m / 8.0, -7))"),
    "fp8_max": ("s = (a / _F32(E4M3_MAX)).astype(_F32)", "s = (a / _F32(240.0)).astype(_F32)"),
    "fp8_ties_up": ("q = np.rint(a / np.ldexp(1.0, (e - 3).astype(np.int64)))   # 8 .. 16",
                    "q = np.floor(a / np.ldexp(1.0, (e - 3).astype(np.int64)) + 0.5)"),
    "fp8_subnormal_step": ("q_sub = np.rint(a / 2.0 ** -9)", "q_sub = np.rint(a / 2.0 ** -10)"),
    "headwise_slots_transposed": ("slots = np.asarray(slot_mapping_headwise, np.int64).reshape(T, Hkv)",
                                  "slots = np.asarray(slot_mapping_headwise, np.int64).reshape(Hkv, T).T"),
    # INT4 with the zero point in the scale's low bits
    "inline_zero_high_bits": ("return ((bits & np.uint32(0xFFFFFFF0)) | np.asarray(zp, np.uint32))",
                              "return ((bits & np.uint32(0xFFFFFF0F)) | (np.asarray(zp, np.uint32) << np.uint32(4)))"),
    "inline_range_without_zero": ("mn = np.minimum(np.min(y, axis=-1), _F32(0.0)).astype(_F32)",
                                  "mn = np.min(y, axis=-1).astype(_F32)"),
    "inline_round_after_add": ("c = np.clip(np.rint(t) + zp[..., None], 0, INLINE_LEVELS)",
                               "c = np.clip(np.rint(t + zp[..., None]), 0, INLINE_LEVELS)"),
    "inline_unperturbed_scale": ("inv = (_F32(1.0) / np.where(ok, st, _F32(1.0))).astype(_F32)",
                                 "inv = (_F32(1.0) / np.where(ok, s1, _F32(1.0))).astype(_F32)"),
    "inline_dequant_no_zero": ("return (codes - zp[:, None]) * st.astype(np.float64)[:, None]",
                               "return codes * st.astype(np.float64)[:, None]"),
    "inline_v_from_k_half": ("xhat = dequant_inline_rows_f64(k_codes[bi, kv, off, h, :], head_dim)",
                             "xhat = dequant_inline_rows_f64(k_codes[bi, 0, off, h, :], head_dim)"),
    "inline_zero_truncated": ("zp = np.clip(np.rint((-mn / s1).astype(_F32)), 0, INLINE_LEVELS).astype(np.int64)",
                              "zp = np.clip(np.floor((-mn / s1).astype(_F32)), 0, INLINE_LEVELS).astype(np.int64)"),
}


def _mutant(old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor not unique/present: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name):
    mod = _mutant(*MUTATIONS[name])
    caught = []
    for check in pins.ALL:
        try:
            check(mod)
        except Exception:   # AssertionError, or a crash the mistake causes
            caught.append(check.__name__)
    assert caught, f"no pin caught the planted mistake {name}"
