// One cache row of the quantize-on-write (the arithmetic the cache format
// defines, in the order of the prhub summary of vLLM PR 40835, 实现拆解 item
// 2): bf16 row -> optional rotation -> scale (and zero) -> round -> pack ->
// paged store.  Shared by the write kernel and the fused decode step.
//
// The D/EPL lanes lr = 0 .. D/EPL-1 of one aligned lane group call it
// together (converged: the FWHT and the statistics are shuffles within the
// group); each lane owns EPL = 8 or 16 consecutive elements.  The element
// split changes which butterfly stages run inside a lane and which across
// lanes, not the stages or their order, so both splits store the same bits.  Row (token t, kv head h, K if kv =
// 0 else V) goes to `slot` (block * block_size + offset); a slot < 0 or at
// or past the planes' capacity computes nothing visible.  The load and the rest are separate steps, so a caller
// can have the loads of several rows in flight before the first is used.
#pragma once

#include "kvq_internal.h"
#include "kvq_device.h"

namespace kvq {
namespace {

// The lane's 8 bf16 elements of row (token t, kv head h, K if kv = 0 else
// V): one 16-byte load.  I32: tokens and strides are below 2^31 (checked on
// the host for the write kernel), so the token offset is one 32 x 32 ->
// 64-bit multiply.  The fused decode step keeps the 64-bit form, whose
// register use the decode kernel's allocation is tuned around.
template <int D, bool I32 = false>
__device__ __forceinline__ uint4 write_row_load(const WriteParams& p, int64_t t, int h, int kv, int lr) {
  if constexpr (I32) {
    const uint64_t tt = (uint32_t)t;
    const uint16_t* src = kv ? p.value + tt * (uint32_t)p.value_stride : p.key + tt * (uint32_t)p.key_stride;
    return *reinterpret_cast<const uint4*>(src + (uint32_t)(h * D + lr * 8));
  }
  const uint16_t* src = kv ? p.value + t * p.value_stride : p.key + t * p.key_stride;
  return *reinterpret_cast<const uint4*>(src + (int64_t)h * D + lr * 8);
}

// The lane's 8 rotation signs (read before any store of the caller, so they
// are not reloaded after each row's stores).
__device__ __forceinline__ void write_row_signs(const WriteParams& p, int lr, float (&sg)[8]) {
  const float4 s0 = *reinterpret_cast<const float4*>(p.signs + lr * 8);
  const float4 s1 = *reinterpret_cast<const float4*>(p.signs + lr * 8 + 4);
  sg[0] = s0.x; sg[1] = s0.y; sg[2] = s0.z; sg[3] = s0.w;
  sg[4] = s1.x; sg[5] = s1.y; sg[6] = s1.z; sg[7] = s1.w;
}

// The same for EPL elements a lane: EPL / 8 16-byte loads of the row, and
// the lane's EPL signs.
template <int D, int EPL>
__device__ __forceinline__ void write_row_load_n(const WriteParams& p, int64_t t, int h, int kv, int lr,
                                                 uint4 (&raw)[EPL / 8]) {
  const uint64_t tt = (uint32_t)t;   // tokens and strides below 2^31 (checked on the host)
  const uint16_t* src = kv ? p.value + tt * (uint32_t)p.value_stride : p.key + tt * (uint32_t)p.key_stride;
  const uint4* row = reinterpret_cast<const uint4*>(src + (uint32_t)(h * D + lr * EPL));
#pragma unroll
  for (int i = 0; i < EPL / 8; ++i) raw[i] = row[i];
}

template <int EPL>
__device__ __forceinline__ void write_row_signs_n(const WriteParams& p, int lr, float (&sg)[EPL]) {
#pragma unroll
  for (int i = 0; i < EPL / 4; ++i) {
    const float4 v = *reinterpret_cast<const float4*>(p.signs + lr * EPL + 4 * i);
    sg[4 * i] = v.x; sg[4 * i + 1] = v.y; sg[4 * i + 2] = v.z; sg[4 * i + 3] = v.w;
  }
}

// NW consecutive dwords to dst: one store of 4, 8 or 16 bytes a time (A4:
// dst is only 4-byte aligned).
template <int NW, bool A4>
__device__ __forceinline__ void store_dwords(uint8_t* dst, const uint32_t (&w)[NW]) {
  if constexpr (NW == 1) {
    *reinterpret_cast<uint32_t*>(dst) = w[0];
  } else if constexpr (NW == 2) {
    if constexpr (A4) *reinterpret_cast<u32x2a4_t*>(dst) = u32x2a4_t{w[0], w[1]};
    else *reinterpret_cast<uint2*>(dst) = make_uint2(w[0], w[1]);
  } else {
#pragma unroll
    for (int i = 0; i < NW / 4; ++i) {
      if constexpr (A4) {
        *reinterpret_cast<u32x4a4_t*>(dst + 16 * i) = u32x4a4_t{w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]};
      } else {
        *reinterpret_cast<uint4*>(dst + 16 * i) = make_uint4(w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]);
      }
    }
  }
}

// Everything after the load: rotation (lane signs sg), scale (and zero),
// codes, packed and paged stores of the row whose lane elements `raw` holds.
template <int MODE, int D, bool ROT, bool I32, int EPL>
__device__ __forceinline__ void write_row_store_n(const WriteParams& p, const uint4 (&raw)[EPL / 8],
                                                  const float (&sg)[EPL], int h, int kv, int64_t slot, int lr,
                                                  const float* chinv) {
#pragma clang fp contract(off)
  static_assert(EPL == 8 || EPL == 16 || EPL == 32, "8, 16 or 32 elements a lane");
  constexpr int LPR = D / EPL;           // lanes per row
  constexpr int P = row_bytes(MODE, D);  // packed bytes per row
  constexpr int BPL = P / LPR;           // packed bytes per lane
  constexpr int M = mode_meta(MODE);
  constexpr float kLevels = (float)mode_levels(MODE);
  const int hkv = p.hkv;
  const bool active = slot >= 0 && slot < p.slot_cap;

  // An inactive row (all lanes of its group alike) computes on whatever its
  // registers hold and stores nothing.  The 8-element form of the fused step
  // zeroes them first (its register allocation is tuned around that), and so
  // does per-channel INT8 (fewer instructions that way).
  float x[EPL];
  if ((EPL > 8 && MODE != kChannelMode) || active) {
#pragma unroll
    for (int v = 0; v < EPL / 8; ++v) {
      const uint32_t w[4] = {raw[v].x, raw[v].y, raw[v].z, raw[v].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[8 * v + 2 * i] = __uint_as_float(w[i] << 16);
        x[8 * v + 2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < EPL; ++i) x[i] = 0.0f;
  }

  if constexpr (ROT) {
#pragma unroll
    for (int i = 0; i < EPL; ++i) x[i] *= sg[i];
    // in-lane butterflies, pairs (i, i + hh) with bit hh of i clear
#pragma unroll
    for (int hh = 1; hh < EPL; hh <<= 1) {
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        if (!(i & hh)) {
          const float a = x[i], b = x[i + hh];
          x[i] = a + b;
          x[i + hh] = a - b;
        }
      }
    }
    // cross-lane butterflies: element stride EPL*m lives m lanes away
#pragma unroll
    for (int m = 1; m < LPR; m <<= 1) {
      // x + o in the lower lane, o - x in the upper one, as one fma with a
      // +-1 factor (the product is exact, so the single rounding is the sum's)
      const float sgn = (lr & m) ? -1.0f : 1.0f;
#pragma unroll
      for (int i = 0; i < EPL; ++i) x[i] = __builtin_fmaf(x[i], sgn, xor_in_row(x[i], m));
    }
#pragma unroll
    for (int i = 0; i < EPL; ++i) x[i] = x[i] * p.inv_sqrt_d;
  }

  // per-channel INT8: fixed scales of the (K or V, kv head) channels, codes
  // clamp(rint(x * (1/s_d)), -127, 127), one correctly rounded reciprocal per
  // channel (0 for a zero or subnormal scale, which gives code 0); no row
  // metadata.  chinv: the reciprocals already in LDS ([2][Hkv][D]), else
  // computed here
  uint32_t c[EPL];
  if constexpr (MODE == kChannelMode) {
    float inv[EPL];
    if (chinv) {
      const float* ci = chinv + (kv * hkv + h) * D + lr * EPL;
#pragma unroll
      for (int v = 0; v < EPL / 4; ++v) {
        const float4 iv = *reinterpret_cast<const float4*>(ci + 4 * v);
        inv[4 * v] = iv.x; inv[4 * v + 1] = iv.y; inv[4 * v + 2] = iv.z; inv[4 * v + 3] = iv.w;
      }
    } else {
      const float* cs = p.chs + ((int64_t)kv * hkv + h) * D + lr * EPL;
#pragma unroll
      for (int v = 0; v < EPL / 4; ++v) {
        const float4 sv = *reinterpret_cast<const float4*>(cs + 4 * v);
        const float sc[4] = {sv.x, sv.y, sv.z, sv.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) inv[4 * v + i] = sc[i] >= 1.17549435e-38f ? 1.0f / sc[i] : 0.0f;
      }
    }
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const float r = fminf(fmaxf(__builtin_rintf(x[i] * inv[i]), -kLevels), kLevels);
      c[i] = inv[i] != 0.0f ? (uint32_t)(int32_t)r : 0u;   // 1/s of a normal scale is never 0
    }
  }
  float s = 0.0f, z = 0.0f;   // per-row scale and zero (not for per-channel INT8)
  uint32_t stbits = 0;        // inline INT4: bits of the stored scale
  if constexpr (MODE == 0 || MODE == kFp8Mode) {
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < EPL; ++i) a = fmaxf(a, fabsf(x[i]));
#pragma unroll
    for (int m = 1; m < LPR; m <<= 1) a = fmaxf(a, xor_in_row(a, m));
    s = a / kLevels;
    z = 0.0f;
  } else if constexpr (MODE != kChannelMode) {
    float mn = x[0], mx = x[0];
#pragma unroll
    for (int i = 1; i < EPL; ++i) {
      mn = fminf(mn, x[i]);
      mx = fmaxf(mx, x[i]);
    }
#pragma unroll
    for (int m = 1; m < LPR; m <<= 1) {
      mn = fminf(mn, xor_in_row(mn, m));
      mx = fmaxf(mx, xor_in_row(mx, m));
    }
    if constexpr (MODE == kInlineMode) {   // the range holds zero (integer zero point)
      mn = fminf(mn, 0.0f);
      mx = fmaxf(mx, 0.0f);
    }
    s = (mx - mn) / kLevels;
    z = mn;
  }

  if constexpr (MODE == kFp8Mode) {
    // FP8: t = clamp(x * (1/s), -448, 448), nearest E4M3 (ties to even) by
    // the hardware conversion, two values per instruction; zero, subnormal or
    // NaN scale: all-zero codes
    const bool ok = s >= 1.17549435e-38f;
    const float inv = ok ? 1.0f / s : 0.0f;
    float t[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) t[i] = ok ? fminf(fmaxf(x[i] * inv, -kLevels), kLevels) : 0.0f;
#pragma unroll
    for (int j = 0; j < EPL / 4; ++j) {
      uint32_t w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(t[4 * j], t[4 * j + 1], 0, false);
      w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(t[4 * j + 2], t[4 * j + 3], (int)w, true);
      c[4 * j] = w & 0xffu; c[4 * j + 1] = (w >> 8) & 0xffu; c[4 * j + 2] = (w >> 16) & 0xffu; c[4 * j + 3] = w >> 24;
    }
  } else if constexpr (MODE == kInlineMode) {
    // zp = clamp(rint(-mn / s), 0, 15) into the low 4 bits of s (the stored
    // scale st), then c = clamp(rint(x * (1/st)) + zp, 0, 15); a zero,
    // subnormal or NaN s stores st = 0 and codes 0
    const bool ok = s >= 1.17549435e-38f;
    const float zp = ok ? fminf(fmaxf(__builtin_rintf(-z / s), 0.0f), kLevels) : 0.0f;
    stbits = ok ? ((__float_as_uint(s) & ~0xFu) | (uint32_t)zp) : 0u;
    const float inv = ok ? 1.0f / __uint_as_float(stbits) : 0.0f;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const float r = fminf(fmaxf(__builtin_rintf(x[i] * inv) + zp, 0.0f), kLevels);
      c[i] = ok ? (uint32_t)(int32_t)r : 0u;
    }
  } else if constexpr (MODE != kChannelMode) {
    // zero, subnormal or NaN scale: all-zero codes
    const bool ok = s >= 1.17549435e-38f;
    const float inv = ok ? 1.0f / s : 0.0f;
    constexpr float lo = MODE == 0 ? -kLevels : 0.0f;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const float tq = MODE == 0 ? x[i] * inv : (x[i] - z) * inv;
      const float r = fminf(fmaxf(__builtin_rintf(tq), lo), kLevels);
      c[i] = ok ? (uint32_t)(int32_t)r : 0u;
    }
  }

  if (!active) return;
  // block_size is a power of two (checked on the host); an active slot is
  // below num_blocks * block_size and every row index below 2^31 (host
  // check), so with I32 the index math is 32-bit
  const int bsl = __builtin_ctz((unsigned)p.block_size);
  const int64_t blk = slot >> bsl;
  const int64_t off = slot & (p.block_size - 1);
  const uint32_t blk32 = (uint32_t)slot >> bsl, off32 = (uint32_t)slot & (uint32_t)(p.block_size - 1);
  if constexpr (MODE == kInlineMode) {
    // row ((blk * 2 bs + off) Hkv + h) from the K or V base: nibbles, then
    // the stored scale
    uint8_t* row = (kv ? p.v_codes : p.k_codes) +
                   (I32 ? (uint64_t)(((blk32 << (bsl + 1)) + off32) * (uint32_t)hkv + (uint32_t)h) *
                              inline_row_bytes(D)
                        : (((blk << (bsl + 1)) + off) * hkv + h) * inline_row_bytes(D));
    uint32_t w[EPL / 8] = {};
#pragma unroll
    for (int i = 0; i < EPL; ++i) w[i >> 3] |= c[i] << (4 * (i & 7));
    store_dwords<EPL / 8, true>(row + lr * BPL, w);   // inline rows are 4-byte aligned only
    if (lr == 0) *reinterpret_cast<uint32_t*>(row + P) = stbits;
    return;
  }
  const int64_t ridx = I32 ? (int64_t)(((blk32 * (uint32_t)hkv + (uint32_t)h) << bsl) + off32)
                           : (blk * hkv + h) * p.block_size + off;
  uint8_t* codes = (kv ? p.v_codes : p.k_codes) + ridx * P + lr * BPL;
  float* meta = (kv ? p.v_meta : p.k_meta) + ridx * M;   // unused when M == 0

  if constexpr (mode_bits(MODE) == 8) {
    uint32_t w[EPL / 4];
#pragma unroll
    for (int k = 0; k < EPL / 4; ++k)
      w[k] = (c[4 * k] & 0xffu) | ((c[4 * k + 1] & 0xffu) << 8) | ((c[4 * k + 2] & 0xffu) << 16) |
             ((c[4 * k + 3] & 0xffu) << 24);
    store_dwords<EPL / 4, false>(codes, w);
  } else if constexpr (MODE == 1) {
    uint32_t w[EPL / 8] = {};
#pragma unroll
    for (int i = 0; i < EPL; ++i) w[i >> 3] |= c[i] << (4 * (i & 7));
    store_dwords<EPL / 8, false>(codes, w);
  } else if constexpr (EPL == 8) {
    uint32_t w = 0;
#pragma unroll
    for (int i = 0; i < EPL; ++i) w |= c[i] << (2 * i);
    *reinterpret_cast<uint16_t*>(codes) = (uint16_t)w;
  } else {
    uint32_t w[EPL / 16] = {};
#pragma unroll
    for (int i = 0; i < EPL; ++i) w[i >> 4] |= c[i] << (2 * (i & 15));
    store_dwords<EPL / 16, false>(codes, w);
  }
  if (M > 0 && lr == 0) {
    if constexpr (M == 1) {
      meta[0] = s;
    } else {
      *reinterpret_cast<float2*>(meta) = make_float2(s, z);
    }
  }
}

// The 8-element form with one loaded vector (the fused decode step's).
template <int MODE, int D, bool ROT, bool I32 = false>
__device__ __forceinline__ void write_row_store(const WriteParams& p, uint4 raw, const float (&sg)[8], int h, int kv,
                                                int64_t slot, int lr, const float* chinv = nullptr) {
  const uint4 r[1] = {raw};
  write_row_store_n<MODE, D, ROT, I32, 8>(p, r, sg, h, kv, slot, lr, chinv);
}

}  // namespace
}  // namespace kvq
