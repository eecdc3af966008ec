// Device helpers shared by the libkvq HIP kernels (gfx950): MFMA wrappers,
// cross-lane reductions, bf16 packing, raw byte loads and the in-register
// query rotation.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));

constexpr float kNegInf = -__builtin_inff();
constexpr uint32_t kMagic = 0x43004300u;  // bf16 128.0 in both halves
constexpr float kRescale = 8.0f;          // log2 of the growth that forces a rescale

__device__ __forceinline__ f32x4_t mfma(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ i32x4_t mfma_i8(u32x4_t a, u32x4_t b, i32x4_t c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4_t, a), __builtin_bit_cast(i32x4_t, b),
                                               c, 0, 0, 0);
}

// (x & m) | (c & ~m).  With m and c held in VGPRs this is one v_bitop3_b32
// (with literal or scalar constants the compiler emits an and plus an or).
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t m, uint32_t c) { return (x & m) | (c & ~m); }

// Copy a wave-uniform value into a VGPR the optimizer cannot fold back into a
// scalar or a literal.  Used once per kernel for the and_or() constants; the
// result only feeds ordinary VALU instructions.
__device__ __forceinline__ uint32_t to_vgpr(uint32_t x) {
  uint32_t r;
  asm("v_mov_b32 %0, %1" : "=v"(r) : "s"(x));
  return r;
}

// Cross-lane reductions without LDS round trips.  v_permlane16_swap /
// v_permlane32_swap applied to (x, x) return x and its partner lane l^16 /
// l^32 in the two results; DPP quad_perm gives lanes l^1 and l^2.  Both lanes
// of a pair compute the same commutative op on the same two values, so they
// agree bit for bit.
__device__ __forceinline__ float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float add_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float add_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// lane l ^ M for M = 1 or 2 (within a quad)
template <int M>
__device__ __forceinline__ float quad_xor(float x) {
  constexpr int sel = M == 1 ? 0xB1 : 0x4E;   // quad_perm [1,0,3,2] / [2,3,0,1]
  return __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(x), sel, 0xF, 0xF, false));
}

// x from lane l ^ m, m = 1, 2, 4 or 8, partners inside aligned 16-lane rows
// (m a constant after unrolling): DPP quad permutes for 1 and 2, a rotate by
// 8 within the 16-lane DPP row for 8 (equal to xor 8 there), a bitmask
// swizzle for 4; none goes through LDS memory.  Both lanes of a pair must be
// active.
__device__ __forceinline__ float xor_in_row(float x, int m) {
  // plain DPP moves (no old value to merge, so no zeroed destination first)
  switch (m) {
    case 1: return __uint_as_float(__builtin_amdgcn_mov_dpp(__float_as_uint(x), 0xB1, 0xF, 0xF, true));
    case 2: return __uint_as_float(__builtin_amdgcn_mov_dpp(__float_as_uint(x), 0x4E, 0xF, 0xF, true));
    case 4: return __uint_as_float(__builtin_amdgcn_ds_swizzle(__float_as_uint(x), 0x101F));
    default: return __uint_as_float(__builtin_amdgcn_mov_dpp(__float_as_uint(x), 0x128, 0xF, 0xF, true));
  }
}

// x from lane l ^ m for m = 1 .. 32 (a constant after unrolling), with no
// LDS round trip: xor_in_row below 16; for 16 and 32 a permlane swap of
// (x, x), whose two results are x and the partner's value in a lane-dependent
// order, so the partner's bits are r0 ^ r1 ^ x.  All 64 lanes must be active.
__device__ __forceinline__ float lane_xor(float x, int m) {
  if (m < 16) return xor_in_row(x, m);
  const uint32_t b = __float_as_uint(x);
  const auto r = m == 16 ? __builtin_amdgcn_permlane16_swap(b, b, false, false)
                         : __builtin_amdgcn_permlane32_swap(b, b, false, false);
  return __uint_as_float(r[0] ^ r[1] ^ b);
}

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  bf16x2_t v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two exact small integers held as floats -> bf16 pair (the dropped mantissa
// bits are zero for values < 256).
__device__ __forceinline__ uint32_t pack_exact(float a, float b) {
  return __builtin_amdgcn_perm(__float_as_uint(b), __float_as_uint(a), 0x07060302u);
}

// N bytes from an address that is only 4-byte aligned (rows of the inline
// layout): dword vectors declared with 4-byte alignment.
typedef uint32_t u32x4a4_t __attribute__((ext_vector_type(4), aligned(4)));
typedef uint32_t u32x2a4_t __attribute__((ext_vector_type(2), aligned(4)));
template <int N>
__device__ __forceinline__ void load_bytes_a4(uint32_t* dst, const uint8_t* src) {
  static_assert(N % 4 == 0, "whole dwords");
  if constexpr (N >= 16) {
#pragma unroll
    for (int i = 0; i < N / 16; ++i) {
      const u32x4a4_t a = reinterpret_cast<const u32x4a4_t*>(src)[i];
      dst[4 * i] = a[0]; dst[4 * i + 1] = a[1]; dst[4 * i + 2] = a[2]; dst[4 * i + 3] = a[3];
    }
  } else if constexpr (N == 8) {
    const u32x2a4_t a = *reinterpret_cast<const u32x2a4_t*>(src);
    dst[0] = a[0]; dst[1] = a[1];
  } else {
    dst[0] = *reinterpret_cast<const uint32_t*>(src);
  }
}

template <int N>
__device__ __forceinline__ void load_bytes(uint32_t* dst, const uint8_t* src) {
  if constexpr (N >= 16) {
#pragma unroll
    for (int i = 0; i < N / 16; ++i) {
      const uint4 a = reinterpret_cast<const uint4*>(src)[i];
      dst[4 * i] = a.x; dst[4 * i + 1] = a.y; dst[4 * i + 2] = a.z; dst[4 * i + 3] = a.w;
    }
  } else if constexpr (N == 8) {
    const uint2 a = *reinterpret_cast<const uint2*>(src);
    dst[0] = a.x; dst[1] = a.y;
  } else if constexpr (N == 4) {
    dst[0] = *reinterpret_cast<const uint32_t*>(src);
  } else if constexpr (N == 2) {
    dst[0] = *reinterpret_cast<const uint16_t*>(src);
  } else {
    dst[0] = *src;
  }
}

// In-register Sylvester FWHT of one row (natural order, unnormalized).  The
// stages h = 1, 2, ..., D/2 run in that order: stage h maps the pair
// (d, d + h), bit h of d clear, to (x_d + x_{d+h}, x_d - x_{d+h}); within the
// lane for h < E, across lanes (lane ^ h/E) otherwise, with DPP and
// permlane moves (all 64 lanes active).
template <int D>
__device__ __forceinline__ void wave_fwht(float (&x)[D / 64], int lane) {
  constexpr int E = D / 64;
  if constexpr (E == 2) {
    const float a = x[0], b = x[1];
    x[0] = a + b;
    x[1] = a - b;
  }
#pragma unroll
  for (int hl = 1; hl < 64; hl <<= 1) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float y = lane_xor(x[e], hl);
      x[e] = (lane & hl) ? y - x[e] : x[e] + y;
    }
  }
}

// The lane's E bf16 values of a query row, as loaded (one dword or one short).
template <int D>
__device__ __forceinline__ uint32_t load_qrow(const uint16_t* src, int lane) {
  if constexpr (D == 128) return reinterpret_cast<const uint32_t*>(src)[lane];
  else return src[lane];
}

}  // namespace
}  // namespace kvq
