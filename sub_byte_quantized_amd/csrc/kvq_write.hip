// Quantize-on-write: bf16 K/V rows -> (optional) Hadamard rotation ->
// per-(token, kv head) scale and zero point -> round -> pack -> paged store.
//
// Follows the write half of the prhub summary of vLLM PR 40835 ("INT4
// per-token-head KV cache quantization for the Triton backend", 实现拆解
// item 2: the write kernel applies the randomized Hadamard transform, computes
// one scale and zero point per token and head, and packs nibbles) and the
// encoder/decoder cache-write kernels of FastDeploy PR 5173 ("support dynamic
// int2 quantization cache kv").  The arithmetic is the float32 sequence the
// cache format defines, so codes are reproducible bit for bit:
//   y = fl(FWHT(d .* x) * fl(1/sqrt(D)))   stages h = 1, 2, 4, ..., D/2
//   INT8: s = max|y| / 127,            c = clamp(rint(y * (1/s)), -127, 127)
//   INT4/INT2: s = (max y - min y) / L, z = min y,
//              c = clamp(rint((y - z) * (1/s)), 0, L)
// with correctly rounded divisions and no fused multiply-adds.
//
// Work split: one row = one (token, kv head) of K or of V.  D/8 lanes own a
// row, 8 elements per lane (one 16-byte load), so a wave64 handles 128/D*4
// rows and a 256-thread workgroup 16 (D=128) or 32 (D=64) rows.  The FWHT
// runs in registers for the three in-lane stages and across lanes for the
// rest; min/max/absmax are lane reductions.  Stores are the lane's slice of
// the packed row (4 bytes for INT4, 8 for INT8, 2 for INT2) plus one meta
// store per row.
#pragma clang fp contract(off)

#include "kvq_internal.h"

namespace kvq {
namespace {

template <int MODE, int D, bool ROT>
__global__ __launch_bounds__(256) void write_kernel(WriteParams p) {
  constexpr int LPR = D / 8;             // lanes per row
  constexpr int RPW = 64 / LPR;          // rows per wave
  constexpr int RPB = 4 * RPW;           // rows per workgroup
  constexpr int P = row_bytes(MODE, D);  // packed bytes per row
  constexpr int BPL = P / LPR;           // packed bytes per lane
  constexpr int M = mode_meta(MODE);
  constexpr float kLevels = (float)mode_levels(MODE);

  const int lane = threadIdx.x & 63;
  const int lr = lane & (LPR - 1);
  const int64_t row = (int64_t)blockIdx.x * RPB + (threadIdx.x >> 6) * RPW + lane / LPR;
  const int hkv = p.hkv;
  const int64_t t = row / (2 * hkv);
  const int h = (int)((row >> 1) % hkv);
  const int kv = (int)(row & 1);

  int64_t slot = -1;
  if (row < p.total_rows) slot = p.slot_hw ? p.slot_hw[t * hkv + h] : p.slot[t];
  const bool active = slot >= 0;

  float x[8];
  if (active) {
    const uint16_t* src = kv ? p.value + t * p.value_stride : p.key + t * p.key_stride;
    const uint4 raw = *reinterpret_cast<const uint4*>(src + (int64_t)h * D + lr * 8);
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = 0.0f;
  }

  if constexpr (ROT) {
    const float4 s0 = *reinterpret_cast<const float4*>(p.signs + lr * 8);
    const float4 s1 = *reinterpret_cast<const float4*>(p.signs + lr * 8 + 4);
    x[0] *= s0.x; x[1] *= s0.y; x[2] *= s0.z; x[3] *= s0.w;
    x[4] *= s1.x; x[5] *= s1.y; x[6] *= s1.z; x[7] *= s1.w;
    // in-lane butterflies, pairs (i, i + hh) with bit hh of i clear
#pragma unroll
    for (int hh = 1; hh < 8; hh <<= 1) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (!(i & hh)) {
          const float a = x[i], b = x[i + hh];
          x[i] = a + b;
          x[i + hh] = a - b;
        }
      }
    }
    // cross-lane butterflies: element stride 8*m lives m lanes away
#pragma unroll
    for (int m = 1; m < LPR; m <<= 1) {
      const bool upper = (lr & m) != 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float o = __shfl_xor(x[i], m);
        x[i] = upper ? (o - x[i]) : (x[i] + o);
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = x[i] * p.inv_sqrt_d;
  }

  float s, z;
  if constexpr (MODE == 0) {
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) a = fmaxf(a, fabsf(x[i]));
#pragma unroll
    for (int m = 1; m < LPR; m <<= 1) a = fmaxf(a, __shfl_xor(a, m));
    s = a / kLevels;
    z = 0.0f;
  } else {
    float mn = x[0], mx = x[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) {
      mn = fminf(mn, x[i]);
      mx = fmaxf(mx, x[i]);
    }
#pragma unroll
    for (int m = 1; m < LPR; m <<= 1) {
      mn = fminf(mn, __shfl_xor(mn, m));
      mx = fmaxf(mx, __shfl_xor(mx, m));
    }
    s = (mx - mn) / kLevels;
    z = mn;
  }

  // zero, subnormal or NaN scale: all-zero codes
  const bool ok = s >= 1.17549435e-38f;
  const float inv = ok ? 1.0f / s : 0.0f;
  constexpr float lo = MODE == 0 ? -kLevels : 0.0f;
  uint32_t c[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float tq = MODE == 0 ? x[i] * inv : (x[i] - z) * inv;
    const float r = fminf(fmaxf(__builtin_rintf(tq), lo), kLevels);
    c[i] = ok ? (uint32_t)(int32_t)r : 0u;
  }

  if (!active) return;
  const int64_t blk = slot / p.block_size;
  const int64_t off = slot - blk * p.block_size;
  const int64_t ridx = (blk * hkv + h) * p.block_size + off;
  uint8_t* codes = (kv ? p.v_codes : p.k_codes) + ridx * P + lr * BPL;
  float* meta = (kv ? p.v_meta : p.k_meta) + ridx * M;

  if constexpr (MODE == 0) {
    uint2 w;
    w.x = (c[0] & 0xffu) | ((c[1] & 0xffu) << 8) | ((c[2] & 0xffu) << 16) | ((c[3] & 0xffu) << 24);
    w.y = (c[4] & 0xffu) | ((c[5] & 0xffu) << 8) | ((c[6] & 0xffu) << 16) | ((c[7] & 0xffu) << 24);
    *reinterpret_cast<uint2*>(codes) = w;
  } else if constexpr (MODE == 1) {
    uint32_t w = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) w |= c[i] << (4 * i);
    *reinterpret_cast<uint32_t*>(codes) = w;
  } else {
    uint32_t w = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) w |= c[i] << (2 * i);
    *reinterpret_cast<uint16_t*>(codes) = (uint16_t)w;
  }
  if (lr == 0) {
    if constexpr (M == 1) {
      meta[0] = s;
    } else {
      *reinterpret_cast<float2*>(meta) = make_float2(s, z);
    }
  }
}

__global__ __launch_bounds__(256) void fill_zero_kernel(uint4* p, size_t n16) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = make_uint4(0, 0, 0, 0);
}

template <int MODE, int D, bool ROT>
hipError_t launch_write_t(const WriteParams& p, hipStream_t s) {
  constexpr int RPB = 4 * (64 / (D / 8));
  const int64_t blocks = (p.total_rows + RPB - 1) / RPB;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((write_kernel<MODE, D, ROT>), dim3((unsigned)blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

template <int MODE>
hipError_t launch_write_m(int d, bool rot, const WriteParams& p, hipStream_t s) {
  if (d == 64) return rot ? launch_write_t<MODE, 64, true>(p, s) : launch_write_t<MODE, 64, false>(p, s);
  return rot ? launch_write_t<MODE, 128, true>(p, s) : launch_write_t<MODE, 128, false>(p, s);
}

}  // namespace

hipError_t launch_write(int mode, int d, bool rot, const WriteParams& p, hipStream_t s) {
  switch (mode) {
    case 0: return launch_write_m<0>(d, rot, p, s);
    case 1: return launch_write_m<1>(d, rot, p, s);
    default: return launch_write_m<2>(d, rot, p, s);
  }
}

hipError_t launch_fill_zero(void* ptr, size_t bytes, hipStream_t s) {
  const size_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  const size_t blocks = n16 / 256 + 1 < 4096 ? n16 / 256 + 1 : 4096;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                     reinterpret_cast<uint4*>(ptr), n16);
  return hipGetLastError();
}

}  // namespace kvq
