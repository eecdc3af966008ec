// Dequantize-gather: materialize the un-rotated K and V of given sequences
// out of the quantized paged cache, as dense [token, kv head, D] rows.
//
// The operation is the cache-fetch-and-dequantize custom operator named in the
// review thread of FastDeploy PR 5173 ("[Feature] support dynamic int2
// quantization cache kv"), and the gather-and-dequantize that prefill applies
// to the paged cache in the vllm-ascend-quantized-kv-cache package (运行机制).
// Per row (position j of sequence b, kv head h, K or V):
//   x_hat = c*s (+ z)             float32, product then sum (no contraction)
//   out   = R^T x_hat = (1/sqrt(D)) d .* (H x_hat)   when the cache is rotated
// with the block id read from the uniform table row b or the head-wise row
// b*Hkv + h; a -1 entry (an evicted sliding-window block, FastDeploy PR 7718)
// gives a zero row and no cache address is formed.
//
// Work split: HBM streaming.  D/8 lanes own a row, 8 elements per lane: the
// lane's packed bytes (8 INT8, 4 INT4, 2 INT2) and the row's meta in one load
// each, 16 (bf16) or 32 (float32) bytes stored.  A 256-thread workgroup takes
// ITER groups of 16 (D 128) or 32 (D 64) consecutive rows of one sequence, in
// (position, kv head, K/V) order: all their table entries are read, then all
// their codes and meta, before the first use.  grid.y is the sequence; grid.x covers max_seq_len positions.
#pragma clang fp contract(off)

#include "kvq_internal.h"
#include "kvq_device.h"

namespace kvq {
namespace {

constexpr int kGatherIter = 4;

template <int MODE, int D, bool ROT, bool BF16>
__global__ __launch_bounds__(256) void gather_kernel(GatherParams p) {
  constexpr int LPR = D / 8;                    // lanes per row
  constexpr int RPW = 64 / LPR;                 // rows per wave
  constexpr int RPB = 4 * RPW;                  // rows per workgroup and iteration
  constexpr int P = row_bytes(MODE, D);
  constexpr int M = mode_meta(MODE);
  constexpr int BPL = P / LPR;                  // packed bytes per lane

  const int b = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int lr = lane & (LPR - 1);
  const int hkv = p.hkv;
  const int c0 = p.cu[b];
  const int n = min(p.cu[b + 1] - c0, p.max_blocks << p.block_size_log2);
  // row, table and output indices stay below 2^31 (checked on the host), so
  // the index math is 32-bit and each address one 32 x 32 -> 64-bit product
  const int rows = n * hkv * 2;
  const int r0 = blockIdx.x * RPB * kGatherIter + (threadIdx.x >> 6) * RPW + lane / LPR;
  if (r0 >= rows) return;

  // the lane's rotation signs, read before any store (so not reloaded per row)
  float sg[8] = {1.0f, 1.0f, 1.0f, 1.0f, 1.0f, 1.0f, 1.0f, 1.0f};
  if constexpr (ROT) {
    const float4 s0 = *reinterpret_cast<const float4*>(p.signs + lr * 8);
    const float4 s1 = *reinterpret_cast<const float4*>(p.signs + lr * 8 + 4);
    sg[0] = s0.x; sg[1] = s0.y; sg[2] = s0.z; sg[3] = s0.w;
    sg[4] = s1.x; sg[5] = s1.y; sg[6] = s1.z; sg[7] = s1.w;
  }
  uint32_t raw[kGatherIter][BPL >= 4 ? BPL / 4 : 1];
  float s[kGatherIter], z[kGatherIter];
  bool present[kGatherIter];
  int orow[kGatherIter], pins[kGatherIter], ids[kGatherIter];
  int hh[kGatherIter], kvs[kGatherIter];
  // Three phases, so each wait covers one kind of load: every row's table
  // entry, then (one wait) every row's codes and meta, then the
  // dequantization and stores.  r = pos * 2 Hkv + 2 h + kv: one division for
  // the first row, then steps of RPB rows.
  int pos = r0 / (2 * hkv);
  int rem = r0 - pos * 2 * hkv;
#pragma unroll
  for (int it = 0; it < kGatherIter; ++it) {
    const int r = r0 + it * RPB;
    if (it > 0) {
      rem += RPB;
      while (rem >= 2 * hkv) {
        rem -= 2 * hkv;
        ++pos;
      }
    }
    const bool in = r < rows;
    const int h = rem >> 1;
    hh[it] = h;
    kvs[it] = rem & 1;
    orow[it] = in ? c0 + pos : -1;
    pins[it] = pos & ((1 << p.block_size_log2) - 1);
    ids[it] = -1;
    if (in) {
      const int32_t* trow = p.tables + (uint32_t)(p.headwise ? b * hkv + h : b) * (uint32_t)p.max_blocks;
      ids[it] = trow[pos >> p.block_size_log2];
    }
  }
#pragma unroll
  for (int it = 0; it < kGatherIter; ++it) {
    const int id = ids[it], h = hh[it], kv = kvs[it];
    present[it] = orow[it] >= 0 && id >= 0 && id < p.num_blocks && orow[it] < p.total_tokens;
    const uint32_t pin = (uint32_t)pins[it];
    // plane row (id Hkv + h) bs + offset; inline row (id 2 bs + offset) Hkv + h
    const uint32_t src = !present[it] ? 0u
                         : MODE == kInlineMode ? ((((uint32_t)id << (p.block_size_log2 + 1)) + pin) * hkv + h)
                                               : ((((uint32_t)id * hkv + h) << p.block_size_log2) + pin);
    const uint8_t* codes = (kv ? p.v_codes : p.k_codes) +
                           (uint64_t)src * (MODE == kInlineMode ? inline_row_bytes(D) : P) + lr * BPL;
    const float* meta = (kv ? p.v_meta : p.k_meta) + (uint64_t)src * M;   // unused when M == 0
    if (present[it]) {
      load_bytes<BPL>(raw[it], codes);
      if constexpr (MODE == kInlineMode) {   // stored scale st; zero point = its low 4 bits
        const uint32_t sb = *reinterpret_cast<const uint32_t*>(codes - lr * BPL + P);
        s[it] = __uint_as_float(sb);
        z[it] = (float)(sb & 0xFu);
      } else if constexpr (M == 0) {   // per-channel scales, read below
        s[it] = 1.0f;
        z[it] = 0.0f;
      } else if constexpr (M == 2) {
        const float2 sz = *reinterpret_cast<const float2*>(meta);
        s[it] = sz.x;
        z[it] = sz.y;
      } else {
        s[it] = meta[0];
        z[it] = 0.0f;
      }
    } else {
#pragma unroll
      for (int w = 0; w < (BPL >= 4 ? BPL / 4 : 1); ++w) raw[it][w] = 0;
      s[it] = 0.0f;
      z[it] = 0.0f;
    }
  }

#pragma unroll
  for (int it = 0; it < kGatherIter; ++it) {
    if (orow[it] < 0 || orow[it] >= p.total_tokens) continue;
    // per-channel INT8: the lane's 8 channel scales of (K or V, kv head)
    float sc[8] = {1.0f, 1.0f, 1.0f, 1.0f, 1.0f, 1.0f, 1.0f, 1.0f};
    if constexpr (MODE == kChannelMode) {
      const float* cs = p.chs + ((int64_t)kvs[it] * hkv + hh[it]) * D + lr * 8;
      const float4 s0 = *reinterpret_cast<const float4*>(cs);
      const float4 s1 = *reinterpret_cast<const float4*>(cs + 4);
      sc[0] = s0.x; sc[1] = s0.y; sc[2] = s0.z; sc[3] = s0.w;
      sc[4] = s1.x; sc[5] = s1.y; sc[6] = s1.z; sc[7] = s1.w;
    }
    float x[8];
    if constexpr (MODE == kFp8Mode) {   // E4M3 values, exact in float32, times the row scale
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)raw[it][w], false);
        const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)raw[it][w], true);
        x[4 * w] = lo[0] * s[it]; x[4 * w + 1] = lo[1] * s[it];
        x[4 * w + 2] = hi[0] * s[it]; x[4 * w + 3] = hi[1] * s[it];
      }
    }
#pragma unroll
    for (int i = 0; i < 8 && MODE != kFp8Mode; ++i) {
      int c;
      if constexpr (MODE == 0 || MODE == kChannelMode) c = (int)(int8_t)((raw[it][i >> 2] >> (8 * (i & 3))) & 0xffu);
      else if constexpr (code_mode(MODE) == 1) c = (int)((raw[it][0] >> (4 * i)) & 0xFu);
      else c = (int)((raw[it][0] >> (2 * i)) & 0x3u);
      if constexpr (MODE == kInlineMode) {   // (c - zp) st: an exact small integer times st
        x[i] = ((float)c - z[it]) * s[it];
        continue;
      }
      const float cs = (float)c * (MODE == kChannelMode ? sc[i] : s[it]);
      x[i] = M == 2 ? cs + z[it] : cs;
    }
    if (!present[it]) {
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = 0.0f;
    }
    if constexpr (ROT) {
      // H x: in-lane butterflies (element strides 1, 2, 4), then across the
      // row's lanes (element stride 8m lives m lanes away)
#pragma unroll
      for (int hs = 1; hs < 8; hs <<= 1) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          if (!(i & hs)) {
            const float a = x[i], c = x[i + hs];
            x[i] = a + c;
            x[i + hs] = a - c;
          }
        }
      }
#pragma unroll
      for (int m = 1; m < LPR; m <<= 1) {
        // x + o in the lower lane, o - x in the upper one, as one fma with a
        // +-1 factor (the product is exact, so the single rounding is the sum's)
        const float sgn = (lr & m) ? -1.0f : 1.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = __builtin_fmaf(x[i], sgn, xor_in_row(x[i], m));
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = x[i] * sg[i] * p.inv_sqrt_d;
    }
    // non-temporal stores: the dense rows are written once and not read back
    // by this kernel, so they need not stay in the caches
    const uint64_t e0 = (uint64_t)(uint32_t)(orow[it] * hkv + hh[it]) * D + lr * 8;
    void* out = kvs[it] ? p.v_out : p.k_out;
    if constexpr (BF16) {
      const u32x4_t w = {pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3]), pack_bf16(x[4], x[5]), pack_bf16(x[6], x[7])};
      __builtin_nontemporal_store(w, reinterpret_cast<u32x4_t*>(reinterpret_cast<uint16_t*>(out) + e0));
    } else {
      f32x4_t* o = reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(out) + e0);
      const f32x4_t a = {x[0], x[1], x[2], x[3]}, c = {x[4], x[5], x[6], x[7]};
      __builtin_nontemporal_store(a, o);
      __builtin_nontemporal_store(c, o + 1);
    }
  }
}

template <int MODE, int D, bool ROT>
hipError_t launch_gather_t(const GatherParams& p, hipStream_t s) {
  constexpr int RPB = 4 * (64 / (D / 8)) * kGatherIter;
  const int64_t rows = (int64_t)p.max_seq_len * p.hkv * 2;
  const int64_t gx = (rows + RPB - 1) / RPB;
  if (gx == 0 || p.num_seqs == 0) return hipSuccess;
  const dim3 grid((unsigned)gx, (unsigned)p.num_seqs);
  if (p.out_bf16)
    hipLaunchKernelGGL((gather_kernel<MODE, D, ROT, true>), grid, dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((gather_kernel<MODE, D, ROT, false>), grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

template <int MODE>
hipError_t launch_gather_m(int d, bool rot, const GatherParams& p, hipStream_t s) {
  if constexpr (MODE == kChannelMode) {   // no rotation in this mode (checked on the host)
    return d == 64 ? launch_gather_t<MODE, 64, false>(p, s) : launch_gather_t<MODE, 128, false>(p, s);
  } else {
    if (d == 64) return rot ? launch_gather_t<MODE, 64, true>(p, s) : launch_gather_t<MODE, 64, false>(p, s);
    return rot ? launch_gather_t<MODE, 128, true>(p, s) : launch_gather_t<MODE, 128, false>(p, s);
  }
}

}  // namespace

int64_t gather_rows_per_workgroup(int d) { return 4LL * (64 / (d / 8)) * kGatherIter; }

hipError_t launch_gather(int mode, int d, bool rot, const GatherParams& p, hipStream_t s) {
  switch (mode) {
    case 0: return launch_gather_m<0>(d, rot, p, s);
    case 1: return launch_gather_m<1>(d, rot, p, s);
    case 2: return launch_gather_m<2>(d, rot, p, s);
    case kChannelMode: return launch_gather_m<kChannelMode>(d, rot, p, s);
    case kFp8Mode: return launch_gather_m<kFp8Mode>(d, rot, p, s);
    default: return launch_gather_m<kInlineMode>(d, rot, p, s);
  }
}

}  // namespace kvq
