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
  // positions at or past max_seq_len (which sizes the grid) are not written
  const int n = min(min(p.cu[b + 1] - c0, p.max_blocks << p.block_size_log2), p.max_seq_len);
  // row, table and output indices stay below 2^31 (checked on the host), so
  // the index math is 32-bit and each address one 32 x 32 -> 64-bit product
  const int rows = n * hkv * 2;
  // Workgroups go to the 8 XCDs round-robin, and gridDim.x is a multiple of
  // 8, so XCD x % 8 runs workgroups x, x + 8, ...  Of the nb8 workgroups
  // (a multiple of 8) that cover this sequence's rows, those of XCD x % 8
  // take the contiguous run (x % 8) nb8/8 .. of its row groups: neighbouring
  // row groups share 128-byte lines of per-row meta, which one L2 then
  // fetches once instead of once per XCD.
  const int nb8 = ((rows + RPB * kGatherIter - 1) / (RPB * kGatherIter) + 7) & ~7;
  if ((int)blockIdx.x >= nb8) return;
  const int bx = (blockIdx.x & 7) * (nb8 >> 3) + (blockIdx.x >> 3);
  const int r0 = bx * RPB * kGatherIter + (threadIdx.x >> 6) * RPW + lane / LPR;
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

// Rotated integer modes: R^T x_hat on the matrix cores.  With
// x_hat = c s + z (inline: s = st, z = -zp st), the Sylvester H gives
//   H x_hat = s (H c) + D z e_0
// (row 0 of H is all ones, every other row sums to zero), so
//   out_n = (d_n / sqrt(D)) (s (H c)_n + D z [n = 0]).
// H c is exact in int32 (|.| <= 128 * 127) on v_mfma_i32_16x16x64_i8 with
// A = diag(d) H (entries +-1, in LDS, built once per workgroup) and B = the
// row's codes as int8, so each output is one conversion and one product
// (plus the zero point in column 0) instead of log2 D butterfly stages.
//
// Work split: a block is 16 rows of one sequence in (K/V, position, kv
// head) order, which are 16 consecutive output rows; a wave takes NB blocks.
// Lane l holds codes 16 (l / 16) .. +15 of each 64-wide k-step of row l % 16
// (the B operand) and receives output columns 16 cb + 4 (l / 16) .. +3 of
// that row; the rows go through a per-wave LDS tile to be stored whole.
// Table entries, then codes and meta, are read for all NB blocks before one
// wait each, as in gather_kernel.
constexpr int kRotBlocks = 4;   // 16-row blocks per wave

// d offset (0..15) of byte j of a lane's 16 int8 codes of one k-step, as the
// unpack below leaves them: INT2 crumb k of byte b -> word k; INT4 the low
// nibbles of the first loaded word, its high nibbles, then the second word's.
template <int MODE>
__device__ __forceinline__ int rot_kslot(int j) {
  if constexpr (MODE == 2) return 4 * (j & 3) + (j >> 2);
  else if constexpr (code_mode(MODE) == 1) return 8 * ((j >> 2) >> 1) + 2 * (j & 3) + ((j >> 2) & 1);
  else return j;
}

template <int MODE, int D, bool BF16>
__global__ __launch_bounds__(256) void gather_rot_kernel(GatherParams p) {
  constexpr int KS = D / 64;                              // int8 k-steps
  constexpr int CB = D / 16;                              // 16-column output blocks
  constexpr int NB = kRotBlocks;
  constexpr int P = row_bytes(MODE, D);
  constexpr int RS = MODE == kInlineMode ? inline_row_bytes(D) : P;   // bytes between rows
  constexpr int M = mode_meta(MODE);
  constexpr int CBY = 16 * mode_bits(MODE) / 8;           // code bytes of a lane per k-step
  constexpr int CW = CBY >= 4 ? CBY / 4 : 1;              // ... in dwords
  constexpr int OB = BF16 ? 2 : 4;                        // output bytes per element
  constexpr int TROW = D * OB + 16;                       // LDS output tile row stride (bytes)
  constexpr int HROW = D + 16;                            // LDS H row stride (bytes)
  __shared__ __align__(16) int8_t htab[D * HROW];
  __shared__ __align__(16) uint8_t tile[4][16 * TROW];
  __shared__ int64_t obase[4][16];                        // output element offset of a tile row, -1: none

  const int b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hkv = p.hkv;
  const int c0 = p.cu[b];
  // positions at or past max_seq_len (which sizes the grid) are not written
  const int n = min(min(p.cu[b + 1] - c0, p.max_blocks << p.block_size_log2), p.max_seq_len);
  const int nh = n * hkv;                                 // rows of one of K, V (< 2^30, checked on the host)
  const int rows = 2 * nh;
  const int wbase = (blockIdx.x * 4 + wave) * 16 * NB;
  if (blockIdx.x * 4 * 16 * NB >= rows) return;           // uniform over the workgroup

  // diag(d) H in k-slot order: htab[n][k] = d_n (-1)^popcount(n & d(k)),
  // d(k) = 64 (k / 64) + 16 ((k % 64) / 16) + rot_kslot(k % 16)
  {
    constexpr int PER = D * D / 256;                      // bytes per thread (64 or 16)
    const int nn = tid / (D / PER), k0 = (tid % (D / PER)) * PER;
    const int sgn = p.signs[nn] < 0.0f ? -1 : 1;
    uint32_t w[PER / 4];
#pragma unroll
    for (int i = 0; i < PER / 4; ++i) {
      uint32_t v = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int k = k0 + 4 * i + j;
        const int d = (k & ~15) + rot_kslot<MODE>(k & 15);
        const int h = (__builtin_popcount((unsigned)(nn & d)) & 1) ? -sgn : sgn;
        v |= ((uint32_t)h & 0xffu) << (8 * j);
      }
      w[i] = v;
    }
#pragma unroll
    for (int i = 0; i < PER / 16; ++i)
      *reinterpret_cast<u32x4_t*>(htab + nn * HROW + k0 + 16 * i) = u32x4_t{w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]};
  }

  // ---- table entries of the lane's row in every block
  const int rl = lane & 15, kq = lane >> 4;
  int ids[NB], pins[NB], hh[NB], kvs[NB], orow[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int u = wbase + 16 * j + rl;
    const bool in = u < rows;
    const int kv = u >= nh ? 1 : 0;
    const int rem = u - kv * nh;
    const int pos = rem / hkv, h = rem - pos * hkv;
    kvs[j] = kv;
    hh[j] = h;
    orow[j] = in ? c0 + pos : -1;
    pins[j] = pos & ((1 << p.block_size_log2) - 1);
    ids[j] = -1;
    if (in) {
      const int32_t* trow = p.tables + (uint32_t)(p.headwise ? b * hkv + h : b) * (uint32_t)p.max_blocks;
      ids[j] = trow[pos >> p.block_size_log2];
    }
  }
  // ---- codes and meta (one wait for the table entries above)
  uint32_t raw[NB][KS][CW];
  float sv[NB], zv[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int id = ids[j], h = hh[j];
    const bool present = orow[j] >= 0 && id >= 0 && id < p.num_blocks && orow[j] < p.total_tokens;
    const uint32_t pin = (uint32_t)pins[j];
    const uint32_t src = !present ? 0u
                         : MODE == kInlineMode ? ((((uint32_t)id << (p.block_size_log2 + 1)) + pin) * hkv + h)
                                               : ((((uint32_t)id * hkv + h) << p.block_size_log2) + pin);
    const uint8_t* row = (kvs[j] ? p.v_codes : p.k_codes) + (uint64_t)src * RS;
    sv[j] = 0.0f;
    zv[j] = 0.0f;
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2)
#pragma unroll
      for (int w = 0; w < CW; ++w) raw[j][s2][w] = 0u;
    if (present) {
#pragma unroll
      for (int s2 = 0; s2 < KS; ++s2) {
        const uint8_t* cp = row + (64 * s2 + 16 * kq) * mode_bits(MODE) / 8;
        if constexpr (MODE == kInlineMode) load_bytes_a4<CBY>(raw[j][s2], cp);
        else load_bytes<CBY>(raw[j][s2], cp);
      }
      if constexpr (MODE == kInlineMode) {   // stored scale st; zero point = its low 4 bits
        const uint32_t sb = *reinterpret_cast<const uint32_t*>(row + P);
        sv[j] = __uint_as_float(sb);
        zv[j] = -(float)(sb & 0xFu) * sv[j];
      } else if constexpr (M == 2) {
        const float2 sz = *reinterpret_cast<const float2*>((kvs[j] ? p.v_meta : p.k_meta) + (uint64_t)src * 2);
        sv[j] = sz.x;
        zv[j] = sz.y;
      } else {
        sv[j] = ((kvs[j] ? p.v_meta : p.k_meta) + (uint64_t)src * M)[0];
      }
    }
  }
  __syncthreads();   // htab written

  // the A operands: (diag(d) H)[16 cb + lane % 16][64 s + 16 kq .. +15]
  u32x4_t ha[CB][KS];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2)
      ha[cb][s2] = *reinterpret_cast<const u32x4_t*>(htab + (16 * cb + rl) * HROW + 64 * s2 + 16 * kq);

  const float isd = p.inv_sqrt_d;
  const float d0 = p.signs[0] < 0.0f ? -isd : isd;        // d_0 / sqrt(D)
  uint8_t* tw = tile[wave];
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    // B operands: the row's codes as int8 in rot_kslot order
    u32x4_t bc[KS];
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2) {
      if constexpr (MODE == 2) {
        const uint32_t v = raw[j][s2][0];
        bc[s2] = u32x4_t{v & 0x03030303u, (v >> 2) & 0x03030303u, (v >> 4) & 0x03030303u, (v >> 6) & 0x03030303u};
      } else if constexpr (code_mode(MODE) == 1) {
        const uint32_t v0 = raw[j][s2][0], v1 = raw[j][s2][1];
        bc[s2] = u32x4_t{v0 & 0x0F0F0F0Fu, (v0 >> 4) & 0x0F0F0F0Fu, v1 & 0x0F0F0F0Fu, (v1 >> 4) & 0x0F0F0F0Fu};
      } else {
        bc[s2] = u32x4_t{raw[j][s2][0], raw[j][s2][1], raw[j][s2][2], raw[j][s2][3]};
      }
    }
    // the tile row's output offset (lanes 0..15 own rows 0..15)
    if (kq == 0) {
      const bool st = orow[j] >= 0 && orow[j] < p.total_tokens;
      obase[wave][rl] = st ? (int64_t)((uint32_t)(orow[j] * hkv + hh[j])) * D + (kvs[j] ? ((int64_t)1 << 62) : 0) : -1;
    }
    const float sr = sv[j] * isd;                         // s / sqrt(D); d_n is in A
    const float zr = (float)D * zv[j] * d0;               // D z d_0 / sqrt(D), column 0 only
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      i32x4_t acc = {0, 0, 0, 0};
#pragma unroll
      for (int s2 = 0; s2 < KS; ++s2) acc = mfma_i8(ha[cb][s2], bc[s2], acc);
      float o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = (float)acc[i] * sr;
      if (cb == 0 && kq == 0) o[0] = o[0] + zr;
      uint8_t* dst = tw + rl * TROW + (16 * cb + 4 * kq) * OB;
      if constexpr (BF16) *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16(o[0], o[1]), pack_bf16(o[2], o[3]));
      else *reinterpret_cast<f32x4_t*>(dst) = f32x4_t{o[0], o[1], o[2], o[3]};
    }
    // The tile and obase rows are exchanged between lanes of this wave.  LDS
    // performs one wave's accesses in issue order, so no wait is needed, but
    // the compiler sees only one lane: without this barrier it may keep an
    // earlier block's obase value in a register for lanes that wrote none.
    asm volatile("" ::: "memory");
    // whole rows out: 16 bytes a lane, non-temporal
    constexpr int LPR = D * OB / 16;                      // lanes per row
    constexpr int RPI = 64 / LPR;                         // rows per store instruction
#pragma unroll
    for (int it = 0; it < 16 / RPI; ++it) {
      const int r = it * RPI + lane / LPR, c = lane % LPR;
      const int64_t ob = obase[wave][r];
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(tw + r * TROW + 16 * c);
      if (ob >= 0) {
        const bool isv = (ob >> 62) != 0;
        const int64_t e0 = (ob & (((int64_t)1 << 62) - 1)) + c * (16 / OB);
        void* out = isv ? p.v_out : p.k_out;
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(reinterpret_cast<uint8_t*>(out) + e0 * OB));
      }
    }
    asm volatile("" ::: "memory");   // the next block's tile writes stay below these reads
  }
}

template <int MODE, int D, bool ROT>
hipError_t launch_gather_t(const GatherParams& p, hipStream_t s) {
  if constexpr (ROT && MODE != kFp8Mode) {
    constexpr int RPW = 4 * 16 * kRotBlocks;   // rows per workgroup
    const int64_t rows = (int64_t)p.max_seq_len * p.hkv * 2;
    const int64_t gx = (rows + RPW - 1) / RPW;
    if (gx == 0 || p.num_seqs == 0) return hipSuccess;
    const dim3 grid((unsigned)gx, (unsigned)p.num_seqs);
    if (p.out_bf16)
      hipLaunchKernelGGL((gather_rot_kernel<MODE, D, true>), grid, dim3(256), 0, s, p);
    else
      hipLaunchKernelGGL((gather_rot_kernel<MODE, D, false>), grid, dim3(256), 0, s, p);
    return hipGetLastError();
  }
  constexpr int RPB = 4 * (64 / (D / 8)) * kGatherIter;
  const int64_t rows = (int64_t)p.max_seq_len * p.hkv * 2;
  const int64_t gx = ((rows + RPB - 1) / RPB + 7) & ~7LL;   // a multiple of the XCD count
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

// The fewest rows any gather workgroup covers (the host bounds the grid with
// it; the launch pads grid.x to a multiple of 8 beyond that).
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
