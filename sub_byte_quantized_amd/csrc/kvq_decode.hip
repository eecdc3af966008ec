// Split-KV paged decode attention over the quantized cache.
//
// Follows the read half of the prhub summary of vLLM PR 40835 ("INT4
// per-token-head KV cache quantization for the Triton backend", 实现拆解
// item 2: unpack, dequantize, attend), the head-wise block-table walk of
// FastDeploy PR 7718 ("Optimize AppendAttention for discrete head-wise
// block_idx": per-head rows, -1 entries skipped before any K/V address is
// formed), and the decode-side dequantization inside attention described in
// the vllm-ascend-quantized-kv-cache package (运行机制).
//
// What is computed, per (sequence b, q head hq, kv head h = hq / G):
//   out = R^T softmax_j(scale * q'.k_hat_j) v_hat_j ,  q' = R q
// where k_hat/v_hat are the stored codes dequantized in the rotated basis
// (x_hat = c*s + z) and R the cache's rotation (identity without signs).
// The dot products never dequantize element by element:
//   q'.k_hat_t = s_t (q'.c_t) + z_t sum(q')
//   sum_t w_t v_hat_t = sum_t (p_t s_t) c_t + (sum_t p_t z_t) 1
// and both contractions run on MFMA (v_mfma_f32_16x16x32_bf16) with the codes
// as exact bf16 integers 128 + c (built with one and-or per two codes), the
// query and the weights split into bf16 hi + lo, and the 128 offset removed by
// seeding the accumulators with -128 * (sum of the other operand).
//
// Work split: one wave per (split, kv head, sequence).  A split is a run of
// 32-position chunks of the sequence's active range (positions inside the
// window).  Each chunk is two 16-token MFMA tiles; a tile lies in one cache
// block (block_size is a multiple of 16) and is skipped when its block id is
// negative or it lies outside [window start, seq_len).
//   K pass  A = codes [16 tokens x 32 d]     lane (token, d-group)
//           B = q'    [32 d x 16 heads]      lane (head,  d-group)
//           C = scores[16 tokens x 16 heads] lane (head, 4 tokens)
//   V pass  A = codes^T [16 d x 32 tokens]   lane (d-group, 8 tokens)
//           B = w^T   [32 tokens x 16 heads] lane (head, 8 tokens): the K
//                       pass's C registers of two tiles, no shuffle needed
//           C = acc   [16 d x 16 heads]      lane (head, 4 d-slots)
// Heads beyond G carry zeros.  With more than one split, every wave writes
// (m, l, acc) to the workspace, and the last wave of a (sequence, kv head)
// (device-scope counter) combines them, applies R^T and stores.
#include "kvq_internal.h"

namespace kvq {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr float kNegInf = -__builtin_inff();
constexpr uint32_t kMagic = 0x43004300u;  // bf16 128.0 in both halves

__device__ __forceinline__ f32x4_t mfma(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  bf16x2_t v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Pack two exact small integers held as floats into a bf16 pair (truncation
// of the low mantissa bits is exact for values < 256).
__device__ __forceinline__ uint32_t pack_exact(float a, float b) {
  return __builtin_amdgcn_perm(__float_as_uint(b), __float_as_uint(a), 0x07060302u);
}

// d index held by MFMA k-slot j of lane group kg in k-step k (K pass); the
// same map lays out the query operand.  It follows the unpacking order below.
template <int MODE, int D>
__device__ __forceinline__ int kmap(int kg, int k, int j) {
  const int base = kg * (D / 4);
  if constexpr (MODE == 1) return base + 8 * k + (j >> 1) + 4 * (j & 1);
  else if constexpr (MODE == 2) return base + 16 * (k >> 1) + 4 * (k & 1) + (j >> 1) + 8 * (j & 1);
  else return base + 8 * k + j;
}

// Number of dwords a lane loads from one K row (P/4 bytes) and from one V row
// (P/16 bytes, at least one dword register).
template <int MODE, int D> struct Geo {
  static constexpr int P = row_bytes(MODE, D);
  static constexpr int KW = P / 16;              // dwords of K codes per lane per tile
  static constexpr int VB = P / 16;              // bytes of V codes per lane per token
  static constexpr int VW = VB >= 4 ? VB / 4 : 1;
  static constexpr int KSTEPS = D / 32;
  static constexpr int DT = D / 16;              // d-tiles of the V pass
  static constexpr int M = mode_meta(MODE);
};

// K-pass A operand: exact bf16 (128 + c) of the 8 codes of k-step k.
template <int MODE, int D>
__device__ __forceinline__ u32x4_t unpack_k(const uint32_t* kc, int k) {
  u32x4_t a;
  if constexpr (MODE == 1) {
    const uint32_t x = kc[k];
    a[0] = (x & 0x000F000Fu) | kMagic;
    a[1] = ((x >> 4) & 0x000F000Fu) | kMagic;
    a[2] = ((x >> 8) & 0x000F000Fu) | kMagic;
    a[3] = ((x >> 12) & 0x000F000Fu) | kMagic;
  } else if constexpr (MODE == 2) {
    const uint32_t x = kc[k >> 1] >> (8 * (k & 1));
    a[0] = (x & 0x00030003u) | kMagic;
    a[1] = ((x >> 2) & 0x00030003u) | kMagic;
    a[2] = ((x >> 4) & 0x00030003u) | kMagic;
    a[3] = ((x >> 6) & 0x00030003u) | kMagic;
  } else {
    const uint32_t x0 = kc[2 * k] ^ 0x80808080u, x1 = kc[2 * k + 1] ^ 0x80808080u;
    a[0] = pack_exact((float)(x0 & 0xffu), (float)((x0 >> 8) & 0xffu));
    a[1] = pack_exact((float)((x0 >> 16) & 0xffu), (float)(x0 >> 24));
    a[2] = pack_exact((float)(x1 & 0xffu), (float)((x1 >> 8) & 0xffu));
    a[3] = pack_exact((float)((x1 >> 16) & 0xffu), (float)(x1 >> 24));
  }
  return a;
}

// V-pass A operand for d-tile dt: token slots 0..7 (pairs 2p, 2p+1) of the
// lane's d = d-group*(D/16) + dt, as exact bf16 (128 + c).
template <int MODE, int D, int DTI>
__device__ __forceinline__ u32x4_t unpack_v(const uint32_t (*vc)[Geo<MODE, D>::VW]) {
  u32x4_t a;
  if constexpr (MODE == 1) {
    constexpr int b = DTI >> 1;
    constexpr uint32_t sel = (uint32_t)b | (0x0Cu << 8) | ((uint32_t)(4 + b) << 16) | (0x0Cu << 24);
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t y = __builtin_amdgcn_perm(vc[2 * p + 1][0], vc[2 * p][0], sel);
      a[p] = (((DTI & 1) ? (y >> 4) : y) & 0x000F000Fu) | kMagic;
    }
  } else if constexpr (MODE == 2) {
    constexpr int b = DTI >> 2;
    constexpr int sh = 2 * (DTI & 3);
    constexpr uint32_t sel = (uint32_t)b | (0x0Cu << 8) | ((uint32_t)(4 + b) << 16) | (0x0Cu << 24);
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t y = __builtin_amdgcn_perm(vc[2 * p + 1][0], vc[2 * p][0], sel);
      a[p] = ((y >> sh) & 0x00030003u) | kMagic;
    }
  } else {
    constexpr int w = DTI >> 2;
    constexpr int sh = 8 * (DTI & 3);
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t x0 = vc[2 * p][w] ^ 0x80808080u, x1 = vc[2 * p + 1][w] ^ 0x80808080u;
      a[p] = pack_exact((float)((x0 >> sh) & 0xffu), (float)((x1 >> sh) & 0xffu));
    }
  }
  return a;
}

template <int MODE, int D, int DTI>
struct VPass {
  __device__ __forceinline__ static void run(const uint32_t (*vc)[Geo<MODE, D>::VW], u32x4_t bhi,
                                             u32x4_t blo, f32x4_t* acc) {
    const u32x4_t a = unpack_v<MODE, D, DTI>(vc);
    acc[DTI] = mfma(a, bhi, acc[DTI]);
    acc[DTI] = mfma(a, blo, acc[DTI]);
    VPass<MODE, D, DTI + 1>::run(vc, bhi, blo, acc);
  }
};
template <int MODE, int D>
struct VPass<MODE, D, D / 16> {
  __device__ __forceinline__ static void run(const uint32_t (*)[Geo<MODE, D>::VW], u32x4_t,
                                             u32x4_t, f32x4_t*) {}
};

template <int N>
__device__ __forceinline__ void load_bytes(uint32_t* dst, const uint8_t* src) {
  if constexpr (N == 32) {
    const uint4 a = reinterpret_cast<const uint4*>(src)[0];
    const uint4 b = reinterpret_cast<const uint4*>(src)[1];
    dst[0] = a.x; dst[1] = a.y; dst[2] = a.z; dst[3] = a.w;
    dst[4] = b.x; dst[5] = b.y; dst[6] = b.z; dst[7] = b.w;
  } else if constexpr (N == 16) {
    const uint4 a = *reinterpret_cast<const uint4*>(src);
    dst[0] = a.x; dst[1] = a.y; dst[2] = a.z; dst[3] = a.w;
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

template <int N>
__device__ __forceinline__ void zero_words(uint32_t* dst) {
#pragma unroll
  for (int i = 0; i < N; ++i) dst[i] = 0u;
}

// In-lane + cross-lane (xor 16, xor 32) FWHT over the D values of one head
// held as v[e], e = 0..D/4-1, by the four lanes l%16 = g, l/16 = q, with
// d = q*(D/4) + e; then d .* / sqrt(D).  Only the orthogonal map matters here
// (tolerance-checked), not a particular rounding sequence.
template <int D>
__device__ __forceinline__ void inverse_rotate(float* v, int q, const float* signs, float inv_sqrt_d) {
  constexpr int E = D / 4;
#pragma unroll
  for (int hh = 1; hh < E; hh <<= 1) {
#pragma unroll
    for (int i = 0; i < E; ++i) {
      if (!(i & hh)) {
        const float a = v[i], b = v[i + hh];
        v[i] = a + b;
        v[i + hh] = a - b;
      }
    }
  }
#pragma unroll
  for (int m = 16; m <= 32; m <<= 1) {
    const bool upper = ((q * 16) & m) != 0;
#pragma unroll
    for (int i = 0; i < E; ++i) {
      const float o = __shfl_xor(v[i], m);
      v[i] = upper ? (o - v[i]) : (v[i] + o);
    }
  }
#pragma unroll
  for (int i = 0; i < E; ++i) v[i] = v[i] * signs[q * E + i] * inv_sqrt_d;
}

template <int D>
__device__ __forceinline__ void store_out(const DecodeParams& p, int64_t orow, int q, const float* v) {
  constexpr int E = D / 4;
  if (p.out_bf16) {
    uint32_t* o = reinterpret_cast<uint32_t*>(reinterpret_cast<uint16_t*>(p.out) + orow * D + q * E);
#pragma unroll
    for (int i = 0; i < E / 8; ++i) {
      uint4 w;
      w.x = pack_bf16(v[8 * i + 0], v[8 * i + 1]);
      w.y = pack_bf16(v[8 * i + 2], v[8 * i + 3]);
      w.z = pack_bf16(v[8 * i + 4], v[8 * i + 5]);
      w.w = pack_bf16(v[8 * i + 6], v[8 * i + 7]);
      reinterpret_cast<uint4*>(o)[i] = w;
    }
  } else {
    float4* o = reinterpret_cast<float4*>(reinterpret_cast<float*>(p.out) + orow * D + q * E);
#pragma unroll
    for (int i = 0; i < E / 4; ++i) o[i] = make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
  }
}

template <int MODE, int D, bool ROT>
__global__ __launch_bounds__(64) void decode_kernel(DecodeParams p) {
  using Gm = Geo<MODE, D>;
  constexpr int P = Gm::P;
  constexpr int M = Gm::M;
  constexpr int KS = Gm::KSTEPS;
  constexpr int E = D / 4;            // output values per lane
  __shared__ float qs[16][D];

  const int split = blockIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int lane = threadIdx.x;
  const int r16 = lane & 15;
  const int kg = lane >> 4;
  const int G = p.group;
  const int hkv = p.hkv;
  const int bs = p.block_size;

  const int L = p.seq_lens[b];
  const int W = p.window ? p.window[h] : 0;
  const int start = (W > 0 && L > W) ? L - W : 0;
  const int c0 = start / kChunk;
  const int c1 = (L + kChunk - 1) / kChunk;
  const int n_chunks = L > 0 ? c1 - c0 : 0;
  const int cps = p.chunks_per_split;
  const int n_splits = n_chunks > 0 ? (n_chunks + cps - 1) / cps : 1;
  if (split >= n_splits) return;
  const int cb = c0 + split * cps;
  const int ce = min(c1, cb + cps);
  const int32_t* trow = p.tables + (int64_t)(p.headwise ? b * hkv + h : b) * p.max_blocks;

  // ---- query prologue: q'' = R q * scale * log2(e), split into bf16 hi + lo
  for (int e = lane; e < G * D; e += 64) {
    const int g = e / D, d = e - g * D;
    float v = __uint_as_float((uint32_t)p.q[((int64_t)b * p.hq + h * G + g) * D + d] << 16);
    if constexpr (ROT) v *= p.signs[d];
    qs[g][d] = v;
  }
  __syncthreads();
  if constexpr (ROT) {
    for (int hh = 1; hh < D; hh <<= 1) {
      for (int e = lane; e < G * (D / 2); e += 64) {
        const int g = e / (D / 2), k = e - g * (D / 2);
        const int i = (k / hh) * 2 * hh + (k % hh);
        const float a = qs[g][i], bb = qs[g][i + hh];
        qs[g][i] = a + bb;
        qs[g][i + hh] = a - bb;
      }
      __syncthreads();
    }
  }
  const float qmul = ROT ? p.qscale * p.inv_sqrt_d : p.qscale;
  u32x4_t bqh[KS], bql[KS];
  float q1 = 0.0f;
#pragma unroll
  for (int k = 0; k < KS; ++k) {
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      float v0 = 0.0f, v1 = 0.0f;
      if (r16 < G) {
        v0 = qs[r16][kmap<MODE, D>(kg, k, 2 * jj)] * qmul;
        v1 = qs[r16][kmap<MODE, D>(kg, k, 2 * jj + 1)] * qmul;
      }
      const uint32_t hi = pack_bf16(v0, v1);
      const uint32_t lo = pack_bf16(v0 - bf16_lo(hi), v1 - bf16_hi(hi));
      bqh[k][jj] = hi;
      bql[k][jj] = lo;
      q1 += (bf16_lo(hi) + bf16_lo(lo)) + (bf16_hi(hi) + bf16_hi(lo));
    }
  }
  q1 += __shfl_xor(q1, 16);
  q1 += __shfl_xor(q1, 32);
  const float koff = -128.0f * q1;

  // ---- main loop over chunks
  float m_run = kNegInf;
  float l_run = 0.0f;   // per-lane partial sum of p
  float z_run = 0.0f;   // per-lane partial sum of p * z_V
  f32x4_t acc[Gm::DT];
#pragma unroll
  for (int i = 0; i < Gm::DT; ++i) acc[i] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  for (int c = cb; c < ce; ++c) {
    int tpos[2];
    int64_t rbase[2];   // row index of the tile's first token in the planes
    bool tok[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      tpos[mt] = c * kChunk + 16 * mt;
      tok[mt] = false;
      rbase[mt] = 0;
      if (tpos[mt] < L && tpos[mt] + 15 >= start) {
        const int id = trow[tpos[mt] / bs];
        if (id >= 0) {
          tok[mt] = true;
          rbase[mt] = ((int64_t)id * hkv + h) * bs + (tpos[mt] % bs);
        }
      }
    }
    if (!tok[0] && !tok[1]) continue;

    // loads: K codes (lane = token r16, bytes kg*P/4..), V codes (lane =
    // d-group r16, token slots j), K/V meta (lane = head, tokens 4kg..4kg+3)
    uint32_t kc[2][Gm::KW];
    uint32_t vc[8][Gm::VW];
    float km[2][4 * M], vm[2][4 * M];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      if (tok[mt]) {
        load_bytes<P / 4>(kc[mt], p.k_codes + (rbase[mt] + r16) * P + kg * (P / 4));
#pragma unroll
        for (int i = 0; i < 4; ++i)
          load_bytes<Gm::VB>(vc[4 * mt + i], p.v_codes + (rbase[mt] + 4 * kg + i) * P + r16 * Gm::VB);
        const float* kmp = p.k_meta + (rbase[mt] + 4 * kg) * M;
        const float* vmp = p.v_meta + (rbase[mt] + 4 * kg) * M;
#pragma unroll
        for (int i = 0; i < M; ++i) {
          const float4 a = reinterpret_cast<const float4*>(kmp)[i];
          const float4 bb = reinterpret_cast<const float4*>(vmp)[i];
          km[mt][4 * i] = a.x; km[mt][4 * i + 1] = a.y; km[mt][4 * i + 2] = a.z; km[mt][4 * i + 3] = a.w;
          vm[mt][4 * i] = bb.x; vm[mt][4 * i + 1] = bb.y; vm[mt][4 * i + 2] = bb.z; vm[mt][4 * i + 3] = bb.w;
        }
      } else {
        zero_words<Gm::KW>(kc[mt]);
#pragma unroll
        for (int i = 0; i < 4; ++i) zero_words<Gm::VW>(vc[4 * mt + i]);
#pragma unroll
        for (int i = 0; i < 4 * M; ++i) { km[mt][i] = 0.0f; vm[mt][i] = 0.0f; }
      }
    }

    // K pass: raw[mt][i] = sum_d q''_d (128 + c_d) - 128 sum q'' for token 4kg+i
    f32x4_t sc[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      f32x4_t a = {koff, koff, koff, koff};
#pragma unroll
      for (int k = 0; k < KS; ++k) {
        const u32x4_t ak = unpack_k<MODE, D>(kc[mt], k);
        a = mfma(ak, bqh[k], a);
        a = mfma(ak, bql[k], a);
      }
      sc[mt] = a;
    }

    // scores (log2 units), masks, chunk max per head
    float s2[2][4];
    float cmax = kNegInf;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int pos = tpos[mt] + 4 * kg + i;
        const bool valid = tok[mt] && pos < L && pos >= start && r16 < G;
        const float s = M == 2 ? km[mt][2 * i] : km[mt][i];
        const float z = M == 2 ? km[mt][2 * i + 1] : 0.0f;
        const float v = s * sc[mt][i] + z * q1;
        s2[mt][i] = valid ? v : kNegInf;
        cmax = fmaxf(cmax, s2[mt][i]);
      }
    }
    cmax = fmaxf(cmax, __shfl_xor(cmax, 16));
    cmax = fmaxf(cmax, __shfl_xor(cmax, 32));
    const float m_new = fmaxf(m_run, cmax);
    const float m_use = m_new == kNegInf ? 0.0f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);

    // probabilities, V weights w = p * s_V (bf16 hi + lo), zero-point term
    uint32_t whi[4], wlo[4];
    float lsum = 0.0f, zsum = 0.0f, wsum = 0.0f;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int i = 0; i < 4; i += 2) {
        float w2[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const float pr = __builtin_amdgcn_exp2f(s2[mt][i + e] - m_use);
          const float sv = M == 2 ? vm[mt][2 * (i + e)] : vm[mt][i + e];
          const float zv = M == 2 ? vm[mt][2 * (i + e) + 1] : 0.0f;
          const bool live = pr > 0.0f;
          lsum += pr;
          zsum += live ? pr * zv : 0.0f;
          w2[e] = live ? pr * sv : 0.0f;
        }
        const uint32_t hi = pack_bf16(w2[0], w2[1]);
        const uint32_t lo = pack_bf16(w2[0] - bf16_lo(hi), w2[1] - bf16_hi(hi));
        whi[2 * mt + i / 2] = hi;
        wlo[2 * mt + i / 2] = lo;
        wsum += (bf16_lo(hi) + bf16_lo(lo)) + (bf16_hi(hi) + bf16_hi(lo));
      }
    }
    l_run = l_run * alpha + lsum;
    z_run = z_run * alpha + zsum;
    wsum += __shfl_xor(wsum, 16);
    wsum += __shfl_xor(wsum, 32);
    const float voff = -128.0f * wsum;
#pragma unroll
    for (int i = 0; i < Gm::DT; ++i) {
      acc[i][0] = acc[i][0] * alpha + voff;
      acc[i][1] = acc[i][1] * alpha + voff;
      acc[i][2] = acc[i][2] * alpha + voff;
      acc[i][3] = acc[i][3] * alpha + voff;
    }
    const u32x4_t bwh = {whi[0], whi[1], whi[2], whi[3]};
    const u32x4_t bwl = {wlo[0], wlo[1], wlo[2], wlo[3]};
    VPass<MODE, D, 0>::run(vc, bwh, bwl, acc);
    m_run = m_new;
  }

  // ---- split epilogue
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  z_run += __shfl_xor(z_run, 16);
  z_run += __shfl_xor(z_run, 32);
  // lane (head g = r16, q = kg) holds d = (4q + i)*(D/16) + dt  ->  e = i*(D/16) + dt
  float v[E];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int dt = 0; dt < Gm::DT; ++dt) v[i * Gm::DT + dt] = acc[dt][i] + z_run;

  const int g = r16;
  const int64_t orow = (int64_t)b * p.hq + h * G + g;
  if (n_splits == 1) {
    const float inv_l = l_run > 0.0f ? 1.0f / l_run : 0.0f;
#pragma unroll
    for (int i = 0; i < E; ++i) v[i] = l_run > 0.0f ? v[i] * inv_l : 0.0f;
    if constexpr (ROT) inverse_rotate<D>(v, kg, p.signs, p.inv_sqrt_d);
    if (g < G) store_out<D>(p, orow, kg, v);
    return;
  }

  float* rec = p.partials + (orow * p.max_splits + split) * (D + 4);
  if (g < G) {
    if (kg == 0) *reinterpret_cast<float2*>(rec) = make_float2(m_run, l_run);
    float4* dst = reinterpret_cast<float4*>(rec + 4 + kg * E);
#pragma unroll
    for (int i = 0; i < E / 4; ++i) dst[i] = make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
  }
  __threadfence();
  uint32_t* ctr = p.counters + (int64_t)b * hkv + h;
  uint32_t old = 0;
  if (lane == 0) old = atomicAdd(ctr, 1u);
  old = __shfl(old, 0);
  if (old != (uint32_t)(n_splits - 1)) return;
  __threadfence();
  if (lane == 0) atomicExch(ctr, 0u);

  // last wave: combine the splits of every head of this kv head
  const float* base = p.partials + orow * p.max_splits * (D + 4);
  float mx = kNegInf;
  for (int s = 0; s < n_splits; ++s) mx = fmaxf(mx, g < G ? base[s * (D + 4)] : kNegInf);
  const float mu = mx == kNegInf ? 0.0f : mx;
  float ltot = 0.0f;
#pragma unroll
  for (int i = 0; i < E; ++i) v[i] = 0.0f;
  if (g < G) {
    for (int s = 0; s < n_splits; ++s) {
      const float* r = base + s * (D + 4);
      const float2 ml = *reinterpret_cast<const float2*>(r);
      const float wgt = __builtin_amdgcn_exp2f(ml.x - mu);
      ltot += wgt * ml.y;
      const float4* src = reinterpret_cast<const float4*>(r + 4 + kg * E);
#pragma unroll
      for (int i = 0; i < E / 4; ++i) {
        const float4 a = src[i];
        v[4 * i] += wgt * a.x;
        v[4 * i + 1] += wgt * a.y;
        v[4 * i + 2] += wgt * a.z;
        v[4 * i + 3] += wgt * a.w;
      }
    }
  }
  const float inv_l = ltot > 0.0f ? 1.0f / ltot : 0.0f;
#pragma unroll
  for (int i = 0; i < E; ++i) v[i] = ltot > 0.0f ? v[i] * inv_l : 0.0f;
  if constexpr (ROT) inverse_rotate<D>(v, kg, p.signs, p.inv_sqrt_d);
  if (g < G) store_out<D>(p, orow, kg, v);
}

template <int MODE, int D, bool ROT>
hipError_t launch_decode_t(const DecodeParams& p, int num_seqs, hipStream_t s) {
  hipLaunchKernelGGL((decode_kernel<MODE, D, ROT>), dim3(p.max_splits, p.hkv, num_seqs), dim3(64), 0, s, p);
  return hipGetLastError();
}

template <int MODE>
hipError_t launch_decode_m(int d, bool rot, const DecodeParams& p, int n, hipStream_t s) {
  if (d == 64) return rot ? launch_decode_t<MODE, 64, true>(p, n, s) : launch_decode_t<MODE, 64, false>(p, n, s);
  return rot ? launch_decode_t<MODE, 128, true>(p, n, s) : launch_decode_t<MODE, 128, false>(p, n, s);
}

}  // namespace

hipError_t launch_decode(int mode, int d, bool rot, const DecodeParams& p, int num_seqs, hipStream_t s) {
  switch (mode) {
    case 0: return launch_decode_m<0>(d, rot, p, num_seqs, s);
    case 1: return launch_decode_m<1>(d, rot, p, num_seqs, s);
    default: return launch_decode_m<2>(d, rot, p, num_seqs, s);
  }
}

}  // namespace kvq
