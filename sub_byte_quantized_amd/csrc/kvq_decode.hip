// Split-KV paged decode attention over the quantized cache.
//
// Follows the read half of the prhub summary of vLLM PR 40835 ("INT4
// per-token-head KV cache quantization for the Triton backend", 实现拆解
// item 2: unpack, dequantize, attend), the head-wise block-table walk of
// FastDeploy PR 7718 ("Optimize AppendAttention for discrete head-wise
// block_idx": per-head rows; -1 entries are skipped before any K/V address is
// formed), and decode-side dequantization inside attention as described for
// the vllm-ascend-quantized-kv-cache package (运行机制).
//
// Per (sequence b, q head hq, kv head h = hq / G) it computes
//   out = R^T sum_j softmax_j(scale * q'.k_hat_j) v_hat_j ,   q' = R q,
// k_hat / v_hat the stored codes dequantized in the rotated basis
// (x_hat = c*s + z) and R the cache's rotation (identity without signs),
// without dequantizing element by element:
//   q'.k_hat_t      = s_t (q'.c_t) + z_t sum(q')
//   sum_t w_t v_hat_t = sum_t (p_t s_t) c_t + (sum_t p_t z_t) 1 .
// q'.c runs on v_mfma_i32_16x16x64_i8: the codes are int8 operands as they
// are (INT8) or after two or three bit operations per 16 codes (INT4/INT2),
// and q' is split into two int8 pieces (scale S: q' ~ S (a + b/2^7),
// |a| <= 127, |b| <= 64, within 2^-15 of max|q'|), so the products
// accumulate exactly in int32.  sum_t w_t c_t runs on v_mfma_f32_16x16x32_bf16 with the codes as
// exact bf16 integers 128 + c (one and-or per two codes) and w split into
// bf16 hi + lo; one extra MFMA per d-tile, a constant -128 operand against the
// weight sum in three bf16 pieces, cancels the 128 offset.
//
// Layout of one 64-position tile (four 16-token sub-tiles sigma = 0..3).
// MFMA columns n = 0..15 are (head g, phase phi) = (n / PHI, n % PHI), PHI the
// largest power of two <= 16/G (at most 4), so G*PHI of the 16 columns carry
// work instead of G.  Lane l has r = l % 16 and q = l / 16.
//   K pass, K-tile tau (4/PHI per tile, sub-tiles tau*PHI .. +PHI-1):
//     A  codes  [16 tokens x 64 k] int8  lane (token r of sub-tile
//                                   tau*PHI + q*PHI/4, d-range q % (4/PHI))
//     B  q' piece [64 k x 16 cols] int8  from LDS; zero unless the lane
//                                   group's phase equals the column's phase
//     C  scores [16 tokens x 16 cols] int32, lane (col r, tokens 4q..4q+3)
//   V pass, k-steps u = 0, 1 (sub-tiles 2u, 2u+1):
//     A  codes^T [16 d x 32 tokens]  lane (d-group r, tokens 16(2u+j/4)+4q+j%4)
//     B  w^T     [32 tokens x 16 cols] the K pass's C registers, zero where the
//                                   column's phase does not own the sub-tile
//     C  acc     [16 d x 16 cols]   lane (col r, d-slots 4q..4q+3)
//   Columns of one head are summed at the end (phases partition the tokens).
//
// Work split: one 256-thread workgroup (4 waves) per (split, kv head,
// sequence); a split is a run of tiles of the sequence's active range (the
// window), interleaved over the waves.  Each wave keeps its own online-softmax
// state, issues the next tile's loads before computing the current one, and
// rescales its accumulators only when a head's running maximum grows by more
// than 2^8.  The workgroup combines its waves in LDS; with one split it
// finishes (normalize, R^T, store), otherwise it writes (m, l, acc) to the
// workspace and decode_reduce_kernel, launched next on the same stream,
// combines the splits and finishes (stream order makes the partials visible;
// no device-scope fence or atomic is needed).
#include "kvq_internal.h"
#include "kvq_device.h"

namespace kvq {
namespace {

constexpr int kWaves = 4;

template <int MODE, int D, int PHI>
struct Geo {
  static constexpr int P = row_bytes(MODE, D);   // packed bytes per row
  static constexpr int M = mode_meta(MODE);      // meta floats per row
  static constexpr int NKT = 4 / PHI;            // K-tiles per 64-position tile
  static constexpr int SUBD = D * PHI / 4;       // d values per lane group per K-tile
  static constexpr int KS = SUBD / 16;           // int8 MFMA k-steps per K-tile
  static constexpr int KB = SUBD * mode_bits(MODE) / 8;  // K bytes a lane loads per K-tile
  static constexpr int KW = KB / 4;              // ... in dwords
  static constexpr int KSW = KW / KS;            // ... per k-step
  static constexpr int VB = P / 16;              // V bytes a lane loads per token
  static constexpr int VW = VB >= 4 ? VB / 4 : 1;
  static constexpr int DT = D / 16;              // V-pass d-tiles
};

// d held by byte j (0..15) of the int8 operand of k-step s for lane-group
// d-range `sub` (K pass); the query pieces in LDS are laid out in this order.
template <int MODE, int D, int PHI>
__device__ __forceinline__ int kmap(int sub, int s, int j) {
  const int base = sub * Geo<MODE, D, PHI>::SUBD + 16 * s;
  if constexpr (MODE == 1) return base + 8 * ((j >> 2) >> 1) + 2 * (j & 3) + ((j >> 2) & 1);
  else if constexpr (MODE == 2) return base + 4 * (j & 3) + (j >> 2);
  else return base + j;
}

// K-pass int8 A operand of k-step s (16 codes) from the lane's K-tile dwords.
template <int MODE, int KSW>
__device__ __forceinline__ u32x4_t unpack_k(const uint32_t* kc, int s, uint32_t m4, uint32_t m2) {
  u32x4_t a;
  if constexpr (MODE == 1) {
    const uint32_t x0 = kc[2 * s], x1 = kc[2 * s + 1];
    a[0] = x0 & m4;
    a[1] = (x0 >> 4) & m4;
    a[2] = x1 & m4;
    a[3] = (x1 >> 4) & m4;
  } else if constexpr (MODE == 2) {
    const uint32_t x = kc[s];
    a[0] = x & m2;
    a[1] = (x >> 2) & m2;
    a[2] = (x >> 4) & m2;
    a[3] = (x >> 6) & m2;
  } else {
    a[0] = kc[4 * s]; a[1] = kc[4 * s + 1]; a[2] = kc[4 * s + 2]; a[3] = kc[4 * s + 3];
  }
  return a;
}

// V-pass A operand for d-tile DTI: token slots j = 0..7 (pairs 2p, 2p+1) of
// the lane's d = r*(D/16) + DTI, from vc[j][*].
template <int MODE, int VW, int DTI>
__device__ __forceinline__ u32x4_t unpack_v(const uint32_t (*vc)[VW], uint32_t magic, uint32_t n4,
                                            uint32_t n2) {
  u32x4_t a;
  if constexpr (MODE == 1) {
    constexpr uint32_t b = DTI >> 1;
    constexpr uint32_t sel = b | (0x0Cu << 8) | ((4u + b) << 16) | (0x0Cu << 24);
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t y = __builtin_amdgcn_perm(vc[2 * p + 1][0], vc[2 * p][0], sel);
      a[p] = and_or((DTI & 1) ? (y >> 4) : y, n4, magic);
    }
  } else if constexpr (MODE == 2) {
    constexpr uint32_t b = DTI >> 2;
    constexpr int sh = 2 * (DTI & 3);
    constexpr uint32_t sel = b | (0x0Cu << 8) | ((4u + b) << 16) | (0x0Cu << 24);
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t y = __builtin_amdgcn_perm(vc[2 * p + 1][0], vc[2 * p][0], sel);
      a[p] = and_or(sh ? (y >> sh) : y, n2, magic);
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

template <int MODE, int VW, int DT, int DTI>
struct VPass {
  __device__ __forceinline__ static void run(const uint32_t (*vc)[VW], u32x4_t bh, u32x4_t bl,
                                             f32x4_t* acc, uint32_t magic, uint32_t n4, uint32_t n2) {
    const u32x4_t a = unpack_v<MODE, VW, DTI>(vc, magic, n4, n2);
    acc[DTI] = mfma(a, bh, acc[DTI]);
    acc[DTI] = mfma(a, bl, acc[DTI]);
    VPass<MODE, VW, DT, DTI + 1>::run(vc, bh, bl, acc, magic, n4, n2);
  }
};
template <int MODE, int VW, int DT>
struct VPass<MODE, VW, DT, DT> {
  __device__ __forceinline__ static void run(const uint32_t (*)[VW], u32x4_t, u32x4_t, f32x4_t*, uint32_t,
                                             uint32_t, uint32_t) {}
};


// Rows and validity of one tile's four 16-token sub-tiles (wave-uniform).
struct TileInfo {
  int pos0;                 // first position of the tile
  int row0, row1, row2, row3;  // plane row of the sub-tile's first token; 0 when invalid
  uint32_t valid;           // bit sigma: sub-tile has a block and meets [start, L)
};

// CB: block_size >= 64, so a tile lies in one block and its sub-tile rows
// are row0 + 16 s (one block id per tile; an evicted block reads rows 0..63,
// which exist because every block slice has at least 64 rows).
template <bool CB>
__device__ __forceinline__ TileInfo tile_info(const int32_t* ids, int blk0, int tile, int te, int L, int start,
                                              int bs_log2, int hkv, int h) {
  TileInfo t;
  t.pos0 = tile * 64;
  t.valid = 0;
  if constexpr (CB) {
    const bool in = tile < te;
    const int id = __builtin_amdgcn_readfirstlane(ids[in ? (t.pos0 >> bs_log2) - blk0 : 0]);
    const bool okb = in && id >= 0;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int pos = t.pos0 + 16 * s;
      t.valid |= (okb && pos < L && pos + 15 >= start) ? 1u << s : 0u;
    }
    t.row0 = okb ? ((id * hkv + h) << bs_log2) + (t.pos0 & ((1 << bs_log2) - 1)) : 0;
    t.row1 = t.row0 + 16; t.row2 = t.row0 + 32; t.row3 = t.row0 + 48;
    return t;
  }
  int row[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int pos = t.pos0 + 16 * s;
    const bool in = tile < te && pos < L && pos + 15 >= start;
    const int id = __builtin_amdgcn_readfirstlane(ids[in ? (pos >> bs_log2) - blk0 : 0]);
    const bool ok = in && id >= 0;
    t.valid |= ok ? 1u << s : 0u;
    row[s] = ok ? ((id * hkv + h) << bs_log2) + (pos & ((1 << bs_log2) - 1)) : 0;
  }
  t.row0 = row[0]; t.row1 = row[1]; t.row2 = row[2]; t.row3 = row[3];
  return t;
}

// Row of sub-tile sigma (sigma may differ per lane).  An invalid sub-tile
// reads row 0, which is always addressable; its data is masked out of the
// scores and gets zero weight.
__device__ __forceinline__ int pick_row(const TileInfo& t, int sigma) {
  return sigma == 0 ? t.row0 : (sigma == 1 ? t.row1 : (sigma == 2 ? t.row2 : t.row3));
}

template <int MODE, int D, int PHI>
struct Buf {
  using Gm = Geo<MODE, D, PHI>;
  uint32_t k[Gm::NKT][Gm::KW];
  uint32_t v[16][Gm::VW];
  float km[Gm::NKT][4 * Gm::M];
  float vm[Gm::NKT][4 * Gm::M];
};

template <int MODE, int D, int PHI, bool CB>
__device__ __forceinline__ void issue_loads(Buf<MODE, D, PHI>& b, const TileInfo& t, const DecodeParams& p,
                                            int r, int q, int phi_col) {
  using Gm = Geo<MODE, D, PHI>;
  constexpr int P = Gm::P, M = Gm::M;
  const int phi_grp = q * PHI / 4;          // phase of this lane group (K pass)
  const int sub = q % (4 / PHI);            // d-range of this lane group (K pass)
  if constexpr (CB) {
    // uniform tile bases (scalar) + per-lane constant 32-bit offsets
    const uint8_t* kb = p.k_codes + (int64_t)t.row0 * P;
    const uint8_t* vb = p.v_codes + (int64_t)t.row0 * P;
    const float* kmb = p.k_meta + (int64_t)t.row0 * M;
    const float* vmb = p.v_meta + (int64_t)t.row0 * M;
#pragma unroll
    for (int tau = 0; tau < Gm::NKT; ++tau) {
      const uint32_t ko = (uint32_t)((16 * (tau * PHI + phi_grp) + r) * P + sub * Gm::KB);
      load_bytes<Gm::KB>(b.k[tau], kb + ko);
      const uint32_t mo = (uint32_t)((16 * (tau * PHI + phi_col) + 4 * q) * M);
#pragma unroll
      for (int i = 0; i < M; ++i) {
        const float4 a = reinterpret_cast<const float4*>(kmb + mo)[i];
        const float4 c = reinterpret_cast<const float4*>(vmb + mo)[i];
        b.km[tau][4 * i] = a.x; b.km[tau][4 * i + 1] = a.y; b.km[tau][4 * i + 2] = a.z; b.km[tau][4 * i + 3] = a.w;
        b.vm[tau][4 * i] = c.x; b.vm[tau][4 * i + 1] = c.y; b.vm[tau][4 * i + 2] = c.z; b.vm[tau][4 * i + 3] = c.w;
      }
    }
    const uint32_t vo = (uint32_t)(4 * q * P + r * Gm::VB);
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int i = 0; i < 4; ++i) load_bytes<Gm::VB>(b.v[4 * s + i], vb + vo + (16 * s + i) * P);
    return;
  }
#pragma unroll
  for (int tau = 0; tau < Gm::NKT; ++tau) {
    const int kr = pick_row(t, tau * PHI + phi_grp) + r;
    load_bytes<Gm::KB>(b.k[tau], p.k_codes + (int64_t)kr * P + sub * Gm::KB);
    const int mr = pick_row(t, tau * PHI + phi_col) + 4 * q;
#pragma unroll
    for (int i = 0; i < M; ++i) {
      const float4 a = reinterpret_cast<const float4*>(p.k_meta + (int64_t)mr * M)[i];
      const float4 c = reinterpret_cast<const float4*>(p.v_meta + (int64_t)mr * M)[i];
      b.km[tau][4 * i] = a.x; b.km[tau][4 * i + 1] = a.y; b.km[tau][4 * i + 2] = a.z; b.km[tau][4 * i + 3] = a.w;
      b.vm[tau][4 * i] = c.x; b.vm[tau][4 * i + 1] = c.y; b.vm[tau][4 * i + 2] = c.z; b.vm[tau][4 * i + 3] = c.w;
    }
  }
  const int voff = 4 * q * P + r * Gm::VB;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int row = s == 0 ? t.row0 : (s == 1 ? t.row1 : (s == 2 ? t.row2 : t.row3));
    const uint8_t* base = p.v_codes + (int64_t)row * P;
#pragma unroll
    for (int i = 0; i < 4; ++i) load_bytes<Gm::VB>(b.v[4 * s + i], base + voff + i * P);
  }
}

struct WaveState {
  float m;     // running reference maximum (log2 units) of the lane's head
  float l;     // lane partial sum of p
  float z;     // lane partial sum of p * z_V
};

struct LaneConst {
  const int8_t* qa;    // query pieces of this lane's B operand rows (LDS)
  const int8_t* qb;
  float sp;            // log2 logit per unit of x (S/128 of the column's head)
  float q1r;           // sum of the column head's pieces, 128 a + b
  int q;
  int phi_col;
  bool head_ok;
  uint32_t magic, n4, n2;   // bf16 128.0 pair; nibble and crumb masks of a bf16 pair
};

// full: every position of the tile is present and inside [start, L), so no
// score needs a mask (wave-uniform; the masking sits behind a branch).
template <int MODE, int D, int PHI>
__device__ __forceinline__ void compute_tile(const Buf<MODE, D, PHI>& b, const TileInfo& t, WaveState& st,
                                             f32x4_t* acc, const LaneConst& lc, int L, int start, bool full) {
  using Gm = Geo<MODE, D, PHI>;
  constexpr int M = Gm::M;
  const int q = lc.q, phi_col = lc.phi_col;
  // ---- K pass: int32 (a, b) dot products of the query pieces with the codes;
  // x = s_K (128 a + b).c + z_K q1r, the log2 logit being sp * x
  float sc[Gm::NKT][4];
#pragma unroll
  for (int tau = 0; tau < Gm::NKT; ++tau) {
    i32x4_t ia = {0, 0, 0, 0}, ib = {0, 0, 0, 0};
#pragma unroll
    for (int s = 0; s < Gm::KS; ++s) {
      const u32x4_t a = unpack_k<MODE, Gm::KSW>(b.k[tau], s, 0x0F0F0F0Fu, 0x03030303u);
      const uint4 xa = *reinterpret_cast<const uint4*>(lc.qa + 16 * s);
      const uint4 xb = *reinterpret_cast<const uint4*>(lc.qb + 16 * s);
      ia = mfma_i8(a, u32x4_t{xa.x, xa.y, xa.z, xa.w}, ia);
      ib = mfma_i8(a, u32x4_t{xb.x, xb.y, xb.z, xb.w}, ib);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float raw = (float)((ia[i] << 7) + ib[i]);
      const float s = M == 2 ? b.km[tau][2 * i] : b.km[tau][i];
      const float z = M == 2 ? b.km[tau][2 * i + 1] : 0.0f;
      sc[tau][i] = __builtin_fmaf(raw, s, z * lc.q1r);
    }
  }
  // V meta of the lane's positions; a masked position may sit on an absent
  // or unwritten row whose meta is not finite, so its weight inputs are zeroed
  float svv[Gm::NKT][4], zvv[Gm::NKT][4];
#pragma unroll
  for (int tau = 0; tau < Gm::NKT; ++tau)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      svv[tau][i] = M == 2 ? b.vm[tau][2 * i] : b.vm[tau][i];
      zvv[tau][i] = M == 2 ? b.vm[tau][2 * i + 1] : 0.0f;
    }
  if (__builtin_expect(!full, 0)) {
#pragma unroll
    for (int tau = 0; tau < Gm::NKT; ++tau) {
      const int sg = tau * PHI + phi_col;
      const bool tv = (t.valid >> sg) & 1u;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int pos = t.pos0 + 16 * sg + 4 * q + i;
        const bool keep = tv && pos < L && pos >= start;
        sc[tau][i] = keep ? sc[tau][i] : kNegInf;
        svv[tau][i] = keep ? svv[tau][i] : 0.0f;
        zvv[tau][i] = keep ? zvv[tau][i] : 0.0f;
      }
    }
  }
  // ---- tile maximum of the head: lane values, lane groups q, phases of the head
  float tmax = kNegInf;
#pragma unroll
  for (int tau = 0; tau < Gm::NKT; ++tau)
#pragma unroll
    for (int i = 0; i < 4; ++i) tmax = fmaxf(tmax, sc[tau][i]);
  tmax = max_xor32(max_xor16(tmax)) * lc.sp;
  if constexpr (PHI >= 2) tmax = __builtin_fmaxf(tmax, quad_xor<1>(tmax));
  if constexpr (PHI >= 4) tmax = __builtin_fmaxf(tmax, quad_xor<2>(tmax));
  if (__any(tmax > st.m + kRescale)) {
    const float mn = fmaxf(st.m, tmax);
    const float alpha = mn == kNegInf ? 1.0f : __builtin_amdgcn_exp2f(st.m - mn);
    st.m = mn;
    st.l *= alpha;
    st.z *= alpha;
#pragma unroll
    for (int i = 0; i < Gm::DT; ++i) acc[i] *= alpha;
  }
  const float mu = st.m == kNegInf ? 0.0f : st.m;

  // ---- probabilities and V weights w = p * s_V as bf16 hi + lo pairs
  uint32_t wh[Gm::NKT][2], wl[Gm::NKT][2];
  float wsum = 0.0f;
#pragma unroll
  for (int tau = 0; tau < Gm::NKT; ++tau) {
#pragma unroll
    for (int i = 0; i < 4; i += 2) {
      float w2[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[tau][i + e], lc.sp, -mu));
        st.l += pr;
        if constexpr (M == 2) st.z = __builtin_fmaf(pr, zvv[tau][i + e], st.z);
        w2[e] = pr * svv[tau][i + e];
      }
      // hi = w with the low 16 bits cleared (exact bf16), lo = w - hi (exact)
      // rounded to bf16; the represented weights hi + lo feed the offset sum
      const float h0 = __uint_as_float(__float_as_uint(w2[0]) & 0xffff0000u);
      const float h1 = __uint_as_float(__float_as_uint(w2[1]) & 0xffff0000u);
      const uint32_t hi = __builtin_amdgcn_perm(__float_as_uint(h1), __float_as_uint(h0), 0x07060302u);
      const uint32_t lo = pack_bf16(w2[0] - h0, w2[1] - h1);
      wh[tau][i / 2] = hi;
      wl[tau][i / 2] = lo;
      wsum += (h0 + bf16_lo(lo)) + (h1 + bf16_hi(lo));
    }
  }
  // ---- offset: acc -= 128 * (sum of the column's weights), as one MFMA per
  // d-tile against the sum split into three bf16 pieces
  wsum = add_xor32(add_xor16(wsum));
  {
    const __bf16 w0 = (__bf16)wsum;
    const float r1 = wsum - (float)w0;
    const __bf16 w1 = (__bf16)r1;
    const __bf16 w2 = (__bf16)(r1 - (float)w1);
    const uint32_t d0 = q == 0 ? ((uint32_t)__builtin_bit_cast(uint16_t, w0) |
                                  ((uint32_t)__builtin_bit_cast(uint16_t, w1) << 16)) : 0u;
    const uint32_t d1 = q == 0 ? (uint32_t)__builtin_bit_cast(uint16_t, w2) : 0u;
    const u32x4_t bw = {d0, d1, 0u, 0u};
    const u32x4_t neg128 = {0xC300C300u, 0xC300C300u, 0xC300C300u, 0xC300C300u};
#pragma unroll
    for (int i = 0; i < Gm::DT; ++i) acc[i] = mfma(neg128, bw, acc[i]);
  }

  // ---- V pass: k-step u covers sub-tiles 2u (slots 0..3) and 2u+1 (slots 4..7)
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    u32x4_t bh, bl;
    if constexpr (PHI == 1) {
      bh = u32x4_t{wh[2 * u][0], wh[2 * u][1], wh[2 * u + 1][0], wh[2 * u + 1][1]};
      bl = u32x4_t{wl[2 * u][0], wl[2 * u][1], wl[2 * u + 1][0], wl[2 * u + 1][1]};
    } else {
      // the lane owns sub-tile 2u + phi_col % 2 of this k-step (PHI == 2: from
      // K-tile u; PHI == 4: only when phi_col / 2 == u, from its one K-tile)
      const int tau = PHI == 2 ? u : 0;
      const bool own = PHI == 2 ? true : (phi_col >> 1) == u;
      const bool first = (phi_col & 1) == 0;
      const uint32_t h0 = own ? wh[tau][0] : 0u, h1 = own ? wh[tau][1] : 0u;
      const uint32_t l0 = own ? wl[tau][0] : 0u, l1 = own ? wl[tau][1] : 0u;
      bh = first ? u32x4_t{h0, h1, 0u, 0u} : u32x4_t{0u, 0u, h0, h1};
      bl = first ? u32x4_t{l0, l1, 0u, 0u} : u32x4_t{0u, 0u, l0, l1};
    }
    VPass<MODE, Gm::VW, Gm::DT, 0>::run(b.v + 8 * u, bh, bl, acc, lc.magic, lc.n4, lc.n2);
  }
}

template <int MODE, int D, int PHI>
__device__ __forceinline__ void run_tile(const Buf<MODE, D, PHI>& b, const TileInfo& t, WaveState& st,
                                         f32x4_t* acc, const LaneConst& lc, int L, int start) {
  if (!t.valid) return;
  const bool full = t.valid == 0xFu && t.pos0 >= start && t.pos0 + 64 <= L;
  compute_tile<MODE, D, PHI>(b, t, st, acc, lc, L, start, full);
}

// FWHT of `rows` rows of D floats in LDS (Sylvester, natural order), all
// threads of the workgroup; ends with a barrier.
template <int D>
__device__ __forceinline__ void lds_fwht(float (*x)[D], int rows, int tid) {
  for (int hh = 1; hh < D; hh <<= 1) {
    for (int e = tid; e < rows * (D / 2); e += 64 * kWaves) {
      const int g = e / (D / 2), k = e - g * (D / 2);
      const int i = (k / hh) * 2 * hh + (k % hh);
      const float a = x[g][i], bb = x[g][i + hh];
      x[g][i] = a + bb;
      x[g][i + hh] = a - bb;
    }
    __syncthreads();
  }
}

template <int D>
__device__ __forceinline__ void store_rows(const DecodeParams& p, float (*fin)[D], int G, int64_t orow0,
                                           int tid, bool rot) {
  for (int e = tid; e < G * D; e += 64 * kWaves) {
    const int g = e / D, d = e - g * D;
    float v = fin[g][d];
    if (rot) v = v * p.signs[d] * p.inv_sqrt_d;
    if (p.out_bf16)
      reinterpret_cast<__bf16*>(p.out)[(orow0 + g) * D + d] = (__bf16)v;
    else
      reinterpret_cast<float*>(p.out)[(orow0 + g) * D + d] = v;
  }
}

template <int D>
struct Smem {
  union {
    struct {
      int8_t qa[17][D + 16];  // query pieces in k-slot order; row 16 = zeros
      int8_t qb[17][D + 16];  // (16 bytes of padding keep rows on distinct banks)
      float qf[16][D];      // prologue scratch: R q * scale * log2(e)
    } pro;
    struct {
      float acc[kWaves][16][D];
      float ml[kWaves][16][2];
    } comb;
    float fin[16][D];
  };
  float qs[16];   // sp: log2 logit per unit of x, (max|q'| / 127) / 128
  float q1[16];   // q1r: sum over d of 128 a + b
  int32_t ids[kMaxSplitBlocks];   // block ids of the split's range
};

// Two waves per SIMD (two workgroups per CU) where the registers fit without
// spilling, so one workgroup's prologue and epilogue overlap another's tiles;
// three for INT2 with four phases, whose tiles are the lightest.
template <int MODE, int D, int PHI>
constexpr int decode_waves_per_simd() {
  return (PHI == 1 || (MODE == 0 && D == 128 && PHI < 4)) ? 1 : ((MODE == 2 && PHI == 4) ? 3 : 2);
}

template <int MODE, int D, int PHI, bool ROT, bool CB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(decode_waves_per_simd<MODE, D, PHI>())))
void decode_kernel(DecodeParams p) {
  using Gm = Geo<MODE, D, PHI>;
  __shared__ Smem<D> sm;

  const int split = blockIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (SGPR)
  const int lane = tid & 63;
  const int r = lane & 15;
  const int q = lane >> 4;
  const int G = p.group;
  const int hkv = p.hkv;

  const int L = p.seq_lens[b];
  const int W = p.window ? p.window[h] : 0;
  const int start = (W > 0 && L > W) ? L - W : 0;
  const int t0 = start / 64;
  const int t1 = (L + 63) / 64;
  const int n_tiles = L > 0 ? t1 - t0 : 0;
  const int tps = p.chunks_per_split;   // tiles per split
  const int n_splits = n_tiles > 0 ? (n_tiles + tps - 1) / tps : 1;
  if (split >= n_splits) return;
  const int tb = t0 + split * tps;
  const int te = min(t1, tb + tps);
  const int32_t* trow = p.tables + (int64_t)(p.headwise ? b * hkv + h : b) * p.max_blocks;
  const int64_t orow0 = (int64_t)b * p.hq + h * G;

  // ---- block ids of the split's positions [64 tb, min(64 te, L)) and the raw
  // query rows into LDS
  const int blk0 = (tb * 64) >> p.block_size_log2;
  {
    const int last_pos = min(te * 64, L) - 1;
    const int n_ids = last_pos >= tb * 64 ? (last_pos >> p.block_size_log2) - blk0 + 1 : 0;
    for (int i = tid; i < n_ids; i += 64 * kWaves) sm.ids[i] = trow[blk0 + i];
    if (n_ids == 0 && tid == 0) sm.ids[0] = -1;
  }
  for (int e = tid; e < G * D; e += 64 * kWaves) {
    const int g = e / D, d = e - g * D;
    float v = __uint_as_float((uint32_t)p.q[(orow0 + g) * D + d] << 16);
    if constexpr (ROT) v *= p.signs[d];
    sm.pro.qf[g][d] = v;
  }
  __syncthreads();

  // ---- first tiles' loads go out before the query prologue, which they do
  // not depend on, so their latency overlaps it
  const int bl = p.block_size_log2;
  Buf<MODE, D, PHI> ba, bb;
  int tile = tb + wave;
  TileInfo ta = tile_info<CB>(sm.ids, blk0, tile, te, L, start, bl, hkv, h);
  TileInfo tn = tile_info<CB>(sm.ids, blk0, tile + kWaves, te, L, start, bl, hkv, h);
  const int phi_col0 = r % PHI;
  issue_loads<MODE, D, PHI, CB>(ba, ta, p, r, q, phi_col0);

  // ---- query prologue: q' = R q * scale * log2(e), then int8 pieces in
  // k-slot order
  if constexpr (ROT) lds_fwht<D>(sm.pro.qf, G, tid);
  const float qmul = ROT ? p.qscale * p.inv_sqrt_d : p.qscale;
  for (int g = wave; g < 17; g += kWaves) {
    if (g >= G) {
      for (int pos = lane; pos < D; pos += 64) {
        sm.pro.qa[g][pos] = 0; sm.pro.qb[g][pos] = 0;
      }
      continue;
    }
    float mx = 0.0f;
    for (int d = lane; d < D; d += 64) mx = fmaxf(mx, fabsf(sm.pro.qf[g][d] * qmul));
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) mx = fmaxf(mx, __shfl_xor(mx, m));
    // q' ~ (S / 128) (128 a + b), S = max|q'| / 127, |a| <= 127, |b| <= 64
    const float invS = mx > 0.0f ? 127.0f / mx : 0.0f;
    float sab = 0.0f;
    for (int pos = lane; pos < D; pos += 64) {
      const int sub = pos / Gm::SUBD, rem = pos - sub * Gm::SUBD;
      const float v = sm.pro.qf[g][kmap<MODE, D, PHI>(sub, rem >> 4, rem & 15)] * qmul;
      const float t = fminf(fmaxf(v * invS, -127.0f), 127.0f);
      const float a = __builtin_rintf(t);
      const float bq = __builtin_rintf((t - a) * 128.0f);
      sm.pro.qa[g][pos] = (int8_t)a;
      sm.pro.qb[g][pos] = (int8_t)bq;
      sab += 128.0f * a + bq;           // exact: |sum| < 2^24
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) sab += __shfl_xor(sab, m);
    if (lane == 0) {
      sm.qs[g] = mx > 0.0f ? (mx / 127.0f) * 0.0078125f : 1.0f;
      sm.q1[g] = sab;
    }
  }
  __syncthreads();

  // ---- per-lane constants
  LaneConst lc;
  const int g_col = r / PHI;            // head of this lane's MFMA column
  lc.q = q;
  lc.phi_col = r % PHI;                 // phase of this lane's MFMA column
  lc.head_ok = g_col < G;
  const int phi_grp = q * PHI / 4;      // phase of this lane group (K pass)
  const int sub = q % (4 / PHI);
  const int brow = (lc.head_ok && phi_grp == lc.phi_col) ? g_col : 16;
  lc.qa = &sm.pro.qa[brow][sub * Gm::SUBD];
  lc.qb = &sm.pro.qb[brow][sub * Gm::SUBD];
  lc.sp = lc.head_ok ? sm.qs[g_col] : 1.0f;
  lc.q1r = lc.head_ok ? sm.q1[g_col] : 0.0f;
  lc.magic = to_vgpr(p.bits_magic);
  lc.n4 = to_vgpr(p.bits_n4);
  lc.n2 = to_vgpr(p.bits_n2);

  WaveState st{kNegInf, 0.0f, 0.0f};
  f32x4_t acc[Gm::DT];
#pragma unroll
  for (int i = 0; i < Gm::DT; ++i) acc[i] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  // ---- tiles tb + wave, tb + wave + 4, ...: two buffers, loads one tile ahead.
  // Every half-iteration issues the same loads (a tile past the split end is
  // invalid and reads row 0), so the wait counts before each compute are exact
  // and cover only the tile being computed.
  for (; tile < te; tile += 2 * kWaves) {
    issue_loads<MODE, D, PHI, CB>(bb, tn, p, r, q, lc.phi_col);
    const TileInfo t2 = tile_info<CB>(sm.ids, blk0, tile + 2 * kWaves, te, L, start, bl, hkv, h);
    run_tile<MODE, D, PHI>(ba, ta, st, acc, lc, L, start);
    issue_loads<MODE, D, PHI, CB>(ba, t2, p, r, q, lc.phi_col);
    const TileInfo t3 = tile_info<CB>(sm.ids, blk0, tile + 3 * kWaves, te, L, start, bl, hkv, h);
    run_tile<MODE, D, PHI>(bb, tn, st, acc, lc, L, start);
    ta = t2;
    tn = t3;
  }

  // ---- wave epilogue: sum the phases of a head, then l and z over lane groups
  if constexpr (PHI >= 2) {
#pragma unroll
    for (int i = 0; i < Gm::DT; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] += quad_xor<1>(acc[i][j]);
    st.l += quad_xor<1>(st.l);
    st.z += quad_xor<1>(st.z);
  }
  if constexpr (PHI >= 4) {
#pragma unroll
    for (int i = 0; i < Gm::DT; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] += quad_xor<2>(acc[i][j]);
    st.l += quad_xor<2>(st.l);
    st.z += quad_xor<2>(st.z);
  }
  st.l = add_xor32(add_xor16(st.l));
  st.z = add_xor32(add_xor16(st.z));
  __syncthreads();   // the prologue area becomes the combine area
  if (lc.head_ok && lc.phi_col == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int dt = 0; dt < Gm::DT; ++dt) sm.comb.acc[wave][g_col][(4 * q + i) * Gm::DT + dt] = acc[dt][i] + st.z;
    if (q == 0) {
      sm.comb.ml[wave][g_col][0] = st.m;
      sm.comb.ml[wave][g_col][1] = st.l;
    }
  }
  __syncthreads();

  // ---- workgroup combine: each thread owns (g, d) pairs
  constexpr int PER = (16 * D + 64 * kWaves - 1) / (64 * kWaves);
  float val[PER];
  float lsum[PER];
  float mmax[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int e = tid + k * 64 * kWaves;
    val[k] = 0.0f; lsum[k] = 0.0f; mmax[k] = kNegInf;
    if (e < G * D) {
      const int g = e / D, d = e - g * D;
      float mx = kNegInf;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) mx = fmaxf(mx, sm.comb.ml[w][g][0]);
      const float mu = mx == kNegInf ? 0.0f : mx;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float f = __builtin_amdgcn_exp2f(sm.comb.ml[w][g][0] - mu);
        val[k] += f * sm.comb.acc[w][g][d];
        lsum[k] += f * sm.comb.ml[w][g][1];
      }
      mmax[k] = mx;
    }
  }
  __syncthreads();

  if (n_splits == 1) {
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int e = tid + k * 64 * kWaves;
      if (e < G * D) sm.fin[e / D][e % D] = lsum[k] > 0.0f ? val[k] / lsum[k] : 0.0f;
    }
    __syncthreads();
    if constexpr (ROT) lds_fwht<D>(sm.fin, G, tid);
    store_rows<D>(p, sm.fin, G, orow0, tid, ROT);
    return;
  }

  // ---- several splits: publish (m, l, acc); decode_reduce_kernel combines
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int e = tid + k * 64 * kWaves;
    if (e < G * D) {
      const int g = e / D, d = e - g * D;
      float* rec = p.partials + ((orow0 + g) * p.max_splits + split) * (D + 4);
      rec[4 + d] = val[k];
      if (d == 0) {
        rec[0] = mmax[k];
        rec[1] = lsum[k];
      }
    }
  }
}

// Cross-split combine, launched after decode_kernel on the same stream when a
// (sequence, kv head) can have several splits: one workgroup per (sequence,
// kv head) merges the splits' (m, l, acc) of its G heads, normalizes, applies
// R^T and stores.
template <int D, bool ROT>
__global__ __launch_bounds__(256) void decode_reduce_kernel(DecodeParams p) {
  __shared__ float fin[16][D];
  __shared__ float wgt[16][kMaxReduceSplits];
  __shared__ float inv_l[16];
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int G = p.group;
  const int L = p.seq_lens[b];
  const int W = p.window ? p.window[h] : 0;
  const int start = (W > 0 && L > W) ? L - W : 0;
  const int n_tiles = L > 0 ? (L + 63) / 64 - start / 64 : 0;
  const int tps = p.chunks_per_split;
  const int n_splits = n_tiles > 0 ? (n_tiles + tps - 1) / tps : 1;
  if (n_splits == 1) return;   // decode_kernel already stored this (sequence, kv head)
  const int64_t orow0 = (int64_t)b * p.hq + h * G;
  // weights exp2(m_s - M) of every (head, split), and 1 / sum_s w_s l_s
  for (int g = tid >> 6; g < G; g += 4) {
    const int lane = tid & 63;
    const float* base = p.partials + (orow0 + g) * p.max_splits * (D + 4);
    float mx = kNegInf;
    for (int s = lane; s < n_splits; s += 64) mx = fmaxf(mx, base[s * (D + 4)]);
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) mx = fmaxf(mx, __shfl_xor(mx, m));
    const float mu = mx == kNegInf ? 0.0f : mx;
    float l = 0.0f;
    for (int s = lane; s < n_splits; s += 64) {
      const float w = __builtin_amdgcn_exp2f(base[s * (D + 4)] - mu);
      wgt[g][s] = w;
      l += w * base[s * (D + 4) + 1];
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) l += __shfl_xor(l, m);
    if (lane == 0) inv_l[g] = l > 0.0f ? 1.0f / l : 0.0f;
  }
  __syncthreads();
  for (int e = tid; e < G * D; e += 256) {
    const int g = e / D, d = e - g * D;
    const float* base = p.partials + (orow0 + g) * p.max_splits * (D + 4) + 4 + d;
    float v0 = 0.0f, v1 = 0.0f, v2 = 0.0f, v3 = 0.0f;
    int s = 0;
    for (; s + 4 <= n_splits; s += 4) {
      v0 += wgt[g][s] * base[s * (D + 4)];
      v1 += wgt[g][s + 1] * base[(s + 1) * (D + 4)];
      v2 += wgt[g][s + 2] * base[(s + 2) * (D + 4)];
      v3 += wgt[g][s + 3] * base[(s + 3) * (D + 4)];
    }
    for (; s < n_splits; ++s) v0 += wgt[g][s] * base[s * (D + 4)];
    fin[g][d] = ((v0 + v1) + (v2 + v3)) * inv_l[g];
  }
  __syncthreads();
  if constexpr (ROT) {
    for (int hh = 1; hh < D; hh <<= 1) {
      for (int e = tid; e < G * (D / 2); e += 256) {
        const int g = e / (D / 2), k = e - g * (D / 2);
        const int i = (k / hh) * 2 * hh + (k % hh);
        const float a = fin[g][i], bb = fin[g][i + hh];
        fin[g][i] = a + bb;
        fin[g][i + hh] = a - bb;
      }
      __syncthreads();
    }
  }
  store_rows<D>(p, fin, G, orow0, tid, ROT);
}

template <int MODE, int D, int PHI, bool ROT>
hipError_t launch_decode_t(const DecodeParams& p, int num_seqs, hipStream_t s) {
  if (p.block_size >= 64)
    hipLaunchKernelGGL((decode_kernel<MODE, D, PHI, ROT, true>), dim3(p.max_splits, p.hkv, num_seqs),
                       dim3(64 * kWaves), 0, s, p);
  else
    hipLaunchKernelGGL((decode_kernel<MODE, D, PHI, ROT, false>), dim3(p.max_splits, p.hkv, num_seqs),
                       dim3(64 * kWaves), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.max_splits == 1) return e;
  hipLaunchKernelGGL((decode_reduce_kernel<D, ROT>), dim3(p.hkv, num_seqs), dim3(256), 0, s, p);
  return hipGetLastError();
}

template <int MODE, int D, bool ROT>
hipError_t launch_decode_p(const DecodeParams& p, int n, hipStream_t s) {
  if (p.group * 4 <= 16) return launch_decode_t<MODE, D, 4, ROT>(p, n, s);
  if (p.group * 2 <= 16) return launch_decode_t<MODE, D, 2, ROT>(p, n, s);
  return launch_decode_t<MODE, D, 1, ROT>(p, n, s);
}

template <int MODE>
hipError_t launch_decode_m(int d, bool rot, const DecodeParams& p, int n, hipStream_t s) {
  if (d == 64) return rot ? launch_decode_p<MODE, 64, true>(p, n, s) : launch_decode_p<MODE, 64, false>(p, n, s);
  return rot ? launch_decode_p<MODE, 128, true>(p, n, s) : launch_decode_p<MODE, 128, false>(p, n, s);
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
