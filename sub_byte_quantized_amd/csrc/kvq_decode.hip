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
// and q' is split into three int8 pieces (scale S: q' ~ S (a + b/2^7 +
// c/2^14), |a| <= 127, |b|, |c| <= 64, within 2^-22 of max|q'|), so the
// products accumulate exactly in int32.  Two pieces (2^-15) were measured
// too coarse for a peaked softmax over x10 outlier channels.  sum_t w_t c_t runs on v_mfma_f32_16x16x32_bf16 with the codes as
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
// Work split: a persistent grid of 256-thread workgroups (4 waves) takes
// equal shares of all (sequence, kv head) pairs' tiles concatenated (see
// decode_kernel); a share's piece of one pair is a segment, whose tiles are
// interleaved over the waves.  Each wave keeps its own online-softmax
// state, issues the next tile's loads before computing the current one (also
// across segment ends), and rescales its accumulators only when a head's
// running maximum grows by more than 2^8.  The workgroup combines its waves
// in LDS; a whole pair is finished there (normalize, R^T, store), a cut one
// is published as (m, l, acc) to the workspace and merged by whichever of
// its workgroups counts in last.
#include "kvq_internal.h"
#include "kvq_device.h"
#include "kvq_write_row.h"

namespace kvq {
namespace {


template <int MODE, int D, int PHI>
struct Geo {
  static constexpr int P = row_bytes(MODE, D);   // packed bytes per row
  static constexpr int M = mode_meta(MODE);      // meta floats per row (meta planes)
  // inline INT4: rows of RS bytes (codes, then the stored scale), tokens
  // Hkv rows apart; the scale and the zero point come from one word
  static constexpr bool INL = MODE == kInlineMode;
  static constexpr int RS = INL ? inline_row_bytes(D) : P;
  static constexpr bool MZ = M == 2 || INL;      // rows carry a zero point
  static constexpr int NKT = 4 / PHI;            // K-tiles per 64-position tile
  static constexpr int SUBD = D * PHI / 4;       // d values per lane group per K-tile
  static constexpr int KS = SUBD / 16;           // int8 MFMA k-steps per K-tile
  static constexpr int KB = SUBD * mode_bits(MODE) / 8;  // K bytes a lane loads per K-tile
  static constexpr int KW = KB / 4;              // ... in dwords
  static constexpr int KSW = KW / KS;            // ... per k-step
  static constexpr int VB = P / 16;              // V bytes a lane loads per token
  static constexpr int VW = VB >= 4 ? VB / 4 : 1;
  // VB < 4: a lane loads the aligned dword that holds its VB bytes of a
  // token (whole dwords: every bit of the loaded register stays live, so no
  // narrowing or zero-extension has to wait for the data) and picks its
  // bytes with a per-lane byte selector
  static constexpr bool NARROW = VB < 4;
  static constexpr int DT = D / 16;              // V-pass d-tiles
};

// Bytes between consecutive query-piece planes of the decode LDS (Smem::qp:
// 32 rows of a batch's (segment, head) pieces plus one zero row, QB D + 16
// bytes each; QB = 1 for the int8 pieces, 2 for the bf16 pieces of FP8).
template <int D, int PHI, int QB = 1>
constexpr int kQPlane = (32 / (16 / PHI) * (16 / PHI) + 1) * (QB * D + 16);

// Query bytes per element in the decode LDS.
template <int MODE>
constexpr int q_elem_bytes() { return MODE == kFp8Mode ? 2 : 1; }

// d held by byte j (0..15) of the int8 operand of k-step s for lane-group
// d-range `sub` (K pass); the query pieces in LDS are laid out in this order.
template <int MODE, int D, int PHI>
__device__ __forceinline__ int kmap(int sub, int s, int j) {
  const int base = sub * Geo<MODE, D, PHI>::SUBD + 16 * s;
  if constexpr (code_mode(MODE) == 1) return base + 8 * ((j >> 2) >> 1) + 2 * (j & 3) + ((j >> 2) & 1);
  else if constexpr (MODE == 2) return base + 4 * (j & 3) + (j >> 2);
  else return base + j;
}

// K-pass int8 A operand of k-step s (16 codes) from the lane's K-tile dwords.
template <int MODE, int KSW>
__device__ __forceinline__ u32x4_t unpack_k(const uint32_t* kc, int s, uint32_t m4, uint32_t m2) {
  u32x4_t a;
  if constexpr (code_mode(MODE) == 1) {
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
template <int MODE, int VW, int DTI, bool NARROW>
__device__ __forceinline__ u32x4_t unpack_v(const uint32_t (*vc)[VW], uint32_t magic, uint32_t n4,
                                            uint32_t n2, uint32_t vsel) {
  u32x4_t a;
  if constexpr (MODE == kFp8Mode) {
    // E4M3 byte of tokens 2p and 2p + 1 side by side, then both to bf16
    // (every E4M3 value is a bf16 value)
    constexpr int w = DTI >> 2;
    constexpr uint32_t sel = (uint32_t)(DTI & 3) | ((4u + (DTI & 3)) << 8) | 0x0C0C0000u;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t y = __builtin_amdgcn_perm(vc[2 * p + 1][w], vc[2 * p][w], sel);
      a[p] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)y, 1.0f, false));
    }
  } else if constexpr (NARROW) {
    // vsel picks byte 0 of the lane's bytes in each of the two dwords; byte
    // b of them is vsel + b in both selector fields
    constexpr bool I4 = code_mode(MODE) == 1;
    constexpr uint32_t b = I4 ? DTI >> 1 : DTI >> 2;
    constexpr int sh = I4 ? 4 * (DTI & 1) : 2 * (DTI & 3);
    const uint32_t sel = vsel + b * 0x00010001u;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t y = __builtin_amdgcn_perm(vc[2 * p + 1][0], vc[2 * p][0], sel);
      a[p] = and_or(sh ? (y >> sh) : y, I4 ? n4 : n2, magic);
    }
  } else if constexpr (code_mode(MODE) == 1) {
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

template <int MODE, int VW, int DT, int DTI, bool NARROW>
struct VPass {
  __device__ __forceinline__ static void run(const uint32_t (*vc)[VW], u32x4_t bh, u32x4_t bl,
                                             f32x4_t* acc, uint32_t magic, uint32_t n4, uint32_t n2,
                                             uint32_t vsel) {
    const u32x4_t a = unpack_v<MODE, VW, DTI, NARROW>(vc, magic, n4, n2, vsel);
    acc[DTI] = mfma(a, bh, acc[DTI]);
    acc[DTI] = mfma(a, bl, acc[DTI]);
    VPass<MODE, VW, DT, DTI + 1, NARROW>::run(vc, bh, bl, acc, magic, n4, n2, vsel);
  }
};
template <int MODE, int VW, int DT, bool NARROW>
struct VPass<MODE, VW, DT, DT, NARROW> {
  __device__ __forceinline__ static void run(const uint32_t (*)[VW], u32x4_t, u32x4_t, f32x4_t*, uint32_t,
                                             uint32_t, uint32_t, uint32_t) {}
};

// Rows and validity of one tile's four 16-token sub-tiles (wave-uniform).
struct TileInfo {
  int pos0;                 // first position of the tile
  int row0, row1, row2, row3;  // plane row of the sub-tile's first token; 0 when invalid
  uint32_t valid;           // bit sigma: sub-tile has a block and meets [start, L)
};

// CB: block_size >= 64, so a tile lies in one block and its sub-tile rows
// are row0 + 16 s (one block id per tile).  A block id that is negative
// (evicted) or at or past num_blocks makes its sub-tiles invalid: no row is
// formed for them and issue_loads reads nothing for them.
// Attended positions of a pair: [start, L), plus [0, sink) when the head is
// windowed (sink is 0 otherwise).
// INL: rows of the inline layout, ((id 2 bs + offset) Hkv + h), tokens Hkv
// rows apart (the V rows use the same index from the V base).
template <bool CB, bool INL>
__device__ __forceinline__ TileInfo tile_info(const int32_t* ids, int blk0, int tile, int te, int L, int start,
                                              int sink, int bs_log2, int hkv, int h, int nblk) {
  TileInfo t;
  t.pos0 = tile * 64;
  t.valid = 0;
  if constexpr (CB) {
    const bool in = tile < te;
    const int id = __builtin_amdgcn_readfirstlane(ids[in ? (t.pos0 >> bs_log2) - blk0 : 0]);
    const bool okb = in && id >= 0 && id < nblk;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int pos = t.pos0 + 16 * s;
      t.valid |= (okb && pos < L && (pos + 15 >= start || pos < sink)) ? 1u << s : 0u;
    }
    const int pin = t.pos0 & ((1 << bs_log2) - 1);
    if constexpr (INL) {
      t.row0 = okb ? ((id << (bs_log2 + 1)) + pin) * hkv + h : 0;
      t.row1 = t.row0 + 16 * hkv; t.row2 = t.row0 + 32 * hkv; t.row3 = t.row0 + 48 * hkv;
      return t;
    }
    t.row0 = okb ? ((id * hkv + h) << bs_log2) + pin : 0;
    t.row1 = t.row0 + 16; t.row2 = t.row0 + 32; t.row3 = t.row0 + 48;
    return t;
  }
  int row[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int pos = t.pos0 + 16 * s;
    const bool in = tile < te && pos < L && (pos + 15 >= start || pos < sink);
    const int id = __builtin_amdgcn_readfirstlane(ids[in ? (pos >> bs_log2) - blk0 : 0]);
    const bool ok = in && id >= 0 && id < nblk;
    t.valid |= ok ? 1u << s : 0u;
    const int pin = pos & ((1 << bs_log2) - 1);
    row[s] = !ok ? 0 : (INL ? ((id << (bs_log2 + 1)) + pin) * hkv + h : ((id * hkv + h) << bs_log2) + pin);
  }
  t.row0 = row[0]; t.row1 = row[1]; t.row2 = row[2]; t.row3 = row[3];
  return t;
}

// Row of sub-tile sigma (sigma may differ per lane); 0 for an invalid
// sub-tile, whose loads are not issued.
__device__ __forceinline__ int pick_row(const TileInfo& t, int sigma) {
  return sigma == 0 ? t.row0 : (sigma == 1 ? t.row1 : (sigma == 2 ? t.row2 : t.row3));
}

template <int MODE, int D, int PHI>
struct Buf {
  using Gm = Geo<MODE, D, PHI>;
  uint32_t k[Gm::NKT][Gm::KW];
  uint32_t v[16][Gm::VW];
  float km[Gm::NKT][4 * (Gm::M > 0 ? Gm::M : 1)];   // unused without per-row metadata
  float vm[Gm::NKT][4 * (Gm::M > 0 ? Gm::M : 1)];
};

template <int MODE, int D, int PHI, bool CB>
__device__ __forceinline__ void issue_loads(Buf<MODE, D, PHI>& b, const TileInfo& t, const DecodeParams& p,
                                            int r, int q, int phi_col) {
  using Gm = Geo<MODE, D, PHI>;
  constexpr int P = Gm::P, M = Gm::M;
  const int phi_grp = q * PHI / 4;          // phase of this lane group (K pass)
  const int sub = q % (4 / PHI);            // d-range of this lane group (K pass)
  // An invalid sub-tile (evicted block, id out of range, or wholly outside
  // [start, L)) is not read: its registers keep whatever they held, which the
  // compute masks (score -inf, weight and V meta zero) and never lets reach a
  // result, since the codes are integers and every use is a select.
  if constexpr (Gm::INL) {
    // inline rows (4-byte aligned): tokens TS bytes apart, the stored scale
    // word at byte P of each row
    constexpr int RS = Gm::RS;
    const int TS = p.hkv * RS;
    if constexpr (CB) {
      if (t.valid == 0) return;
      const uint8_t* kb = p.k_codes + (int64_t)t.row0 * RS;
      const uint8_t* vb = p.v_codes + (int64_t)t.row0 * RS;
#pragma unroll
      for (int tau = 0; tau < Gm::NKT; ++tau) {
        load_bytes_a4<Gm::KB>(b.k[tau], kb + (16 * (tau * PHI + phi_grp) + r) * TS + sub * Gm::KB);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int mo = (16 * (tau * PHI + phi_col) + 4 * q + i) * TS + P;
          b.km[tau][i] = *reinterpret_cast<const float*>(kb + mo);
          b.vm[tau][i] = *reinterpret_cast<const float*>(vb + mo);
        }
      }
      const int vo = 4 * q * TS + ((r * Gm::VB) & ~3);
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int i = 0; i < 4; ++i) load_bytes_a4<Gm::NARROW ? 4 : Gm::VB>(b.v[4 * s + i], vb + vo + (16 * s + i) * TS);
      return;
    }
#pragma unroll
    for (int tau = 0; tau < Gm::NKT; ++tau) {
      const int sk = tau * PHI + phi_grp;
      if ((t.valid >> sk) & 1u)
        load_bytes_a4<Gm::KB>(b.k[tau], p.k_codes + (int64_t)pick_row(t, sk) * RS + r * TS + sub * Gm::KB);
      const int sm = tau * PHI + phi_col;
      if ((t.valid >> sm) & 1u) {
        const int64_t mb = (int64_t)pick_row(t, sm) * RS + P;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          b.km[tau][i] = *reinterpret_cast<const float*>(p.k_codes + mb + (4 * q + i) * TS);
          b.vm[tau][i] = *reinterpret_cast<const float*>(p.v_codes + mb + (4 * q + i) * TS);
        }
      }
    }
    const int vo = 4 * q * TS + ((r * Gm::VB) & ~3);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (!((t.valid >> s) & 1u)) continue;   // wave-uniform
      const int row = s == 0 ? t.row0 : (s == 1 ? t.row1 : (s == 2 ? t.row2 : t.row3));
      const uint8_t* base = p.v_codes + (int64_t)row * RS + vo;
#pragma unroll
      for (int i = 0; i < 4; ++i) load_bytes_a4<Gm::NARROW ? 4 : Gm::VB>(b.v[4 * s + i], base + i * TS);
    }
    return;
  }
  if constexpr (CB) {
    if (t.valid == 0) return;   // one block per tile: all four sub-tiles or none
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
    const uint32_t vo = (uint32_t)(4 * q * P + ((r * Gm::VB) & ~3));   // NARROW: the aligned dword
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int i = 0; i < 4; ++i) load_bytes<Gm::NARROW ? 4 : Gm::VB>(b.v[4 * s + i], vb + vo + (16 * s + i) * P);
    return;
  }
#pragma unroll
  for (int tau = 0; tau < Gm::NKT; ++tau) {
    const int sk = tau * PHI + phi_grp;     // per lane group
    if ((t.valid >> sk) & 1u) {
      const int kr = pick_row(t, sk) + r;
      load_bytes<Gm::KB>(b.k[tau], p.k_codes + (int64_t)kr * P + sub * Gm::KB);
    }
    const int sm = tau * PHI + phi_col;     // per lane
    if ((t.valid >> sm) & 1u) {
      const int mr = pick_row(t, sm) + 4 * q;
#pragma unroll
      for (int i = 0; i < M; ++i) {
        const float4 a = reinterpret_cast<const float4*>(p.k_meta + (int64_t)mr * M)[i];
        const float4 c = reinterpret_cast<const float4*>(p.v_meta + (int64_t)mr * M)[i];
        b.km[tau][4 * i] = a.x; b.km[tau][4 * i + 1] = a.y; b.km[tau][4 * i + 2] = a.z; b.km[tau][4 * i + 3] = a.w;
        b.vm[tau][4 * i] = c.x; b.vm[tau][4 * i + 1] = c.y; b.vm[tau][4 * i + 2] = c.z; b.vm[tau][4 * i + 3] = c.w;
      }
    }
  }
  const int voff = 4 * q * P + ((r * Gm::VB) & ~3);
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    if (!((t.valid >> s) & 1u)) continue;   // wave-uniform
    const int row = s == 0 ? t.row0 : (s == 1 ? t.row1 : (s == 2 ? t.row2 : t.row3));
    const uint8_t* base = p.v_codes + (int64_t)row * P;
#pragma unroll
    for (int i = 0; i < 4; ++i) load_bytes<Gm::NARROW ? 4 : Gm::VB>(b.v[4 * s + i], base + voff + i * P);
  }
}

struct WaveState {
  float m;     // running reference maximum (log2 units) of the lane's head
  float l;     // lane partial sum of p
  float z;     // lane partial sum of p * z_V
};

struct LaneConst {
  const int8_t* qa;    // query piece a of this lane's B operand row (LDS); pieces b
                       // and c sit kQPlane and 2 kQPlane bytes further
  float sp;            // log2 logit per unit of x (S/128 of the column's head)
  float q1r;           // sum of the column head's pieces, 2^14 a + 2^7 b + c
  int q;
  int phi_col;
  bool head_ok;
  uint32_t magic, n4, n2;   // bf16 128.0 pair; nibble and crumb masks of a bf16 pair
  uint32_t vsel;            // NARROW V rows: byte selector of the lane's first byte
};

// FP8 codes of masked rows set to zero.  A masked row may be unwritten or
// stale (an absent sub-tile keeps the registers of an earlier tile), and an
// E4M3 NaN byte (0x7F, 0xFF) there would reach every MFMA column through the
// products with zero that the integer modes rely on (the K pass mixes the
// phases' rows, the V pass sums over tokens).  Rows as issue_loads assigns
// them: K-tile tau of lane group q holds token 16 (tau PHI + phase) + r, V
// slot 4 s + i holds token 16 s + 4 q + i.
template <int MODE, int D, int PHI>
__device__ __forceinline__ void clear_masked_rows(Buf<MODE, D, PHI>& b, const TileInfo& t, int L, int start,
                                                  int sink) {
  using Gm = Geo<MODE, D, PHI>;
  int ln;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
  const int rr = ln & 15, qq = ln >> 4, pg = qq * PHI / 4;
#pragma unroll
  for (int tau = 0; tau < Gm::NKT; ++tau) {
    const int sk = tau * PHI + pg;
    const int pos = t.pos0 + 16 * sk + rr;
    const bool keep = ((t.valid >> sk) & 1u) && pos < L && (pos >= start || pos < sink);
#pragma unroll
    for (int w = 0; w < Gm::KW; ++w) b.k[tau][w] = keep ? b.k[tau][w] : 0u;
  }
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int pos = t.pos0 + 16 * s + 4 * qq + i;
      const bool keep = ((t.valid >> s) & 1u) && pos < L && (pos >= start || pos < sink);
#pragma unroll
      for (int w = 0; w < Gm::VW; ++w) b.v[4 * s + i][w] = keep ? b.v[4 * s + i][w] : 0u;
    }
}

// full: every position of the tile is present and inside [start, L), so no
// score needs a mask (wave-uniform; the masking sits behind a branch).
template <int MODE, int D, int PHI>
__device__ __forceinline__ void compute_tile(Buf<MODE, D, PHI>& b, const TileInfo& t, WaveState& st,
                                             f32x4_t* acc, const LaneConst& lc, int L, int start, int sink,
                                             bool full) {
  using Gm = Geo<MODE, D, PHI>;
  constexpr int M = Gm::M;
  const int q = lc.q, phi_col = lc.phi_col;
  if constexpr (MODE == kFp8Mode) {
    if (__builtin_expect(!full, 0)) clear_masked_rows<MODE, D, PHI>(b, t, L, start, sink);
  }
  // ---- K pass: int32 (a, b, c) dot products of the query pieces with the
  // codes; x = s_K (2^14 a + 2^7 b + c).code + z_K q1r, the log2 logit
  // being sp * x
  float sc[Gm::NKT][4];
#pragma unroll
  for (int tau = 0; tau < Gm::NKT && MODE == kFp8Mode; ++tau) {
    // FP8: E4M3 codes to bf16 (exact), bf16 MFMA against the query's three
    // bf16 pieces (hi, mid, lo) into one float32 accumulator; x = s_K q'.code
    constexpr int QP = kQPlane<D, PHI, 2>;
    f32x4_t fa = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int s = 0; s < Gm::KS; ++s) {
      const u32x4_t c8 = unpack_k<MODE, Gm::KSW>(b.k[tau], s, 0u, 0u);
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        u32x4_t a;
#pragma unroll
        for (int w = 0; w < 2; ++w) {
          a[2 * w] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)c8[2 * hh + w],
                                                                                           1.0f, false));
          a[2 * w + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)c8[2 * hh + w],
                                                                                               1.0f, true));
        }
        const int8_t* qp = lc.qa + 32 * s + 16 * hh;
        const uint4 xh = *reinterpret_cast<const uint4*>(qp);
        const uint4 xm = *reinterpret_cast<const uint4*>(qp + QP);
        const uint4 xl = *reinterpret_cast<const uint4*>(qp + 2 * QP);
        fa = mfma(a, u32x4_t{xh.x, xh.y, xh.z, xh.w}, fa);
        fa = mfma(a, u32x4_t{xm.x, xm.y, xm.z, xm.w}, fa);
        fa = mfma(a, u32x4_t{xl.x, xl.y, xl.z, xl.w}, fa);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) sc[tau][i] = fa[i] * b.km[tau][i];
  }
#pragma unroll
  for (int tau = 0; tau < Gm::NKT && MODE != kFp8Mode; ++tau) {
    i32x4_t ia = {0, 0, 0, 0}, ib = {0, 0, 0, 0}, ic = {0, 0, 0, 0};
#pragma unroll
    for (int s = 0; s < Gm::KS; ++s) {
      const u32x4_t a = unpack_k<MODE, Gm::KSW>(b.k[tau], s, 0x0F0F0F0Fu, 0x03030303u);
      // one address, three immediate offsets
      const uint4 xa = *reinterpret_cast<const uint4*>(lc.qa + 16 * s);
      const uint4 xb = *reinterpret_cast<const uint4*>(lc.qa + kQPlane<D, PHI> + 16 * s);
      const uint4 xc = *reinterpret_cast<const uint4*>(lc.qa + 2 * kQPlane<D, PHI> + 16 * s);
      ia = mfma_i8(a, u32x4_t{xa.x, xa.y, xa.z, xa.w}, ia);
      ib = mfma_i8(a, u32x4_t{xb.x, xb.y, xb.z, xb.w}, ib);
      ic = mfma_i8(a, u32x4_t{xc.x, xc.y, xc.z, xc.w}, ic);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // 2^7 a + b is exact in int32 (|.| < 2^29); one rounding joins c
      const float raw = __builtin_fmaf((float)((ia[i] << 7) + ib[i]), 128.0f, (float)ic[i]);
      // per-channel INT8: the K scales are folded into the query pieces
      // inline: the stored scale st, z = -zp st with zp its low 4 bits
      const float s = (M == 0 && !Gm::INL) ? 1.0f : (M == 2 ? b.km[tau][2 * i] : b.km[tau][i]);
      const float z = Gm::INL ? -(float)(__float_as_uint(s) & 0xFu) * s : (M == 2 ? b.km[tau][2 * i + 1] : 0.0f);
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
      svv[tau][i] = (M == 0 && !Gm::INL) ? 1.0f : (M == 2 ? b.vm[tau][2 * i] : b.vm[tau][i]);
      zvv[tau][i] = Gm::INL ? -(float)(__float_as_uint(svv[tau][i]) & 0xFu) * svv[tau][i]
                            : (M == 2 ? b.vm[tau][2 * i + 1] : 0.0f);
    }
  if (__builtin_expect(!full, 0)) {
    // the lane index re-derived here (mbcnt, from no register), so this rare
    // path's per-lane masks and offsets are not hoisted out of the tile loop,
    // where they would hold registers or spill
    int ln;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
    const int qm = ln >> 4, pm = (ln & 15) % PHI;
#pragma unroll
    for (int tau = 0; tau < Gm::NKT; ++tau) {
      const int sg = tau * PHI + pm;
      const bool tv = (t.valid >> sg) & 1u;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int pos = t.pos0 + 16 * sg + 4 * qm + i;
        const bool keep = tv && pos < L && (pos >= start || pos < sink);
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
        if constexpr (Gm::MZ) st.z = __builtin_fmaf(pr, zvv[tau][i + e], st.z);
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
      if constexpr (MODE != kFp8Mode) wsum += (h0 + bf16_lo(lo)) + (h1 + bf16_hi(lo));
    }
  }
  // ---- offset: acc -= 128 * (sum of the column's weights), as one MFMA per
  // d-tile against the sum split into three bf16 pieces (not for FP8, whose
  // codes enter the V pass as their own values)
  if constexpr (MODE != kFp8Mode) {
    wsum = add_xor32(add_xor16(wsum));
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
    VPass<MODE, Gm::VW, Gm::DT, 0, Gm::NARROW>::run(b.v + 8 * u, bh, bl, acc, lc.magic, lc.n4, lc.n2, lc.vsel);
  }
}

template <int MODE, int D, int PHI>
__device__ __forceinline__ void run_tile(Buf<MODE, D, PHI>& b, const TileInfo& t, WaveState& st,
                                         f32x4_t* acc, const LaneConst& lc, int L, int start, int sink) {
  if (!t.valid) return;
  const bool full = t.valid == 0xFu && (t.pos0 >= start || t.pos0 + 64 <= sink) && t.pos0 + 64 <= L;
  compute_tile<MODE, D, PHI>(b, t, st, acc, lc, L, start, sink, full);
}

// Waves per SIMD, i.e. resident four-wave workgroups per CU: two where the
// registers fit without spilling, so one workgroup's prologue and epilogue
// overlap another's tiles; three for INT2 with four phases, whose tiles are
// the lightest; one where a tile needs the whole register file.
template <int MODE, int D, int PHI>
constexpr int decode_waves_per_simd() {
  return (PHI == 1 || (mode_bits(MODE) == 8 && D == 128 && PHI < 4)) ? 1 : ((MODE == 2 && PHI == 4) ? 3 : 2);
}

// Waves per workgroup.  INT4 and INT2: all of a CU's waves in one
// workgroup (one per SIMD per round), so no two workgroups on a CU compete
// for issue; INT8, whose tiles
// are the heaviest in bytes: four-wave workgroups, several per CU, so one
// workgroup's segment barriers and prologue overlap another's loads
// (measured faster for each).
template <int MODE, int D, int PHI>
constexpr int decode_wg_waves() { return mode_bits(MODE) != 8 ? 4 * decode_waves_per_simd<MODE, D, PHI>() : 4; }

// ---------------------------------------------------------------------------
// Whole rows of D values, one row per wave: lane holds d = E*lane + e with
// E = D/64.

// One query row: q' = R q * scale * log2(e), then its three int8 pieces in
// k-slot order (q' ~ (S/2^14)(2^14 a + 2^7 b + c), S = max|q'|/127,
// |a| <= 127, |b|, |c| <= 64), sp = S/2^14 and q1r = sum(2^14 a + 2^7 b + c).
// sg and ch are the lane's rotation signs and K channel scales (d = E lane ..
// E lane + E - 1), read with the query row so that nothing here waits on a
// load.  `scratch` is the wave's own D floats of LDS (written and read back
// by the same wave, in order).
template <int MODE, int D, int PHI, bool ROT>
__device__ __forceinline__ void prep_query(const DecodeParams& p, uint32_t raw, const float (&sg)[D / 64],
                                           const float (&ch)[D / 64], float* scratch, int8_t* qa, int8_t* qb,
                                           int8_t* qc, float* qs, float* q1, int lane) {
  using Gm = Geo<MODE, D, PHI>;
  constexpr int E = D / 64;
  float x[E];
  if constexpr (E == 2) {
    x[0] = __uint_as_float(raw << 16);
    x[1] = __uint_as_float(raw & 0xffff0000u);
  } else {
    x[0] = __uint_as_float(raw << 16);
  }
  if constexpr (ROT) {
#pragma unroll
    for (int e = 0; e < E; ++e) x[e] *= sg[e];
    wave_fwht<D>(x, lane);
  }
  if constexpr (MODE == kChannelMode) {   // q . (c (.) s_K) = (q (.) s_K) . c
#pragma unroll
    for (int e = 0; e < E; ++e) x[e] *= ch[e];
  }
  const float qmul = ROT ? p.qscale * p.inv_sqrt_d : p.qscale;
  if constexpr (MODE == kFp8Mode) {
    // three bf16 pieces hi + mid + lo of q' (each residual exact in float32,
    // the sum within 2^-24 of q' relative); sp = 1, q1r = 0
#pragma unroll
    for (int e = 0; e < E; ++e) scratch[E * lane + e] = x[e] * qmul;
#pragma unroll
    for (int j = 0; j < E; ++j) {
      const int pos = lane + 64 * j;
      const int sub = pos / Gm::SUBD, rem = pos - sub * Gm::SUBD;
      const float v = scratch[kmap<MODE, D, PHI>(sub, rem >> 4, rem & 15)];
      const __bf16 hi = (__bf16)v;
      const float r1 = v - (float)hi;
      const __bf16 mid = (__bf16)r1;
      const __bf16 lo = (__bf16)(r1 - (float)mid);
      reinterpret_cast<__bf16*>(qa)[pos] = hi;
      reinterpret_cast<__bf16*>(qb)[pos] = mid;
      reinterpret_cast<__bf16*>(qc)[pos] = lo;
    }
    if (lane == 0) {
      *qs = 1.0f;
      *q1 = 0.0f;
    }
    return;
  }
  float mx = 0.0f;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    x[e] *= qmul;
    mx = fmaxf(mx, fabsf(x[e]));
    scratch[E * lane + e] = x[e];
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) mx = fmaxf(mx, lane_xor(mx, m));
  const float invS = mx > 0.0f ? 127.0f / mx : 0.0f;
  float sab = 0.0f;
#pragma unroll
  for (int j = 0; j < E; ++j) {
    const int pos = lane + 64 * j;
    const int sub = pos / Gm::SUBD, rem = pos - sub * Gm::SUBD;
    const float v = scratch[kmap<MODE, D, PHI>(sub, rem >> 4, rem & 15)];
    const float t = fminf(fmaxf(v * invS, -127.0f), 127.0f);
    const float a = __builtin_rintf(t);
    const float r1 = (t - a) * 128.0f;          // exact, |r1| <= 64
    const float bq = __builtin_rintf(r1);
    const float cq = __builtin_rintf((r1 - bq) * 128.0f);
    qa[pos] = (int8_t)a;
    qb[pos] = (int8_t)bq;
    qc[pos] = (int8_t)cq;
    sab += __builtin_fmaf(16384.0f, a, __builtin_fmaf(128.0f, bq, cq));   // each term exact (< 2^22)
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) sab += lane_xor(sab, m);
  if (lane == 0) {
    *qs = mx > 0.0f ? (mx / 127.0f) * 6.103515625e-05f : 1.0f;   // S / 2^14
    *q1 = sab;
  }
}

// One output row from its D normalized values in LDS: R^T (FWHT, signs,
// 1/sqrt(D)) when rotated, the V channel scales for per-channel INT8, then
// float32 or bf16 stores.
template <int MODE, int D, bool ROT>
__device__ __forceinline__ void finish_row(const DecodeParams& p, const float* src, int64_t orow, int lane) {
  constexpr int E = D / 64;
  float x[E];
#pragma unroll
  for (int e = 0; e < E; ++e) x[e] = src[E * lane + e];
  if constexpr (MODE == kChannelMode) {   // sum_t p_t c_t (.) s_V
    const int h = (int)((orow % p.hq) / p.group);
#pragma unroll
    for (int e = 0; e < E; ++e) x[e] *= p.chs[((int64_t)p.hkv + h) * D + E * lane + e];
  }
  if constexpr (ROT) {
    wave_fwht<D>(x, lane);
#pragma unroll
    for (int e = 0; e < E; ++e) x[e] = x[e] * p.signs[E * lane + e] * p.inv_sqrt_d;
  }
  if (p.out_bf16) {
    __bf16* o = reinterpret_cast<__bf16*>(p.out) + orow * D + E * lane;
    if constexpr (E == 2) *reinterpret_cast<uint32_t*>(o) = pack_bf16(x[0], x[1]);
    else o[0] = (__bf16)x[0];
  } else {
    float* o = reinterpret_cast<float*>(p.out) + orow * D + E * lane;
    if constexpr (E == 2) *reinterpret_cast<float2*>(o) = make_float2(x[0], x[1]);
    else o[0] = x[0];
  }
}

constexpr int kPrefChunk = 1024;   // pairs whose tile prefix one LDS pass holds

// A workgroup's piece of one (sequence, kv head) pair's tile range.
struct SegRec {
  int b, h;          // sequence, kv head
  int tb, te;        // tiles [tb, te) of the pair (tile t = positions 64t ..)
  int L, start;      // attended positions [start, L)
  int ids_off;       // LDS ids[ids_off + j] = table entry blk0 + j
  int blk0;
  int n_ids;
  int slot;          // partial slot, or -1: the segment is the whole pair
  int pad[2];
};

template <int D, int PHI, int NWV, int QB>
struct Smem {
  static constexpr int GM = 16 / PHI;   // most heads of a kv head's group (G * PHI <= 16)
  static constexpr int NS = 32 / GM;    // segments of one batch (their pieces stay in LDS)
  static constexpr int QW = QB * D + 16;   // piece row stride: 16 bytes of padding spread banks
  // query pieces a, b, c (int8; FP8: bf16 hi, mid, lo) in k-slot order:
  // piece p of row (segment k, head g) at qp[p][k GM + g]; row NS GM of every
  // piece is zero (the B rows of columns without work)
  alignas(16) int8_t qp[3][NS * GM + 1][QW];
  static_assert(sizeof(qp[0]) == (size_t)kQPlane<D, PHI, QB>, "query plane stride");
  float qs[NS][GM];                     // sp: (max|q'| / 127) / 2^14
  float q1[NS][GM];                     // q1r: sum over d of 2^14 a + 2^7 b + c
  SegRec seg[NS];
  int32_t ids[kMaxSplitBlocks];         // block ids of the batch's segments
  union {
    struct {
      float acc[NWV][GM][D];
      float ml[NWV][GM][2];
    } comb;                             // per-wave (m, l, acc) of a segment
    struct {
      float fin[2][GM][D];              // normalized rows before R^T (up to two pairs)
    } fw;
    float qrow[NWV][D];                 // query prologue scratch, one row per wave
  };
  int32_t pref[kPrefChunk + 1];         // inclusive tile prefix of a chunk of pairs
  int32_t plen[kPrefChunk];             // its pairs' attended end L and start
  int32_t pst[kPrefChunk];
  int32_t part[64 * NWV];
  int32_t pend[2][3];                   // pieces this workgroup published: pair, s0, s1
  int32_t pflag[2];                     // this workgroup counted the last piece in
};

// Tiles of (sequence b, kv head h): 64-position tiles from the window start
// (or 0; or 0 as well when the window cuts and sinks are on, the tiles in
// between then reading nothing) to seq_len; *t0 = first tile, *L = attended
// end, *start = window start.
__device__ __forceinline__ int first_tile(int start, int sink) { return (start > 0 && sink > 0) ? 0 : start / 64; }

// Sequence b and kv head h of pair `pair`.  The planes layouts number the
// pairs sequence-major (b Hkv + h).  The inline layout numbers them
// head-major (h B + b): its rows interleave a token's heads, so a 128-byte
// line holds parts of several heads' rows.  With equal shares over Hkv equal
// head blocks, shares w, w + nw / Hkv, ... then walk the same positions of
// one sequence's heads at the same time, and since workgroups go to the XCDs
// round-robin they sit on one XCD (one L2) whenever nw / Hkv is a multiple of
// the XCD count: a line is fetched once for all its heads, not once per head.
template <bool HM>
__device__ __forceinline__ void pair_bh(const DecodeParams& p, int hkv, int pair, int& b, int& h) {
  if constexpr (HM) {
    const int nb = p.num_pairs / hkv;
    h = pair / nb;
    b = pair - h * nb;
  } else {
    b = pair / hkv;
    h = pair - b * hkv;
  }
}

template <bool HM>
__device__ __forceinline__ int pair_geo(const DecodeParams& p, int pair, int* t0, int* L, int* start) {
  int b, h;
  pair_bh<HM>(p, p.hkv, pair, b, h);
  const int l = min(p.seq_lens[b], p.max_seq_len);   // host checked max_seq_len <= max_blocks * bs
  const int W = p.window ? p.window[h] : 0;
  const int s = (W > 0 && l > W) ? l - W : 0;
  *t0 = first_tile(s, p.sink);
  *L = l;
  *start = s;
  return l > 0 ? (l + 63) / 64 - *t0 : 0;
}

// The share partition: workgroup w takes tiles [start(w), start(w + 1)) of
// the T concatenated tiles, equal shares (nw <= T, so none is empty).
struct Part {
  int T, nw;
  __device__ int start(int w) const { return (int)(((int64_t)T * w) / nw); }
  // workgroup whose share holds tile x (0 <= x < T)
  __device__ int owner(int x) const {
    int lo = 0, hi = nw - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (start(mid) <= x) lo = mid; else hi = mid - 1;
    }
    return lo;
  }
};

// Workgroups in the partition: never more than tiles.
__device__ __forceinline__ int active_wgs(int grid, int T) { return max(1, min(grid, T)); }

// Tiles of one segment that wave `wave` computes: tb + wave + 4 i, padded to
// an even count (the pad is past te, hence invalid) so the two load buffers
// keep their roles across segments.
template <int NWV>
__device__ __forceinline__ int wave_tiles2(int n, int wave) {
  const int k = n > wave ? (n - wave + NWV - 1) / NWV : 0;
  return k + (k & 1);
}

// The wave's next tile to load, walking its tiles of the batch's segments in
// order (wave-uniform, scalar registers).
struct Cursor {
  int ls, li, nseg;
  int tb, te, off, blk0, L, start, h, n2;
};

template <int D, int PHI, int NWV, int QB>
__device__ __forceinline__ void cursor_seek(Cursor& c, const Smem<D, PHI, NWV, QB>& sm, int wave) {
  for (; c.ls < c.nseg; ++c.ls) {
    const SegRec& s = sm.seg[c.ls];
    c.tb = __builtin_amdgcn_readfirstlane(s.tb);
    c.te = __builtin_amdgcn_readfirstlane(s.te);
    c.n2 = wave_tiles2<NWV>(c.te - c.tb, wave);
    if (c.n2 > 0) {
      c.off = __builtin_amdgcn_readfirstlane(s.ids_off);
      c.blk0 = __builtin_amdgcn_readfirstlane(s.blk0);
      c.L = __builtin_amdgcn_readfirstlane(s.L);
      c.start = __builtin_amdgcn_readfirstlane(s.start);
      c.h = __builtin_amdgcn_readfirstlane(s.h);
      return;
    }
  }
}

template <bool CB, bool INL, int D, int PHI, int NWV, int QB>
__device__ __forceinline__ TileInfo cursor_info(const Cursor& c, const Smem<D, PHI, NWV, QB>& sm, int wave, int bl,
                                                int hkv, int nblk, int sink) {
  if (c.ls >= c.nseg) {
    TileInfo t;
    t.pos0 = 0; t.row0 = 0; t.row1 = 0; t.row2 = 0; t.row3 = 0; t.valid = 0;
    return t;
  }
  return tile_info<CB, INL>(sm.ids + c.off, c.blk0, c.tb + wave + NWV * c.li, c.te, c.L, c.start,
                       c.start > 0 ? sink : 0, bl, hkv, c.h, nblk);
}

template <int D, int PHI, int NWV, int QB>
__device__ __forceinline__ void cursor_next(Cursor& c, const Smem<D, PHI, NWV, QB>& sm, int wave) {
  if (++c.li < c.n2) return;
  c.li = 0;
  ++c.ls;
  cursor_seek(c, sm, wave);
}

// Pieces cross workgroups (and XCDs, whose L2s are not coherent with each
// other): they are stored and loaded with device scope, so they go to and
// come from the device-coherent level instead of a stale L2 line, and no
// cache-wide writeback or invalidate is needed.
__device__ __forceinline__ void store_dev(float* a, float v) {
  __hip_atomic_store(a, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_dev(const float* a) {
  return __hip_atomic_load(a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Merge the published pieces of up to two pairs (pair i: slots s0[i] ..
// s0[i] + n[i] - 1, output rows o0[i] ..), normalize, R^T and store.  All
// threads.  Each pass gives every thread U (head, d) values of both pairs;
// the thread folds each over its pieces in slot order with the online-softmax
// update, and requests the (m, l, acc) of KP pieces of every value at once,
// so a pass over pairs of at most KP pieces waits on memory once.
template <int MODE, int D, int PHI, int NWV, bool ROT, int KP, int QB>
__device__ __forceinline__ void merge_pieces(const DecodeParams& p, Smem<D, PHI, NWV, QB>& sm, int np, int s0a, int na,
                                             int64_t o0a, int s0b, int nb, int64_t o0b, int tid) {
  constexpr int NT = 64 * NWV;
  // values per thread and pass: enough to cover the largest group in one
  // pass where the threads are few, at most two (registers)
  constexpr int U = (Smem<D, PHI, NWV, QB>::GM * D + NT - 1) / NT >= 2 ? 2 : 1;
  const int G = p.group;
  const int GD = G * D;
  const int lane = tid & 63, wave = tid >> 6;
  const int64_t stride = (int64_t)G * (D + 4);   // floats between consecutive pieces
  const int nmax = max(na, np > 1 ? nb : 0);
  for (int e0 = 0; e0 < GD; e0 += U * NT) {
    float M[2][U], l[2][U], v[2][U];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int u = 0; u < U; ++u) { M[i][u] = kNegInf; l[i][u] = 0.0f; v[i][u] = 0.0f; }
    for (int s = 0; s < nmax; s += KP) {
      float pm[2][U][KP], pl[2][U][KP], pa[2][U][KP];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int n = i ? nb : na;
        const int slot0 = i ? s0b : s0a;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int e = e0 + u * NT + tid;
          const int g = e / D, d = e - g * D;
          const float* base = p.partials + ((int64_t)slot0 * G + g) * (D + 4);
#pragma unroll
          for (int k = 0; k < KP; ++k) {
            if (i < np && e < GD && s + k < n) {
              const float* rec = base + (s + k) * stride;
              pm[i][u][k] = load_dev(rec);
              pl[i][u][k] = load_dev(rec + 1);
              pa[i][u][k] = load_dev(rec + 4 + d);
            }
          }
        }
      }
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int n = i ? nb : na;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int e = e0 + u * NT + tid;
#pragma unroll
          for (int k = 0; k < KP; ++k) {
            if (i < np && e < GD && s + k < n) {
              const float mn = fmaxf(M[i][u], pm[i][u][k]);
              const float fo = M[i][u] == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(M[i][u] - mn);
              const float fn = pm[i][u][k] == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(pm[i][u][k] - mn);
              v[i][u] = v[i][u] * fo + pa[i][u][k] * fn;
              l[i][u] = l[i][u] * fo + pl[i][u][k] * fn;
              M[i][u] = mn;
            }
          }
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int e = e0 + u * NT + tid;
        if (i < np && e < GD) sm.fw.fin[i][e / D][e % D] = l[i][u] > 0.0f ? v[i][u] / l[i][u] : 0.0f;
      }
  }
  __syncthreads();
  for (int g = wave; g < G; g += NWV) {
    finish_row<MODE, D, ROT>(p, sm.fw.fin[0][g], o0a + g, lane);
    if (np > 1) finish_row<MODE, D, ROT>(p, sm.fw.fin[1][g], o0b + g, lane);
  }
}

// Inclusive tile prefix of pairs [c0, c0 + cn) into pref[1 .. cn] (pref[0] =
// 0); returns the chunk's tile total.  All threads of the workgroup; each
// thread takes a run of consecutive pairs, the runs are scanned within the
// wave by shuffles and across the waves in LDS.  Ends with a barrier.
template <int NWV, bool HM>
__device__ __forceinline__ int scan_chunk(const DecodeParams& p, int32_t* pref, int32_t* plen, int32_t* pst,
                                          int32_t* part, int c0, int cn, int tid) {
  constexpr int NT = 64 * NWV;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int per = (cn + NT - 1) / NT;
  int run = 0;
  for (int k = 0; k < per; ++k) {
    const int i = tid * per + k;
    if (i < cn) {
      int t0, L, s;
      run += pair_geo<HM>(p, c0 + i, &t0, &L, &s);
      pref[i + 1] = run;
      plen[i] = L;
      pst[i] = s;
    }
  }
  int x = run;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) part[wave] = x;
  __syncthreads();
  int before = x - run;
  for (int v = 0; v < wave; ++v) before += part[v];
  int tot = 0;
#pragma unroll
  for (int v = 0; v < NWV; ++v) tot += part[v];
  for (int k = 0; k < per; ++k) {
    const int i = tid * per + k;
    if (i < cn) pref[i + 1] += before;
  }
  if (tid == 0) pref[0] = 0;
  __syncthreads();
  return __builtin_amdgcn_readfirstlane(tot);
}

// First pair of a chunk whose range ends after tile x (cn if none).
__device__ __forceinline__ int first_after(const int32_t* pref, int cn, int cbase, int x) {
  int lo = 0, hi = cn;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (cbase + __builtin_amdgcn_readfirstlane(pref[mid + 1]) <= x) lo = mid + 1; else hi = mid;
  }
  return lo;
}

// Stream-K decode: a persistent grid of n_wgs workgroups.  The (sequence, kv
// head) pairs' tile ranges are concatenated in pair order (T tiles in all);
// workgroup w takes tiles [w T / NW, (w + 1) T / NW): the tail of one pair,
// some whole pairs, the head of another.  Each piece of a pair is a segment.
// Segments go in batches: the batch's block ids and query pieces are staged
// in LDS first; then every wave walks its tiles of all the batch's segments
// as one stream with one tile of look-ahead, so the loads of a segment's
// first tile are in flight while the previous segment is combined.  A whole
// pair is finished in place; a cut one writes (m, l, acc) to slot
// first_wg(pair) + pair + (w - first_wg(pair)) of the workspace and, at the
// end, bumps the pair's counter: the workgroup that brings it to the pieces'
// count merges them and resets it to zero.  Every workgroup scans the pairs'
// tile counts itself; there is no other launch and no waiting on another
// workgroup.
template <int MODE, int D, int PHI, bool ROT, bool CB, int NWV>
__global__ __launch_bounds__(64 * NWV) __attribute__((amdgpu_waves_per_eu(decode_waves_per_simd<MODE, D, PHI>())))
void decode_kernel(DecodeParams p) {
  using Sm = Smem<D, PHI, NWV, q_elem_bytes<MODE>()>;
  using Gm = Geo<MODE, D, PHI>;
  constexpr int NT = 64 * NWV, NS = Sm::NS;
  constexpr int QR = (NS * Sm::GM + NWV - 1) / NWV;      // query rows per wave in a batch prologue
  constexpr int IDR = (kMaxSplitBlocks + NT - 1) / NT;    // block ids per thread
  __shared__ Sm sm;
  const int tid = threadIdx.x;
  const int lane = tid & 63, r = lane & 15, q = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int P = p.num_pairs, G = p.group, hkv = p.hkv, bl = p.block_size_log2;
  const int nblk = (int)p.num_blocks;   // < 2^31 (checked on the host)
  const int w = blockIdx.x;
  constexpr bool HM = MODE == kInlineMode;   // pair order (pair_bh)

  // ---- tile prefix of the first chunk of pairs; total tiles
  for (int i = tid; i < 3 * Sm::QW; i += NT) sm.qp[i / Sm::QW][NS * Sm::GM][i % Sm::QW] = 0;
  int cn = min(kPrefChunk, P);
  int ctot = scan_chunk<NWV, HM>(p, sm.pref, sm.plen, sm.pst, sm.part, 0, cn, tid);
  int T = ctot;
  if (P > cn) {
    int my = 0;
    for (int i = cn + tid; i < P; i += NT) {
      int t0, L, s;
      my += pair_geo<HM>(p, i, &t0, &L, &s);
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) my += __shfl_xor(my, m);
    if (lane == 0) sm.part[wave] = my;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NWV; ++i) T += __builtin_amdgcn_readfirstlane(sm.part[i]);
    __syncthreads();
  }
  Part part;
  part.T = T;
  part.nw = active_wgs(gridDim.x, T);
  const int nw = part.nw;
  if (w >= nw) return;
  const int e_my = part.start(w + 1);

  // ---- pairs without tiles (an empty sequence) get zero rows; pair i falls
  // to workgroup i % nw.  Pairs of the first prefix chunk take their length
  // from LDS (the scan's), so only batches of more than kPrefChunk pairs
  // read seq_lens again here.
  for (int i = w + tid * nw; i < P; i += NT * nw) {
    int t0, L, s;
    if (i < cn ? sm.plen[i] <= 0 : pair_geo<HM>(p, i, &t0, &L, &s) == 0) {
      int b, h;
      pair_bh<HM>(p, hkv, i, b, h);
      const int64_t o = ((int64_t)b * p.hq + h * G) * D;
      for (int e = 0; e < G * D; ++e) {
        if (p.out_bf16) reinterpret_cast<__bf16*>(p.out)[o + e] = (__bf16)0.0f;
        else reinterpret_cast<float*>(p.out)[o + e] = 0.0f;
      }
    }
  }

  // ---- per-lane constants of the MFMA columns
  const int g_col = r / PHI;            // head of this lane's MFMA column
  const int phi_col = r % PHI;          // phase of this lane's MFMA column
  const int phi_grp = q * PHI / 4;      // phase of this lane group (K pass)
  const int sub = q % (4 / PHI);
  const uint32_t magic = to_vgpr(p.bits_magic), n4 = to_vgpr(p.bits_n4), n2m = to_vgpr(p.bits_n2);
  // byte (r * VB) % 4 of the dword in both selector fields, zero bytes between
  const uint32_t vsel0 = (uint32_t)((r * Gm::VB) & 3);
  const uint32_t vsel = vsel0 | 0x0C00u | ((4u + vsel0) << 16) | 0x0C000000u;

  // chunk of pairs whose prefix is in LDS: pairs [c0, c0 + cn), cbase tiles
  // before it, ci the next pair to look at
  int c0 = 0, cbase = 0;
  int x = part.start(w);  // next tile of the share
  int ci = first_after(sm.pref, cn, cbase, x);
  int npend = 0;

  while (x < e_my) {
    // ---- a batch: up to NS segments whose block ids fit the LDS table
    __syncthreads();   // every wave is done with the previous batch's records
    int nseg = 0, ids_used = 0;
    while (nseg < NS && x < e_my) {
      if (ci >= cn) {
        c0 += cn;
        cbase += ctot;
        cn = min(kPrefChunk, P - c0);
        if (cn <= 0) {   // no pair left (cannot happen while x < T)
          x = e_my;
          break;
        }
        __syncthreads();   // earlier readers of pref / part are done
        ctot = scan_chunk<NWV, HM>(p, sm.pref, sm.plen, sm.pst, sm.part, c0, cn, tid);
        ci = first_after(sm.pref, cn, cbase, x);
        continue;
      }
      const int s0 = cbase + __builtin_amdgcn_readfirstlane(sm.pref[ci]);
      const int s1 = cbase + __builtin_amdgcn_readfirstlane(sm.pref[ci + 1]);
      if (s1 <= x) {
        ++ci;
        continue;
      }
      const int pair = c0 + ci;
      const int L = __builtin_amdgcn_readfirstlane(sm.plen[ci]);
      const int start = __builtin_amdgcn_readfirstlane(sm.pst[ci]);
      const int t0 = first_tile(start, p.sink);
      const int e = min(s1, e_my);
      const int tb = t0 + (x - s0), te = t0 + (e - s0);
      const int blk0 = (tb * 64) >> bl;
      const int n_ids = ((min(te * 64, L) - 1) >> bl) - blk0 + 1;
      if (ids_used + n_ids > kMaxSplitBlocks) {
        if (nseg > 0) break;
        x = e_my;   // cannot happen for a launch the host sized; give up the share
        break;
      }
      const bool whole = x == s0 && e == s1;
      if (tid == 0) {
        SegRec& s = sm.seg[nseg];
        pair_bh<HM>(p, hkv, pair, s.b, s.h);
        s.tb = tb;
        s.te = te;
        s.L = L;
        s.start = start;
        s.ids_off = ids_used;
        s.blk0 = blk0;
        s.n_ids = n_ids;
        s.slot = whole ? -1 : pair + w;
        if (!whole && npend < 2) {
          sm.pend[npend][0] = pair;
          sm.pend[npend][1] = s0;
          sm.pend[npend][2] = s1;
        }
      }
      npend = min(2, npend + (whole ? 0 : 1));   // a share cuts at most two pairs
      ids_used += n_ids;
      ++nseg;
      x = e;
      if (x == s1) ++ci;
    }
    if (nseg == 0) break;
    __syncthreads();   // records visible; the previous batch's LDS reads are done

    int pt = threadIdx.x;   // thread index opaque to the compiler, as in the segment epilogue
    asm volatile("" : "+v"(pt));
    const int plane = pt & 63;
    // the tile buffers live within one batch (each batch loads its first
    // tile afresh), so nothing holds them across the share's merges
    Buf<MODE, D, PHI> ba, bb;

    // fused step: does this batch hold the last tile of a pair (the tile with
    // the new token at position L - 1)?
    bool wr = false;
    if (p.fused) {
      for (int k = 0; k < nseg; ++k) {
        const int te = __builtin_amdgcn_readfirstlane(sm.seg[k].te);
        const int Lk = __builtin_amdgcn_readfirstlane(sm.seg[k].L);
        wr = wr || (Lk > 0 && te - 1 == (Lk - 1) >> 6);
      }
    }

    // ---- batch prologue: the block ids (into LDS) and the query rows (into
    // registers) are requested first, then the block id of the wave's first
    // tile (from the table itself), and that tile's loads go out as soon as
    // the id is back.  Vector loads complete in order, so the waits for the
    // ids and the queries below never wait for tile data: the first tiles
    // stream while the prologue finishes.  A tile holding a new token waits
    // until after the barrier that follows the token's store.
    uint32_t raw[QR];
    float qch[QR][D / 64];
    float qsg[D / 64];
    int idv[IDR];
#pragma unroll
    for (int u = 0; u < IDR; ++u) {
      const int j = pt + u * NT;
      idv[u] = 0;
      if (j < ids_used) {
        int k = 0;
        while (k + 1 < nseg && sm.seg[k + 1].ids_off <= j) ++k;
        const SegRec& s = sm.seg[k];
        const int32_t* trow = p.tables + (int64_t)(p.headwise ? s.b * hkv + s.h : s.b) * p.max_blocks;
        idv[u] = trow[s.blk0 + (j - s.ids_off)];
      }
    }
#pragma unroll
    for (int e = 0; e < D / 64; ++e) qsg[e] = ROT ? p.signs[(D / 64) * plane + e] : 1.0f;
#pragma unroll
    for (int i = 0; i < QR; ++i) {
      const int rr = wave + i * NWV;
      raw[i] = 0;
#pragma unroll
      for (int e = 0; e < D / 64; ++e) qch[i][e] = 1.0f;
      if (rr < nseg * G) {
        const int k = rr / G, g = rr - k * G;
        const int b = __builtin_amdgcn_readfirstlane(sm.seg[k].b), h = __builtin_amdgcn_readfirstlane(sm.seg[k].h);
        raw[i] = load_qrow<D>(p.q + ((int64_t)b * p.hq + h * G + g) * D, plane);
        if constexpr (MODE == kChannelMode) {
#pragma unroll
          for (int e = 0; e < D / 64; ++e) qch[i][e] = p.chs[(int64_t)h * D + (D / 64) * plane + e];
        }
      }
    }
    const bool writer = wr && wave == NWV - 1;
    Cursor cur;
    cur.ls = 0;
    cur.li = 0;
    cur.nseg = nseg;
    cursor_seek(cur, sm, wave);
    TileInfo ta;
    // the last wave writes the new tokens, so only it waits on stores; its
    // first tile, and any wave's first tile that holds a new token, go out
    // after the barrier
    const bool defer = writer ||
                       (wr && cur.ls < nseg && cur.L > 0 && cur.tb + wave + NWV * cur.li == (cur.L - 1) >> 6);
    if (cur.ls < nseg) {
      const int b0 = __builtin_amdgcn_readfirstlane(sm.seg[cur.ls].b);
      const int32_t* trow = p.tables + (int64_t)(p.headwise ? b0 * hkv + cur.h : b0) * p.max_blocks;
      ta = tile_info<CB, MODE == kInlineMode>(trow + cur.blk0, cur.blk0, cur.tb + wave + NWV * cur.li, cur.te,
                                              cur.L, cur.start,
                         cur.start > 0 ? p.sink : 0, bl, hkv, cur.h, nblk);
    } else {
      ta = cursor_info<CB, MODE == kInlineMode>(cur, sm, wave, bl, hkv, nblk, p.sink);
    }
    cursor_next(cur, sm, wave);
    // the ids, query rows, signs and channel scales are back (the table read
    // above waited for all older loads): consume them before the tile loads
    // go out, so no later
    // wait has to count those loads (a deferred tile would otherwise make the
    // compiler wait for every load at the join)
#pragma unroll
    for (int u = 0; u < IDR; ++u) {
      const int j = pt + u * NT;
      if (j < ids_used) sm.ids[j] = idv[u];
    }
#pragma unroll
    for (int i = 0; i < QR; ++i) asm volatile("" : "+v"(raw[i]));
#pragma unroll
    for (int e = 0; e < D / 64; ++e) {
      if constexpr (ROT) asm volatile("" : "+v"(qsg[e]));
      if constexpr (MODE == kChannelMode) {
#pragma unroll
        for (int i = 0; i < QR; ++i) asm volatile("" : "+v"(qch[i][e]));
      }
    }
    __atomic_signal_fence(__ATOMIC_SEQ_CST);   // keep those stores above the tile loads
    if (!defer) issue_loads<MODE, D, PHI, CB>(ba, ta, p, r, q, phi_col);

    // ---- fused step: the new token of every pair whose last tile is in
    // this batch is quantized and stored (K and V rows, one lane group of the
    // writer wave each), and the writer waits for its stores before the
    // barrier below, after which the tile holding it may be read.  Only this
    // workgroup reads that tile, so no other workgroup has to wait for it.
    if (writer) {
      // the writer wave has no tile loads out yet, so each pass's loads (the
      // slot, the row and the signs, none waiting on another) cost one round
      // trip; a row without a slot stores nothing
      constexpr int WLPR = D / 8;   // lanes per new-token row
      float wsg[8] = {1.0f, 1.0f, 1.0f, 1.0f, 1.0f, 1.0f, 1.0f, 1.0f};
      if constexpr (ROT) write_row_signs(p.wp, plane % WLPR, wsg);
      for (int g0 = 0; g0 < 2 * nseg; g0 += 64 / WLPR) {
        const int grp = g0 + plane / WLPR;
        if (grp < 2 * nseg) {
          const SegRec& sr = sm.seg[grp >> 1];
          if (sr.L > 0 && sr.te - 1 == (sr.L - 1) >> 6) {
            int64_t slot = p.wp.slot_hw ? p.wp.slot_hw[(int64_t)sr.b * hkv + sr.h] : p.wp.slot[sr.b];
            uint4 raw = write_row_load<D>(p.wp, sr.b, sr.h, grp & 1, plane % WLPR);
            // both loads out before either is used (the compiler would
            // otherwise sink the row load under the slot test)
            asm volatile("" : "+v"(raw.x), "+v"(raw.y), "+v"(raw.z), "+v"(raw.w), "+v"(slot));
            write_row_store<MODE, D, ROT>(p.wp, raw, wsg, sr.h, grp & 1, slot, plane % WLPR);
          }
        }
      }
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      __builtin_amdgcn_s_waitcnt(0);
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
    }

    __syncthreads();
    if (defer) issue_loads<MODE, D, PHI, CB>(ba, ta, p, r, q, phi_col);

#pragma unroll
    for (int i = 0; i < QR; ++i) {
      const int rr = wave + i * NWV;
      if (rr < nseg * G) {
        const int k = rr / G, g = rr - k * G;
        prep_query<MODE, D, PHI, ROT>(p, raw[i], qsg, qch[i], sm.qrow[wave], sm.qp[0][k * Sm::GM + g],
                                      sm.qp[1][k * Sm::GM + g], sm.qp[2][k * Sm::GM + g], &sm.qs[k][g],
                                      &sm.q1[k][g], plane);
      }
    }
    __syncthreads();

    // ---- the stream: segment by segment, look-ahead across segment ends
    for (int k = 0; k < nseg; ++k) {
      const SegRec& sr = sm.seg[k];
      const int L = __builtin_amdgcn_readfirstlane(sr.L);
      const int start = __builtin_amdgcn_readfirstlane(sr.start);
      const int sinkE = start > 0 ? p.sink : 0;
      const int n2 = wave_tiles2<NWV>(__builtin_amdgcn_readfirstlane(sr.te) -
                                      __builtin_amdgcn_readfirstlane(sr.tb), wave);
      LaneConst lc;
      lc.q = q;
      lc.phi_col = phi_col;
      lc.head_ok = g_col < G;
      const bool brow = lc.head_ok && phi_grp == phi_col;
      lc.qa = &sm.qp[0][brow ? k * Sm::GM + g_col : NS * Sm::GM][q_elem_bytes<MODE>() * sub * Gm::SUBD];
      lc.sp = lc.head_ok ? sm.qs[k][g_col] : 1.0f;
      lc.q1r = lc.head_ok ? sm.q1[k][g_col] : 0.0f;
      lc.magic = magic;
      lc.n4 = n4;
      lc.n2 = n2m;
      lc.vsel = vsel;

      WaveState st{kNegInf, 0.0f, 0.0f};
      f32x4_t acc[Gm::DT];
#pragma unroll
      for (int i = 0; i < Gm::DT; ++i) acc[i] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

      for (int it = 0; it < n2; it += 2) {
        const TileInfo tn = cursor_info<CB, MODE == kInlineMode>(cur, sm, wave, bl, hkv, nblk, p.sink);
        cursor_next(cur, sm, wave);
        issue_loads<MODE, D, PHI, CB>(bb, tn, p, r, q, phi_col);
        run_tile<MODE, D, PHI>(ba, ta, st, acc, lc, L, start, sinkE);
        const TileInfo t2 = cursor_info<CB, MODE == kInlineMode>(cur, sm, wave, bl, hkv, nblk, p.sink);
        cursor_next(cur, sm, wave);
        issue_loads<MODE, D, PHI, CB>(ba, t2, p, r, q, phi_col);
        run_tile<MODE, D, PHI>(bb, tn, st, acc, lc, L, start, sinkE);
        ta = t2;
      }

      // ---- segment epilogue: sum the phases of a head, then l and z over
      // lane groups; combine the waves in LDS
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
      // thread index the compiler cannot see through: the combine's
      // lane-dependent addresses are formed here, not hoisted out of the
      // segment loop and held across the tiles
      int et = threadIdx.x;
      asm volatile("" : "+v"(et));
      const int elane = et & 63;
      __syncthreads();   // the combine area is free
      if (lc.head_ok && phi_col == 0) {
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

      constexpr int PER = (Sm::GM * D + NT - 1) / NT;
      float val[PER], lsum[PER], mmax[PER];
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        const int e = et + j * NT;
        val[j] = 0.0f; lsum[j] = 0.0f; mmax[j] = kNegInf;
        if (e < G * D) {
          const int g = e / D, d = e - g * D;
          float mx = kNegInf;
#pragma unroll
          for (int v = 0; v < NWV; ++v) mx = fmaxf(mx, sm.comb.ml[v][g][0]);
          const float mu = mx == kNegInf ? 0.0f : mx;
#pragma unroll
          for (int v = 0; v < NWV; ++v) {
            const float f = __builtin_amdgcn_exp2f(sm.comb.ml[v][g][0] - mu);
            val[j] += f * sm.comb.acc[v][g][d];
            lsum[j] += f * sm.comb.ml[v][g][1];
          }
          mmax[j] = mx;
        }
      }
      const int slot = __builtin_amdgcn_readfirstlane(sr.slot);
      const int b = __builtin_amdgcn_readfirstlane(sr.b), h = __builtin_amdgcn_readfirstlane(sr.h);
      const int64_t orow0 = (int64_t)b * p.hq + h * G;
      if (slot < 0) {
        __syncthreads();   // fin overlays the combine area
#pragma unroll
        for (int j = 0; j < PER; ++j) {
          const int e = et + j * NT;
          if (e < G * D) sm.fw.fin[0][e / D][e % D] = lsum[j] > 0.0f ? val[j] / lsum[j] : 0.0f;
        }
        __syncthreads();
        for (int g = wave; g < G; g += NWV) finish_row<MODE, D, ROT>(p, sm.fw.fin[0][g], orow0 + g, elane);
      } else {
#pragma unroll
        for (int j = 0; j < PER; ++j) {
          const int e = et + j * NT;
          if (e < G * D) {
            const int g = e / D, d = e - g * D;
            float* rec = p.partials + ((int64_t)slot * G + g) * (D + 4);
            store_dev(rec + 4 + d, val[j]);
            if (d == 0) {
              store_dev(rec, mmax[j]);
              store_dev(rec + 1, lsum[j]);
            }
          }
        }
      }
    }
  }

  // ---- published pieces: count them in; the last of a pair merges it
  if (npend > 0) {
    // the pieces' device-scope stores are complete before any count
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __syncthreads();
    // one lane per published piece: all counts go out together
    if (tid < npend) {
      const int fw = part.owner(sm.pend[tid][1]), lw = part.owner(sm.pend[tid][2] - 1);
      sm.pflag[tid] = atomicAdd(p.counters + sm.pend[tid][0], 1) == lw - fw;
    }
    __syncthreads();
    // the pairs this workgroup completes (at most two), merged together
    int np = 0, s0a = 0, na = 0, s0b = 0, nb = 0, pa = 0, pb = 0;
    int64_t o0a = 0, o0b = 0;
    for (int i = 0; i < npend; ++i) {
      if (__builtin_amdgcn_readfirstlane(sm.pflag[i])) {
        const int pair = __builtin_amdgcn_readfirstlane(sm.pend[i][0]);
        const int fw = part.owner(__builtin_amdgcn_readfirstlane(sm.pend[i][1]));
        const int lw = part.owner(__builtin_amdgcn_readfirstlane(sm.pend[i][2]) - 1);
        int b, h;
        pair_bh<HM>(p, hkv, pair, b, h);
        if (np == 0) {
          s0a = pair + fw; na = lw - fw + 1; o0a = (int64_t)b * p.hq + h * G; pa = pair;
        } else {
          s0b = pair + fw; nb = lw - fw + 1; o0b = (int64_t)b * p.hq + h * G; pb = pair;
        }
        ++np;
      }
    }
    if (np > 0) {
      // eight pieces per round trip, four in the variants with three waves per
      // SIMD (168 registers)
      constexpr int KP = decode_waves_per_simd<MODE, D, PHI>() >= 3 ? 4 : 8;
      merge_pieces<MODE, D, PHI, NWV, ROT, KP>(p, sm, np, s0a, na, o0a, s0b, nb, o0b, tid);
      if (tid < np) atomicExch(p.counters + (tid ? pb : pa), 0);
    }
  }
}

template <int MODE, int D, int PHI, bool ROT>
hipError_t launch_decode_t(const DecodeParams& p, hipStream_t s) {
  constexpr int NWV = decode_wg_waves<MODE, D, PHI>();
  if (p.block_size >= 64)
    hipLaunchKernelGGL((decode_kernel<MODE, D, PHI, ROT, true, NWV>), dim3(p.n_wgs), dim3(64 * NWV), 0, s, p);
  else
    hipLaunchKernelGGL((decode_kernel<MODE, D, PHI, ROT, false, NWV>), dim3(p.n_wgs), dim3(64 * NWV), 0, s, p);
  return hipGetLastError();
}

template <int MODE, int D, bool ROT>
hipError_t launch_decode_p(const DecodeParams& p, hipStream_t s) {
  if (p.group * 4 <= 16) return launch_decode_t<MODE, D, 4, ROT>(p, s);
  if (p.group * 2 <= 16) return launch_decode_t<MODE, D, 2, ROT>(p, s);
  return launch_decode_t<MODE, D, 1, ROT>(p, s);
}

template <int MODE>
hipError_t launch_decode_m(int d, bool rot, const DecodeParams& p, hipStream_t s) {
  if constexpr (MODE == kChannelMode) {   // no rotation in this mode (checked on the host)
    return d == 64 ? launch_decode_p<MODE, 64, false>(p, s) : launch_decode_p<MODE, 128, false>(p, s);
  } else {
    if (d == 64) return rot ? launch_decode_p<MODE, 64, true>(p, s) : launch_decode_p<MODE, 64, false>(p, s);
    return rot ? launch_decode_p<MODE, 128, true>(p, s) : launch_decode_p<MODE, 128, false>(p, s);
  }
}

}  // namespace

int decode_wgs_per_cu(int mode, int d, int group) {
  const int phi = group * 4 <= 16 ? 4 : (group * 2 <= 16 ? 2 : 1);
#define KVQ_W(M_, D_, P_) if (mode == M_ && d == D_ && phi == P_) return 4 * decode_waves_per_simd<M_, D_, P_>() / decode_wg_waves<M_, D_, P_>();
  KVQ_W(0, 64, 4) KVQ_W(0, 64, 2) KVQ_W(0, 64, 1) KVQ_W(0, 128, 4) KVQ_W(0, 128, 2) KVQ_W(0, 128, 1)
  KVQ_W(1, 64, 4) KVQ_W(1, 64, 2) KVQ_W(1, 64, 1) KVQ_W(1, 128, 4) KVQ_W(1, 128, 2) KVQ_W(1, 128, 1)
  KVQ_W(2, 64, 4) KVQ_W(2, 64, 2) KVQ_W(2, 64, 1) KVQ_W(2, 128, 4) KVQ_W(2, 128, 2) KVQ_W(2, 128, 1)
  KVQ_W(3, 64, 4) KVQ_W(3, 64, 2) KVQ_W(3, 64, 1) KVQ_W(3, 128, 4) KVQ_W(3, 128, 2) KVQ_W(3, 128, 1)
  KVQ_W(4, 64, 4) KVQ_W(4, 64, 2) KVQ_W(4, 64, 1) KVQ_W(4, 128, 4) KVQ_W(4, 128, 2) KVQ_W(4, 128, 1)
  KVQ_W(5, 64, 4) KVQ_W(5, 64, 2) KVQ_W(5, 64, 1) KVQ_W(5, 128, 4) KVQ_W(5, 128, 2) KVQ_W(5, 128, 1)
#undef KVQ_W
  return 4;
}

hipError_t launch_decode(int mode, int d, bool rot, const DecodeParams& p, hipStream_t s) {
  switch (mode) {
    case 0: return launch_decode_m<0>(d, rot, p, s);
    case 1: return launch_decode_m<1>(d, rot, p, s);
    case 2: return launch_decode_m<2>(d, rot, p, s);
    case kChannelMode: return launch_decode_m<kChannelMode>(d, rot, p, s);
    case kFp8Mode: return launch_decode_m<kFp8Mode>(d, rot, p, s);
    default: return launch_decode_m<kInlineMode>(d, rot, p, s);
  }
}

}  // namespace kvq
