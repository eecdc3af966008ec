// Chunked-prefill attention over the quantized paged cache.
//
// Follows the read half of the prhub summary of vLLM PR 40835 ("INT4
// per-token-head KV cache quantization for the Triton backend", 实现拆解
// item 2: unpack, dequantize, attend), prefill over a gathered and
// dequantized paged cache as described for the vllm-ascend-quantized-kv-cache
// package (运行机制), and the head-wise block-table walk with -1 skips and the
// per-head sliding window of FastDeploy PR 7718 ("Optimize AppendAttention for
// discrete head-wise block_idx").
//
// Sequence b appends n_b query tokens that sit at positions L_b - n_b + i
// (their K/V rows are already in the cache).  Query row (token i, q head hq)
// attends to the cached positions j <= L_b - n_b + i whose block is present
// and, for a windowed kv head, j >= L_b - n_b + i - W + 1:
//   out = R^T sum_j softmax_j(scale * q'.k_hat_j) v_hat_j ,  q' = R q.
// As in decode, nothing is dequantized element by element:
//   q'.k_hat_j = s_j (q'.c_j) + z_j sum(q')
//   sum_j p_j v_hat_j = sum_j (p_j s_j) c_j + sum_j p_j z_j .
//
// Work split: one 256-thread workgroup (4 waves) per (query tile, kv head,
// sequence); a query tile is floor(128 / G) consecutive tokens times the G q
// heads of the kv head, 128 rows (token-major), 32 per wave.  The workgroup
// walks 64-position key tiles from the earliest window start of its rows to
// its last row's position.  Each tile is staged through LDS once for all
// waves: K as int8 codes in k-slot order (two or three bit operations per 16
// codes for INT4 / INT2), V transposed to [d][position] as exact bf16
// integers c, and per-position (s_K, z_K, s_V, z_V).  The next tile's global
// loads are in flight while the current tile is computed.
//
// Per wave and tile (lane l: r = l % 16, q = l / 16):
//   S^T = K Q^T on v_mfma_i32_16x16x64_i8
//     A  codes [16 positions x 64 k] from LDS, position 16 kb + r
//     B  query pieces [64 k x 16 rows] in registers; q' * scale * log2(e) is
//        split into three int8 pieces (q' ~ S (a + b / 2^7 + c / 2^14),
//        |a| <= 127, |b|, |c| <= 64) that accumulate exactly in int32
//     C  lane (row r, positions 16 kb + 4 q + i)
//   O += W V on v_mfma_f32_16x16x32_bf16, W = p * s_V as bf16 hi + lo
//     A  W [16 rows x 32 positions]: the C registers of two key blocks
//     B  V^T [32 positions x 16 d] from LDS, the position order matching A
//     C  lane (d 16 db + r, rows 4 q + i)
// The online softmax keeps one reference maximum per row (log2 units) and
// rescales only when a row's maximum grows by more than 2^8.
#include "kvq_internal.h"
#include "kvq_device.h"

namespace kvq {
namespace {

constexpr int kPWaves = 4;
constexpr int kPRows = 128;   // query rows per workgroup
constexpr int kPKeys = 64;    // positions per key tile

template <int MODE, int D>
struct PGeo {
  static constexpr int P = row_bytes(MODE, D);             // packed bytes per row
  static constexpr int M = mode_meta(MODE);                // meta floats per row
  static constexpr int DC = D / 4;                         // d per K-staging thread
  static constexpr int KNW = DC * mode_bits(MODE) / 32;    // K code dwords per staging thread
  static constexpr int DPT = D / 16;                       // d per V-staging thread
  static constexpr int VNB = DPT * mode_bits(MODE) / 8;    // V bytes per position per thread
  static constexpr int VNW = VNB >= 4 ? VNB / 4 : 1;
  static constexpr int KS = D / 64;                        // int8 k-steps
  static constexpr int DB = D / 16;                        // d-blocks of the PV product
  static constexpr int KROW = D + 16;                      // LDS K row stride, bytes
  static constexpr int VROW = 2 * kPKeys + 16;             // LDS V^T row stride, bytes
};

// d of k-slot c (0 .. DC-1) inside a K-staging chunk, for the order the
// staging threads write: INT4 puts the low nibbles of the chunk's dwords
// first, then the high ones; INT2 puts its four 2-bit planes one after the
// other.
template <int MODE, int D>
__device__ __forceinline__ int kslot_d(int s) {
  constexpr int DC = PGeo<MODE, D>::DC;
  const int base = (s / DC) * DC, c = s % DC;
  if constexpr (code_mode(MODE) == 1) {
    const int pl = c / (DC / 2), rem = c % (DC / 2);
    return base + 8 * (rem >> 2) + 2 * (rem & 3) + pl;
  } else if constexpr (MODE == 2) {
    const int pl = c / (DC / 4), rem = c % (DC / 4);
    return base + 16 * (rem >> 2) + 4 * (rem & 3) + pl;
  } else {
    return s;
  }
}

template <int MODE, int D>
struct PBuf {
  using Gp = PGeo<MODE, D>;
  u32x4_t k[kPKeys][Gp::KROW / 16];    // int8 codes, k-slot order
  u32x4_t vt[D + 16][Gp::VROW / 16];   // bf16 c, [d][position slot]; rows D..D+3: see stage_store
  f32x4_t sk[kPKeys / 4];              // per position, four to a vector
  f32x4_t zk[kPKeys / 4];
  f32x4_t sv[kPKeys / 4];
  i32x4_t ok[kPKeys / 4];              // position present and within the tile range
};

template <int MODE, int D>
struct PSmem {
  union {
    float qf[kPRows][D + 4];         // prologue: R q; epilogue: rows before R^T
    PBuf<MODE, D> buf[2];
  };
  float rs[kPRows];                  // max |q' * scale * log2(e)| of each row
  float r1[kPRows];                  // sum over d of the row's 2^14 a + 2^7 b + c
};

// Registers a staging thread carries from the global loads to the LDS stores.
template <int MODE, int D>
struct Stage {
  using Gp = PGeo<MODE, D>;
  uint32_t k[Gp::KNW];
  uint32_t v[4][Gp::VNW];
  float sk, zk, sv, zv;
  int ok;
};

// Plane row of position j of the walked table row, or -1 when no row of the
// workgroup sees the position or it is absent: past khi, in the gap between
// the sinks and the earliest window start [sink, klo), in an evicted (-1)
// block, or in a block id at or past num_blocks.
struct KeyRange {
  int klo, khi, sink;   // positions the workgroup's rows may see: [0, sink) and [klo, khi]
};

__device__ __forceinline__ bool key_seen(const KeyRange& kr, int j) {
  return j <= kr.khi && (j >= kr.klo || j < kr.sink);
}

// INL: the row of the inline layout, ((id 2 bs + offset) Hkv + h), read
// from the K or the V base (consecutive positions are Hkv rows apart).
template <bool INL>
__device__ __forceinline__ int plane_row(const int32_t* trow, int j, const KeyRange& kr, int bs_log2, int hkv,
                                         int h, int nblk) {
  int id = -1;
  if (key_seen(kr, j)) id = trow[j >> bs_log2];
  if (id < 0 || id >= nblk) return -1;
  const int pin = j & ((1 << bs_log2) - 1);
  return INL ? ((id << (bs_log2 + 1)) + pin) * hkv + h : ((id * hkv + h) << bs_log2) + pin;
}

// Global loads of key tile `tau` into registers.  Thread t stages K codes of
// position t / 4, d-chunk t % 4 (and the meta of the position when t % 4 ==
// 0) and V codes of positions 4 (t % 16) .. +3, d = DPT (t / 16) .. +DPT-1.
// An absent position is not read: its codes stage as zeros and `ok` masks it
// (score -inf, weight 0).
template <int MODE, int D>
__device__ __forceinline__ void stage_load(Stage<MODE, D>& st, const PrefillParams& p, const int32_t* trow,
                                           int tau, const KeyRange& kr, int h, int tid) {
  using Gp = PGeo<MODE, D>;
  const int n = tid >> 2, qd = tid & 3;
  const int nblk = (int)p.num_blocks;   // < 2^31 (checked on the host)
  constexpr bool INL = MODE == kInlineMode;
  constexpr int RS = INL ? inline_row_bytes(D) : Gp::P;   // bytes between rows
  const int row = plane_row<INL>(trow, tau * kPKeys + n, kr, p.block_size_log2, p.hkv, h, nblk);
  st.ok = row >= 0;
#pragma unroll
  for (int i = 0; i < Gp::KNW; ++i) st.k[i] = 0u;
  st.sk = 0.0f; st.zk = 0.0f; st.sv = 0.0f; st.zv = 0.0f;
  if (row >= 0) {
    if constexpr (INL) {
      // 4-byte aligned rows; the stored scale st at byte P, zero point = its
      // low 4 bits (z = -zp st)
      const uint8_t* kr8 = p.k_codes + (int64_t)row * RS;
      load_bytes_a4<Gp::KNW * 4>(st.k, kr8 + qd * (Gp::KNW * 4));
      if (qd == 0) {
        const uint32_t kb = *reinterpret_cast<const uint32_t*>(kr8 + Gp::P);
        const uint32_t vb = *reinterpret_cast<const uint32_t*>(p.v_codes + (int64_t)row * RS + Gp::P);
        st.sk = __uint_as_float(kb);
        st.zk = -(float)(kb & 0xFu) * st.sk;
        st.sv = __uint_as_float(vb);
        st.zv = -(float)(vb & 0xFu) * st.sv;
      }
    } else {
      load_bytes<Gp::KNW * 4>(st.k, p.k_codes + (int64_t)row * Gp::P + qd * (Gp::KNW * 4));
    }
    if (qd == 0 && !INL) {
      if constexpr (Gp::M == 0) {   // per-channel INT8: scales live in the query and the output
        st.sk = 1.0f;
        st.sv = 1.0f;
      } else {
        st.sk = p.k_meta[(int64_t)row * Gp::M];
        st.zk = Gp::M == 2 ? p.k_meta[(int64_t)row * Gp::M + 1] : 0.0f;
        st.sv = p.v_meta[(int64_t)row * Gp::M];
        st.zv = Gp::M == 2 ? p.v_meta[(int64_t)row * Gp::M + 1] : 0.0f;
      }
    }
  }
  // V: positions 4 kq .. 4 kq + 3 (one block: block sizes are >= 16),
  // d = DPT wd .. DPT wd + DPT - 1, with kq = t % 16 so that the 16 lanes of
  // a group write one whole V^T row in LDS (no bank conflicts).
  const int kq = tid & 15, wd = tid >> 4;
  const int j0 = tau * kPKeys + 4 * kq;
  // the four positions share a block (block sizes are >= 16)
  const KeyRange all = {0, kr.khi, 0};
  const int vrow0 = plane_row<INL>(trow, j0, all, p.block_size_log2, p.hkv, h, nblk);
  const int vstep = INL ? p.hkv : 1;   // rows between consecutive positions
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int w = 0; w < Gp::VNW; ++w) st.v[i][w] = 0u;
    if (vrow0 >= 0 && key_seen(kr, j0 + i))
      load_bytes<Gp::VNB>(st.v[i], p.v_codes + (int64_t)(vrow0 + i * vstep) * RS + wd * Gp::VNB);
  }
}

// Unpack the staged registers into LDS buffer `b`.
template <int MODE, int D>
__device__ __forceinline__ void stage_store(const Stage<MODE, D>& st, PBuf<MODE, D>& b, int tid) {
  using Gp = PGeo<MODE, D>;
  const int n = tid >> 2, qd = tid & 3;
  // K: int8 codes, k-slot order
  uint32_t kc[Gp::DC / 4];
  if constexpr (code_mode(MODE) == 1) {
#pragma unroll
    for (int i = 0; i < Gp::KNW; ++i) {
      kc[i] = st.k[i] & 0x0F0F0F0Fu;
      kc[Gp::KNW + i] = (st.k[i] >> 4) & 0x0F0F0F0Fu;
    }
  } else if constexpr (MODE == 2) {
#pragma unroll
    for (int pl = 0; pl < 4; ++pl)
#pragma unroll
      for (int i = 0; i < Gp::KNW; ++i) kc[pl * Gp::KNW + i] = (st.k[i] >> (2 * pl)) & 0x03030303u;
  } else {
#pragma unroll
    for (int i = 0; i < Gp::KNW; ++i) kc[i] = st.k[i];
  }
#pragma unroll
  for (int i = 0; i < Gp::DC / 16; ++i)
    b.k[n][qd * (Gp::DC / 16) + i] = u32x4_t{kc[4 * i], kc[4 * i + 1], kc[4 * i + 2], kc[4 * i + 3]};
  if (qd == 0) {
    // The PV product also yields the row sums l = sum p and Z = sum p z_V
    // through four extra V^T rows holding 1/s_V and z_V/s_V as bf16 hi + lo
    // (W = p s_V).  s_V enters both as max(s_V, 2^-96): below that, the lo
    // half of W would fall under bf16's subnormal range and W / s_V would
    // carry up to 2^-8 of error into l.  A row with a zero or subnormal scale
    // has all-zero codes, so any s_V reconstructs it; a row with a scale in
    // [2^-126, 2^-96) has entries below 127 * 2^-96, and the clamp moves its
    // share of the output by less than 2^-89 p.
    const float sv = fmaxf(st.sv, 0x1p-96f);
    const float u = st.ok ? __builtin_amdgcn_rcpf(sv) : 0.0f;
    const float t = st.ok ? st.zv * u : 0.0f;
    const __bf16 uh = (__bf16)u, th = (__bf16)t;
    const __bf16 ul = (__bf16)(u - (float)uh), tl = (__bf16)(t - (float)th);
    const int kq7 = (n >> 2) & 7;
    const int nslot = 32 * (n >> 5) + 8 * (kq7 & 3) + 4 * (kq7 >> 2) + (n & 3);
    reinterpret_cast<__bf16*>(&b.vt[D + 0][0])[nslot] = uh;
    reinterpret_cast<__bf16*>(&b.vt[D + 1][0])[nslot] = ul;
    reinterpret_cast<__bf16*>(&b.vt[D + 2][0])[nslot] = th;
    reinterpret_cast<__bf16*>(&b.vt[D + 3][0])[nslot] = tl;
    b.sk[n >> 2][n & 3] = st.ok ? st.sk : 0.0f;
    b.zk[n >> 2][n & 3] = st.ok ? st.zk : 0.0f;
    b.sv[n >> 2][n & 3] = st.ok ? sv : 0.0f;
    b.ok[n >> 2][n & 3] = st.ok;
  }
  // V: positions 4 kq .. 4 kq + 3 -> slots of the PV operand order, as exact
  // bf16 integers c (no offset: the accumulator then holds only the signal,
  // whose fp32 rounding does not grow with an offset over long contexts)
  const int kq = tid & 15, wd = tid >> 4;
  const int kq7 = kq & 7;
  const int slot = 32 * (kq >> 3) + 8 * (kq7 & 3) + 4 * (kq7 >> 2);
  // codes into bytes, then one v_cvt_f32_ubyte per code: byte b of plane
  // word pw[pl][w] holds the code of d = DPT*wd + e with (INT8) e = 4 w + b,
  // (INT4) e = 8 w + 2 b + pl, (INT2) e = 16 w + 4 b + pl
  constexpr int BITS = mode_bits(MODE);
  constexpr int NPL = 8 / BITS;                       // code planes per byte
  constexpr int NW = (Gp::DPT * BITS + 31) / 32;      // dwords per position
  float c[4][Gp::DPT];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int w = 0; w < NW; ++w)
#pragma unroll
      for (int pl = 0; pl < NPL; ++pl) {
        const uint32_t x = BITS == 8 ? (st.v[i][w] ^ 0x80808080u)
                                     : ((st.v[i][w] >> (BITS * pl)) &
                                        (code_mode(MODE) == 1 ? 0x0F0F0F0Fu : 0x03030303u));
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
          const int e = (32 / BITS) * w + NPL * bb + pl;
          if (e < Gp::DPT) c[i][e] = BITS == 8 ? (float)((x >> (8 * bb)) & 0xffu) - 128.0f
                                               : (float)((x >> (8 * bb)) & 0xffu);
        }
      }
#pragma unroll
  for (int e = 0; e < Gp::DPT; ++e)
    reinterpret_cast<uint2*>(&b.vt[Gp::DPT * wd + e][0])[slot >> 2] =
        make_uint2(pack_exact(c[0][e], c[1][e]), pack_exact(c[2][e], c[3][e]));
}

template <int MODE, int D>
struct WaveCtx {
  using Gp = PGeo<MODE, D>;
  u32x4_t qa[2][Gp::KS], qb[2][Gp::KS], qc[2][Gp::KS];   // query pieces, B-operand layout
  f32x4_t o[2][Gp::DB + 1];               // output accumulators (C layout); block DB: l, Z
  float m[2];                             // reference max (log2 units)
  float sp[2], qp[2];                     // logit = sp * (s_K raw + z_K qp), raw = 2^14 A + 2^7 B + C
  int rpos[2], rlo[2];                    // row position and window start
  int W, wpos_lo, wpos_hi;
  int sink;                               // windowed head: positions < sink are seen too (else 0)
  bool wave_live;
  int lane, r, q;
};

// One key tile: global loads of the next tile, this tile's compute from
// buffer PAR, the next tile's LDS stores into the other buffer, barrier.
template <int MODE, int D, int PAR>
__device__ __forceinline__ void tile_step(PSmem<MODE, D>& sm, WaveCtx<MODE, D>& wc, Stage<MODE, D>& stg,
                                          const PrefillParams& p, const int32_t* trow, int tau, int tau_next,
                                          const KeyRange& kr, int h, int tid) {
  using Gp = PGeo<MODE, D>;
  const PBuf<MODE, D>& cb = sm.buf[PAR];
  const bool more = tau_next >= 0;
  if (more) stage_load<MODE, D>(stg, p, trow, tau_next, kr, h, tid);
  const int W = wc.W, r = wc.r, q = wc.q;
    const int pos0 = tau * kPKeys;
    const bool active = wc.wave_live && pos0 <= wc.wpos_hi &&
                        (W <= 0 || pos0 + kPKeys - 1 >= wc.wpos_lo - W + 1 || pos0 < wc.sink);
    if (active) {
      const bool all_ok = __all(cb.ok[wc.lane >> 2][wc.lane & 3] != 0);
      const bool full = all_ok && pos0 + kPKeys - 1 <= wc.wpos_lo &&
                        (W <= 0 || pos0 >= wc.wpos_hi - W + 1 || pos0 + kPKeys <= wc.sink);
      // ---- S^T = K Q^T, three int32 accumulators (pieces a, b and c)
      float x[4][2][4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        i32x4_t ia[2] = {{0, 0, 0, 0}, {0, 0, 0, 0}}, ib[2] = {{0, 0, 0, 0}, {0, 0, 0, 0}};
        i32x4_t ic[2] = {{0, 0, 0, 0}, {0, 0, 0, 0}};
#pragma unroll
        for (int ks = 0; ks < Gp::KS; ++ks) {
          const u32x4_t a = cb.k[16 * kb + r][4 * ks + q];
#pragma unroll
          for (int rb = 0; rb < 2; ++rb) {
            ia[rb] = mfma_i8(a, wc.qa[rb][ks], ia[rb]);
            ib[rb] = mfma_i8(a, wc.qb[rb][ks], ib[rb]);
            ic[rb] = mfma_i8(a, wc.qc[rb][ks], ic[rb]);
          }
        }
        const f32x4_t skv = cb.sk[4 * kb + q];
        const f32x4_t zkv = cb.zk[4 * kb + q];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            // 2^7 A + B is exact in int32 (|.| < 2^29); one rounding joins C
            const float raw = __builtin_fmaf((float)((ia[rb][i] << 7) + ib[rb][i]), 128.0f, (float)ic[rb][i]);
            x[kb][rb][i] = __builtin_fmaf(raw, skv[i], zkv[i] * wc.qp[rb]);
          }
      }
      if (__builtin_expect(!full, 0)) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          const i32x4_t okv = cb.ok[4 * kb + q];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int j = pos0 + 16 * kb + 4 * q + i;
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
              const bool keep = okv[i] != 0 && j <= wc.rpos[rb] && (j >= wc.rlo[rb] || j < wc.sink);
              x[kb][rb][i] = keep ? x[kb][rb][i] : kNegInf;
            }
          }
        }
      }
      // ---- row maxima (log2 units) and lazy rescale
      float tm[2];
      bool grow = false;
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        float mx = kNegInf;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) mx = fmaxf(mx, x[kb][rb][i]);
        mx = max_xor32(max_xor16(mx));
        tm[rb] = mx * wc.sp[rb];
        grow |= tm[rb] > wc.m[rb] + kRescale;
      }
      if (__any(grow)) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          const float mn = fmaxf(wc.m[rb], tm[rb]);
          const float alpha = mn == kNegInf ? 1.0f : __builtin_amdgcn_exp2f(wc.m[rb] - mn);
          wc.m[rb] = mn;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float ai = __shfl(alpha, 4 * q + i);
#pragma unroll
            for (int db = 0; db <= Gp::DB; ++db) wc.o[rb][db][i] *= ai;
          }
        }
      }
      // ---- p = 2^(logit - m), W = p s_V as bf16 hi + lo in PV A-operand
      // order (slab s = positions 32 s .. 32 s + 31)
      u32x4_t wh[2][2], wl[2][2];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const float mu = wc.m[rb] == kNegInf ? 0.0f : wc.m[rb];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          const f32x4_t svv = cb.sv[4 * kb + q];
          float wv[4];
#pragma unroll
          for (int i = 0; i < 4; ++i)
            wv[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[kb][rb][i], wc.sp[rb], -mu)) * svv[i];
          // hi = w with the low 16 bits cleared (exact bf16), lo = w - hi
          // (exact in fp32) rounded to bf16: together 16 significant bits
          float th[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) th[i] = __uint_as_float(__float_as_uint(wv[i]) & 0xffff0000u);
          const int s = kb >> 1, hf = 2 * (kb & 1);
          wh[s][rb][hf] = __builtin_amdgcn_perm(__float_as_uint(th[1]), __float_as_uint(th[0]), 0x07060302u);
          wh[s][rb][hf + 1] = __builtin_amdgcn_perm(__float_as_uint(th[3]), __float_as_uint(th[2]), 0x07060302u);
          wl[s][rb][hf] = pack_bf16(wv[0] - th[0], wv[1] - th[1]);
          wl[s][rb][hf + 1] = pack_bf16(wv[2] - th[2], wv[3] - th[3]);
        }
      }
      // ---- O += W V, V operands read one d-block ahead of their MFMAs
      u32x4_t b0 = cb.vt[r][q], b1 = cb.vt[r][4 + q];
#pragma unroll
      for (int db = 0; db <= Gp::DB; ++db) {
        u32x4_t n0 = b0, n1 = b1;
        if (db < Gp::DB) {
          n0 = cb.vt[16 * (db + 1) + r][q];
          n1 = cb.vt[16 * (db + 1) + r][4 + q];
        }
        // keep the next operands' reads ahead of this block's MFMAs (the
        // scheduler otherwise sinks them next to their use and exposes the
        // LDS latency)
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          wc.o[rb][db] = mfma(wh[0][rb], b0, wc.o[rb][db]);
          wc.o[rb][db] = mfma(wl[0][rb], b0, wc.o[rb][db]);
          wc.o[rb][db] = mfma(wh[1][rb], b1, wc.o[rb][db]);
          wc.o[rb][db] = mfma(wl[1][rb], b1, wc.o[rb][db]);
        }
        b0 = n0;
        b1 = n1;
      }
    }
  if (more) stage_store<MODE, D>(stg, sm.buf[PAR ^ 1], tid);
  __syncthreads();
}

template <int MODE, int D>
constexpr int prefill_waves_per_simd() { return 2; }

template <int MODE, int D, bool ROT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(prefill_waves_per_simd<MODE, D>())))
void prefill_kernel(PrefillParams p) {
  using Gp = PGeo<MODE, D>;
  __shared__ PSmem<MODE, D> sm;

  // ---- work item: consecutive items (the query tiles of one (sequence, kv
  // head)) land on one XCD, whose L2 then serves their shared key tiles
  const int nb = gridDim.x;                       // a multiple of 8
  const int bid = blockIdx.x;
  const int w_item = (bid & 7) * (nb >> 3) + (bid >> 3);
  if (w_item >= p.n_work) return;
  const int qt = w_item % p.n_qtiles;
  const int hb = w_item / p.n_qtiles;
  const int h = hb % p.hkv;
  const int b = hb / p.hkv;

  const int q0 = p.cu_q[b];
  const int nq = p.cu_q[b + 1] - q0;
  const int G = p.group;
  const int tq = p.tq;
  const int tok0 = qt * tq;
  if (tok0 >= nq) return;
  const int ntok = min(tq, nq - tok0);
  const int nrows = ntok * G;
  const int L = min(p.seq_lens[b], p.max_seq_len);   // host checked max_seq_len <= max_blocks * bs
  const int W = p.window ? p.window[h] : 0;
  const int pbase = L - nq + tok0;                // position of the tile's first token
  const int khi = pbase + ntok - 1;               // last position any row may see
  const int klo = W > 0 ? max(0, pbase - W + 1) : 0;
  // sinks: a windowed head also sees positions < sink; the key tiles walked
  // are those of [0, sink) then those of [klo, khi] (a tile in both counts once)
  const int sinkE = (W > 0 && klo > 0) ? min(p.sink, klo) : 0;
  const int ns_tiles = (sinkE + kPKeys - 1) / kPKeys;       // tiles 0 .. ns_tiles - 1
  const int tau0 = max(klo / kPKeys, ns_tiles);
  const int tau1 = khi >= 0 ? khi / kPKeys : -1;  // inclusive; none when khi < 0
  const int32_t* trow = p.tables + (int64_t)(p.headwise ? b * p.hkv + h : b) * p.max_blocks;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int r = lane & 15;
  const int q = lane >> 4;

  // ---- first key tile's loads overlap the query prologue
  Stage<MODE, D> stg;
  const KeyRange kr = {klo, khi, sinkE};
  // the walk: k = 0 .. nwalk - 1 visits tile walk_tile(k)
  const int nwin = tau1 >= tau0 ? tau1 - tau0 + 1 : 0;
  const int nwalk = (khi >= 0 ? min(ns_tiles, khi / kPKeys + 1) : 0) + nwin;
  const int nsw = nwalk - nwin;                               // sink tiles walked
  auto walk_tile = [&](int k) { return k < nsw ? k : tau0 + (k - nsw); };
  if (nwalk > 0) stage_load<MODE, D>(stg, p, trow, walk_tile(0), kr, h, tid);

  // ---- query prologue: rows (token t, head g) -> R q
  for (int e = tid; e < kPRows * D; e += 64 * kPWaves) {
    const int row = e / D, d = e - row * D;
    float v = 0.0f;
    if (row < nrows) {
      const int t = row / G, g = row - t * G;
      v = __uint_as_float((uint32_t)p.q[((int64_t)(q0 + tok0 + t) * p.hq + h * G + g) * D + d] << 16);
      if constexpr (ROT) v *= p.signs[d];
      if constexpr (MODE == kChannelMode) v *= p.chs[(int64_t)h * D + d];   // q . (c (.) s_K)
    }
    sm.qf[row][d] = v;
  }
  __syncthreads();
  if constexpr (ROT) {
    for (int hh = 1; hh < D; hh <<= 1) {
      for (int e = tid; e < kPRows * (D / 2); e += 64 * kPWaves) {
        const int g = e / (D / 2), k = e - g * (D / 2);
        const int i = (k / hh) * 2 * hh + (k % hh);
        const float a = sm.qf[g][i], c = sm.qf[g][i + hh];
        sm.qf[g][i] = a + c;
        sm.qf[g][i + hh] = a - c;
      }
      __syncthreads();
    }
  }
  const float qmul = ROT ? p.qscale * p.inv_sqrt_d : p.qscale;
  // piece scale and represented sum per row (each wave its own 32 rows)
  for (int i = 0; i < 32; ++i) {
    const int row = 32 * wave + i;
    float mx = 0.0f;
    for (int d = lane; d < D; d += 64) mx = fmaxf(mx, fabsf(sm.qf[row][d] * qmul));
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) mx = fmaxf(mx, __shfl_xor(mx, m));
    const float invS = mx > 0.0f ? 127.0f / mx : 0.0f;
    float sq = 0.0f;
    for (int d = lane; d < D; d += 64) {
      const float t = fminf(fmaxf(sm.qf[row][d] * qmul * invS, -127.0f), 127.0f);
      const float a = __builtin_rintf(t);
      const float r1 = (t - a) * 128.0f;
      const float b = __builtin_rintf(r1);
      const float c = __builtin_rintf((r1 - b) * 128.0f);
      sq += __builtin_fmaf(16384.0f, a, __builtin_fmaf(128.0f, b, c));   // each term exact (< 2^22)
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) sq += __shfl_xor(sq, m);
    if (lane == 0) {
      sm.rs[row] = mx;
      sm.r1[row] = sq;
    }
  }
  __syncthreads();
  // B operands: lane (row r of block rb, k-slots 64 ks + 16 q .. +15)
  u32x4_t qa[2][Gp::KS], qb[2][Gp::KS], qc[2][Gp::KS];
  float sp[2], qp[2];
  int rpos[2], rlo[2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int row = 32 * wave + 16 * rb + r;
    const float mx = sm.rs[row];
    const float S = mx / 127.0f;
    const float invS = mx > 0.0f ? 127.0f / mx : 0.0f;   // as in the pass above
#pragma unroll
    for (int ks = 0; ks < Gp::KS; ++ks) {
      uint32_t wa[4], wb[4], wcc[4];
#pragma unroll
      for (int j4 = 0; j4 < 4; ++j4) {
        uint32_t pa = 0, pb = 0, pc = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int d = kslot_d<MODE, D>(64 * ks + 16 * q + 4 * j4 + j);
          const float t = fminf(fmaxf(sm.qf[row][d] * qmul * invS, -127.0f), 127.0f);
          const float a = __builtin_rintf(t);
          const float r1 = (t - a) * 128.0f;
          const float b = __builtin_rintf(r1);
          const float c = __builtin_rintf((r1 - b) * 128.0f);
          pa |= ((uint32_t)(int32_t)a & 0xffu) << (8 * j);
          pb |= ((uint32_t)(int32_t)b & 0xffu) << (8 * j);
          pc |= ((uint32_t)(int32_t)c & 0xffu) << (8 * j);
        }
        wa[j4] = pa;
        wb[j4] = pb;
        wcc[j4] = pc;
      }
      qa[rb][ks] = u32x4_t{wa[0], wa[1], wa[2], wa[3]};
      qb[rb][ks] = u32x4_t{wb[0], wb[1], wb[2], wb[3]};
      qc[rb][ks] = u32x4_t{wcc[0], wcc[1], wcc[2], wcc[3]};
    }
    // logit (log2 units) = sp * x, x = s_K raw + z_K qp, raw = 2^14 A + 2^7 B + C
    sp[rb] = S > 0.0f ? S * 6.103515625e-05f : 1.0f;   // S / 2^14
    qp[rb] = S > 0.0f ? sm.r1[row] : 0.0f;
    const bool live = row < nrows;
    rpos[rb] = live ? pbase + row / G : -1;
    rlo[rb] = W > 0 ? rpos[rb] - W + 1 : INT32_MIN;
  }
  // wave-uniform position range of the wave's live rows
  const int wrow0 = 32 * wave;
  const bool wave_live = wrow0 < nrows;
  const int wpos_lo = pbase + wrow0 / G;
  const int wpos_hi = pbase + (min(wrow0 + 31, nrows - 1)) / G;
  __syncthreads();   // qf is dead; the buffers may be written
  // extra V^T rows D+4 .. D+15 feed unused output columns: keep them zero
  for (int e = tid; e < 2 * 12 * (Gp::VROW / 16); e += 64 * kPWaves) {
    const int bsel = e / (12 * (Gp::VROW / 16)), rem = e - bsel * (12 * (Gp::VROW / 16));
    sm.buf[bsel].vt[D + 4 + rem / (Gp::VROW / 16)][rem % (Gp::VROW / 16)] = u32x4_t{0u, 0u, 0u, 0u};
  }

  if (nwalk > 0) stage_store<MODE, D>(stg, sm.buf[0], tid);
  __syncthreads();

  WaveCtx<MODE, D> wc{};
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    wc.m[rb] = kNegInf;
    wc.sp[rb] = sp[rb]; wc.qp[rb] = qp[rb]; wc.rpos[rb] = rpos[rb]; wc.rlo[rb] = rlo[rb];
#pragma unroll
    for (int ks = 0; ks < Gp::KS; ++ks) {
      wc.qa[rb][ks] = qa[rb][ks]; wc.qb[rb][ks] = qb[rb][ks]; wc.qc[rb][ks] = qc[rb][ks];
    }
#pragma unroll
    for (int db = 0; db <= Gp::DB; ++db) wc.o[rb][db] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  }
  // the rows' masks take the whole sink range: a later row's window starts
  // after klo, so positions in [min(sink, klo), sink) are sinks for it
  wc.W = W; wc.wave_live = wave_live; wc.wpos_lo = wpos_lo; wc.wpos_hi = wpos_hi; wc.sink = W > 0 ? p.sink : 0;
  wc.lane = lane; wc.r = r; wc.q = q;

  // two tiles per iteration so that each buffer's LDS offsets are constants
  for (int k = 0; k < nwalk; k += 2) {
    tile_step<MODE, D, 0>(sm, wc, stg, p, trow, walk_tile(k), k + 1 < nwalk ? walk_tile(k + 1) : -1, kr, h, tid);
    if (k + 1 >= nwalk) break;
    tile_step<MODE, D, 1>(sm, wc, stg, p, trow, walk_tile(k + 1), k + 2 < nwalk ? walk_tile(k + 2) : -1, kr, h,
                          tid);
  }

  // ---- epilogue: normalize into LDS rows, R^T, store
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // l and Z of row 4 q + i: columns 0 + 1 and 2 + 3 of the extra block
      const float li = __shfl(wc.o[rb][Gp::DB][i], 16 * q) + __shfl(wc.o[rb][Gp::DB][i], 16 * q + 1);
      const float zi = __shfl(wc.o[rb][Gp::DB][i], 16 * q + 2) + __shfl(wc.o[rb][Gp::DB][i], 16 * q + 3);
      const float inv = li > 0.0f ? 1.0f / li : 0.0f;
      const int row = 32 * wave + 16 * rb + 4 * q + i;
#pragma unroll
      for (int db = 0; db < Gp::DB; ++db) sm.qf[row][16 * db + r] = (wc.o[rb][db][i] + zi) * inv;
    }
  }
  __syncthreads();
  if constexpr (ROT) {
    for (int hh = 1; hh < D; hh <<= 1) {
      for (int e = tid; e < nrows * (D / 2); e += 64 * kPWaves) {
        const int g = e / (D / 2), k = e - g * (D / 2);
        const int i = (k / hh) * 2 * hh + (k % hh);
        const float a = sm.qf[g][i], c = sm.qf[g][i + hh];
        sm.qf[g][i] = a + c;
        sm.qf[g][i + hh] = a - c;
      }
      __syncthreads();
    }
  }
  for (int e = tid; e < nrows * D; e += 64 * kPWaves) {
    const int row = e / D, d = e - row * D;
    const int t = row / G, g = row - t * G;
    float v = sm.qf[row][d];
    if constexpr (ROT) v = v * p.signs[d] * p.inv_sqrt_d;
    if constexpr (MODE == kChannelMode) v *= p.chs[((int64_t)p.hkv + h) * D + d];   // (sum_j p_j c_j) (.) s_V
    const int64_t o_idx = ((int64_t)(q0 + tok0 + t) * p.hq + h * G + g) * D + d;
    if (p.out_bf16)
      reinterpret_cast<__bf16*>(p.out)[o_idx] = (__bf16)v;
    else
      reinterpret_cast<float*>(p.out)[o_idx] = v;
  }
}

template <int MODE, int D, bool ROT>
hipError_t launch_prefill_t(const PrefillParams& p, hipStream_t s) {
  const int grid = (p.n_work + 7) / 8 * 8;
  hipLaunchKernelGGL((prefill_kernel<MODE, D, ROT>), dim3(grid), dim3(64 * kPWaves), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(int mode, int d, bool rot, const PrefillParams& p, hipStream_t s) {
#define KVQ_PREFILL_CASE(M_, D_)                                                           \
  if (mode == M_ && d == D_) return rot ? launch_prefill_t<M_, D_, true>(p, s)           \
                                        : launch_prefill_t<M_, D_, false>(p, s);
  KVQ_PREFILL_CASE(0, 64)
  KVQ_PREFILL_CASE(0, 128)
  KVQ_PREFILL_CASE(1, 64)
  KVQ_PREFILL_CASE(1, 128)
  KVQ_PREFILL_CASE(2, 64)
  KVQ_PREFILL_CASE(2, 128)
  KVQ_PREFILL_CASE(kInlineMode, 64)
  KVQ_PREFILL_CASE(kInlineMode, 128)
#undef KVQ_PREFILL_CASE
  // per-channel INT8 has no rotation (checked on the host)
  if (mode == kChannelMode && d == 64) return launch_prefill_t<kChannelMode, 64, false>(p, s);
  if (mode == kChannelMode && d == 128) return launch_prefill_t<kChannelMode, 128, false>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace kvq
