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
  u32x4_t vt[D + 16][Gp::VROW / 16];   // bf16 c, [d][position slot]; rows D..D+3: see stage_part
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
  int kid, vid;   // block ids of the tile staged next (K position, V positions), read a tile ahead
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

// Plane row of position j in block `id` (-1: evicted, or at or past
// num_blocks: no row).  INL: the row of the inline layout,
// ((id 2 bs + offset) Hkv + h), read from the K or the V base (consecutive
// positions are Hkv rows apart).
template <bool INL>
__device__ __forceinline__ int plane_row(int id, int j, int bs_log2, int hkv, int h, int nblk) {
  if (id < 0 || id >= nblk) return -1;
  const int pin = j & ((1 << bs_log2) - 1);
  return INL ? ((id << (bs_log2 + 1)) + pin) * hkv + h : ((id * hkv + h) << bs_log2) + pin;
}

// Block ids of key tile `tau` for this thread's K position t / 4 and V
// positions 4 (t % 16) .. +3 (one block: block sizes are >= 16).  They are
// read one tile ahead, so the code loads of a tile never wait on the table.
template <int MODE, int D>
__device__ __forceinline__ void stage_ids(Stage<MODE, D>& st, const int32_t* trow, int tau, const KeyRange& kr,
                                          int bs_log2, int tid) {
  // entries at positions clamped to khi (< L, inside the table row) are read
  // with no branch around the loads; stage_load discards those of positions
  // no row sees (testing them here would wait for the loads at once)
  const int j = tau * kPKeys + (tid >> 2), j0 = tau * kPKeys + 4 * (tid & 15);
  st.kid = trow[min(j, kr.khi) >> bs_log2];
  st.vid = trow[min(j0, kr.khi) >> bs_log2];
}

// Global loads of key tile `tau` into registers, from the block ids
// stage_ids read.  Thread t stages K codes of position t / 4, d-chunk t % 4,
// the meta of that position and V codes of positions 4 (t % 16) .. +3,
// d = DPT (t / 16) .. +DPT-1.  Nothing of an absent block (-1, or an id at
// or past num_blocks) is read, nor a K position that no row sees: their
// codes stage as zeros and `ok` masks them (score -inf, weight 0).
template <int MODE, int D>
__device__ __forceinline__ void stage_load(Stage<MODE, D>& st, const PrefillParams& p, int tau, const KeyRange& kr,
                                           int h, int tid) {
  using Gp = PGeo<MODE, D>;
  const int n = tid >> 2, qd = tid & 3;
  const int nblk = (int)p.num_blocks;   // < 2^31 (checked on the host)
  constexpr bool INL = MODE == kInlineMode;
  constexpr int RS = INL ? inline_row_bytes(D) : Gp::P;   // bytes between rows
  const int jk = tau * kPKeys + n;
  const int row = plane_row<INL>(key_seen(kr, jk) ? st.kid : -1, jk, p.block_size_log2, p.hkv, h, nblk);
  st.ok = row >= 0;
#pragma unroll
  for (int i = 0; i < Gp::KNW; ++i) st.k[i] = 0u;
  st.sk = 0.0f; st.zk = 0.0f; st.sv = 0.0f; st.zv = 0.0f;
  if (row >= 0) {
    // the four lanes of a position all read its meta (one request per
    // address): each stores one field of it, with no branch in the store
    if constexpr (INL) {
      // 4-byte aligned rows; the stored scale st at byte P, zero point = its
      // low 4 bits (z = -zp st)
      const uint8_t* kr8 = p.k_codes + (int64_t)row * RS;
      load_bytes_a4<Gp::KNW * 4>(st.k, kr8 + qd * (Gp::KNW * 4));
      const uint32_t kb = *reinterpret_cast<const uint32_t*>(kr8 + Gp::P);
      const uint32_t vb = *reinterpret_cast<const uint32_t*>(p.v_codes + (int64_t)row * RS + Gp::P);
      st.sk = __uint_as_float(kb);
      st.zk = -(float)(kb & 0xFu) * st.sk;
      st.sv = __uint_as_float(vb);
      st.zv = -(float)(vb & 0xFu) * st.sv;
    } else {
      load_bytes<Gp::KNW * 4>(st.k, p.k_codes + (int64_t)row * Gp::P + qd * (Gp::KNW * 4));
    }
    if constexpr (!INL) {
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
  // All four are read when the block is present: a position outside the
  // rows' range has zero weight (p = 0 and s_V = 0 staged), and integer
  // codes are finite, so its codes add exactly nothing.
  const int vrow0 = plane_row<INL>(j0 <= kr.khi ? st.vid : -1, j0, p.block_size_log2, p.hkv, h, nblk);
  const int64_t vstep = INL ? (int64_t)p.hkv * RS : RS;   // bytes between consecutive positions
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int w = 0; w < Gp::VNW; ++w) st.v[i][w] = 0u;
  if (vrow0 >= 0) {
    const uint8_t* vb = p.v_codes + (int64_t)vrow0 * RS + wd * Gp::VNB;
#pragma unroll
    for (int i = 0; i < 4; ++i) load_bytes<Gp::VNB>(st.v[i], vb + i * vstep);
  }
}

// Unpacking the staged registers into LDS buffer `b` goes in parts that the
// tile loop spreads between the MFMAs of the PV product (part 0: K codes,
// parts 1 .. DPT: V^T columns, part DPT + 1: the per-position meta); none
// branches.  Parts 1 .. DPT read the V codes through `vp`: INT4 keeps its
// two nibble planes there, formed in part 0.
template <int MODE, int D>
struct VPlanes {
  uint32_t x[4][2];
};

// V code of position 4 kq + i, d = DPT wd + e, as a float (exact).
template <int MODE, int D>
__device__ __forceinline__ float v_code(const Stage<MODE, D>& st, const VPlanes<MODE, D>& vp, int i, int e) {
  if constexpr (code_mode(MODE) == 1) {   // byte b of plane pl: d = 2 b + pl
    return (float)((vp.x[i][e & 1] >> (8 * (e >> 1))) & 0xffu);
  } else if constexpr (MODE == 2) {       // byte b, crumb pl: d = 4 b + pl
    return (float)((st.v[i][0] >> (8 * (e >> 2) + 2 * (e & 3))) & 3u);
  } else {                                // INT8: byte e % 4 of word e / 4, signed
    return (float)(int8_t)(st.v[i][e >> 2] >> (8 * (e & 3)));
  }
}

template <int MODE, int D>
__device__ __forceinline__ void stage_part(const Stage<MODE, D>& st, VPlanes<MODE, D>& vp, PBuf<MODE, D>& b,
                                           int tid, int part) {
  using Gp = PGeo<MODE, D>;
  const int n = tid >> 2, qd = tid & 3;
  if (part == 0) {
    // K: int8 codes, k-slot order
    uint32_t kc[Gp::DC / 4];
    if constexpr (code_mode(MODE) == 1) {
#pragma unroll
      for (int i = 0; i < Gp::KNW; ++i) {
        kc[i] = st.k[i] & 0x0F0F0F0Fu;
        kc[Gp::KNW + i] = (st.k[i] >> 4) & 0x0F0F0F0Fu;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        vp.x[i][0] = st.v[i][0] & 0x0F0F0F0Fu;
        vp.x[i][1] = (st.v[i][0] >> 4) & 0x0F0F0F0Fu;
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
  } else if (part <= Gp::DPT) {
    // V: positions 4 kq .. 4 kq + 3 -> slots of the PV operand order, as
    // exact bf16 integers c (no offset: the accumulator then holds only the
    // signal, whose fp32 rounding does not grow with an offset over long
    // contexts)
    const int e = part - 1;
    const int kq = tid & 15, wd = tid >> 4;
    const int kq7 = kq & 7;
    const int slot = 32 * (kq >> 3) + 8 * (kq7 & 3) + 4 * (kq7 >> 2);
    reinterpret_cast<uint2*>(&b.vt[Gp::DPT * wd + e][0])[slot >> 2] =
        make_uint2(pack_exact(v_code(st, vp, 0, e), v_code(st, vp, 1, e)),
                   pack_exact(v_code(st, vp, 2, e), v_code(st, vp, 3, e)));
  } else {
    // The PV product also yields the row sums l = sum p and Z = sum p z_V
    // through four extra V^T rows holding 1/s_V and z_V/s_V as bf16 hi + lo
    // (W = p s_V); lane qd of a position writes row D + qd and one of its
    // s_K, z_K, s_V, present flags.  s_V enters both as max(s_V, 2^-96):
    // below that, the lo half of W would fall under bf16's subnormal range
    // and W / s_V would carry up to 2^-8 of error into l.  A row with a zero
    // or subnormal scale has all-zero codes, so any s_V reconstructs it; a
    // row with a scale in [2^-126, 2^-96) has entries below 127 * 2^-96, and
    // the clamp moves its share of the output by less than 2^-89 p.
    const float sv = fmaxf(st.sv, 0x1p-96f);
    const float u = st.ok ? __builtin_amdgcn_rcpf(sv) : 0.0f;
    const float t = st.ok ? st.zv * u : 0.0f;
    const float val = qd < 2 ? u : t;
    const __bf16 hi = (__bf16)val;
    const __bf16 lo = (__bf16)(val - (float)hi);
    const int kq7 = (n >> 2) & 7;
    const int nslot = 32 * (n >> 5) + 8 * (kq7 & 3) + 4 * (kq7 >> 2) + (n & 3);
    reinterpret_cast<__bf16*>(&b.vt[D + qd][0])[nslot] = (qd & 1) ? lo : hi;
    // sk, zk, sv and ok are consecutive arrays of kPKeys words
    using PB = PBuf<MODE, D>;
    static_assert(offsetof(PB, zk) == offsetof(PB, sk) + 4 * kPKeys &&
                      offsetof(PB, sv) == offsetof(PB, sk) + 8 * kPKeys &&
                      offsetof(PB, ok) == offsetof(PB, sk) + 12 * kPKeys,
                  "per-position meta arrays must be consecutive");
    const float f = qd == 0 ? st.sk : qd == 1 ? st.zk : sv;
    reinterpret_cast<uint32_t*>(&b.sk[0])[qd * kPKeys + n] =
        qd == 3 ? (uint32_t)st.ok : (st.ok ? __float_as_uint(f) : 0u);
  }
}

template <int MODE, int D>
__device__ __forceinline__ void stage_store(const Stage<MODE, D>& st, PBuf<MODE, D>& b, int tid) {
  VPlanes<MODE, D> vp;
#pragma unroll
  for (int part = 0; part <= PGeo<MODE, D>::DPT + 1; ++part) stage_part<MODE, D>(st, vp, b, tid, part);
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
                                          int tau_next2, const KeyRange& kr, int h, int tid) {
  using Gp = PGeo<MODE, D>;
  const PBuf<MODE, D>& cb = sm.buf[PAR];
  const bool more = tau_next >= 0;
  // the ids of tile tau_next2 are read only on the path that has consumed
  // the previous ids (a write on a path that had not would make the compiler
  // wait for every load in flight, this tile's codes included)
  if (more) {
    stage_load<MODE, D>(stg, p, tau_next, kr, h, tid);
    if (tau_next2 >= 0) stage_ids<MODE, D>(stg, trow, tau_next2, kr, p.block_size_log2, tid);
  }
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
      // order (slab s = positions 32 s .. 32 s + 31), and O += W V.  The
      // MFMAs of slab 0 run while slab 1's weights are formed, and those of
      // slab 1 while the next tile is unpacked into LDS: the source order
      // below, fenced per d-block, is the issue order.  Every accumulator
      // still sums slab 0's hi, lo, then slab 1's hi, lo.
      float mu[2];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) mu[rb] = wc.m[rb] == kNegInf ? 0.0f : wc.m[rb];
      u32x4_t wh[2][2], wl[2][2];
      // weights of positions 16 kb + 4 q + 2 h2 + {0, 1}, rows of block rb:
      // hi = w with the low 16 bits cleared (exact bf16), lo = w - hi (exact
      // in fp32) rounded to bf16: together 16 significant bits
      auto wpair = [&](int kb, int rb, int h2) {
        const f32x4_t svv = cb.sv[4 * kb + q];
        const float w0 = __builtin_amdgcn_exp2f(__builtin_fmaf(x[kb][rb][2 * h2], wc.sp[rb], -mu[rb])) *
                         svv[2 * h2];
        const float w1 = __builtin_amdgcn_exp2f(__builtin_fmaf(x[kb][rb][2 * h2 + 1], wc.sp[rb], -mu[rb])) *
                         svv[2 * h2 + 1];
        const float t0 = __uint_as_float(__float_as_uint(w0) & 0xffff0000u);
        const float t1 = __uint_as_float(__float_as_uint(w1) & 0xffff0000u);
        const int s = kb >> 1, hf = 2 * (kb & 1) + h2;
        wh[s][rb][hf] = __builtin_amdgcn_perm(__float_as_uint(t1), __float_as_uint(t0), 0x07060302u);
        wl[s][rb][hf] = pack_bf16(w0 - t0, w1 - t1);
      };
#pragma unroll
      for (int k = 0; k < 8; ++k) wpair(k >> 2, (k >> 1) & 1, k & 1);
      constexpr int NST = Gp::DB + 1;   // d-blocks, one fenced step each
      VPlanes<MODE, D> vp;
      u32x4_t bv = cb.vt[r][q];
#pragma unroll
      for (int st2 = 0; st2 < 2 * NST; ++st2) {
        const int sl = st2 / NST, db = st2 % NST;
        // the operand of the next step, read one step ahead
        u32x4_t nb = bv;
        if (st2 + 1 < 2 * NST) {
          const int sl1 = (st2 + 1) / NST, db1 = (st2 + 1) % NST;
          nb = cb.vt[16 * db1 + r][4 * sl1 + q];
        }
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          wc.o[rb][db] = mfma(wh[sl][rb], bv, wc.o[rb][db]);
          wc.o[rb][db] = mfma(wl[sl][rb], bv, wc.o[rb][db]);
        }
        if (sl == 0) {
          // slab 1's eight weight pairs over the NST steps
#pragma unroll
          for (int k = db * 8 / NST; k < (db + 1) * 8 / NST; ++k) wpair(2 + (k >> 2), (k >> 1) & 1, k & 1);
        } else {
          // the next tile's LDS stores (stale data after the last tile, into
          // the buffer no wave reads before the barrier)
          stage_part<MODE, D>(stg, vp, sm.buf[PAR ^ 1], tid, db);
          if (db == NST - 1) stage_part<MODE, D>(stg, vp, sm.buf[PAR ^ 1], tid, Gp::DPT + 1);
        }
        __builtin_amdgcn_sched_barrier(0);
        bv = nb;
      }
    } else if (more) {
      stage_store<MODE, D>(stg, sm.buf[PAR ^ 1], tid);
    }
  __syncthreads();
}

template <int MODE, int D>
constexpr int prefill_waves_per_simd() { return 2; }

template <int MODE, int D, bool ROT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(prefill_waves_per_simd<MODE, D>())))
void prefill_kernel(PrefillParams p) {
  using Gp = PGeo<MODE, D>;
  __shared__ PSmem<MODE, D> sm;

  // ---- work item: (sequence, kv head) group and query tile.  The query
  // tiles of a group run on one XCD, whose L2 then serves their shared key
  // tiles; groups go to the XCDs round-robin, and on each XCD in group order
  // (workgroups reach the XCDs round-robin in blockIdx order, grid.x = 8
  // groups-per-XCD query-tile counts).  Groups are numbered heads without a
  // window first: their key walks are the long ones, so every XCD starts its
  // long items first and the short (windowed) ones fill in behind them.
  int b, h, qt;
  {
    const int nqt = p.n_qtiles;
    const int ng = p.n_work / nqt;                  // Hkv * num_seqs
    const int bid = blockIdx.x;
    const int k = bid >> 3;
    const int lg = k / nqt;
    qt = k - lg * nqt;
    const int g = lg * 8 + (bid & 7);
    if (g >= ng) return;
    const int hkv = p.hkv, nseq = ng / hkv;
    int nf = hkv;                                   // heads without a window
    if (p.window) {
      nf = 0;
      for (int i = 0; i < hkv; ++i) nf += p.window[i] <= 0 ? 1 : 0;
    }
    // group g: the j-th head of its class, sequence b
    const bool full = g < nf * nseq;
    const int nc = full ? nf : hkv - nf;
    const int gc = full ? g : g - nf * nseq;
    b = gc / nc;
    const int j = gc - b * nc;
    h = j;
    if (p.window) {
      int seen = 0;
      for (int i = 0; i < hkv; ++i) {
        if ((p.window[i] <= 0) == full) {
          if (seen == j) h = i;
          ++seen;
        }
      }
    }
  }

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
  if (nwalk > 0) {
    stage_ids<MODE, D>(stg, trow, walk_tile(0), kr, p.block_size_log2, tid);
    stage_load<MODE, D>(stg, p, walk_tile(0), kr, h, tid);
    if (nwalk > 1) stage_ids<MODE, D>(stg, trow, walk_tile(1), kr, p.block_size_log2, tid);
  }

  // ---- query prologue: each wave its 32 rows (token t, head g): one
  // lane-contiguous load per row, all in flight together, then in registers
  // q' = R q * qmul (Sylvester FWHT across the wave, stages h = 1 .. D/2 in
  // order), its maximum |q'| and the sum of its pieces; q' goes to LDS for
  // the B-operand gather below.  Lane l holds d = E l .. E l + E - 1.
  constexpr int E = D / 64;
  const float qmul = ROT ? p.qscale * p.inv_sqrt_d : p.qscale;
  float sg[E], chk[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    sg[e] = ROT ? p.signs[E * lane + e] : 1.0f;
    chk[e] = MODE == kChannelMode ? p.chs[(int64_t)h * D + E * lane + e] : 1.0f;   // q . (c (.) s_K)
  }
  {
    uint32_t raw[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const int row = 32 * wave + i;
      const int t = row / G, g = row - t * G;
      raw[i] = row < nrows ? load_qrow<D>(p.q + ((int64_t)(q0 + tok0 + t) * p.hq + h * G + g) * D, lane) : 0u;
    }
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const int row = 32 * wave + i;
      float x[E];
      x[0] = __uint_as_float(raw[i] << 16);
      if constexpr (E == 2) x[1] = __uint_as_float(raw[i] & 0xffff0000u);
      if constexpr (ROT) {
#pragma unroll
        for (int e = 0; e < E; ++e) x[e] *= sg[e];
        wave_fwht<D>(x, lane);
      }
      float mx = 0.0f;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        if constexpr (MODE == kChannelMode) x[e] *= chk[e];
        x[e] *= qmul;
        mx = fmaxf(mx, fabsf(x[e]));
        sm.qf[row][E * lane + e] = x[e];
      }
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) mx = fmaxf(mx, lane_xor(mx, m));
      const float invS = mx > 0.0f ? 127.0f / mx : 0.0f;
      float sq = 0.0f;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float tt = fminf(fmaxf(x[e] * invS, -127.0f), 127.0f);
        const float a = __builtin_rintf(tt);
        const float r1 = (tt - a) * 128.0f;
        const float b = __builtin_rintf(r1);
        const float c = __builtin_rintf((r1 - b) * 128.0f);
        sq += __builtin_fmaf(16384.0f, a, __builtin_fmaf(128.0f, b, c));   // each term exact (< 2^22)
      }
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) sq += lane_xor(sq, m);
      if (lane == 0) {
        sm.rs[row] = mx;
        sm.r1[row] = sq;
      }
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
          const float t = fminf(fmaxf(sm.qf[row][d] * invS, -127.0f), 127.0f);
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
  // wave-uniform position range of the wave's live rows (kept in scalar
  // registers, so the per-tile tests below are scalar branches)
  const int wrow0 = 32 * wave;
  const bool wave_live = wrow0 < nrows;
  const int wpos_lo = __builtin_amdgcn_readfirstlane(pbase + wrow0 / G);
  const int wpos_hi = __builtin_amdgcn_readfirstlane(pbase + (min(wrow0 + 31, nrows - 1)) / G);
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
  auto walk_or_none = [&](int k) { return k < nwalk ? walk_tile(k) : -1; };
  for (int k = 0; k < nwalk; k += 2) {
    tile_step<MODE, D, 0>(sm, wc, stg, p, trow, walk_tile(k), walk_or_none(k + 1), walk_or_none(k + 2), kr, h, tid);
    if (k + 1 >= nwalk) break;
    tile_step<MODE, D, 1>(sm, wc, stg, p, trow, walk_tile(k + 1), walk_or_none(k + 2), walk_or_none(k + 3), kr, h,
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
  // R^T (FWHT across the wave, signs, 1/sqrt(D)), the V channel scales for
  // per-channel INT8, and lane-contiguous stores: each wave its own rows.
  // The lane index is opaque here, so the prologue's sign loads are not kept
  // live across the tile loop.
  int el = lane;
  asm volatile("" : "+v"(el));
  float so[E], chv[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    so[e] = ROT ? p.signs[E * el + e] : 1.0f;
    chv[e] = MODE == kChannelMode ? p.chs[((int64_t)p.hkv + h) * D + E * el + e] : 1.0f;   // (sum_j p_j c_j) (.) s_V
  }
  for (int i = 0; i < 32; ++i) {
    const int row = 32 * wave + i;
    if (row >= nrows) break;
    float x[E];
#pragma unroll
    for (int e = 0; e < E; ++e) x[e] = sm.qf[row][E * el + e];
    if constexpr (ROT) {
      wave_fwht<D>(x, el);
#pragma unroll
      for (int e = 0; e < E; ++e) x[e] = x[e] * so[e] * p.inv_sqrt_d;
    }
    if constexpr (MODE == kChannelMode) {
#pragma unroll
      for (int e = 0; e < E; ++e) x[e] *= chv[e];
    }
    const int t = row / G, g = row - t * G;
    const int64_t o_idx = ((int64_t)(q0 + tok0 + t) * p.hq + h * G + g) * D + E * el;
    if (p.out_bf16) {
      if constexpr (E == 2) reinterpret_cast<uint32_t*>(p.out)[o_idx / 2] = pack_bf16(x[0], x[1]);
      else reinterpret_cast<__bf16*>(p.out)[o_idx] = (__bf16)x[0];
    } else {
      if constexpr (E == 2) reinterpret_cast<float2*>(p.out)[o_idx / 2] = make_float2(x[0], x[1]);
      else reinterpret_cast<float*>(p.out)[o_idx] = x[0];
    }
  }
}

template <int MODE, int D, bool ROT>
hipError_t launch_prefill_t(const PrefillParams& p, hipStream_t s) {
  const int ng = p.n_work / p.n_qtiles;                // (sequence, kv head) groups
  const int grid = (ng + 7) / 8 * 8 * p.n_qtiles;      // bounded on the host
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
