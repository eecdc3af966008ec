// Internal declarations shared by the libkvq host code and its HIP kernels.
// Not part of the C ABI (include/kvq.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

// Code bits, metadata floats per row (in separate meta planes) and levels,
// by mode: 0 INT8 per token and head, 1 INT4, 2 INT2, 3 INT8 with
// per-channel scales and no per-row metadata, 4 FP8 E4M3 per token and head
// (one scale, codes up to 448), 5 INT4 in the inline layout (codes and the
// float32 stored scale in one row, the integer zero point in the scale's low
// 4 bits, no meta planes).
__host__ __device__ constexpr int mode_bits(int mode) {
  return (mode == 0 || mode == 3 || mode == 4) ? 8 : ((mode == 1 || mode == 5) ? 4 : 2);
}
__host__ __device__ constexpr int mode_meta(int mode) {
  return (mode == 0 || mode == 4) ? 1 : ((mode == 3 || mode == 5) ? 0 : 2);
}
__host__ __device__ constexpr int mode_levels(int mode) {
  return (mode == 0 || mode == 3) ? 127 : ((mode == 1 || mode == 5) ? 15 : (mode == 4 ? 448 : 3));
}
// Per-channel scales: [2][Hkv][D] float32, K then V.
constexpr int kChannelMode = 3;
constexpr int kFp8Mode = 4;
// Inline INT4: one uint8 tensor [nb][2][bs][Hkv][D/2 + 4]; K rows at index 0
// of the second axis, V rows at 1 (the host passes the V half of block 0 as
// the V base, so both use one row index ((blk * 2 bs + offset) Hkv + h)).
constexpr int kInlineMode = 5;
__host__ __device__ constexpr int inline_row_bytes(int d) { return d / 2 + 4; }
// How a mode packs its codes (the inline mode packs like INT4).
__host__ __device__ constexpr int code_mode(int mode) { return mode == 5 ? 1 : mode; }
__host__ __device__ constexpr int row_bytes(int mode, int d) { return d * mode_bits(mode) / 8; }

// Positions the decode kernel processes as one tile (four 16-token MFMA tiles).
constexpr int kTile = 64;
// Most block ids one decode segment may span (held in LDS).
constexpr int kMaxSplitBlocks = 1024;
// CUs of an MI355X: the persistent decode grid is this times the resident
// workgroups per CU.
constexpr int kNumCUs = 256;

struct WriteParams {
  const uint16_t* key;      // bf16
  const uint16_t* value;    // bf16
  int64_t key_stride;       // elements between tokens
  int64_t value_stride;
  const int64_t* slot;      // [T] or nullptr
  const int64_t* slot_hw;   // [T, Hkv] or nullptr
  int64_t total_rows;       // 2 * T * Hkv
  int64_t slot_cap;         // num_blocks * block_size: slots at or past it are skipped
  int32_t hkv;
  int32_t block_size;
  uint8_t* k_codes;
  float* k_meta;
  uint8_t* v_codes;
  float* v_meta;
  const float* signs;       // [D] or nullptr
  const float* chs;         // per-channel mode: [2][Hkv][D] scales, K then V
  float inv_sqrt_d;         // float32 rounding of 1/sqrt(D)
};

struct DecodeParams {
  const uint8_t* k_codes;
  const float* k_meta;
  const uint8_t* v_codes;
  const float* v_meta;
  const uint16_t* q;            // bf16 [B, Hq, D]
  void* out;                    // [B, Hq, D]
  const int32_t* tables;        // [B, max_blocks] or [B*Hkv, max_blocks]
  const int32_t* seq_lens;      // [B]
  const int32_t* window;        // [Hkv] or nullptr
  const float* signs;           // [D] or nullptr
  const float* chs;             // per-channel mode: [2][Hkv][D] scales, K then V
  float* partials;              // [n_wgs + num_pairs][group][D + 4] pieces (m, l, pad, pad, acc)
  int32_t* counters;            // [num_pairs] pieces counted in; zero between calls
  float qscale;                 // softmax_scale * log2(e)
  float inv_sqrt_d;
  int64_t num_blocks;           // ids at or past it are treated as evicted
  int32_t headwise;
  int32_t max_blocks;
  int32_t max_seq_len;          // seq_lens entries are clamped to it
  int32_t sink;                 // windowed heads also attend positions < sink (>= 0)
  int32_t block_size;
  int32_t block_size_log2;
  int32_t hq;
  int32_t hkv;
  int32_t group;                // Hq / Hkv
  int32_t num_pairs;            // B * Hkv
  int32_t n_wgs;                // persistent decode workgroups
  int32_t out_bf16;
  uint32_t bits_magic;          // 0x43004300: bf16 128.0 in both halves
  uint32_t bits_n4;             // 0x000F000F
  uint32_t bits_n2;             // 0x00030003
  int32_t fused;                // 1: write each sequence's new token first (wp)
  WriteParams wp;               // the new tokens: token b = sequence b
};

struct PrefillParams {
  const uint8_t* k_codes;
  const float* k_meta;
  const uint8_t* v_codes;
  const float* v_meta;
  const uint16_t* q;            // bf16 [Tq, Hq, D]
  void* out;                    // [Tq, Hq, D]
  const int32_t* cu_q;          // [B + 1]
  const int32_t* seq_lens;      // [B]
  const int32_t* tables;        // [B, max_blocks] or [B*Hkv, max_blocks]
  const int32_t* window;        // [Hkv] or nullptr
  const float* signs;           // [D] or nullptr
  const float* chs;             // per-channel mode: [2][Hkv][D] scales, K then V
  float qscale;                 // softmax_scale * log2(e)
  float inv_sqrt_d;
  int64_t num_blocks;           // ids at or past it are treated as evicted
  int32_t headwise;
  int32_t max_blocks;
  int32_t max_seq_len;          // seq_lens entries are clamped to it
  int32_t sink;                 // windowed heads also attend positions < sink (>= 0)
  int32_t block_size_log2;
  int32_t hq;
  int32_t hkv;
  int32_t group;                // Hq / Hkv
  int32_t tq;                   // query tokens per workgroup = 128 / group
  int32_t n_qtiles;             // ceil(max_q_len / tq)
  int32_t n_work;               // n_qtiles * hkv * num_seqs
  int32_t out_bf16;
};

struct GatherParams {
  const uint8_t* k_codes;
  const float* k_meta;
  const uint8_t* v_codes;
  const float* v_meta;
  void* k_out;                  // [total_tokens, Hkv, D] float32 or bf16
  void* v_out;
  const int32_t* tables;        // [B, max_blocks] or [B*Hkv, max_blocks]
  const int32_t* cu;            // [B + 1] output row offsets
  const float* signs;           // [D] or nullptr
  const float* chs;             // per-channel mode: [2][Hkv][D] scales, K then V
  int64_t num_blocks;
  float inv_sqrt_d;
  int32_t headwise;
  int32_t max_blocks;
  int32_t block_size_log2;
  int32_t hkv;
  int32_t num_seqs;
  int32_t max_seq_len;          // positions the grid covers per sequence
  int32_t total_tokens;         // rows of the outputs
  int32_t out_bf16;
};

hipError_t launch_write(int mode, int d, bool rot, const WriteParams& p, hipStream_t s);
hipError_t launch_gather(int mode, int d, bool rot, const GatherParams& p, hipStream_t s);
// Rows one dequantize-gather workgroup covers (grid.x = ceil(rows / this)).
int64_t gather_rows_per_workgroup(int d);
// Resident decode workgroups per CU for this variant (its waves per SIMD).
int decode_wgs_per_cu(int mode, int d, int group);
hipError_t launch_decode(int mode, int d, bool rot, const DecodeParams& p, hipStream_t s);
hipError_t launch_prefill(int mode, int d, bool rot, const PrefillParams& p, hipStream_t s);
hipError_t launch_fill_zero(void* ptr, size_t bytes, hipStream_t s);
// Per-channel scales of a first batch: out[kv][h][d] = max_t |x| / 127.
hipError_t launch_calibrate(int d, const WriteParams& p, int32_t num_tokens, float* out, hipStream_t s);

}  // namespace kvq
