/*
 * kvq.h -- C ABI of libkvq: a dynamically quantized paged KV cache and the
 * attention that reads it, for AMD Instinct MI355X (gfx950).
 *
 * The operations follow these pages (cited by title and section):
 *  - FastDeploy PR 5173 "[Feature] support dynamic int2 quantization cache kv"
 *    (Motivation; pull-request overview): a 2-bit KV cache with run-time
 *    scales, written by encoder/decoder cache-write kernels and read by an
 *    attention kernel; no scales come from checkpoints.
 *  - prhub summary of vLLM PR 40835 "INT4 per-token-head KV cache quantization
 *    for the Triton backend" (功能与动机; 实现拆解; 关键源码片段): a write
 *    entry point (reshape-and-cache) that applies a randomized Hadamard
 *    transform, computes one scale and zero point per (token, kv head) and
 *    packs two 4-bit codes per byte; a read entry point (unified attention)
 *    that unpacks, dequantizes and attends; uint8 storage.
 *  - FastDeploy PR 7718 "Optimize AppendAttention for discrete head-wise
 *    block_idx" (Motivation; Modifications; correctness gates): an optional,
 *    additive head-wise block table [batch*kv_heads, max_blocks] whose -1
 *    entries are evicted sliding-window blocks that are skipped before any
 *    K/V address is formed; int32 index tensors; the GQA head-divisibility
 *    check raises instead of asserting.
 *  - FastDeploy PR 7757 "fix cache_manager_v1 allocating kv cache with wrong
 *    dtype" (问题描述; 修复): every quantized cache is uint8; a storage
 *    dtype/size mismatch must be reported, not crash.
 *
 * Conventions for every entry point:
 *  - Pointers marked (device) are HIP device pointers; (host) are host
 *    pointers.  The caller owns every buffer and keeps it alive until the work
 *    queued on `stream` has finished.  The library allocates no device memory
 *    and keeps no pointer after returning.
 *  - `stream` is a hipStream_t passed as void*; NULL means the null stream.
 *    Every launch is asynchronous on it.
 *  - Arguments are validated on the host before anything is launched.  A
 *    status other than KVQ_OK means nothing was launched; kvq_last_error()
 *    then returns a message (thread-local, valid until the next call on the
 *    same thread).  The library never aborts.
 *  - Values the host cannot see (device-side seq_lens, block ids, slots) are
 *    the caller's contract: block ids should be < num_blocks or negative
 *    (table entries) and slots < num_blocks*block_size or negative (slot
 *    mappings).  A violation never makes a kernel touch memory outside the
 *    planes: a table entry >= num_blocks is treated like -1 (an evicted
 *    block, never read), a slot >= num_blocks*block_size like a negative one
 *    (the row is not written), and seq_lens entries are clamped to
 *    max_seq_len.  Results for such inputs are what those rules give.
 *
 * Cache layout (one code plane and one meta plane each for K and for V):
 *    codes: uint8   [num_blocks, num_kv_heads, block_size, P]
 *           P = head_dim * b / 8, b = 8, 4, 2 bits
 *    meta : float32 [num_blocks, num_kv_heads, block_size, M]
 *           M = 1 (INT8, FP8: scale), 2 (INT4/INT2: scale, zero point) or 0
 *           (INT8_CHANNEL: the scales are per channel, in
 *           desc->channel_scales; meta pointers may then be NULL)
 *  A (token, kv head) row of codes is contiguous.  INT4 puts element 2j in the
 *  low nibble of byte j; INT2 puts element 4j+k in bits 2k..2k+1 of byte j;
 *  INT8 stores two's complement codes in [-127, 127]; FP8 one E4M3 byte per
 *  element.  Reconstruction:
 *  x_hat = c*s (INT8), c*s + z (INT4/INT2), E4M3(c)*s (FP8), c*s_d
 *  (INT8_CHANNEL), in the rotated basis when the cache has a rotation.
 *  KVQ_INT4_INLINE keeps codes and scale in one tensor instead (see kvq_mode):
 *  x_hat = (c - zp)*st.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KVQ_OK = 0,
  KVQ_EINVAL = 1,        /* an argument is invalid (NULL, out of range, inconsistent) */
  KVQ_EUNSUPPORTED = 2,  /* valid but not built (e.g. head_dim 96, GQA group > 16) */
  KVQ_ENOSPACE = 3,      /* the workspace is smaller than the *_workspace_size result */
  KVQ_EHIP = 4           /* the HIP runtime reported an error at launch */
} kvq_status;

/* Quantization modes.  INT8: per-token-head symmetric, s = max|y| / 127.
 * INT4 / INT2: per-token-head asymmetric, s = (max y - min y) / L,
 * z = min y, L = 15 / 3, codes = clamp(rint((y - z) / s), 0, L), computed as
 * (y - z) * (1/s) in float32 with round-half-to-even.  A row whose scale is
 * zero or subnormal gets all-zero codes.
 * INT8_CHANNEL: dynamic per-channel symmetric INT8 (the
 * vllm-ascend-quantized-kv-cache package, 运行机制): one scale per (K or V,
 * kv head, channel), s_d = max_t |x_d| / 127 over the first K/V a layer
 * receives (kvq_calibrate_channel_scales), then fixed; codes
 * clamp(rint(x_d * (1/s_d)), -127, 127), saturating; x_hat = c * s_d.  No
 * rotation and no per-row metadata (the meta planes are empty).
 * FP8_E4M3: per-token-head FP8 (the INT8/FP8 per-token-head schemes of the
 * vLLM PR 40835 summary, 功能与动机): OCP E4M3 codes (bias 7, largest 448),
 * s = max|y| / 448, code = y * (1/s) clamped to +-448 and rounded to the
 * nearest E4M3 value (ties to even); x_hat = E4M3(code) * s; one meta float
 * (s); optional rotation.  Chunked prefill is not built for this mode
 * (KVQ_EUNSUPPORTED; kvq_gather_dequant gives the dense rows).
 * INT4_INLINE: the vLLM-shaped inline layout (vLLM PR 40835 summary,
 * 关键源码片段: cache shape (num_blocks, 2, block_size, num_kv_heads,
 * head_size // 2 + scale_pad), the float32 scale at the end of each row;
 * 评论区精华: the 4-bit zero point kept in the scale's low 4 bits).  ONE
 * uint8 tensor [num_blocks][2][block_size][num_kv_heads][D/2 + 4], index 0
 * of the second axis K, 1 V; a row is D/2 bytes of nibbles (element 2j in
 * the low nibble of byte j) then the 4 little-endian bytes of the stored
 * scale st.  Per row: mn = min(min y, 0), mx = max(max y, 0), s = (mx - mn)
 * / 15, zp = clamp(rint(-mn / s), 0, 15), st = s with its low 4 bits
 * replaced by zp (within 15 ulp of s), c = clamp(rint(y * (1/st)) + zp, 0,
 * 15), x_hat = (c - zp) * st; a zero, subnormal or NaN s stores st = 0 and
 * codes 0.  Optional rotation.  Calls take the tensor as k_codes and NULL
 * for k_meta, v_codes and v_meta (KVQ_EINVAL otherwise). */
typedef enum {
  KVQ_INT8_SYM = 0, KVQ_INT4_ASYM = 1, KVQ_INT2_ASYM = 2, KVQ_INT8_CHANNEL = 3, KVQ_FP8_E4M3 = 4,
  KVQ_INT4_INLINE = 5
} kvq_mode;

typedef enum { KVQ_OUT_F32 = 0, KVQ_OUT_BF16 = 1 } kvq_out_dtype;

typedef struct {
  int32_t mode;            /* kvq_mode */
  int32_t head_dim;        /* D: 64 or 128 */
  int32_t num_kv_heads;    /* Hkv >= 1 */
  int32_t block_size;      /* tokens per block: a power of two, 16..1024 */
  int64_t num_blocks;      /* physical blocks in each plane, >= 1; rows
                              num_blocks * num_kv_heads * block_size < 2^31
                              (< 2^30 for KVQ_INT4_INLINE) */
  /* (device) [head_dim] float32 of +1.0f / -1.0f, or NULL for no rotation.
   * With signs d, every K and V row x is stored as the codes of
   * y = (1/sqrt(D)) * H_D (d .* x), H_D the Sylvester Hadamard matrix in
   * natural order; attention pre-rotates the query with the same matrix and
   * rotates its output back, so results are in the original basis.  Must be
   * NULL for KVQ_INT8_CHANNEL. */
  const float* rot_signs;
  /* (device) KVQ_INT8_CHANNEL only: float32 [2][num_kv_heads][head_dim]
   * scales, K then V (from kvq_calibrate_channel_scales); ignored by the
   * other modes.  Required by every call that quantizes or reads codes. */
  const float* channel_scales;
} kvq_cache_desc;

/* Options of a decode launch.  Pass NULL for the defaults. */
typedef struct {
  /* Workgroups of the persistent decode grid; 0 = as many as the device
   * holds resident at once (the default and the fastest).  Any positive count
   * gives the same result up to floating-point summation order (each count's
   * result is deterministic); the workspace size depends on it, so the same
   * options must be given to kvq_decode_workspace_size. */
  int32_t num_workgroups;
} kvq_decode_options;

typedef struct {
  uint64_t code_bytes;       /* bytes of one code plane (the K plane; V is equal);
                                KVQ_INT4_INLINE: of the one cache tensor (K and V) */
  uint64_t meta_bytes;       /* bytes of one meta plane (0 for INLINE) */
  uint32_t row_code_bytes;   /* P; KVQ_INT4_INLINE: D/2 + 4, the whole inline row */
  uint32_t row_meta_floats;  /* M */
} kvq_layout;

/* Sizes of the planes the caller must allocate for `desc` (host only, no GPU
 * needed).  Cache allocation from these sizes rules out the storage-dtype
 * mismatch of FastDeploy PR 7757 by construction. */
kvq_status kvq_query_layout(const kvq_cache_desc* desc, kvq_layout* out /* host */);

/* Quantize-on-write (vLLM PR 40835 summary, 实现拆解 item 2; FastDeploy PR
 * 5173 encoder/decoder cache write).  For each token t < num_tokens and kv
 * head h: read the bf16 rows key[t, h, :] and value[t, h, :], rotate them
 * (if desc->rot_signs), compute the per-row scale (and zero point), round,
 * pack and store codes and meta at slot = slot_mapping[t] (or
 * slot_mapping_headwise[t*Hkv + h]): block = slot / block_size,
 * offset = slot % block_size.  A negative slot skips the row.
 *   key, value       (device) bf16, row (t, h) at t*tok_stride + h*D elements
 *   *_tok_stride     elements between consecutive tokens, >= Hkv*D, a
 *                    multiple of 8 and below 2^31 (KVQ_EUNSUPPORTED past it)
 *   slot_mapping     (device) int64 [num_tokens], or NULL
 *   slot_mapping_headwise (device) int64 [num_tokens, Hkv], or NULL;
 *                    exactly one of the two slot mappings is non-NULL
 *                    (num_tokens == 0 is a no-op that reads no argument)
 *   k_codes, v_codes (device) uint8 planes; k_meta, v_meta (device) float32
 * Two tokens mapped to the same (slot, head) in one call race.  One call
 * writes at most 2^31 rows (2 * num_tokens * Hkv; KVQ_EUNSUPPORTED past it). */
kvq_status kvq_reshape_and_cache(const kvq_cache_desc* desc,
                                 const void* key, const void* value,
                                 int64_t key_tok_stride, int64_t value_tok_stride,
                                 const int64_t* slot_mapping,
                                 const int64_t* slot_mapping_headwise,
                                 int32_t num_tokens,
                                 uint8_t* k_codes, float* k_meta,
                                 uint8_t* v_codes, float* v_meta,
                                 void* stream);

/* Per-channel scales of KVQ_INT8_CHANNEL from a layer's first K/V (the
 * vllm-ascend-quantized-kv-cache package, 运行机制: computed along the token
 * axis the first time the layer receives K/V, symmetric, K and V apart):
 * scales_out[0][h][d] = max_t |key[t, h, d]| / 127 and scales_out[1][h][d]
 * from value, in float32 (correctly rounded division), over t < num_tokens.
 * A channel whose maximum is 0 gets scale 0 (its codes are then 0).
 *   key, value, *_tok_stride: as for kvq_reshape_and_cache
 *   scales_out   (device) float32 [2, Hkv, D], 16-byte aligned; written, not read
 * desc->mode must be KVQ_INT8_CHANNEL (desc->channel_scales is not read).
 * num_tokens == 0 writes zeros.  One kernel launch. */
kvq_status kvq_calibrate_channel_scales(const kvq_cache_desc* desc,
                                        const void* key, const void* value,
                                        int64_t key_tok_stride, int64_t value_tok_stride,
                                        int32_t num_tokens, float* scales_out, void* stream);

/* Workspace bytes kvq_paged_decode_attention and kvq_decode_step need for
 * these sizes and options (host only; options NULL = defaults, and the same
 * options must then be passed to the decode call).  max_seq_len is the
 * largest seq_lens entry the call will see.  The workspace holds one counter
 * per (sequence, kv head) and the partial softmax states of pairs that
 * several workgroups share; its size grows with num_seqs * kv heads and the
 * GQA group, not with max_seq_len (except for very long batches). */
kvq_status kvq_decode_workspace_size(const kvq_cache_desc* desc, int32_t num_seqs,
                                     int32_t num_q_heads, int32_t max_seq_len,
                                     const kvq_decode_options* options,
                                     size_t* bytes /* host */);

/* Zero a workspace (asynchronous on `stream`; 256-byte aligned, size a
 * multiple of 16).  A decode workspace must be zeroed once before its first
 * use (this call, or any other zero fill); every decode call leaves its
 * counters at zero again, so later calls need no init. */
kvq_status kvq_workspace_init(void* workspace, size_t workspace_bytes, void* stream);

/* Paged decode attention (vLLM PR 40835 summary, 实现拆解 item 2: unpack,
 * dequantize, attend; FastDeploy PR 7718: optional head-wise table with -1
 * skips).  One query token per sequence; for sequence b, q head hq and kv
 * head h = hq / (Hq/Hkv) the output is softmax attention of query[b, hq] over
 * the dequantized, un-rotated keys/values of positions j < seq_lens[b] that
 * lie in a non-evicted block and, if window && window[h] > 0, satisfy
 * j >= seq_lens[b] - window[h] or j < sink_size.  No allowed position =>
 * output 0.
 *   out          (device) [B, Hq, D] float32 (KVQ_OUT_F32) or bf16 (KVQ_OUT_BF16)
 *   query        (device) bf16 [B, Hq, D]
 *   block_tables (device) int32 [B, max_blocks_per_seq], or NULL
 *   block_tables_headwise (device) int32 [B*Hkv, max_blocks_per_seq], or NULL;
 *                exactly one is non-NULL; row b*Hkv + h serves kv head h;
 *                an entry < 0 marks an evicted block (never read)
 *   seq_lens     (device) int32 [B], positions cached for each sequence
 *                (the current token included), each <= max_seq_len (larger
 *                entries are clamped to it)
 *   max_seq_len  host upper bound on seq_lens, <= max_blocks_per_seq*block_size
 *   window       (device) int32 [Hkv], <= 0 = full context; or NULL
 *   sink_size    (host) attention sinks: a windowed kv head also attends
 *                positions j < sink_size (FastDeploy PR 7718, Modifications,
 *                threads a sink_size into the attention op); <= 0 = none.
 *                With sinks, a windowed head's walk starts at position 0 and
 *                the tiles between the sinks and the window read nothing.
 *   softmax_scale  logits scale (usually 1/sqrt(D)); finite
 *   options      NULL, or the options given to kvq_decode_workspace_size
 *   workspace    (device) >= kvq_decode_workspace_size bytes, 256-byte
 *                aligned, zeroed before its first use (kvq_workspace_init);
 *                holds per-pair counters, zero again when the call ends, and
 *                the partial results of pairs several workgroups share
 * Calls sharing one workspace must not overlap in time.  One kernel launch. */
kvq_status kvq_paged_decode_attention(const kvq_cache_desc* desc,
                                      void* out, int32_t out_dtype,
                                      const void* query,
                                      int32_t num_seqs, int32_t num_q_heads,
                                      const uint8_t* k_codes, const float* k_meta,
                                      const uint8_t* v_codes, const float* v_meta,
                                      const int32_t* block_tables,
                                      const int32_t* block_tables_headwise,
                                      int32_t max_blocks_per_seq,
                                      const int32_t* seq_lens, int32_t max_seq_len,
                                      const int32_t* window, int32_t sink_size,
                                      float softmax_scale,
                                      const kvq_decode_options* options,
                                      void* workspace, size_t workspace_bytes,
                                      void* stream);

/* Largest workspace kvq_paged_decode_attention_noalloc can serve (bytes). */
#define KVQ_NOALLOC_SCRATCH_BYTES (8u << 20)

/* Paged decode attention without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  Arguments, result and errors are
 * those of kvq_paged_decode_attention with the default options; the
 * workspace is instead a device array inside the library of
 * KVQ_NOALLOC_SCRATCH_BYTES bytes per GPU, held until the process ends.
 *  - A call whose workspace (kvq_decode_workspace_size with NULL options)
 *    exceeds KVQ_NOALLOC_SCRATCH_BYTES returns KVQ_ENOSPACE and launches
 *    nothing.
 *  - Each call launches a small fill kernel that zeroes the array's counters,
 *    then the decode kernel, both on `stream`; nothing is allocated (no
 *    hipMalloc, no memset node).  The calling thread's current device must be
 *    the one that `stream` and the buffers belong to.
 *  - Every call on a GPU shares that GPU's array: calls that overlap in time
 *    on one GPU (on different streams, or from different threads) race and
 *    give undefined results. */
kvq_status kvq_paged_decode_attention_noalloc(const kvq_cache_desc* desc,
                                              void* out, int32_t out_dtype,
                                              const void* query,
                                              int32_t num_seqs, int32_t num_q_heads,
                                              const uint8_t* k_codes, const float* k_meta,
                                              const uint8_t* v_codes, const float* v_meta,
                                              const int32_t* block_tables,
                                              const int32_t* block_tables_headwise,
                                              int32_t max_blocks_per_seq,
                                              const int32_t* seq_lens, int32_t max_seq_len,
                                              const int32_t* window, int32_t sink_size,
                                              float softmax_scale,
                                              void* stream);

/* One decode step in one launch: the quantize-on-write of each sequence's
 * new token followed by paged decode attention (the decoder's cache write and
 * attention of FastDeploy PR 5173, Modifications, and the append-then-attend
 * shape of FastDeploy PR 7718; the write and read halves of the vLLM PR 40835
 * summary, 实现拆解 item 2).  The result equals kvq_reshape_and_cache of the
 * B tokens followed by kvq_paged_decode_attention, codes and output bit for
 * bit.
 *   key, value   (device) bf16 [B, Hkv, D] rows, token b belongs to sequence
 *                b; token strides in elements (>= Hkv*D, multiple of 8),
 *                16-byte aligned
 *   slot_mapping (device) int64 [B], or slot_mapping_headwise int64 [B, Hkv];
 *                exactly one non-NULL.  A slot < 0 skips that token (or head).
 *                A written slot must be the one the block table gives position
 *                seq_lens[b] - 1 of sequence b (and head h when head-wise):
 *                the workgroup that attends that position writes it first; a
 *                slot anywhere else leaves the attention's view of it undefined.
 *                Sequences with seq_lens[b] = 0 have no new token and nothing
 *                is written for them.
 * Every other argument, the workspace and the errors are those of
 * kvq_paged_decode_attention (the planes are written, so they are not const).
 * Calls sharing one workspace must not overlap in time.  One kernel launch. */
kvq_status kvq_decode_step(const kvq_cache_desc* desc,
                           void* out, int32_t out_dtype,
                           const void* query,
                           int32_t num_seqs, int32_t num_q_heads,
                           const void* key, const void* value,
                           int64_t key_tok_stride, int64_t value_tok_stride,
                           const int64_t* slot_mapping,
                           const int64_t* slot_mapping_headwise,
                           uint8_t* k_codes, float* k_meta,
                           uint8_t* v_codes, float* v_meta,
                           const int32_t* block_tables,
                           const int32_t* block_tables_headwise,
                           int32_t max_blocks_per_seq,
                           const int32_t* seq_lens, int32_t max_seq_len,
                           const int32_t* window, int32_t sink_size,
                           float softmax_scale,
                           const kvq_decode_options* options,
                           void* workspace, size_t workspace_bytes,
                           void* stream);

/* Chunked-prefill attention (vLLM PR 40835 summary, 实现拆解 item 2; the
 * vllm-ascend-quantized-kv-cache package, 运行机制: prefill reads the paged
 * quantized cache; FastDeploy PR 7718: head-wise table with -1 skips and
 * per-head sliding windows).  Sequence b owns the query rows
 * cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1; its n_b = cu_seqlens_q[b+1] -
 * cu_seqlens_q[b] new tokens are already written to the cache (call
 * kvq_reshape_and_cache first) and sit at positions L_b - n_b + i, L_b =
 * seq_lens[b].  Row (i, q head hq) attends, over kv head h = hq / (Hq/Hkv), to
 * the dequantized, un-rotated keys/values of positions j <= L_b - n_b + i that
 * lie in a non-evicted block and, if window && window[h] > 0, satisfy
 * j >= L_b - n_b + i - window[h] + 1 or j < sink_size.  No allowed position
 * => output 0.
 *   out          (device) [total_q, Hq, D] float32 or bf16 (out_dtype)
 *   query        (device) bf16 [total_q, Hq, D]
 *   cu_seqlens_q (device) int32 [num_seqs + 1], non-decreasing, from 0
 *   max_q_len    host upper bound on every n_b (sizes the grid; rows past it
 *                are not computed)
 *   seq_lens     (device) int32 [num_seqs], each >= n_b and <= max_seq_len
 *   block tables, window, sink_size, softmax_scale and the cache planes as
 *   for kvq_paged_decode_attention
 *   workspace    (device) kvq_prefill_workspace_size bytes; may be NULL when
 *                that size is 0 (it is for every shape this library builds:
 *                each workgroup covers the whole key range of its rows)
 * GQA groups up to 128.  One kernel launch.  KVQ_FP8_E4M3 returns
 * KVQ_EUNSUPPORTED (not built; kvq_gather_dequant gives its dense rows). */
kvq_status kvq_paged_prefill_attention(const kvq_cache_desc* desc,
                                       void* out, int32_t out_dtype,
                                       const void* query,
                                       const int32_t* cu_seqlens_q,
                                       int32_t num_seqs, int32_t num_q_heads,
                                       int32_t max_q_len,
                                       const uint8_t* k_codes, const float* k_meta,
                                       const uint8_t* v_codes, const float* v_meta,
                                       const int32_t* block_tables,
                                       const int32_t* block_tables_headwise,
                                       int32_t max_blocks_per_seq,
                                       const int32_t* seq_lens, int32_t max_seq_len,
                                       const int32_t* window, int32_t sink_size,
                                       float softmax_scale,
                                       void* workspace, size_t workspace_bytes,
                                       void* stream);

/* Workspace bytes kvq_paged_prefill_attention needs for these sizes (host
 * only): 0 for every shape this library builds, since a workgroup owns the
 * whole key range of its query rows and merges nothing across workgroups.
 * Validates the same sizes as the prefill call. */
kvq_status kvq_prefill_workspace_size(const kvq_cache_desc* desc, int32_t num_seqs,
                                      int32_t num_q_heads, int32_t max_q_len,
                                      int32_t max_seq_len, size_t* bytes /* host */);

/* Dequantize-gather (the cache-fetch-and-dequantize operator of FastDeploy
 * PR 5173, review thread; the gather-and-dequantize of the paged cache that
 * prefill uses in the vllm-ascend-quantized-kv-cache package, 运行机制).
 * Sequence b's positions j = 0 .. n_b - 1, n_b = cu_seq_lens[b+1] -
 * cu_seq_lens[b], are written to row cu_seq_lens[b] + j of key_out and
 * value_out: for every kv head h the dequantized row x_hat = c*s (+ z) of the
 * block the table gives, rotated back (R^T x_hat) when the cache has a
 * rotation.  A position in an evicted (-1) block gives a zero row.
 *   key_out, value_out (device) [total_tokens, Hkv, D] float32 (KVQ_OUT_F32)
 *                or bf16 (KVQ_OUT_BF16, round to nearest even), 16-byte aligned
 *   block_tables / block_tables_headwise, max_blocks_per_seq: as for
 *                kvq_paged_decode_attention (exactly one non-NULL)
 *   cu_seq_lens  (device) int32 [num_seqs + 1], non-decreasing from 0,
 *                cu_seq_lens[num_seqs] <= total_tokens, every n_b <= max_seq_len
 *   max_seq_len  host upper bound on every n_b (sizes the grid: positions at
 *                or past it are not written), <= max_blocks_per_seq*block_size
 * Rows past total_tokens are never written.  No workspace; one kernel launch.
 * The outputs must not overlap the cache planes. */
kvq_status kvq_gather_dequant(const kvq_cache_desc* desc,
                              void* key_out, void* value_out, int32_t out_dtype,
                              const uint8_t* k_codes, const float* k_meta,
                              const uint8_t* v_codes, const float* v_meta,
                              const int32_t* block_tables,
                              const int32_t* block_tables_headwise,
                              int32_t max_blocks_per_seq,
                              const int32_t* cu_seq_lens,
                              int32_t num_seqs, int32_t total_tokens,
                              int32_t max_seq_len,
                              void* stream);

/* Thread-local message for the last non-OK status ("" if none). */
const char* kvq_last_error(void);

/* Library version as major*10000 + minor*100 + patch. */
int32_t kvq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
