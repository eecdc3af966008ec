// libkvq host side: argument validation, cache layout, split planning and
// kernel launches behind the C ABI of include/kvq.h.
//
// Validation mirrors the interface facts of the pages: int32 index tensors and
// a head-divisibility check that reports instead of asserting (FastDeploy PR
// 7718, Modifications), an additive optional head-wise table (same PR,
// Motivation), uint8 storage whose size comes from the layout query (FastDeploy
// PR 7757, 修复), and no static scales (FastDeploy PR 5173, overview).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "kvq.h"
#include "kvq_internal.h"

// Device scratch of kvq_paged_decode_attention_noalloc: the decode
// workspace (piece counters, then partial softmax states) of callers that
// cannot allocate.  Each GPU the library runs on holds its own copy until
// the process ends.  Host code never uses this name as an address: it takes
// the device address from hipGetSymbolAddress (scratch_address below).
static __device__ __align__(256) unsigned char scratch[KVQ_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local char g_err[512] = "";

kvq_status fail(kvq_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

kvq_status ok() {
  g_err[0] = '\0';
  return KVQ_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

kvq_status check_desc(const kvq_cache_desc* d) {
  if (!d) return fail(KVQ_EINVAL, "desc is NULL");
  if (d->mode < KVQ_INT8_SYM || d->mode > KVQ_INT4_INLINE)
    return fail(KVQ_EINVAL, "mode %d is not a kvq_mode", d->mode);
  if (d->head_dim != 64 && d->head_dim != 128) {
    if (d->head_dim > 0 && (d->head_dim & (d->head_dim - 1)) == 0)
      return fail(KVQ_EUNSUPPORTED, "head_dim %d: only 64 and 128 are built", d->head_dim);
    return fail(KVQ_EINVAL, "head_dim %d must be a power of two (64 or 128)", d->head_dim);
  }
  if (d->num_kv_heads < 1) return fail(KVQ_EINVAL, "num_kv_heads %d < 1", d->num_kv_heads);
  if (d->block_size < 16 || d->block_size > 1024 || (d->block_size & (d->block_size - 1)) != 0)
    return fail(KVQ_EINVAL, "block_size %d must be a power of two in [16, 1024]", d->block_size);
  if (d->num_blocks < 1) return fail(KVQ_EINVAL, "num_blocks %lld < 1", (long long)d->num_blocks);
  if ((long long)d->num_blocks * d->num_kv_heads * d->block_size * (d->mode == KVQ_INT4_INLINE ? 2 : 1) >
      0x7fffffffLL)
    return fail(KVQ_EUNSUPPORTED, "num_blocks*num_kv_heads*block_size must stay below 2^31 rows (2^30 for the "
                "inline layout, which holds K and V rows in one tensor)");
  if (d->rot_signs && !aligned(d->rot_signs, 16))
    return fail(KVQ_EINVAL, "rot_signs must be 16-byte aligned");
  if (d->mode == KVQ_INT8_CHANNEL && d->rot_signs)
    return fail(KVQ_EUNSUPPORTED, "KVQ_INT8_CHANNEL takes no rotation (rot_signs must be NULL)");
  return KVQ_OK;
}

// The per-channel scales a KVQ_INT8_CHANNEL call reads.
kvq_status check_channel(const kvq_cache_desc* d) {
  if (d->mode != KVQ_INT8_CHANNEL) return KVQ_OK;
  if (!d->channel_scales) return fail(KVQ_EINVAL, "KVQ_INT8_CHANNEL needs desc->channel_scales");
  if (!aligned(d->channel_scales, 16)) return fail(KVQ_EINVAL, "channel_scales must be 16-byte aligned");
  return KVQ_OK;
}

// Code planes always; meta planes unless the mode has no per-row metadata.
// The inline layout is one tensor passed as k_codes, the other three NULL.
kvq_status check_planes(int mode, const uint8_t* kc, const float* km, const uint8_t* vc, const float* vm) {
  if (mode == KVQ_INT4_INLINE) {
    if (!kc) return fail(KVQ_EINVAL, "k_codes (the inline cache) is NULL");
    if (km || vc || vm) return fail(KVQ_EINVAL, "KVQ_INT4_INLINE takes one tensor as k_codes; k_meta, v_codes and "
                                    "v_meta must be NULL");
    if (!aligned(kc, 16)) return fail(KVQ_EINVAL, "the inline cache must be 16-byte aligned");
    return KVQ_OK;
  }
  const bool meta = kvq::mode_meta(mode) > 0;
  if (!kc || !vc || (meta && (!km || !vm))) return fail(KVQ_EINVAL, "a cache plane pointer is NULL");
  if (!aligned(kc, 16) || !aligned(vc, 16) || (meta && (!aligned(km, 16) || !aligned(vm, 16))))
    return fail(KVQ_EINVAL, "cache planes must be 16-byte aligned");
  return KVQ_OK;
}

// The four plane pointers the kernels take: for the inline layout the V
// base is the V half of block 0 (block_size * num_kv_heads rows in), so K and
// V rows share one row index, and there are no meta planes.
template <typename C, typename F>
void resolve_planes(const kvq_cache_desc* d, C*& kc, F*& km, C*& vc, F*& vm) {
  if (d->mode != KVQ_INT4_INLINE) return;
  vc = kc + (size_t)d->block_size * d->num_kv_heads * kvq::inline_row_bytes(d->head_dim);
  km = nullptr;
  vm = nullptr;
}

float inv_sqrt_f32(int d) { return (float)(1.0 / std::sqrt((double)d)); }

// Compute units of the current device (the MI355X's 256 when there is no
// device to ask, as in a host-only size query).
int num_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
    (void)hipGetLastError();
    return kvq::kNumCUs;
  }
  return n;
}

struct DecodePlan {
  int n_wgs;
  size_t counter_bytes;
  size_t partial_bytes;
  size_t total() const { return counter_bytes + partial_bytes; }
};

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Stream-K plan: a persistent grid of as many workgroups as fit on the
// MI355X at once (256 CUs times the variant's resident workgroups per CU),
// or the caller's count, shares all pairs' tiles equally; more workgroups
// only when a share could span more blocks than one segment's LDS table
// holds.  The workspace holds one piece counter per pair (zero between calls)
// and one (m, l, acc) record per (piece, head): at most n_wgs + pairs pieces.
// Deterministic in its inputs.
DecodePlan plan_decode(const kvq_cache_desc* d, int num_seqs, int num_q_heads, int max_seq_len,
                       const kvq_decode_options* opt) {
  DecodePlan pl{};
  const long long max_tiles = (max_seq_len + kvq::kTile - 1) / kvq::kTile;
  const long long pairs = (long long)num_seqs * d->num_kv_heads;
  const long long seg_cap = ((long long)(kvq::kMaxSplitBlocks - 1) * d->block_size) / kvq::kTile - 1;
  long long nw = (long long)num_cus() * kvq::decode_wgs_per_cu(d->mode, d->head_dim, num_q_heads / d->num_kv_heads);
  if (opt && opt->num_workgroups > 0) nw = opt->num_workgroups;
  const long long need = (pairs * max_tiles + seg_cap - 1) / seg_cap + 1;
  if (nw < need) nw = need;
  pl.n_wgs = (int)nw;
  const int G = num_q_heads / d->num_kv_heads;
  pl.counter_bytes = round_up((size_t)pairs * sizeof(int32_t), 256);
  pl.partial_bytes = round_up((size_t)(nw + pairs) * G * (d->head_dim + 4) * sizeof(float), 256);
  return pl;
}

kvq_status check_options(const kvq_decode_options* opt) {
  if (opt && opt->num_workgroups < 0)
    return fail(KVQ_EINVAL, "options->num_workgroups %d < 0", opt->num_workgroups);
  if (opt && opt->num_workgroups > (1 << 20))
    return fail(KVQ_EUNSUPPORTED, "options->num_workgroups %d > 2^20", opt->num_workgroups);
  return KVQ_OK;
}

kvq_status check_decode_sizes(const kvq_cache_desc* d, int num_seqs, int num_q_heads, int max_seq_len) {
  if (num_seqs < 0) return fail(KVQ_EINVAL, "num_seqs %d < 0", num_seqs);
  if (num_seqs > 65535) return fail(KVQ_EUNSUPPORTED, "num_seqs %d > 65535", num_seqs);
  if (num_q_heads < 1) return fail(KVQ_EINVAL, "num_q_heads %d < 1", num_q_heads);
  if (num_q_heads % d->num_kv_heads != 0)
    return fail(KVQ_EINVAL, "num_q_heads %d is not a multiple of num_kv_heads %d", num_q_heads,
                d->num_kv_heads);
  if (num_q_heads / d->num_kv_heads > 16)
    return fail(KVQ_EUNSUPPORTED, "GQA group %d > 16 is not built", num_q_heads / d->num_kv_heads);
  if (d->num_kv_heads > 65535) return fail(KVQ_EUNSUPPORTED, "num_kv_heads > 65535");
  if (max_seq_len < 0) return fail(KVQ_EINVAL, "max_seq_len %d < 0", max_seq_len);
  // the decode schedule counts all tiles of the batch in int32
  if ((long long)num_seqs * d->num_kv_heads * ((max_seq_len + kvq::kTile - 1) / kvq::kTile) >= 0x7fffffffLL)
    return fail(KVQ_EUNSUPPORTED, "num_seqs*num_kv_heads*ceil(max_seq_len/64) must stay below 2^31 tiles");
  return KVQ_OK;
}

// Device address of `scratch` on the current device: looked up once per
// device (with that device current) and kept for the life of the process.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices] = {};

kvq_status scratch_address(void** addr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(KVQ_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(KVQ_EUNSUPPORTED, "device %d >= %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(KVQ_EHIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_addr[dev] = p;
  }
  *addr = g_scratch_addr[dev];
  return KVQ_OK;
}

// use_scratch: the workspace is the library's device scratch (workspace and
// workspace_bytes are ignored); its counters are cleared by a fill kernel
// before the decode launch.
kvq_status decode_impl(const kvq_cache_desc* desc, void* out, int32_t out_dtype,
                                      const void* query, int32_t num_seqs, int32_t num_q_heads,
                                      const uint8_t* k_codes, const float* k_meta,
                                      const uint8_t* v_codes, const float* v_meta,
                                      const int32_t* block_tables, const int32_t* block_tables_headwise,
                                      int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                      int32_t max_seq_len, const int32_t* window, int32_t sink_size,
                                      float softmax_scale, const kvq_decode_options* options,
                                      void* workspace, size_t workspace_bytes, void* stream,
                                      const kvq::WriteParams* wp, bool use_scratch = false) {
  kvq_status st = check_desc(desc);
  if (st != KVQ_OK) return st;
  st = check_decode_sizes(desc, num_seqs, num_q_heads, max_seq_len);
  if (st != KVQ_OK) return st;
  st = check_options(options);
  if (st != KVQ_OK) return st;
  if (out_dtype != KVQ_OUT_F32 && out_dtype != KVQ_OUT_BF16)
    return fail(KVQ_EINVAL, "out_dtype %d is not a kvq_out_dtype", out_dtype);
  if ((block_tables == nullptr) == (block_tables_headwise == nullptr))
    return fail(KVQ_EINVAL, "exactly one of block_tables and block_tables_headwise must be non-NULL");
  if (max_blocks_per_seq < 1) return fail(KVQ_EINVAL, "max_blocks_per_seq %d < 1", max_blocks_per_seq);
  if ((int64_t)max_seq_len > (int64_t)max_blocks_per_seq * desc->block_size)
    return fail(KVQ_EINVAL, "max_seq_len %d exceeds max_blocks_per_seq*block_size = %lld", max_seq_len,
                (long long)max_blocks_per_seq * desc->block_size);
  if (!std::isfinite(softmax_scale)) return fail(KVQ_EINVAL, "softmax_scale is not finite");
  if (num_seqs == 0) return ok();
  if (!out || !query || !seq_lens) return fail(KVQ_EINVAL, "out, query or seq_lens is NULL");
  if (!aligned(out, 16)) return fail(KVQ_EINVAL, "out must be 16-byte aligned");
  st = check_planes(desc->mode, k_codes, k_meta, v_codes, v_meta);
  if (st != KVQ_OK) return st;
  resolve_planes(desc, k_codes, k_meta, v_codes, v_meta);
  st = check_channel(desc);
  if (st != KVQ_OK) return st;
  const DecodePlan pl = plan_decode(desc, num_seqs, num_q_heads, max_seq_len, options);
  if (use_scratch) {
    if (pl.total() > (size_t)KVQ_NOALLOC_SCRATCH_BYTES)
      return fail(KVQ_ENOSPACE, "this decode needs %zu bytes of workspace; the allocation-free call has %zu",
                  pl.total(), (size_t)KVQ_NOALLOC_SCRATCH_BYTES);
    st = scratch_address(&workspace);
    if (st != KVQ_OK) return st;
    workspace_bytes = KVQ_NOALLOC_SCRATCH_BYTES;
    // the counters must start at zero: a fill kernel, not a memset node
    hipError_t e = kvq::launch_fill_zero(workspace, pl.counter_bytes, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(KVQ_EHIP, "scratch clear: %s", hipGetErrorString(e));
  }
  if (!workspace) return fail(KVQ_EINVAL, "workspace is NULL (%zu bytes needed)", pl.total());
  if (workspace_bytes < pl.total())
    return fail(KVQ_ENOSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, pl.total());
  if (!aligned(workspace, 256)) return fail(KVQ_EINVAL, "workspace must be 256-byte aligned");
  kvq::DecodeParams p{};
  p.k_codes = k_codes;
  p.k_meta = k_meta;
  p.v_codes = v_codes;
  p.v_meta = v_meta;
  p.q = static_cast<const uint16_t*>(query);
  p.out = out;
  p.headwise = block_tables_headwise != nullptr;
  p.tables = p.headwise ? block_tables_headwise : block_tables;
  p.seq_lens = seq_lens;
  p.window = window;
  p.signs = desc->rot_signs;
  p.chs = desc->channel_scales;
  p.counters = static_cast<int32_t*>(workspace);
  p.partials = reinterpret_cast<float*>(static_cast<char*>(workspace) + pl.counter_bytes);
  p.qscale = softmax_scale * 1.4426950408889634f;
  p.inv_sqrt_d = inv_sqrt_f32(desc->head_dim);
  p.num_blocks = desc->num_blocks;
  p.max_blocks = max_blocks_per_seq;
  p.max_seq_len = max_seq_len;
  p.sink = sink_size > 0 ? sink_size : 0;
  p.block_size = desc->block_size;
  p.block_size_log2 = __builtin_ctz((unsigned)desc->block_size);
  p.hq = num_q_heads;
  p.hkv = desc->num_kv_heads;
  p.group = num_q_heads / desc->num_kv_heads;
  p.num_pairs = num_seqs * desc->num_kv_heads;
  p.n_wgs = pl.n_wgs;
  p.out_bf16 = out_dtype == KVQ_OUT_BF16;
  p.bits_magic = 0x43004300u;
  p.bits_n4 = 0x000F000Fu;
  p.bits_n2 = 0x00030003u;
  if (wp) {
    p.fused = 1;
    p.wp = *wp;
    p.wp.k_codes = const_cast<uint8_t*>(k_codes);
    p.wp.k_meta = const_cast<float*>(k_meta);
    p.wp.v_codes = const_cast<uint8_t*>(v_codes);
    p.wp.v_meta = const_cast<float*>(v_meta);
    p.wp.hkv = desc->num_kv_heads;
    p.wp.block_size = desc->block_size;
    p.wp.slot_cap = desc->num_blocks * desc->block_size;
    p.wp.signs = desc->rot_signs;
    p.wp.chs = desc->channel_scales;
    p.wp.inv_sqrt_d = inv_sqrt_f32(desc->head_dim);
    p.wp.total_rows = 2 * (int64_t)num_seqs * desc->num_kv_heads;
  }
  hipError_t e = kvq::launch_decode(desc->mode, desc->head_dim, desc->rot_signs != nullptr, p,
                                    static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(KVQ_EHIP, "decode launch: %s", hipGetErrorString(e));
  return ok();
}

kvq_status check_prefill_sizes(const kvq_cache_desc* desc, int num_seqs, int num_q_heads, int max_q_len,
                               int max_seq_len) {
  kvq_status st = check_desc(desc);
  if (st != KVQ_OK) return st;
  if (desc->mode == KVQ_FP8_E4M3)
    return fail(KVQ_EUNSUPPORTED, "chunked prefill is not built for KVQ_FP8_E4M3 (kvq_gather_dequant gives the "
                "dense rows)");
  if (num_seqs < 0) return fail(KVQ_EINVAL, "num_seqs %d < 0", num_seqs);
  if (num_q_heads < 1) return fail(KVQ_EINVAL, "num_q_heads %d < 1", num_q_heads);
  if (num_q_heads % desc->num_kv_heads != 0)
    return fail(KVQ_EINVAL, "num_q_heads %d is not a multiple of num_kv_heads %d", num_q_heads,
                desc->num_kv_heads);
  const int group = num_q_heads / desc->num_kv_heads;
  if (group > 128) return fail(KVQ_EUNSUPPORTED, "GQA group %d > 128 is not built", group);
  if (max_q_len < 0) return fail(KVQ_EINVAL, "max_q_len %d < 0", max_q_len);
  if (max_seq_len < 0) return fail(KVQ_EINVAL, "max_seq_len %d < 0", max_seq_len);
  const int tq = 128 / group;
  // the launch pads the (sequence, kv head) groups to a multiple of 8
  const long long n_grid = (((long long)max_q_len + tq - 1) / tq) *
                           (((long long)desc->num_kv_heads * num_seqs + 7) / 8 * 8);
  if (n_grid > 0x7fffff00LL) return fail(KVQ_EUNSUPPORTED, "prefill grid of %lld workgroups", n_grid);
  return KVQ_OK;
}

}  // namespace

extern "C" {

kvq_status kvq_query_layout(const kvq_cache_desc* desc, kvq_layout* out) {
  kvq_status st = check_desc(desc);
  if (st != KVQ_OK) return st;
  if (!out) return fail(KVQ_EINVAL, "out is NULL");
  const uint32_t P = (uint32_t)kvq::row_bytes(desc->mode, desc->head_dim);
  const uint32_t M = (uint32_t)kvq::mode_meta(desc->mode);
  const uint64_t rows = (uint64_t)desc->num_blocks * desc->num_kv_heads * desc->block_size;
  if (desc->mode == KVQ_INT4_INLINE) {   // one tensor: K and V rows of D/2 + 4 bytes
    out->row_code_bytes = (uint32_t)kvq::inline_row_bytes(desc->head_dim);
    out->row_meta_floats = 0;
    out->code_bytes = 2 * rows * out->row_code_bytes;
    out->meta_bytes = 0;
    return ok();
  }
  out->row_code_bytes = P;
  out->row_meta_floats = M;
  out->code_bytes = rows * P;
  out->meta_bytes = rows * M * sizeof(float);
  return ok();
}

kvq_status kvq_reshape_and_cache(const kvq_cache_desc* desc, const void* key, const void* value,
                                 int64_t key_tok_stride, int64_t value_tok_stride,
                                 const int64_t* slot_mapping, const int64_t* slot_mapping_headwise,
                                 int32_t num_tokens, uint8_t* k_codes, float* k_meta,
                                 uint8_t* v_codes, float* v_meta, void* stream) {
  kvq_status st = check_desc(desc);
  if (st != KVQ_OK) return st;
  if (num_tokens < 0) return fail(KVQ_EINVAL, "num_tokens %d < 0", num_tokens);
  if (num_tokens == 0) return ok();  // nothing is read or written
  if ((slot_mapping == nullptr) == (slot_mapping_headwise == nullptr))
    return fail(KVQ_EINVAL, "exactly one of slot_mapping and slot_mapping_headwise must be non-NULL");
  st = check_planes(desc->mode, k_codes, k_meta, v_codes, v_meta);
  if (st != KVQ_OK) return st;
  resolve_planes(desc, k_codes, k_meta, v_codes, v_meta);
  st = check_channel(desc);
  if (st != KVQ_OK) return st;
  const int D = desc->head_dim, H = desc->num_kv_heads;
  {
    if (!key || !value) return fail(KVQ_EINVAL, "key or value is NULL");
    if (key_tok_stride < (int64_t)H * D || value_tok_stride < (int64_t)H * D)
      return fail(KVQ_EINVAL, "token strides (%lld, %lld) must be >= num_kv_heads*head_dim = %d",
                  (long long)key_tok_stride, (long long)value_tok_stride, H * D);
    if (key_tok_stride % 8 != 0 || value_tok_stride % 8 != 0 || !aligned(key, 16) || !aligned(value, 16))
      return fail(KVQ_EINVAL, "key/value must be 16-byte aligned with token strides a multiple of 8");
    if (key_tok_stride > 0x7fffffffLL || value_tok_stride > 0x7fffffffLL)
      return fail(KVQ_EUNSUPPORTED, "token strides must stay below 2^31 elements");
    if (2LL * num_tokens * H > 0x7fffffffLL)
      return fail(KVQ_EUNSUPPORTED, "2*num_tokens*num_kv_heads rows must stay below 2^31 per call");
  }
  kvq::WriteParams p{};
  p.key = static_cast<const uint16_t*>(key);
  p.value = static_cast<const uint16_t*>(value);
  p.key_stride = key_tok_stride;
  p.value_stride = value_tok_stride;
  p.slot = slot_mapping;
  p.slot_hw = slot_mapping_headwise;
  p.total_rows = 2 * (int64_t)num_tokens * H;
  p.slot_cap = desc->num_blocks * desc->block_size;
  p.hkv = H;
  p.block_size = desc->block_size;
  p.k_codes = k_codes;
  p.k_meta = k_meta;
  p.v_codes = v_codes;
  p.v_meta = v_meta;
  p.signs = desc->rot_signs;
  p.chs = desc->channel_scales;
  p.inv_sqrt_d = inv_sqrt_f32(D);
  hipError_t e = kvq::launch_write(desc->mode, D, desc->rot_signs != nullptr, p,
                                   static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(KVQ_EHIP, "write launch: %s", hipGetErrorString(e));
  return ok();
}

kvq_status kvq_calibrate_channel_scales(const kvq_cache_desc* desc, const void* key, const void* value,
                                        int64_t key_tok_stride, int64_t value_tok_stride, int32_t num_tokens,
                                        float* scales_out, void* stream) {
  kvq_status st = check_desc(desc);
  if (st != KVQ_OK) return st;
  if (desc->mode != KVQ_INT8_CHANNEL)
    return fail(KVQ_EINVAL, "kvq_calibrate_channel_scales needs mode KVQ_INT8_CHANNEL (got %d)", desc->mode);
  if (num_tokens < 0) return fail(KVQ_EINVAL, "num_tokens %d < 0", num_tokens);
  if (!scales_out || !aligned(scales_out, 16)) return fail(KVQ_EINVAL, "scales_out must be non-NULL, 16-byte aligned");
  const int D = desc->head_dim, H = desc->num_kv_heads;
  if (num_tokens > 0) {
    if (!key || !value) return fail(KVQ_EINVAL, "key or value is NULL");
    if (key_tok_stride < (int64_t)H * D || value_tok_stride < (int64_t)H * D)
      return fail(KVQ_EINVAL, "token strides (%lld, %lld) must be >= num_kv_heads*head_dim = %d",
                  (long long)key_tok_stride, (long long)value_tok_stride, H * D);
    if (key_tok_stride % 8 != 0 || value_tok_stride % 8 != 0 || !aligned(key, 16) || !aligned(value, 16))
      return fail(KVQ_EINVAL, "key/value must be 16-byte aligned with token strides a multiple of 8");
    if (key_tok_stride > 0x7fffffffLL || value_tok_stride > 0x7fffffffLL)
      return fail(KVQ_EUNSUPPORTED, "token strides must stay below 2^31 elements");
    if (2LL * num_tokens * H > 0x7fffffffLL)
      return fail(KVQ_EUNSUPPORTED, "2*num_tokens*num_kv_heads rows must stay below 2^31 per call");
  }
  kvq::WriteParams p{};
  p.key = static_cast<const uint16_t*>(key);
  p.value = static_cast<const uint16_t*>(value);
  p.key_stride = key_tok_stride;
  p.value_stride = value_tok_stride;
  p.hkv = H;
  hipError_t e = kvq::launch_calibrate(D, p, num_tokens, scales_out, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(KVQ_EHIP, "calibrate launch: %s", hipGetErrorString(e));
  return ok();
}

kvq_status kvq_decode_workspace_size(const kvq_cache_desc* desc, int32_t num_seqs, int32_t num_q_heads,
                                     int32_t max_seq_len, const kvq_decode_options* options, size_t* bytes) {
  kvq_status st = check_desc(desc);
  if (st != KVQ_OK) return st;
  st = check_decode_sizes(desc, num_seqs, num_q_heads, max_seq_len);
  if (st != KVQ_OK) return st;
  st = check_options(options);
  if (st != KVQ_OK) return st;
  if (!bytes) return fail(KVQ_EINVAL, "bytes is NULL");
  *bytes = plan_decode(desc, num_seqs, num_q_heads, max_seq_len, options).total();
  return ok();
}

kvq_status kvq_workspace_init(void* workspace, size_t workspace_bytes, void* stream) {
  if (workspace_bytes == 0) return ok();
  if (!workspace) return fail(KVQ_EINVAL, "workspace is NULL");
  if (!aligned(workspace, 256) || workspace_bytes % 16 != 0)
    return fail(KVQ_EINVAL, "workspace must be 256-byte aligned and a multiple of 16 bytes");
  hipError_t e = kvq::launch_fill_zero(workspace, workspace_bytes, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(KVQ_EHIP, "workspace init: %s", hipGetErrorString(e));
  return ok();
}

kvq_status kvq_paged_decode_attention(const kvq_cache_desc* desc, void* out, int32_t out_dtype,
                                      const void* query, int32_t num_seqs, int32_t num_q_heads,
                                      const uint8_t* k_codes, const float* k_meta,
                                      const uint8_t* v_codes, const float* v_meta,
                                      const int32_t* block_tables, const int32_t* block_tables_headwise,
                                      int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                      int32_t max_seq_len, const int32_t* window, int32_t sink_size,
                                      float softmax_scale, const kvq_decode_options* options,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(desc, out, out_dtype, query, num_seqs, num_q_heads, k_codes, k_meta, v_codes, v_meta,
                     block_tables, block_tables_headwise, max_blocks_per_seq, seq_lens, max_seq_len, window,
                     sink_size, softmax_scale, options, workspace, workspace_bytes, stream, nullptr);
}

kvq_status kvq_paged_decode_attention_noalloc(const kvq_cache_desc* desc, void* out, int32_t out_dtype,
                                              const void* query, int32_t num_seqs, int32_t num_q_heads,
                                              const uint8_t* k_codes, const float* k_meta,
                                              const uint8_t* v_codes, const float* v_meta,
                                              const int32_t* block_tables,
                                              const int32_t* block_tables_headwise,
                                              int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                              int32_t max_seq_len, const int32_t* window, int32_t sink_size,
                                              float softmax_scale, void* stream) {
  return decode_impl(desc, out, out_dtype, query, num_seqs, num_q_heads, k_codes, k_meta, v_codes, v_meta,
                     block_tables, block_tables_headwise, max_blocks_per_seq, seq_lens, max_seq_len, window,
                     sink_size, softmax_scale, nullptr, nullptr, 0, stream, nullptr, true);
}

kvq_status kvq_decode_step(const kvq_cache_desc* desc, void* out, int32_t out_dtype, const void* query,
                           int32_t num_seqs, int32_t num_q_heads, const void* key, const void* value,
                           int64_t key_tok_stride, int64_t value_tok_stride, const int64_t* slot_mapping,
                           const int64_t* slot_mapping_headwise, uint8_t* k_codes, float* k_meta,
                           uint8_t* v_codes, float* v_meta, const int32_t* block_tables,
                           const int32_t* block_tables_headwise, int32_t max_blocks_per_seq,
                           const int32_t* seq_lens, int32_t max_seq_len, const int32_t* window,
                           int32_t sink_size, float softmax_scale, const kvq_decode_options* options,
                           void* workspace, size_t workspace_bytes, void* stream) {
  kvq_status st = check_desc(desc);
  if (st != KVQ_OK) return st;
  if (num_seqs > 0) {
    if ((slot_mapping == nullptr) == (slot_mapping_headwise == nullptr))
      return fail(KVQ_EINVAL, "exactly one of slot_mapping and slot_mapping_headwise must be non-NULL");
    const int D = desc->head_dim, H = desc->num_kv_heads;
    if (!key || !value) return fail(KVQ_EINVAL, "key or value is NULL");
    if (key_tok_stride < (int64_t)H * D || value_tok_stride < (int64_t)H * D)
      return fail(KVQ_EINVAL, "token strides (%lld, %lld) must be >= num_kv_heads*head_dim = %d",
                  (long long)key_tok_stride, (long long)value_tok_stride, H * D);
    if (key_tok_stride % 8 != 0 || value_tok_stride % 8 != 0 || !aligned(key, 16) || !aligned(value, 16))
      return fail(KVQ_EINVAL, "key/value must be 16-byte aligned with token strides a multiple of 8");
    if (key_tok_stride > 0x7fffffffLL || value_tok_stride > 0x7fffffffLL)
      return fail(KVQ_EUNSUPPORTED, "token strides must stay below 2^31 elements");
  }
  kvq::WriteParams w{};
  w.key = static_cast<const uint16_t*>(key);
  w.value = static_cast<const uint16_t*>(value);
  w.key_stride = key_tok_stride;
  w.value_stride = value_tok_stride;
  w.slot = slot_mapping;
  w.slot_hw = slot_mapping_headwise;
  return decode_impl(desc, out, out_dtype, query, num_seqs, num_q_heads, k_codes, k_meta, v_codes, v_meta,
                     block_tables, block_tables_headwise, max_blocks_per_seq, seq_lens, max_seq_len, window,
                     sink_size, softmax_scale, options, workspace, workspace_bytes, stream, &w);
}

kvq_status kvq_paged_prefill_attention(const kvq_cache_desc* desc, void* out, int32_t out_dtype,
                                       const void* query, const int32_t* cu_seqlens_q, int32_t num_seqs,
                                       int32_t num_q_heads, int32_t max_q_len,
                                       const uint8_t* k_codes, const float* k_meta,
                                       const uint8_t* v_codes, const float* v_meta,
                                       const int32_t* block_tables, const int32_t* block_tables_headwise,
                                       int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                       int32_t max_seq_len, const int32_t* window, int32_t sink_size,
                                       float softmax_scale, void* workspace, size_t workspace_bytes,
                                       void* stream) {
  kvq_status st = check_prefill_sizes(desc, num_seqs, num_q_heads, max_q_len, max_seq_len);
  if (st != KVQ_OK) return st;
  const int group = num_q_heads / desc->num_kv_heads;
  if (out_dtype != KVQ_OUT_F32 && out_dtype != KVQ_OUT_BF16)
    return fail(KVQ_EINVAL, "out_dtype %d is not a kvq_out_dtype", out_dtype);
  if ((block_tables == nullptr) == (block_tables_headwise == nullptr))
    return fail(KVQ_EINVAL, "exactly one of block_tables and block_tables_headwise must be non-NULL");
  if (max_blocks_per_seq < 1) return fail(KVQ_EINVAL, "max_blocks_per_seq %d < 1", max_blocks_per_seq);
  if ((int64_t)max_seq_len > (int64_t)max_blocks_per_seq * desc->block_size)
    return fail(KVQ_EINVAL, "max_seq_len %d exceeds max_blocks_per_seq*block_size = %lld", max_seq_len,
                (long long)max_blocks_per_seq * desc->block_size);
  if (!std::isfinite(softmax_scale)) return fail(KVQ_EINVAL, "softmax_scale is not finite");
  // no shape this library builds needs a prefill workspace (the size query
  // returns 0), so any workspace, NULL included, is enough
  (void)workspace;
  (void)workspace_bytes;
  if (num_seqs == 0 || max_q_len == 0) return ok();
  if (!out || !query || !cu_seqlens_q || !seq_lens)
    return fail(KVQ_EINVAL, "out, query, cu_seqlens_q or seq_lens is NULL");
  st = check_planes(desc->mode, k_codes, k_meta, v_codes, v_meta);
  if (st != KVQ_OK) return st;
  resolve_planes(desc, k_codes, k_meta, v_codes, v_meta);
  st = check_channel(desc);
  if (st != KVQ_OK) return st;
  const int tq = 128 / group;
  const long long n_qtiles = ((long long)max_q_len + tq - 1) / tq;
  const long long n_work = n_qtiles * desc->num_kv_heads * (long long)num_seqs;
  kvq::PrefillParams p{};
  p.k_codes = k_codes;
  p.k_meta = k_meta;
  p.v_codes = v_codes;
  p.v_meta = v_meta;
  p.q = static_cast<const uint16_t*>(query);
  p.out = out;
  p.cu_q = cu_seqlens_q;
  p.seq_lens = seq_lens;
  p.headwise = block_tables_headwise != nullptr;
  p.tables = p.headwise ? block_tables_headwise : block_tables;
  p.window = window;
  p.signs = desc->rot_signs;
  p.chs = desc->channel_scales;
  p.qscale = softmax_scale * 1.4426950408889634f;
  p.inv_sqrt_d = inv_sqrt_f32(desc->head_dim);
  p.num_blocks = desc->num_blocks;
  p.max_blocks = max_blocks_per_seq;
  p.max_seq_len = max_seq_len;
  p.sink = sink_size > 0 ? sink_size : 0;
  p.block_size_log2 = __builtin_ctz((unsigned)desc->block_size);
  p.hq = num_q_heads;
  p.hkv = desc->num_kv_heads;
  p.group = group;
  p.tq = tq;
  p.n_qtiles = (int)n_qtiles;
  p.n_work = (int)n_work;
  p.out_bf16 = out_dtype == KVQ_OUT_BF16;
  hipError_t e = kvq::launch_prefill(desc->mode, desc->head_dim, desc->rot_signs != nullptr, p,
                                     static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(KVQ_EHIP, "prefill launch: %s", hipGetErrorString(e));
  return ok();
}

kvq_status kvq_prefill_workspace_size(const kvq_cache_desc* desc, int32_t num_seqs, int32_t num_q_heads,
                                      int32_t max_q_len, int32_t max_seq_len, size_t* bytes) {
  kvq_status st = check_prefill_sizes(desc, num_seqs, num_q_heads, max_q_len, max_seq_len);
  if (st != KVQ_OK) return st;
  if (!bytes) return fail(KVQ_EINVAL, "bytes is NULL");
  *bytes = 0;
  return ok();
}

kvq_status kvq_gather_dequant(const kvq_cache_desc* desc, void* key_out, void* value_out, int32_t out_dtype,
                              const uint8_t* k_codes, const float* k_meta, const uint8_t* v_codes,
                              const float* v_meta, const int32_t* block_tables,
                              const int32_t* block_tables_headwise, int32_t max_blocks_per_seq,
                              const int32_t* cu_seq_lens, int32_t num_seqs, int32_t total_tokens,
                              int32_t max_seq_len, void* stream) {
  kvq_status st = check_desc(desc);
  if (st != KVQ_OK) return st;
  if (num_seqs < 0) return fail(KVQ_EINVAL, "num_seqs %d < 0", num_seqs);
  if (num_seqs > 65535) return fail(KVQ_EUNSUPPORTED, "num_seqs %d > 65535", num_seqs);
  if (total_tokens < 0) return fail(KVQ_EINVAL, "total_tokens %d < 0", total_tokens);
  if (max_seq_len < 0) return fail(KVQ_EINVAL, "max_seq_len %d < 0", max_seq_len);
  if (out_dtype != KVQ_OUT_F32 && out_dtype != KVQ_OUT_BF16)
    return fail(KVQ_EINVAL, "out_dtype %d is not a kvq_out_dtype", out_dtype);
  if ((block_tables == nullptr) == (block_tables_headwise == nullptr))
    return fail(KVQ_EINVAL, "exactly one of block_tables and block_tables_headwise must be non-NULL");
  if (max_blocks_per_seq < 1) return fail(KVQ_EINVAL, "max_blocks_per_seq %d < 1", max_blocks_per_seq);
  if ((int64_t)max_seq_len > (int64_t)max_blocks_per_seq * desc->block_size)
    return fail(KVQ_EINVAL, "max_seq_len %d exceeds max_blocks_per_seq*block_size = %lld", max_seq_len,
                (long long)max_blocks_per_seq * desc->block_size);
  const long long gx = ((long long)max_seq_len * desc->num_kv_heads * 2 +
                        kvq::gather_rows_per_workgroup(desc->head_dim) - 1) /
                       kvq::gather_rows_per_workgroup(desc->head_dim);
  if (gx > 0x7fffffffLL) return fail(KVQ_EUNSUPPORTED, "gather grid of %lld workgroups per sequence", gx);
  if ((long long)total_tokens * desc->num_kv_heads > 0x7fffffffLL)
    return fail(KVQ_EUNSUPPORTED, "outputs of %lld rows are too large (total_tokens*num_kv_heads must stay below "
                "2^31)", (long long)total_tokens);
  if ((long long)max_blocks_per_seq * desc->block_size * desc->num_kv_heads * 2 > 0x7fffffffLL ||
      (long long)num_seqs * desc->num_kv_heads * max_blocks_per_seq > 0x7fffffffLL)
    return fail(KVQ_EUNSUPPORTED, "block tables of %d x %d entries are too large for one gather", num_seqs,
                max_blocks_per_seq);
  if (num_seqs == 0 || total_tokens == 0 || max_seq_len == 0) return ok();
  if (!key_out || !value_out || !cu_seq_lens) return fail(KVQ_EINVAL, "key_out, value_out or cu_seq_lens is NULL");
  if (!aligned(key_out, 16) || !aligned(value_out, 16))
    return fail(KVQ_EINVAL, "key_out and value_out must be 16-byte aligned");
  st = check_planes(desc->mode, k_codes, k_meta, v_codes, v_meta);
  if (st != KVQ_OK) return st;
  resolve_planes(desc, k_codes, k_meta, v_codes, v_meta);
  st = check_channel(desc);
  if (st != KVQ_OK) return st;
  kvq::GatherParams p{};
  p.k_codes = k_codes;
  p.k_meta = k_meta;
  p.v_codes = v_codes;
  p.v_meta = v_meta;
  p.k_out = key_out;
  p.v_out = value_out;
  p.headwise = block_tables_headwise != nullptr;
  p.tables = p.headwise ? block_tables_headwise : block_tables;
  p.cu = cu_seq_lens;
  p.signs = desc->rot_signs;
  p.chs = desc->channel_scales;
  p.num_blocks = desc->num_blocks;
  p.inv_sqrt_d = inv_sqrt_f32(desc->head_dim);
  p.max_blocks = max_blocks_per_seq;
  p.block_size_log2 = __builtin_ctz((unsigned)desc->block_size);
  p.hkv = desc->num_kv_heads;
  p.num_seqs = num_seqs;
  p.max_seq_len = max_seq_len;
  p.total_tokens = total_tokens;
  p.out_bf16 = out_dtype == KVQ_OUT_BF16;
  hipError_t e = kvq::launch_gather(desc->mode, desc->head_dim, desc->rot_signs != nullptr, p,
                                    static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(KVQ_EHIP, "gather launch: %s", hipGetErrorString(e));
  return ok();
}

const char* kvq_last_error(void) { return g_err; }

int32_t kvq_version(void) { return 100; }

}  // extern "C"
