// Quantize-on-write: bf16 K/V rows -> (optional) Hadamard rotation ->
// per-(token, kv head) scale and zero point -> round -> pack -> paged store.
//
// Follows the write half of the prhub summary of vLLM PR 40835 ("INT4
// per-token-head KV cache quantization for the Triton backend", 实现拆解
// item 2: the write kernel applies the randomized Hadamard transform, computes
// one scale and zero point per token and head, and packs nibbles) and the
// encoder/decoder cache-write kernels of FastDeploy PR 5173 ("support dynamic
// int2 quantization cache kv").  The arithmetic is the float32 sequence the
// cache format defines, so codes are reproducible bit for bit:
//   y = fl(FWHT(d .* x) * fl(1/sqrt(D)))   stages h = 1, 2, 4, ..., D/2
//   INT8: s = max|y| / 127,            c = clamp(rint(y * (1/s)), -127, 127)
//   INT4/INT2: s = (max y - min y) / L, z = min y,
//              c = clamp(rint((y - z) * (1/s)), 0, L)
// with correctly rounded divisions and no fused multiply-adds.
//
// Work split: one row = one (token, kv head) of K or of V.  D/EPL lanes own a
// row, EPL = 32 elements per lane with the rotation and 16 without (four or
// two 16-byte loads), so a wave64 handles 64 EPL / D rows at once; each lane
// group takes two (rotated) or four rows, their slots and loads all requested
// before the first is used.  The FWHT runs in registers for the in-lane
// stages (h < EPL) and across lanes for the rest; min/max/absmax are lane
// reductions.  Long lane slices (against the fused decode step's eight
// elements) cut the per-row work each element carries: the cross-lane
// reduction stages, the scale and zero divisions and the address math.
// Stores are the lane's slice of the packed row (EPL bytes for INT8 and FP8,
// EPL/2 for INT4, EPL/4 for INT2) plus one meta store per row.
#pragma clang fp contract(off)

#include "kvq_internal.h"
#include "kvq_write_row.h"

namespace kvq {
namespace {

// Elements per lane: 32 with the rotation (its butterfly stages and the
// per-row statistics make the kernel VALU-bound, and longer lane slices
// carry less per-row work per element), 16 without (the 8-bit modes then
// stream faster with more, shorter rows in flight).
template <bool ROT>
constexpr int write_epl() { return ROT ? 32 : 16; }
// rows per lane group, their loads in flight together (64 bytes a lane)
template <bool ROT>
constexpr int write_iter() { return ROT ? 2 : 4; }
constexpr int kChanInvMax = 4096;   // per-channel reciprocals a workgroup keeps in LDS (2 Hkv D)

template <int MODE, int D, bool ROT>
__global__ __launch_bounds__(256) void write_kernel(WriteParams p) {
  constexpr int EPL = write_epl<ROT>();
  constexpr int kWriteIter = write_iter<ROT>();
  constexpr int LPR = D / EPL;           // lanes per row
  constexpr int RPW = 64 / LPR;          // rows per wave
  constexpr int RPB = 4 * RPW;           // rows per workgroup and iteration

  const int lane = threadIdx.x & 63;
  const int lr = lane & (LPR - 1);
  // rows, tokens and slot-map indices stay below 2^31 (checked on the host)
  const int row0 = blockIdx.x * RPB * kWriteIter + (threadIdx.x >> 6) * RPW + lane / LPR;
  const int hkv = p.hkv;

  float sg[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) sg[i] = 1.0f;
  if constexpr (ROT) write_row_signs_n<EPL>(p, lr, sg);
  // per-channel INT8: the workgroup's rows span all (K or V, kv head)
  // channels, so their correctly rounded reciprocals are computed once into
  // LDS (when they fit) instead of once per row
  const float* chinv = nullptr;
  if constexpr (MODE == kChannelMode) {
    __shared__ __align__(16) float inv_lds[kChanInvMax];
    const int n = 2 * hkv * D;
    if (n <= kChanInvMax) {
      for (int i = threadIdx.x; i < n; i += 256) {
        const float s = p.chs[i];
        inv_lds[i] = s >= 1.17549435e-38f ? 1.0f / s : 0.0f;
      }
      __syncthreads();
      chinv = inv_lds;
    }
  }
  int64_t slot[kWriteIter];
  uint4 raw[kWriteIter][EPL / 8];
  int hs[kWriteIter];
  bool ins[kWriteIter];
  // row = t * 2 Hkv + 2 h + kv: one division for the first row, then steps
  // of RPB rows
  int t = row0 / (2 * hkv);
  int rem = row0 - t * 2 * hkv;
#pragma unroll
  for (int it = 0; it < kWriteIter; ++it) {
    const int row = row0 + it * RPB;
    if (it > 0) {
      rem += RPB;
      while (rem >= 2 * hkv) {
        rem -= 2 * hkv;
        ++t;
      }
    }
    const int h = rem >> 1;
    // a row past the end reads token 0's row and slot (always present, as a
    // launch has rows) and stores nothing: no branch, no zeroing of its
    // registers
    const bool in = row < p.total_rows;
    const int tc = in ? t : 0, hc = in ? h : 0;
    hs[it] = in ? rem : (rem & 1);
    ins[it] = in;
    slot[it] = p.slot_hw ? p.slot_hw[tc * hkv + hc] : p.slot[tc];
    write_row_load_n<D, EPL>(p, tc, hc, rem & 1, lr, raw[it]);
  }
#pragma unroll
  for (int it = 0; it < kWriteIter; ++it)
    write_row_store_n<MODE, D, ROT, true, EPL>(p, raw[it], sg, hs[it] >> 1, hs[it] & 1, ins[it] ? slot[it] : -1, lr,
                                               chinv);
}

// Per-channel scales of a first batch (dynamic per-channel INT8, the
// vllm-ascend-quantized-kv-cache package, 运行机制): workgroup (kv, h)
// reduces max_t |x[t, h, d]| over the tokens for every channel d, then
// divides by 127 (correctly rounded).  Thread i takes channel i % D and
// tokens i / D, i / D + 256 / D, ...; the partial maxima meet in LDS.  The
// maximum of absolute values is exact and order-free.
template <int D>
__global__ __launch_bounds__(256) void calibrate_kernel(WriteParams p, int32_t num_tokens, float* out) {
  constexpr int TPS = 256 / D;             // token lanes per channel
  __shared__ float part[TPS][D];
  const int kv = blockIdx.x & 1, h = blockIdx.x >> 1;
  const int d = threadIdx.x % D, t0 = threadIdx.x / D;
  const uint16_t* src = kv ? p.value : p.key;
  const int64_t stride = kv ? p.value_stride : p.key_stride;
  float m = 0.0f;
  for (int64_t t = t0; t < num_tokens; t += TPS) {
    const uint16_t raw = src[t * stride + (int64_t)h * D + d];
    m = fmaxf(m, fabsf(__uint_as_float((uint32_t)raw << 16)));
  }
  part[t0][d] = m;
  __syncthreads();
  if (t0 == 0) {
#pragma unroll
    for (int i = 1; i < TPS; ++i) m = fmaxf(m, part[i][d]);
    out[((int64_t)kv * p.hkv + h) * D + d] = m / 127.0f;
  }
}

__global__ __launch_bounds__(256) void fill_zero_kernel(uint4* p, size_t n16) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = make_uint4(0, 0, 0, 0);
}

template <int MODE, int D, bool ROT>
hipError_t launch_write_t(const WriteParams& p, hipStream_t s) {
  constexpr int RPB = 4 * (64 / (D / write_epl<ROT>())) * write_iter<ROT>();
  const int64_t blocks = (p.total_rows + RPB - 1) / RPB;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((write_kernel<MODE, D, ROT>), dim3((unsigned)blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

template <int MODE>
hipError_t launch_write_m(int d, bool rot, const WriteParams& p, hipStream_t s) {
  if constexpr (MODE == kChannelMode) {   // no rotation in this mode (checked on the host)
    return d == 64 ? launch_write_t<MODE, 64, false>(p, s) : launch_write_t<MODE, 128, false>(p, s);
  } else {
    if (d == 64) return rot ? launch_write_t<MODE, 64, true>(p, s) : launch_write_t<MODE, 64, false>(p, s);
    return rot ? launch_write_t<MODE, 128, true>(p, s) : launch_write_t<MODE, 128, false>(p, s);
  }
}

}  // namespace

hipError_t launch_write(int mode, int d, bool rot, const WriteParams& p, hipStream_t s) {
  switch (mode) {
    case 0: return launch_write_m<0>(d, rot, p, s);
    case 1: return launch_write_m<1>(d, rot, p, s);
    case 2: return launch_write_m<2>(d, rot, p, s);
    case kChannelMode: return launch_write_m<kChannelMode>(d, rot, p, s);
    case kFp8Mode: return launch_write_m<kFp8Mode>(d, rot, p, s);
    default: return launch_write_m<kInlineMode>(d, rot, p, s);
  }
}

hipError_t launch_calibrate(int d, const WriteParams& p, int32_t num_tokens, float* out, hipStream_t s) {
  const dim3 grid((unsigned)(2 * p.hkv));
  if (d == 64) hipLaunchKernelGGL(calibrate_kernel<64>, grid, dim3(256), 0, s, p, num_tokens, out);
  else hipLaunchKernelGGL(calibrate_kernel<128>, grid, dim3(256), 0, s, p, num_tokens, out);
  return hipGetLastError();
}

hipError_t launch_fill_zero(void* ptr, size_t bytes, hipStream_t s) {
  const size_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  const size_t blocks = n16 / 256 + 1 < 4096 ? n16 / 256 + 1 : 4096;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                     reinterpret_cast<uint4*>(ptr), n16);
  return hipGetLastError();
}

}  // namespace kvq
