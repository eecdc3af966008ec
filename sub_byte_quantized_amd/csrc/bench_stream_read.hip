// A read-only HBM streaming kernel: a measured read ceiling that the
// benchmark reports next to a device copy.  Not part of the cache's C ABI
// (include/kvq.h); built into its own library, libkvq_bench.so.
//
// Every lane issues U 16-byte loads per round before using any of them
// (U * 16 bytes in flight per lane), over a grid-stride loop; the loaded
// words are folded into one value that decides a store that the benchmark's
// fill never triggers, so no load is optimized away.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

template <int U>
__global__ __launch_bounds__(256) void stream_read(const uint4* __restrict__ p, size_t n16, uint32_t key,
                                                   uint32_t* __restrict__ sink) {
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * 256;
  uint32_t acc = 0;
  for (; i + (U - 1) * stride < n16; i += U * stride) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = p[i + u * stride];
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const uint4 v = p[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == key) sink[0] = acc;
}

template <int U>
hipError_t launch(const void* p, size_t n16, uint32_t key, uint32_t* sink, int blocks, hipStream_t s) {
  hipLaunchKernelGGL(stream_read<U>, dim3(blocks), dim3(256), 0, s, static_cast<const uint4*>(p), n16, key, sink);
  return hipGetLastError();
}

}  // namespace

// Read `bytes` (a multiple of 16) from device memory `p` with `blocks`
// 256-thread workgroups and `unroll` (1, 2, 4 or 8) loads in flight per lane;
// `sink` is one device uint32 that is written only when the XOR of all words
// read equals `key`.  Returns 0 or the HIP error; 1 for bad arguments.
extern "C" int kvq_bench_stream_read(const void* p, size_t bytes, uint32_t key, uint32_t* sink, int blocks,
                                     int unroll, void* stream) {
  if (!p || !sink || bytes % 16 != 0 || blocks <= 0) return 1;
  const size_t n16 = bytes / 16;
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (unroll) {
    case 1: return (int)launch<1>(p, n16, key, sink, blocks, s);
    case 2: return (int)launch<2>(p, n16, key, sink, blocks, s);
    case 4: return (int)launch<4>(p, n16, key, sink, blocks, s);
    case 8: return (int)launch<8>(p, n16, key, sink, blocks, s);
    default: return 1;
  }
}
