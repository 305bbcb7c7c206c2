// Streaming-read probe for MI355X HBM: the rate a plain read of a large
// buffer reaches, as the achievable ceiling beside the 8 TB/s peak when the
// decode kernels' read rate is reported.  It is a measuring instrument, not
// part of the decode path, and lives in its own library.
//
// Every lane reads 16-byte words with non-temporal loads, several in flight,
// and folds them into one word; the word is stored only when it equals a key
// the caller picks so that it never matches, which keeps the loads from being
// removed without writing anything.  Two access patterns:
//   mode 0  grid-stride, 8 loads in flight per lane: one pass of the whole
//           grid covers a contiguous span;
//   mode 1, 2, 3  chunked, 8, 16 or 32 loads in flight per lane: workgroup b
//           streams its own contiguous range, 4 KB blocks in order (the
//           pattern of a decode workgroup walking its share of the cache).
#include <hip/hip_runtime.h>

#include <stddef.h>
#include <stdint.h>

namespace {

typedef uint32_t uint4_t __attribute__((ext_vector_type(4)));

constexpr int kBlock = 256;
constexpr int kInFlight = 8;                      // grid-stride pattern

__global__ __launch_bounds__(kBlock) void read_probe_kernel(const uint4_t* p, size_t n16,
                                                            uint32_t key, uint32_t* sink) {
  const size_t stride = (size_t)gridDim.x * kBlock;
  size_t i = (size_t)blockIdx.x * kBlock + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kInFlight - 1) * stride < n16; i += kInFlight * stride) {
    uint4_t v[kInFlight];
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const uint4_t v = __builtin_nontemporal_load(p + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == key) sink[(size_t)blockIdx.x * kBlock + threadIdx.x] = acc;
}

template <int U>
__global__ __launch_bounds__(kBlock) void read_probe_chunked_kernel(const uint4_t* p, size_t n16,
                                                                    size_t chunk, uint32_t key,
                                                                    uint32_t* sink) {
  const size_t begin = (size_t)blockIdx.x * chunk;
  const size_t end = begin + chunk < n16 ? begin + chunk : n16;
  size_t i = begin + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (U - 1) * kBlock < end; i += U * kBlock) {
    uint4_t v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(p + i + u * kBlock);
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < end; i += kBlock) {
    const uint4_t v = __builtin_nontemporal_load(p + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == key) sink[(size_t)blockIdx.x * kBlock + threadIdx.x] = acc;
}

}  // namespace

extern "C" {

// Read `bytes` (a multiple of 16) from the 16-byte aligned device buffer
// `buf` once, with `grid` workgroups of 256 lanes in access pattern `mode`
// (0 to 3, above), on `stream`.  `sink` is a device buffer of grid * 256
// uint32 that a lane writes only when its fold equals `key`.  Returns 0, 1
// for invalid arguments, 2 for a failed launch.
int hbm_read_probe(const void* buf, size_t bytes, uint32_t key, void* sink, int grid, int mode,
                   void* stream) {
  if (!buf || !sink || grid <= 0 || bytes % 16 != 0 || mode < 0 || mode > 3 ||
      (reinterpret_cast<uintptr_t>(buf) & 15) != 0)
    return 1;
  const size_t n16 = bytes / 16;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const uint4_t* p = static_cast<const uint4_t*>(buf);
  uint32_t* out = static_cast<uint32_t*>(sink);
  if (mode == 0) {
    hipLaunchKernelGGL(read_probe_kernel, dim3(grid), dim3(kBlock), 0, st, p, n16, key, out);
  } else {
    // whole 4 KB blocks per workgroup, the last workgroup's range clipped
    const size_t per = (size_t)kBlock;
    const size_t chunk = ((n16 + grid - 1) / grid + per - 1) / per * per;
    if (mode == 1)
      hipLaunchKernelGGL(read_probe_chunked_kernel<8>, dim3(grid), dim3(kBlock), 0, st, p, n16,
                         chunk, key, out);
    else if (mode == 2)
      hipLaunchKernelGGL(read_probe_chunked_kernel<16>, dim3(grid), dim3(kBlock), 0, st, p, n16,
                         chunk, key, out);
    else
      hipLaunchKernelGGL(read_probe_chunked_kernel<32>, dim3(grid), dim3(kBlock), 0, st, p, n16,
                         chunk, key, out);
  }
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
