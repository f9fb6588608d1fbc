// Streaming-read ceiling: what one plain kernel reads per second on this GPU, so that every
// kernel's HBM fraction can be stated against a measured ceiling as well as the published peak.
// Each lane issues 8 nontemporal 16-byte loads per iteration over a grid-stride sweep (a wave
// reads 1 KB of contiguous memory per load instruction); the data are folded into one word that
// is stored only if it equals a marker, so the loads cannot be dropped and nothing else is written.
#include "common.h"
#include "kernels.h"

namespace medusa {

typedef unsigned u32x4_nt __attribute__((ext_vector_type(4)));

constexpr int kReadUnroll = 8;
constexpr unsigned kReadGrid = 4096;

__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4_nt* __restrict__ p, long n16,
                                                          uint32_t* __restrict__ sink) {
  uint32_t acc = 0;
  const long stride = static_cast<long>(gridDim.x) * 256 * kReadUnroll;
  long i = static_cast<long>(blockIdx.x) * 256 * kReadUnroll + threadIdx.x;
  for (; i + 256 * (kReadUnroll - 1) < n16; i += stride) {
    u32x4_nt v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) v[u] = __builtin_nontemporal_load(p + i + u * 256);
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += 256) acc ^= p[i].x;         // ragged tail of the last sweep
  if (acc == 0x9e3779b9u) sink[0] = acc;
}

hipError_t launch_stream_read(const void* buf, long n16, uint32_t* sink, hipStream_t s) {
  stream_read_kernel<<<kReadGrid, 256, 0, s>>>(static_cast<const u32x4_nt*>(buf), n16, sink);
  return hipGetLastError();
}

}  // namespace medusa
