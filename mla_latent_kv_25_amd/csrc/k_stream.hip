// Read-only streaming kernel: the measured HBM read ceiling that the latent-cache read of the
// attention kernels is compared with. Workgroup k reads the k-th contiguous chunk of the buffer;
// each thread keeps sixteen independent 16-byte loads in flight per step and folds every loaded
// word into an XOR, so no load can be removed; one 32-bit word per workgroup leaves the kernel.
// (Contiguous chunks per workgroup streamed 6.1-6.3 TB/s on a 1 GiB buffer, a grid-stride loop
// over the whole buffer 5.1-5.7 TB/s.)
#include "common.hpp"
#include "launch.hpp"

namespace mla {

constexpr int STREAM_UNROLL = 16;

__global__ __launch_bounds__(256) void k_stream_read(const u32x4* __restrict__ src, int64_t n16,
                                                     uint32_t* __restrict__ sink) {
  const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const int64_t c0 = (int64_t)blockIdx.x * per;
  const int64_t c1 = c0 + per < n16 ? c0 + per : n16;
  int64_t i = c0 + threadIdx.x;
  uint32_t acc = 0;
  // full steps: STREAM_UNROLL loads per thread, all issued before any is used
  for (; i + (STREAM_UNROLL - 1) * 256 < c1; i += STREAM_UNROLL * 256) {
    u32x4 v[STREAM_UNROLL];
#pragma unroll
    for (int u = 0; u < STREAM_UNROLL; ++u) v[u] = src[i + u * 256];
#pragma unroll
    for (int u = 0; u < STREAM_UNROLL; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < c1; i += 256) {
    const u32x4 v = src[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o, 64);
  __shared__ uint32_t red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

int stream_read_grid(int64_t n16) {
  const int64_t per_block = 256LL * STREAM_UNROLL;
  int64_t g = (n16 + per_block - 1) / per_block;
  const int64_t cap = (int64_t)device_cu_count() * 16;
  if (g > cap) g = cap;
  if (g > MLA_STREAM_SINK_WORDS) g = MLA_STREAM_SINK_WORDS;
  return g < 1 ? 1 : (int)g;
}

hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t st) {
  const int64_t n16 = (int64_t)(bytes / 16);
  const int g = stream_read_grid(n16);
  hipLaunchKernelGGL(k_stream_read, dim3(g), dim3(256), 0, st, (const u32x4*)src, n16, sink);
  return hipGetLastError();
}

}  // namespace mla
