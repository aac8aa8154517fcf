// HBM read ceiling probe: a plain streaming read of a buffer with 16-byte loads, the measured
// bound the layer kernels' bandwidth is compared with (besides the 8 TB/s published peak).  Each
// lane folds what it reads into one word so that no load is dropped; block b writes its word to
// out[b].  Not a step of the method.
#include "moe_device.h"
#include "moe_launch.h"

namespace moe {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr int PROBE_THREADS = 256;
constexpr int PROBE_UNROLL = 8;

__global__ void __launch_bounds__(PROBE_THREADS) k_read_probe(const u32x4* __restrict__ buf, size_t n16,
                                                              uint32_t* __restrict__ out) {
  uint32_t acc = 0;
  const size_t stride = (size_t)gridDim.x * PROBE_THREADS;
  size_t i = (size_t)blockIdx.x * PROBE_THREADS + threadIdx.x;
  for (; i + (PROBE_UNROLL - 1) * stride < n16; i += PROBE_UNROLL * stride) {
    u32x4 v[PROBE_UNROLL];
#pragma unroll
    for (int u = 0; u < PROBE_UNROLL; ++u) v[u] = __builtin_nontemporal_load(buf + i + u * stride);
#pragma unroll
    for (int u = 0; u < PROBE_UNROLL; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const u32x4 v = buf[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc ^= __shfl_xor(acc, off);
  __shared__ uint32_t part[PROBE_THREADS / WAVE];
  if (threadIdx.x % WAVE == 0) part[threadIdx.x / WAVE] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
    for (int w = 0; w < PROBE_THREADS / WAVE; ++w) r ^= part[w];
    out[blockIdx.x] = r;
  }
}

}  // namespace

hipError_t launch_read_probe(hipStream_t s, const void* buf, size_t bytes, uint32_t* out) {
  return launch(k_read_probe, dim3(MOE_READ_PROBE_BLOCKS), dim3(PROBE_THREADS), 0, s, (const u32x4*)buf, bytes / 16, out);
}

}  // namespace moe
