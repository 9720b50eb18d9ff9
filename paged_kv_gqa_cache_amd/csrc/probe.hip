// Streaming-read probe: reads a device buffer once, as fast as this GPU
// allows, so that the decode kernels' byte rates can be put beside a
// measured read ceiling as well as the published peak.  It carries no part
// of the attention path.
//
// Every thread keeps four 16-byte non-temporal loads in flight per step and
// folds the words it reads into one XOR (so the loads cannot be dropped);
// each workgroup writes one word of `out`.
#include "pkv_common.h"
#include "pkv_launch.h"

namespace pkv {

constexpr int kProbeUnroll = 4;

__global__ __launch_bounds__(256) void read_probe_kernel(const u32x4* __restrict__ src, int64_t n16,
                                                         uint32_t* __restrict__ out) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
  int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kProbeUnroll - 1) * stride < n16; i += kProbeUnroll * stride) {
    u32x4 v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(src + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off);
  __shared__ uint32_t s_acc[4];
  if ((threadIdx.x & 63) == 0) s_acc[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) out[blockIdx.x] = s_acc[0] ^ s_acc[1] ^ s_acc[2] ^ s_acc[3];
}

hipError_t launch_read_probe(const void* src, int64_t bytes, uint32_t* out, int32_t out_words,
                             hipStream_t stream) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  // Two 256-thread workgroups per CU (measured: 6.7-7.0 TB/s; one per CU
  // 6.0-6.3, three 6.8-6.9, four 5.6), at most as many as `out` has words.
  const int grid = std::max(1, std::min(out_words, 2 * cus));
  hipLaunchKernelGGL(read_probe_kernel, dim3(grid), dim3(256), 0, stream, static_cast<const u32x4*>(src), bytes / 16,
                     out);
  return hipGetLastError();
}

}  // namespace pkv
