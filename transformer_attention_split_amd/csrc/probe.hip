// Streaming-read probe: the attainable HBM read bandwidth, the context in
// which the decode kernels' bandwidth is read (their own peak fraction is
// taken against the published 8 TB/s). Not part of the attention path.
//
// Workgroup w reads the 16-byte words [w*per, min((w+1)*per, n16)) of src
// (per = ceil(n16 / workgroups)), eight 16-byte non-temporal loads in flight
// per thread, and writes the XOR of its words to sink[w] (so that no load
// can be dropped; an empty range writes zero).
#include "launch.h"

namespace attn {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 8;

__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(
    const u32x4_t *__restrict__ src, size_t n16, size_t per,
    u32x4_t *__restrict__ sink) {
  const size_t begin = (size_t)blockIdx.x * per;
  const size_t end = begin + per < n16 ? begin + per : n16;
  u32x4_t acc = {0u, 0u, 0u, 0u};
  for (size_t i = begin + threadIdx.x; i < end;
       i += (size_t)kProbeThreads * kProbeUnroll) {
    u32x4_t v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) {
      const size_t j = i + (size_t)u * kProbeThreads;
      v[u] = j < end ? __builtin_nontemporal_load(src + j) : u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u];
  }
  __shared__ u32x4_t red[kProbeThreads];
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int s = kProbeThreads / 2; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) red[threadIdx.x] ^= red[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) sink[blockIdx.x] = red[0];
}

}  // namespace

hipError_t launch_read_probe(const void *src, size_t n16, void *sink,
                             int workgroups, hipStream_t stream) {
  const size_t per = (n16 + (size_t)workgroups - 1) / (size_t)workgroups;
  read_probe_kernel<<<dim3((unsigned)workgroups), kProbeThreads, 0, stream>>>(
      static_cast<const u32x4_t *>(src), n16, per, static_cast<u32x4_t *>(sink));
  return hipGetLastError();
}

}  // namespace attn
