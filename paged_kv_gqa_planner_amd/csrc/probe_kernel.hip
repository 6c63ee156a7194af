// Streaming read of one contiguous device buffer: a measurement aid, not a
// step of the attention path. It gives the HBM read rate this chip reaches
// with the simplest access pattern (every byte once, 16-byte loads, whole
// 64-byte segments per quarter wave), which is reported beside the
// published peak when the attention kernels' bandwidth is judged.
#include "device_common.h"

namespace vat {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 4;

// Each lane XORs the words it loads; a lane stores only when its XOR hits a
// fixed value, so the loads cannot be removed and the sink is almost never
// written.
__global__ __launch_bounds__(kProbeThreads) void vat_read_probe_kernel(const u32x4* __restrict__ p,
                                                                       long long n16,
                                                                       unsigned* sink) {
  const long long stride = (long long)gridDim.x * kProbeThreads;
  long long i = (long long)blockIdx.x * kProbeThreads + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + (kProbeUnroll - 1) * stride < n16; i += kProbeUnroll * stride) {
    u32x4 v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u];
  }
  for (; i < n16; i += stride) acc ^= __builtin_nontemporal_load(p + i);
  const unsigned x = acc.x ^ acc.y ^ acc.z ^ acc.w;
  if (x == 0x9e3779b9u) sink[0] = x;
}

const void* read_probe_kernel() { return (const void*)vat_read_probe_kernel; }

}  // namespace vat
