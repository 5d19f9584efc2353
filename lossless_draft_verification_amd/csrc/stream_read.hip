// stream_read.hip - the attainable read bandwidth of one MI355X, measured
// with the same access pattern as the row-statistics pass: each workgroup
// streams a contiguous share of a buffer with 16-byte nontemporal loads
// (consecutive lanes on consecutive 16-byte pieces, four loads per thread in
// flight) and folds them with XOR, the cheapest fold that keeps every load
// live; one word per workgroup is written so that nothing is optimised
// away.  It verifies nothing: it is the ceiling the verification kernels'
// bandwidth is quoted against.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "specverify.h"

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kThreads) void stream_read_kernel(const u32x4* src, int64_t n16, int64_t per_wg,
                                                              uint32_t* sink) {
  const int64_t lo = (int64_t)blockIdx.x * per_wg;
  const int64_t hi = lo + per_wg < n16 ? lo + per_wg : n16;
  u32x4 acc = {0u, 0u, 0u, 0u};
  int64_t i = lo + threadIdx.x;
  // whole steps: kUnroll loads per thread issued together
  for (; i + (kUnroll - 1) * kThreads < hi; i += kUnroll * kThreads) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * kThreads);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u];
  }
  for (; i < hi; i += kThreads) acc ^= __builtin_nontemporal_load(src + i);
  uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
  for (int o = 32; o > 0; o >>= 1) x ^= __shfl_xor(x, o, 64);
  __shared__ uint32_t red[kThreads / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

}  // namespace

extern "C" sv_status sv_stream_read(const void* src, size_t bytes, uint32_t* sink, int32_t workgroups, void* stream) {
  if (src == nullptr || sink == nullptr || workgroups < 1 || bytes < 16 || (bytes & 15) != 0 ||
      ((uintptr_t)src & 15u) != 0)
    return SV_ERR_INVALID_ARGUMENT;
  const int64_t n16 = (int64_t)(bytes / 16);
  const int64_t per_wg = (n16 + workgroups - 1) / workgroups;
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)workgroups), dim3(kThreads), 0, (hipStream_t)stream,
                     (const u32x4*)src, n16, per_wg, sink);
  return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_LAUNCH;
}
