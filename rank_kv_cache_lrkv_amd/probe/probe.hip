// Measurement kernels (include/lrkv_probe.h): a plain read stream, the ceiling
// a kernel reading the decode's bytes from HBM can reach, and a bounded spin that
// keeps the GPU busy while a host loop enqueues the launches it times.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lrkv_probe.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// chunk k (256 * U pieces of 16 bytes) of the sweep is read by workgroup
// k mod gridDim.x; each thread has its U loads of a chunk in flight together
template <int U, bool NT>
__global__ __launch_bounds__(256) void k_read(const u32x4 *__restrict__ src, int64_t n16,
                                              uint32_t *__restrict__ sink) {
  constexpr int64_t kChunk = 256 * U;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int64_t base = int64_t(blockIdx.x) * kChunk; base < n16; base += int64_t(gridDim.x) * kChunk) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = base + u * 256 + threadIdx.x;
      if (i < n16) {
        if constexpr (NT) v[u] = __builtin_nontemporal_load(src + i);
        else v[u] = src[i];
      } else {
        v[u] = u32x4{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u];
  }
  const uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  if (x == 0x9e3779b9u) sink[blockIdx.x] = x;
}

__global__ void k_spin(int64_t ticks, uint32_t *sink) {
  const int64_t t0 = int64_t(wall_clock64());
  int64_t seen = 0;
  while ((seen = int64_t(wall_clock64()) - t0) < ticks) __builtin_amdgcn_s_sleep(8);
  if (threadIdx.x == 0 && seen < 0) sink[0] = 1u;
}

template <int U>
hipError_t launch_read(const void *src, int64_t n16, uint32_t *sink, int grid, bool nt, hipStream_t s) {
  if (nt)
    hipLaunchKernelGGL((k_read<U, true>), dim3(grid), dim3(256), 0, s, static_cast<const u32x4 *>(src), n16, sink);
  else
    hipLaunchKernelGGL((k_read<U, false>), dim3(grid), dim3(256), 0, s, static_cast<const u32x4 *>(src), n16, sink);
  return hipGetLastError();
}

}  // namespace

extern "C" {

int32_t lrkv_probe_read(const void *src, int64_t bytes, uint32_t *sink, int32_t grid, int32_t unroll,
                        int32_t nontemporal, lrkv_stream_t stream) {
  if (!src || !sink) return 1;
  if (bytes <= 0 || bytes % 16 || grid < 1 || grid > 65535) return 2;
  if (unroll != 1 && unroll != 2 && unroll != 4 && unroll != 8) return 2;
  if (reinterpret_cast<uintptr_t>(src) & 15u) return 5;
  const int64_t n16 = bytes / 16;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const bool nt = nontemporal != 0;
  hipError_t e;
  switch (unroll) {
    case 1: e = launch_read<1>(src, n16, sink, grid, nt, s); break;
    case 2: e = launch_read<2>(src, n16, sink, grid, nt, s); break;
    case 4: e = launch_read<4>(src, n16, sink, grid, nt, s); break;
    default: e = launch_read<8>(src, n16, sink, grid, nt, s); break;
  }
  return e == hipSuccess ? 0 : 8;
}

int32_t lrkv_probe_spin(int64_t ticks, uint32_t *sink, lrkv_stream_t stream) {
  if (!sink) return 1;
  if (ticks < 0 || ticks > (int64_t(1) << 32)) return 2;
  hipLaunchKernelGGL(k_spin, dim3(1), dim3(64), 0, reinterpret_cast<hipStream_t>(stream), ticks, sink);
  return hipGetLastError() == hipSuccess ? 0 : 8;
}

int32_t lrkv_probe_wall_clock_khz(void) {
  int dev = 0, khz = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess) return 0;
  return khz;
}

}  // extern "C"
