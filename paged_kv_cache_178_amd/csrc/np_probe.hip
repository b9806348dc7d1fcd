// Reference kernels for the benchmark: the launch floor (an empty kernel) and
// a plain streaming read of a given byte count. They put the decode kernel's
// time next to what any kernel, and any kernel that only reads the same bytes
// once, takes on the same device.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "np_internal.h"

namespace {

__global__ void probe_empty_kernel() {}

// Each thread reads its share of 16-byte chunks (grid-strided, U loads of a
// thread issued before any is used) and writes one word so the loads stay live.
template <int U>
__global__ __launch_bounds__(1024) void probe_stream_read_kernel(const uint4* __restrict__ src,
                                                                 int64_t n16,
                                                                 uint32_t* __restrict__ sink) {
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (U - 1) * stride < n16; i += U * stride) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = src[i + u * stride];
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const uint4 v = src[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  sink[int64_t(blockIdx.x) * blockDim.x + threadIdx.x] = acc;
}

}  // namespace

extern "C" np_status np_probe_empty(void* stream) {
  probe_empty_kernel<<<dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream)>>>();
  return hipGetLastError() == hipSuccess ? NP_OK : NP_ERR_HIP;
}

extern "C" np_status np_probe_stream_read(const void* src, size_t bytes, uint32_t num_wgs,
                                          void* sink, size_t sink_bytes, void* stream) {
  if (src == nullptr || sink == nullptr) return NP_ERR_NULL_PTR;
  if (reinterpret_cast<uintptr_t>(src) % 16 != 0 || bytes % 16 != 0 ||
      reinterpret_cast<uintptr_t>(sink) % 4 != 0)
    return NP_ERR_MISALIGNED;
  if (num_wgs == 0 || num_wgs > (1u << 20)) return NP_ERR_BAD_SHAPE;
  if (sink_bytes < size_t(num_wgs) * 256 * sizeof(uint32_t)) return NP_ERR_WORKSPACE_TOO_SMALL;
  probe_stream_read_kernel<8><<<dim3(num_wgs), dim3(256), 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const uint4*>(src), int64_t(bytes / 16), static_cast<uint32_t*>(sink));
  return hipGetLastError() == hipSuccess ? NP_OK : NP_ERR_HIP;
}

extern "C" np_status np_probe_stream_read_ex(const void* src, size_t bytes, uint32_t num_wgs,
                                             uint32_t wg_size, uint32_t loads_per_thread,
                                             void* sink, size_t sink_bytes, void* stream) {
  if (src == nullptr || sink == nullptr) return NP_ERR_NULL_PTR;
  if (reinterpret_cast<uintptr_t>(src) % 16 != 0 || bytes % 16 != 0 ||
      reinterpret_cast<uintptr_t>(sink) % 4 != 0)
    return NP_ERR_MISALIGNED;
  if (num_wgs == 0 || num_wgs > (1u << 20) || wg_size % 64 != 0 || wg_size == 0 ||
      wg_size > 1024)
    return NP_ERR_BAD_SHAPE;
  if (sink_bytes < size_t(num_wgs) * wg_size * sizeof(uint32_t)) return NP_ERR_WORKSPACE_TOO_SMALL;
  const dim3 grid(num_wgs), block(wg_size);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const uint4* s16 = static_cast<const uint4*>(src);
  uint32_t* out = static_cast<uint32_t*>(sink);
  const int64_t n16 = int64_t(bytes / 16);
  switch (loads_per_thread) {
    case 1: probe_stream_read_kernel<1><<<grid, block, 0, st>>>(s16, n16, out); break;
    case 2: probe_stream_read_kernel<2><<<grid, block, 0, st>>>(s16, n16, out); break;
    case 4: probe_stream_read_kernel<4><<<grid, block, 0, st>>>(s16, n16, out); break;
    case 8: probe_stream_read_kernel<8><<<grid, block, 0, st>>>(s16, n16, out); break;
    case 16: probe_stream_read_kernel<16><<<grid, block, 0, st>>>(s16, n16, out); break;
    default: return NP_ERR_UNSUPPORTED;
  }
  return hipGetLastError() == hipSuccess ? NP_OK : NP_ERR_HIP;
}
