// gqla_stream_read: the streaming-read rate this GPU reaches with the load form the decodes
// use (non-temporal 128-bit loads that cover whole cache lines), for the roofline context
// of a measurement. It is not part of either decode path.
#include "../../include/gqla.h"
#include "gqla_internal.h"

#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

using f32x4 = float __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kUnroll = 8;   // 16-byte loads in flight per lane

// Each workgroup strides over the buffer in spans of kThreads * kUnroll * 16 bytes (32 KiB),
// every lane issuing its kUnroll loads before it adds any of them. The words are summed as
// fp32 so the loads cannot be dropped; one sum per workgroup is stored.
__global__ __launch_bounds__(kThreads) void stream_read_kernel(const f32x4* __restrict__ src, int64_t n16,
                                                               float* __restrict__ partial) {
  const int64_t span = static_cast<int64_t>(kThreads) * kUnroll;
  const int64_t full = n16 / span;   // whole spans
  float acc = 0.f;
  for (int64_t s = blockIdx.x; s < full; s += gridDim.x) {
    const f32x4* p = src + s * span + threadIdx.x;
    f32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(p + u * kThreads);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      acc += (v[u].x + v[u].y) + (v[u].z + v[u].w);
  }
  // The tail of fewer than one span: workgroup 0 reads it one 16-byte word per lane at a time.
  if (blockIdx.x == 0) {
    for (int64_t i = full * span + threadIdx.x; i < n16; i += kThreads) {
      const f32x4 v = __builtin_nontemporal_load(src + i);
      acc += (v.x + v.y) + (v.z + v.w);
    }
  }
  // Wave sum, then the four waves' sums through LDS.
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) acc += __shfl_xor(acc, o, 64);
  __shared__ float wsum[kThreads / 64];
  if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) partial[blockIdx.x] = (wsum[0] + wsum[1]) + (wsum[2] + wsum[3]);
}

}  // namespace

extern "C" gqla_status gqla_stream_read(const void* src, size_t bytes, float* partial, int32_t num_wgs,
                                        void* stream) {
  if (src == nullptr || partial == nullptr) {
    gqla::set_last_error("gqla_stream_read: NULL pointer");
    return GQLA_ERR_INVALID_ARG;
  }
  if (bytes == 0 || bytes % 16 != 0 || reinterpret_cast<uintptr_t>(src) % 16 != 0) {
    gqla::set_last_error("gqla_stream_read: bytes must be a non-zero multiple of 16 and src 16-byte aligned");
    return GQLA_ERR_INVALID_ARG;
  }
  if (num_wgs < 1 || num_wgs > 65536) {
    gqla::set_last_error("gqla_stream_read: num_wgs must lie in [1, 65536]");
    return GQLA_ERR_INVALID_ARG;
  }
  hipLaunchKernelGGL(stream_read_kernel, dim3(num_wgs), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const f32x4*>(src), static_cast<int64_t>(bytes / 16), partial);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    gqla::set_last_error(hipGetErrorString(e));
    return GQLA_ERR_HIP;
  }
  return GQLA_OK;
}
