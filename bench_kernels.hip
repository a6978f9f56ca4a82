// Bandwidth diagnostics of the benchmark (not part of libpkv): a plain
// streaming read (non-temporal loads) and a plain copy of a contiguous buffer
// on gfx950, 16-byte accesses, grid-stride.  The read gives the achievable
// HBM read bandwidth of the device the decode is measured on; the copy, a
// transfer of known size for scaling the hardware byte counters.  Built by
// bench.build_bench_kernels() into libpkv_bench.so beside this file.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace {

typedef uint32_t u4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;
constexpr int kUnroll = 8;

__global__ __launch_bounds__(kThreads) void stream_read_kernel(const u4 *src, size_t n16,
                                                               uint32_t *sink) {
  const size_t stride = (size_t)gridDim.x * kThreads;
  size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
  u4 acc = u4{0, 0, 0, 0};
  for (; i + (kUnroll - 1) * stride < n16; i += kUnroll * stride) {
    u4 v[kUnroll];
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) v[k] = __builtin_nontemporal_load(src + i + k * stride);
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) acc ^= v[k];
  }
  for (; i < n16; i += stride) acc ^= __builtin_nontemporal_load(src + i);
  const uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  if (x == 0x9E3779B9u) sink[blockIdx.x] = x;   // keeps the loads live
}

// NT: non-temporal loads and stores (the decode kernel reads K/V that way).
template <bool NT>
__global__ __launch_bounds__(kThreads) void stream_copy_kernel(u4 *dst, const u4 *src,
                                                               size_t n16) {
  const size_t stride = (size_t)gridDim.x * kThreads;
  size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
  for (; i + (kUnroll - 1) * stride < n16; i += kUnroll * stride) {
    u4 v[kUnroll];
#pragma unroll
    for (int k = 0; k < kUnroll; ++k)
      v[k] = NT ? __builtin_nontemporal_load(src + i + k * stride) : src[i + k * stride];
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) {
      if (NT) __builtin_nontemporal_store(v[k], dst + i + k * stride);
      else dst[i + k * stride] = v[k];
    }
  }
  for (; i < n16; i += stride) dst[i] = src[i];
}

bool ok_args(const void *p, size_t bytes, int32_t workgroups) {
  return p && bytes % 16 == 0 && ((uintptr_t)p % 16) == 0 && workgroups > 0;
}

}  // namespace

extern "C" {

// 0 on success, -1 for bad arguments, -5 for a launch failure.
int bench_stream_read(const void *src, size_t bytes, uint32_t *sink, int32_t workgroups,
                      void *stream) {
  if (bytes == 0) return 0;
  if (!ok_args(src, bytes, workgroups) || !sink) return -1;
  hipLaunchKernelGGL(stream_read_kernel, dim3(workgroups), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u4 *>(src), bytes / 16,
                     sink);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

int bench_stream_copy(void *dst, const void *src, size_t bytes, int32_t workgroups,
                      int32_t nontemporal, void *stream) {
  if (bytes == 0) return 0;
  if (!ok_args(src, bytes, workgroups) || !ok_args(dst, bytes, workgroups)) return -1;
  if (nontemporal)
    hipLaunchKernelGGL(stream_copy_kernel<true>, dim3(workgroups), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), static_cast<u4 *>(dst),
                       static_cast<const u4 *>(src), bytes / 16);
  else
    hipLaunchKernelGGL(stream_copy_kernel<false>, dim3(workgroups), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), static_cast<u4 *>(dst),
                       static_cast<const u4 *>(src), bytes / 16);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

}  // extern "C"
