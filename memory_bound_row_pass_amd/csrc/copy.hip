// Plain streaming copy: the bandwidth ceiling the row kernels are compared
// with, and the known-size reference for scaling hardware byte counters.
// 16-byte non-temporal loads and stores, four chunks per lane per iteration,
// grid-stride over the buffer; a byte loop covers unaligned ends.
#include "fr_device.hpp"
#include "fr_kernels.hpp"

namespace fr {

__global__ __launch_bounds__(256) void stream_copy_kernel(const u32x4* __restrict__ src,
                                                          u32x4* __restrict__ dst, int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a = __builtin_nontemporal_load(src + i);
    const u32x4 b = __builtin_nontemporal_load(src + i + stride);
    const u32x4 c = __builtin_nontemporal_load(src + i + 2 * stride);
    const u32x4 d = __builtin_nontemporal_load(src + i + 3 * stride);
    __builtin_nontemporal_store(a, dst + i);
    __builtin_nontemporal_store(b, dst + i + stride);
    __builtin_nontemporal_store(c, dst + i + 2 * stride);
    __builtin_nontemporal_store(d, dst + i + 3 * stride);
  }
  for (; i < n16; i += stride) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

__global__ __launch_bounds__(256) void byte_copy_kernel(const uint8_t* src, uint8_t* dst, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) dst[i] = src[i];
}

hipError_t launch_stream_copy(const void* src, void* dst, int64_t bytes, hipStream_t s) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(src), b = reinterpret_cast<uintptr_t>(dst);
  if (a % 16 == 0 && b % 16 == 0 && bytes % 16 == 0) {
    const int64_t n16 = bytes / 16;
    // 256 CUs x 8 workgroups of 256 lanes, each lane moving 64 B per iteration
    int64_t blocks = (n16 + 1023) / 1024;
    blocks = blocks < 2048 ? blocks : 2048;
    blocks = blocks > 0 ? blocks : 1;
    return launch_kernel(&stream_copy_kernel, dim3((unsigned)blocks), dim3(256), s,
                         static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), n16);
  } else {
    int64_t blocks = (bytes + 255) / 256;
    blocks = blocks < 4096 ? blocks : 4096;
    return launch_kernel(&byte_copy_kernel, dim3((unsigned)blocks), dim3(256), s,
                         static_cast<const uint8_t*>(src), static_cast<uint8_t*>(dst), bytes);
  }
}

}  // namespace fr
