// Plain streaming copy: the bandwidth ceiling the row kernels are compared
// with, and the known-size reference for scaling hardware byte counters.
// 16-byte non-temporal loads and stores; buffers that are not 16-byte
// aligned (or not a multiple of 16 bytes) use a plain byte loop.
#include "fr_device.hpp"
#include "fr_kernels.hpp"

namespace fr {

// Each workgroup copies one contiguous block of 8 x 256 chunks: all eight
// loads are issued before the stores. Contiguous per-workgroup blocks keep
// every wavefront on neighbouring DRAM pages (measured faster on MI355X than
// a grid-stride walk).
constexpr int kCopyUnroll = 8;
__global__ __launch_bounds__(256) void stream_copy_kernel(const u32x4* __restrict__ src,
                                                          u32x4* __restrict__ dst, int64_t n16) {
  const int64_t first = (int64_t)blockIdx.x * (kCopyUnroll * 256);
  if (first + kCopyUnroll * 256 <= n16) {  // whole block in range (all but the last)
    const u32x4* s = src + first + threadIdx.x;
    u32x4* d = dst + first + threadIdx.x;
    u32x4 v[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) v[u] = __builtin_nontemporal_load(s + u * 256);
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) __builtin_nontemporal_store(v[u], d + u * 256);
  } else {
    for (int64_t i = first + threadIdx.x; i < n16; i += 256)
      __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
  }
}

__global__ __launch_bounds__(256) void byte_copy_kernel(const uint8_t* src, uint8_t* dst, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) dst[i] = src[i];
}

hipError_t launch_stream_copy(const void* src, void* dst, int64_t bytes, hipStream_t s) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(src), b = reinterpret_cast<uintptr_t>(dst);
  if (a % 16 == 0 && b % 16 == 0 && bytes % 16 == 0) {
    const int64_t n16 = bytes / 16;
    const int64_t blocks = (n16 + kCopyUnroll * 256 - 1) / (kCopyUnroll * 256);
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
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
