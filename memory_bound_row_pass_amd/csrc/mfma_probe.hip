// Matrix-core probe: how fast the bf16 matrix cores retire
// v_mfma_f32_32x32x16_bf16 when nothing else competes for the issue slots —
// no operand loads, no vector work — so the ceiling the attention forward's
// flop rate is compared with, beside the published dense peak (which assumes
// the top clock; a chip running matrix instructions flat out may hold a lower
// one, and how much lower depends on how much the operand bits toggle).
// "Engineering a CUDA Machine Learning Framework from Scratch",
// §6.4 Multi-Head Attention & FlashAttention-2 Extension: the two products of
// attention are the matrix work here.
//
// Every wavefront runs `iters` rounds of 8 instructions on four independent
// accumulators (two per accumulator per round) with two operand vectors u, w
// per lane, taken as (A, B) = (u, w) and then (w, u).
//   pattern 0: every operand element 1/8. Each instruction adds 16/64 to
//     every accumulator element, so each lane's sum of its 64 accumulator
//     elements is exactly 32 iters (iters <= 2^19): every instruction ran.
//   pattern 1: element e of lane l's vector s (s = 0 for u, 1 for w) is the
//     bf16 rounding of a pseudo-random value in [-1, 1) drawn from
//     h = (64 s + l) * 8 + e (operand_value below): full mantissas, as real
//     data has. Every wavefront holds the same operands and adds in the same
//     order, so all wavefronts write the same 64 sums.
#include "fr_device.hpp"
#include "fr_kernels.hpp"

namespace fr {

typedef __bf16 probe_bf16x8 __attribute__((ext_vector_type(8)));
typedef float probe_f32x16 __attribute__((ext_vector_type(16)));

// Pseudo-random value in [-1, 1) for index h: the 32-bit finaliser of
// MurmurHash3 applied to h + 1, top 24 bits as a fraction.
__device__ __forceinline__ float operand_value(uint32_t h) {
  uint32_t x = h + 1u;
  x ^= x >> 16;
  x *= 0x85EBCA6Bu;
  x ^= x >> 13;
  x *= 0xC2B2AE35u;
  x ^= x >> 16;
  return (float)(x >> 8) * 0x1p-23f - 1.f;
}

__global__ __launch_bounds__(256) void mfma_probe_kernel(float* sink, int iters, int pattern) {
  const uint32_t lane = threadIdx.x & 63;
  probe_bf16x8 u, w;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    u[e] = (__bf16)(pattern ? operand_value(lane * 8 + e) : 0.125f);
    w[e] = (__bf16)(pattern ? operand_value((64 + lane) * 8 + e) : 0.125f);
  }
  probe_f32x16 acc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) acc[c] = probe_f32x16{};
  for (int n = 0; n < iters; ++n) {
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(u, w, acc[c], 0, 0, 0);
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w, u, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int j = 0; j < 16; ++j) s += acc[c][j];
  sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

hipError_t launch_mfma_probe(int workgroups, int iters, int pattern, float* sink, hipStream_t s) {
  return launch_kernel(&mfma_probe_kernel, dim3((unsigned)workgroups), dim3(256), s, sink, iters,
                       pattern);
}

}  // namespace fr
