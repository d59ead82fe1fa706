// Register-resident online-softmax core shared by the softmax and the
// softmax cross-entropy kernels.
//
// Per row ("Engineering a CUDA Machine Learning Framework from Scratch",
// §3.1 Online FlashSoftmax, read as: one pass over memory, running max and
// rescaled exponential sum, no exponentials written out):
//   1. each lane loads its share of the row into VGPRs (the only read),
//   2. each lane forms its partial state (m_l, s_l): m_l = max of its values,
//      s_l = sum_j exp(x_j - m_l),
//   3. the partial states are combined with the online-normaliser merge,
//      across the wavefront with DPP and across waves through LDS -> (M, S),
//   4. each lane writes p_j = exp(x_j - M) / S (the only write).
// Two ways to produce step 4 from registers:
//   * bf16 outputs keep e_j = exp(x_j - m_l) from step 2 in place of x_j and
//     rescale by exp(m_l - M) / S (one exponential per element);
//   * fp32 outputs keep x_j and evaluate exp(x_j - M) again, which needs half
//     the registers and rounds each p_j from a single exponential.
#pragma once

#include "fr_device.hpp"

namespace fr {

// Lane max over NV x EPV register values plus the extra slot.
template <int NV, int EPV>
__device__ __forceinline__ float lane_max(const float (&v)[NV][EPV], float xe) {
  constexpr int N = NV * EPV;
  const float* f = &v[0][0];
  // four independent max3 chains, then combine
  float a0 = xe, a1 = kNegInf, a2 = kNegInf, a3 = kNegInf;
  int j = 0;
#pragma unroll
  for (; j + 8 <= N; j += 8) {
    a0 = max3(a0, f[j + 0], f[j + 1]);
    a1 = max3(a1, f[j + 2], f[j + 3]);
    a2 = max3(a2, f[j + 4], f[j + 5]);
    a3 = max3(a3, f[j + 6], f[j + 7]);
  }
#pragma unroll
  for (; j + 2 <= N; j += 2) a0 = max3(a0, f[j], f[j + 1]);
  if constexpr (N % 2) a0 = max3(a0, f[N - 1], f[N - 1]);
  return max3(max3(a0, a1, a2), a3, a3);
}

// ---------------------------------------------------------------- bf16 path
// e_j = 2^((x_j - m_l)*log2e + 64), computed as 2^(x_j*log2e + K) with
// K = 64 - m_l*log2e: e_j lies in (0, 2^64] and is normal down to
// x_j - m_l = -131, which covers every value that can round to a non-zero
// bf16 (p >= 2^-134). The lane state (m_l, s_l) stays in natural units.
// When m_l*log2e would overflow (|m_l| >= 2e38) the wave takes the slower
// (x_j - m_l)*log2e + 64 form.
template <int NV, int EPV>
__device__ __forceinline__ MaxSumState lane_exp_log2(float (&v)[NV][EPV], float& xe, float m) {
  const bool empty = (m == kNegInf);
  const bool huge = !empty && __builtin_fabsf(m) >= 2.0e38f && __builtin_fabsf(m) != __builtin_inff();
  float s0 = 0.f, s1 = 0.f;
  if (!__any(huge)) {
    const float K = empty ? 0.f : 64.f - m * kLog2e;
#pragma unroll
    for (int i = 0; i < NV; ++i)
#pragma unroll
      for (int k = 0; k < EPV; ++k) {
        v[i][k] = exp2_hw(__builtin_fmaf(v[i][k], kLog2e, K));
        if (k & 1) s1 += v[i][k]; else s0 += v[i][k];
      }
    xe = exp2_hw(__builtin_fmaf(xe, kLog2e, K));
  } else {
    const float mr = empty ? 0.f : m;
#pragma unroll
    for (int i = 0; i < NV; ++i)
#pragma unroll
      for (int k = 0; k < EPV; ++k) {
        v[i][k] = exp2_hw(__builtin_fmaf(v[i][k] - mr, kLog2e, 64.f));
        if (k & 1) s1 += v[i][k]; else s0 += v[i][k];
      }
    xe = exp2_hw(__builtin_fmaf(xe - mr, kLog2e, 64.f));
  }
  return {m, (s0 + s1) + xe};
}

// p_j = e_j * 2^((m_l - M)*log2e) / S, where S carries the same 2^64 bias.
// The factor is split as G * 2^n with G = 2^(d - n) / S normal
// (d = (m_l - M)*log2e, n = floor(d)), and 2^n is applied with v_ldexp, so
// results in the bf16 subnormal range are rounded from a full-precision fp32
// value instead of a flushed factor.
struct Log2Scale {
  float g;
  int n;
};

__device__ __forceinline__ Log2Scale log2_scale(float m, float M, float S) {
  // d <= 0; -inf for an empty lane (its e_j are all 0); NaN if the row is
  // all -inf (the result is then NaN, as for the definition).
  const float d = (m - M) * kLog2e;
  float fl = __builtin_floorf(d);
  fl = fl < -300.f ? -300.f : fl;  // also maps -inf to -300
  return {exp2_hw(d - fl) / S, (int)fl};
}

__device__ __forceinline__ float apply_scale(float e, const Log2Scale& s) {
  return __builtin_ldexpf(e * s.g, s.n);
}

// ---------------------------------------------------------------- fp32 path
// Natural units with the compensated exponential; x_j is left in place.
template <int NV, int EPV>
__device__ __forceinline__ MaxSumState lane_sum_nat(const float (&v)[NV][EPV], float xe, float m) {
  const float mr = (m == kNegInf) ? 0.f : m;
  float s0 = 0.f, s1 = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i)
#pragma unroll
    for (int k = 0; k < EPV; ++k) {
      const float e = exp_acc(v[i][k] - mr);
      if (k & 1) s1 += e; else s0 += e;
    }
  return {m, (s0 + s1) + exp_acc(xe - mr)};
}

// p = exp(x - M) / S from the kept x.
template <int NV, int EPV>
__device__ __forceinline__ void probs_nat(float (&v)[NV][EPV], float& xe, float M, float S) {
  const float inv = 1.f / S;
#pragma unroll
  for (int i = 0; i < NV; ++i)
#pragma unroll
    for (int k = 0; k < EPV; ++k) v[i][k] = exp_acc(v[i][k] - M) * inv;
  xe = exp_acc(xe - M) * inv;
}

}  // namespace fr
