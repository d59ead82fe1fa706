// Register-resident online-softmax core shared by the softmax and the
// softmax cross-entropy kernels.
//
// Per row ("Engineering a CUDA Machine Learning Framework from Scratch",
// §3.1 Online FlashSoftmax, read as: one pass over memory, running max and
// rescaled exponential sum, no exponentials written out):
//   1. each lane loads its share of the row into VGPRs (the only read),
//   2. each wavefront finds the maximum m_w of its values (DPP max) and each
//      lane sums exp(x_j - m_w) over its values; the wave's sum s_w is a
//      plain DPP sum, so no exponential or rescale sits inside the tree,
//   3. the waves' states (m_w, s_w) are combined with the online-normaliser
//      merge through LDS and a DPP tree -> (M, S),
//   4. each lane writes p_j = exp(x_j - M) / S (the only write).
// e_j = exp(x_j - m_w) from step 2 replaces x_j in the registers and step 4
// rescales it by exp(m_w - M) / S, one factor per wave: one exponential per
// element. bf16 outputs use base-2 hardware exponentials with a bias that
// keeps bf16 subnormal results exact; fp32 outputs use a compensated
// exponential. The online recurrence is what merges waves (and, on the split
// path, the segments of a row); inside a wave the row is in registers, so its
// maximum is known before any exponential is taken.
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
// e_j = 2^(y_j + kExpBias) with y_j = (x_j - m_w)*log2e <= 0, so e_j lies in
// (0, 2^8]. p_j <= 2^y_j (m_w <= M and the row sum is >= 1 in natural
// units), so every e_j whose p_j can round to a non-zero bf16 (p_j >= 2^-134)
// is >= 2^-126: a normal fp32 value at full precision. 8 is the least bias
// that does this; a larger one would keep fewer bits of y_j + bias and make
// the row sum (which the cross-entropy loss takes) less accurate. Forming
// x_j - m_w first keeps the argument finite for any finite input (m_w*log2e
// alone overflows for |m_w| > 2.3e38). The returned state (m_w, s_l) keeps m_w
// in natural units; s_l, this lane's sum, carries the 2^8 factor, which
// cancels in p_j.
constexpr int kExpBias = 8;

template <int NV, int EPV>
__device__ __forceinline__ MaxSumState lane_exp_log2(float (&v)[NV][EPV], float& xe, float m) {
  const float mr = (m == kNegInf) ? 0.f : m;
  float s0 = 0.f, s1 = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i)
#pragma unroll
    for (int k = 0; k < EPV; ++k) {
      v[i][k] = exp2_hw(__builtin_fmaf(v[i][k] - mr, kLog2e, (float)kExpBias));
      if (k & 1) s1 += v[i][k]; else s0 += v[i][k];
    }
  xe = exp2_hw(__builtin_fmaf(xe - mr, kLog2e, (float)kExpBias));
  return {m, (s0 + s1) + xe};
}

// p_j = e_j * 2^((m_w - M)*log2e) / S, where S carries the same 2^8 factor.
// The wave's factor is split as G * 2^n with G = 2^(d - n) / S normal
// (d = (m_w - M)*log2e, n = floor(d)); callers form f = ldexp(G, n) once per
// wave and take one multiply (or fma) per element. Where f is normal the
// product rounds the exact e_j * G * 2^n once. Where f is subnormal (a wave
// whose maximum lies ~80 below the row's) its own rounding, at most 2^-150,
// moves p_j by at most e_j * 2^-150 <= 2^-142: a 2^-9 fraction of the finest
// bf16 step, so bf16 subnormal results stay within one ulp.
struct Log2Scale {
  float g;
  int n;
};

__device__ __forceinline__ Log2Scale log2_scale(float m, float M, float S) {
  // d <= 0; -inf for an empty wave (its e_j are all 0); NaN if the row is
  // all -inf (the result is then NaN, as for the definition).
  const float d = (m - M) * kLog2e;
  float fl = __builtin_floorf(d);
  fl = fl < -300.f ? -300.f : fl;  // also maps -inf to -300
  return {exp2_hw(d - fl) / S, (int)fl};
}

// ---------------------------------------------------------------- fp32 path
// Natural units with the compensated exponential: e_j = exp(x_j - m_w)
// replaces x_j in place; p_j = e_j * exp(m_w - M) / S at the store. The two
// compensated exponentials each contribute about one ulp, so p_j stays well
// inside 1e-5 relative for results above the fp32 normal range.
template <int NV, int EPV>
__device__ __forceinline__ MaxSumState lane_exp_nat(float (&v)[NV][EPV], float& xe, float m) {
  const float mr = (m == kNegInf) ? 0.f : m;
  float s0 = 0.f, s1 = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i)
#pragma unroll
    for (int k = 0; k < EPV; ++k) {
      v[i][k] = exp_acc(v[i][k] - mr);
      if (k & 1) s1 += v[i][k]; else s0 += v[i][k];
    }
  xe = exp_acc(xe - mr);
  return {m, (s0 + s1) + xe};
}

// Wave factor exp(m_w - M) / S: 0 for an empty wave, NaN for an all -inf row.
__device__ __forceinline__ float nat_scale(float m, float M, float S) {
  return exp_acc(m - M) / S;
}

}  // namespace fr
