// Attention forward with the online softmax fused in, on the bf16 matrix
// cores of gfx950 (v_mfma_f32_32x32x16_bf16).
//
// "Engineering a CUDA Machine Learning Framework from Scratch", §3.1 names
// the online normaliser as the softmax inside attention: the scores of a
// query against a block of keys update a running (max, sum) pair, the output
// accumulator is rescaled by exp(m_old - m_new), and no score or probability
// matrix is written to memory.
//
// Workgroup: 4 waves, 128 queries (32 per wave) of one (batch, head); key
// blocks of 32. Per key block, per wave:
//   S^T (32 keys x 32 queries) = K_blk (A operand, from LDS) * Q^T (B operand,
//     the wave's queries held in registers for the whole kernel);
//   in the MFMA C layout lane l owns query l % 32 and 16 of the 32 keys (the
//     other 16 are in lane l ^ 32), so the per-query max and sum take the
//     lane's 16 values and one exchange with lane l ^ 32, and the rescale of
//     the output accumulator is one per-lane factor;
//   O^T (D x 32 queries) += V_blk^T (A operand, from a transposed V tile in
//     LDS) * P^T (B operand: the lane's 16 probabilities as they are). The C
//     layout gives lane half h the keys {h*4 + 0..3, 8 + h*4 + 0..3} of each
//     16-key group, so the V^T operand is read with the same key order — the
//     contraction over keys does not depend on their order.
// Scores are kept in base 2 (scale * log2(e) folded in); the next key block's
// K and V are loaded into registers while the current one is computed.
#include "fr_kernels.hpp"
#include "fr_device.hpp"

namespace fr {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kAttnBlockM = 128;  // queries per workgroup (4 waves x 32)
constexpr int kAttnBlockN = 32;   // keys per block

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

template <int D>
__global__ __launch_bounds__(256) void attention_fwd_kernel(const bf16_t* q, const bf16_t* k,
                                                            const bf16_t* v, bf16_t* o, float* lse,
                                                            int Sq, int Sk, int causal,
                                                            float scale_log2) {
  constexpr int KP = D + 8;                 // K tile row stride (bf16), padded
  constexpr int VP = kAttnBlockN + 8;       // V^T tile row stride (bf16), padded
  constexpr int NKK = D / 16;               // k-steps of the score product
  constexpr int NDB = D / 32;               // 32-row blocks of O^T
  constexpr int CH = kAttnBlockN * D / 8;   // 16-byte chunks per K (or V) tile
  constexpr int CPT = CH / 256;             // chunks per thread
  static_assert(CPT >= 1 && CH % 256 == 0, "tile");
  __shared__ __attribute__((aligned(16))) bf16_t ks[kAttnBlockN * KP];
  __shared__ __attribute__((aligned(16))) bf16_t vt[D * VP];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int h = lane >> 5;      // lane half
  const int lq = lane & 31;     // the lane's query within the wave / row in A operands
  const int64_t bh = blockIdx.y;
  const int q0 = blockIdx.x * kAttnBlockM + wave * 32;
  const int qi = q0 + lq;       // this lane's query
  const bf16_t* qb = q + bh * (int64_t)Sq * D;
  const bf16_t* kb = k + bh * (int64_t)Sk * D;
  const bf16_t* vb = v + bh * (int64_t)Sk * D;

  // Q^T as B operands: lane (query lq, half h), k-step kk holds d = 16kk + 8h + 0..7
  u32x4 qop[NKK];
  {
    const int qr = qi < Sq ? qi : Sq - 1;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      u32x4 t = *reinterpret_cast<const u32x4*>(qb + (int64_t)qr * D + 16 * kk + 8 * h);
      qop[kk] = qi < Sq ? t : u32x4{0, 0, 0, 0};
    }
  }

  f32x16 acc[NDB];
#pragma unroll
  for (int b = 0; b < NDB; ++b) acc[b] = f32x16{};
  float m_run = kNegInf, l_run = 0.f;

  // keys visible to the workgroup's last query
  const int q_last = blockIdx.x * kAttnBlockM + kAttnBlockM - 1;
  int kend = Sk;
  if (causal) {
    const int lim = q_last + (Sk - Sq) + 1;
    kend = lim < kend ? lim : kend;
  }
  const int nblk = kend > 0 ? (kend + kAttnBlockN - 1) / kAttnBlockN : 0;

  // tile loads: chunk c of a tile = key c / (D/8), d0 = (c % (D/8)) * 8
  u32x4 kreg[CPT], vreg[CPT];
  auto load_tile = [&](int n0) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + 256 * i;
      const int key = n0 + c / (D / 8);
      const int d0 = (c % (D / 8)) * 8;
      const int kr = key < Sk ? key : Sk - 1;
      u32x4 a = *reinterpret_cast<const u32x4*>(kb + (int64_t)kr * D + d0);
      u32x4 b = *reinterpret_cast<const u32x4*>(vb + (int64_t)kr * D + d0);
      kreg[i] = key < Sk ? a : u32x4{0, 0, 0, 0};
      vreg[i] = key < Sk ? b : u32x4{0, 0, 0, 0};
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + 256 * i;
      const int key = c / (D / 8);
      const int d0 = (c % (D / 8)) * 8;
      *reinterpret_cast<u32x4*>(ks + key * KP + d0) = kreg[i];
      const uint32_t w[4] = {vreg[i].x, vreg[i].y, vreg[i].z, vreg[i].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        vt[(d0 + 2 * j) * VP + key].u = (uint16_t)(w[j] & 0xffffu);
        vt[(d0 + 2 * j + 1) * VP + key].u = (uint16_t)(w[j] >> 16);
      }
    }
  };

  if (nblk > 0) load_tile(0);
  for (int blk = 0; blk < nblk; ++blk) {
    const int n0 = blk * kAttnBlockN;
    __syncthreads();  // previous block's tiles fully read
    store_tile();
    __syncthreads();
    if (blk + 1 < nblk) load_tile(n0 + kAttnBlockN);  // in flight during the compute

    // S^T = K_blk * Q^T
    f32x16 s = f32x16{};
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const u32x4 a = *reinterpret_cast<const u32x4*>(ks + lq * KP + 16 * kk + 8 * h);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(qop[kk]), s, 0, 0, 0);
    }

    // online softmax for query qi over keys n0 + key(j), key(j) = (j/4)*8 + 4h + j%4
    const int klim = causal ? qi + (Sk - Sq) : Sk - 1;  // last visible key
    float mloc = kNegInf;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int key = n0 + (j >> 2) * 8 + 4 * h + (j & 3);
      const float sv = (key < Sk && key <= klim) ? s[j] * scale_log2 : kNegInf;
      s[j] = sv;
      mloc = sv > mloc ? sv : mloc;
    }
    const float mpart = __shfl_xor(mloc, 32);
    float m_new = m_run > mloc ? m_run : mloc;
    m_new = m_new > mpart ? m_new : mpart;
    const float m_use = m_new == kNegInf ? 0.f : m_new;
    const float alpha = exp2_hw(m_run - m_use);  // 0 while nothing was visible
    float lsum = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      s[j] = exp2_hw(s[j] - m_use);
      lsum += s[j];
    }
    lsum += __shfl_xor(lsum, 32);
    l_run = l_run * alpha + lsum;
    m_run = m_new;
#pragma unroll
    for (int b = 0; b < NDB; ++b) acc[b] *= alpha;

    // P^T as B operands: k-step 0 = the lane's j 0..7, k-step 1 = j 8..15
    const u32x4 p0 = {pack_bf16x2(s[0], s[1]), pack_bf16x2(s[2], s[3]),
                      pack_bf16x2(s[4], s[5]), pack_bf16x2(s[6], s[7])};
    const u32x4 p1 = {pack_bf16x2(s[8], s[9]), pack_bf16x2(s[10], s[11]),
                      pack_bf16x2(s[12], s[13]), pack_bf16x2(s[14], s[15])};

    // O^T += V^T * P^T; V^T operand rows d = 32b + lq, keys in the C-layout order
#pragma unroll
    for (int b = 0; b < NDB; ++b) {
      const bf16_t* row = vt + (32 * b + lq) * VP + 4 * h;
      const u32x2 a0 = *reinterpret_cast<const u32x2*>(row);        // keys 4h + 0..3
      const u32x2 a1 = *reinterpret_cast<const u32x2*>(row + 8);    // keys 8 + 4h + 0..3
      const u32x2 a2 = *reinterpret_cast<const u32x2*>(row + 16);   // keys 16 + 4h + 0..3
      const u32x2 a3 = *reinterpret_cast<const u32x2*>(row + 24);   // keys 24 + 4h + 0..3
      acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(u32x4{a0.x, a0.y, a1.x, a1.y}),
                                                       as_bf16x8(p0), acc[b], 0, 0, 0);
      acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(u32x4{a2.x, a2.y, a3.x, a3.y}),
                                                       as_bf16x8(p1), acc[b], 0, 0, 0);
    }
  }

  // O = O^T / l, lane (query qi) writes d = 32b + 8g + 4h + 0..3 (8 bytes)
  if (qi < Sq) {
    const float inv_l = l_run > 0.f ? 1.f / l_run : 0.f;
    bf16_t* orow = o + (bh * (int64_t)Sq + qi) * D;
#pragma unroll
    for (int b = 0; b < NDB; ++b)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const u32x2 w = {pack_bf16x2(acc[b][4 * g] * inv_l, acc[b][4 * g + 1] * inv_l),
                         pack_bf16x2(acc[b][4 * g + 2] * inv_l, acc[b][4 * g + 3] * inv_l)};
        *reinterpret_cast<u32x2*>(orow + 32 * b + 8 * g + 4 * h) = w;
      }
    if (lse && h == 0)
      lse[bh * (int64_t)Sq + qi] = l_run > 0.f ? (m_run + __log2f(l_run)) * kLn2 : kNegInf;
  }
}

hipError_t launch_attention_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                                int64_t BH, int Sq, int Sk, int D, int causal, float scale,
                                hipStream_t s) {
  const dim3 grid((unsigned)((Sq + kAttnBlockM - 1) / kAttnBlockM), (unsigned)BH);
  const float sl2 = scale * kLog2e;
  const bf16_t* qp = static_cast<const bf16_t*>(q);
  const bf16_t* kp = static_cast<const bf16_t*>(k);
  const bf16_t* vp = static_cast<const bf16_t*>(v);
  bf16_t* op = static_cast<bf16_t*>(o);
  if (D == 64)
    return launch_kernel(&attention_fwd_kernel<64>, grid, dim3(256), s, qp, kp, vp, op, lse, Sq, Sk,
                         causal, sl2);
  return launch_kernel(&attention_fwd_kernel<128>, grid, dim3(256), s, qp, kp, vp, op, lse, Sq, Sk,
                       causal, sl2);
}

}  // namespace fr
