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
// blocks of BN = 32 keys (one 32-key score tile). Per key block, per wave:
//   S^T (32 keys x 32 queries) = K_blk (A operand, from LDS) * Q^T (B operand,
//     the wave's queries held in registers for the whole kernel);
//   in the MFMA C layout lane l owns query l % 32 and 16 of the 32 keys (the
//     other 16 are in lane l ^ 32), so each lane tests the max of its own 16
//     values against the lazy threshold, and only when the running max is
//     raised is the query's block max formed with one exchange with lane
//     l ^ 32 (v_permlane32_swap, no LDS round trip); the rescale of the
//     output accumulator is one per-lane factor;
//   O^T (D x 32 queries) += V_blk^T (A operand, read from the row-major V
//     tile in LDS through the transposing read ds_read_b64_tr_b16) * P^T
//     (B operand: the lane's 16 probabilities as they are). The C
//     layout gives lane half h the keys {h*4 + 0..3, 8 + h*4 + 0..3} of each
//     16-key group, so the V^T operand is read with the same key order — the
//     contraction over keys does not depend on their order.
// Scores are kept in base 2 (scale * log2(e) folded into the exponential's
// fma); the next key block's K and V are loaded into registers while the
// current one is computed, and written to the second LDS stage after it.
// The running max is raised lazily: only when a query's block max exceeds
// it by more than kLazy (base-2 units) is it updated and the output
// accumulator rescaled — otherwise the probabilities are taken against the
// stale max (at most 2^kLazy, exact in fp32 and bf16 range), which keeps the
// D/2 accumulator multiplies off most key blocks.
// Masks are applied only on the key blocks that reach the causal diagonal or
// the end of the keys. Causal query blocks are launched longest first.
// Each lane keeps its own share of the running sum (its 16 keys of every
// block; the two halves of a query are added once, at the end), and the
// exponentials' offset changes only when the running max is raised.
// The LDS operands of each product are read four at a time, each group
// waited for inside one asm block (`read_k4`, `read_tr4`): one LDS round
// trip per four reads, the next group's reads overlapping the previous
// group's matrix work (bench shape 571.5 -> 561.1 us, causal 304.3 -> 303.1,
// the slowest tenth of the calls 684 -> 572 us).
#include "fr_kernels.hpp"
#include "fr_device.hpp"

namespace fr {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kAttnBlockM = 128;  // queries per workgroup (4 waves x 32)
constexpr float kLazy = 8.f;      // stale-max allowance, base-2 units
constexpr float kFltMax = 3.40282347e38f;
// The wave's issue priority is raised over its matrix-core chains, so that
// the other waves of the SIMD fill the gaps with their softmax work
// (measured 594 -> 585 us and 320 -> 317 us at B=4 H=16 S=4096 D=128).
__device__ __forceinline__ void mfma_prio_hi() { __builtin_amdgcn_s_setprio(1); }
__device__ __forceinline__ void mfma_prio_lo() { __builtin_amdgcn_s_setprio(0); }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// The values of lanes l % 32 and l % 32 + 32 in every lane l, through
// v_permlane32_swap (a VALU exchange of the two wave halves) instead of an
// LDS permute: with both operands x, one result holds the low half's value
// and the other the high half's, in every lane.
struct HalfPair {
  float lo, hi;
};
__device__ __forceinline__ HalfPair half_pair(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return {__uint_as_float(r[0]), __uint_as_float(r[1])};
}

// LDS-address-space views for the transposing LDS read (ds_read_b64_tr_b16)
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) const bf16_t lds_bf16;

// Four transposing reads from one base at immediate offsets O0..O3 (bytes),
// waited for inside the asm block: r[i] from base + Oi.
template <int O0, int O1, int O2, int O3>
__device__ __forceinline__ void read_tr4(uint32_t base, u32x2 (&r)[4]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %4 offset:%5\n\t"
      "ds_read_b64_tr_b16 %1, %4 offset:%6\n\t"
      "ds_read_b64_tr_b16 %2, %4 offset:%7\n\t"
      "ds_read_b64_tr_b16 %3, %4 offset:%8\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
      : "v"(base), "n"(O0), "n"(O1), "n"(O2), "n"(O3)
      : "memory");
}

// Four 16-byte reads from one base at byte offsets O, O + 32, O + 64 and
// O + 96, waited for inside the asm block.
template <int O>
__device__ __forceinline__ void read_k4(uint32_t base, u32x4 (&r)[4]) {
  asm volatile(
      "ds_read_b128 %0, %4 offset:%5\n\t"
      "ds_read_b128 %1, %4 offset:%6\n\t"
      "ds_read_b128 %2, %4 offset:%7\n\t"
      "ds_read_b128 %3, %4 offset:%8\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
      : "v"(base), "n"(O), "n"(O + 32), "n"(O + 64), "n"(O + 96)
      : "memory");
}

template <int D, int BN>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void attention_fwd_kernel(const bf16_t* q, const bf16_t* k,
                                                            const bf16_t* v, bf16_t* o, float* lse,
                                                            int64_t BH, int Sq, int Sk, int causal,
                                                            float scale_log2) {
  constexpr int NT = BN / 32;               // 32-key score tiles per block
  static_assert(NT == 1, "one 32-key score tile per block");
  constexpr int KP = D + 8;                 // K tile row stride (bf16), padded
  // V tile row stride (bf16): row-major [key][d], padded by 64 bytes so that
  // the transposing reads of 8 keys x 32 d spread over all LDS banks
  constexpr int VS = D + 32;
  constexpr int NKK = D / 16;               // k-steps of the score product
  constexpr int NDB = D / 32;               // 32-row blocks of O^T
  constexpr int CH = BN * D / 8;            // 16-byte chunks per K (or V) tile
  constexpr int CPT = CH / 256;             // chunks per thread
  static_assert(CPT >= 1 && CH % 256 == 0, "tile");
  // two stages: the next key block is written while the current one is read
  __shared__ __attribute__((aligned(16))) bf16_t ks_st[2][BN * KP];
  __shared__ __attribute__((aligned(16))) bf16_t vt_st[2][BN * VS];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int h = lane >> 5;      // lane half
  const int lq = lane & 31;     // the lane's query within the wave / row in A operands
  const int nqb = (Sq + kAttnBlockM - 1) / kAttnBlockM;
  int64_t bh;
  int qidx;
  if (BH % 8 == 0) {
    // Workgroups are dealt to the 8 XCDs round-robin: XCD x receives
    // blockIdx x, x + 8, ...; give it the heads x BH/8 .. (x + 1) BH/8 - 1
    // with all their query blocks, so the K/V tiles of those heads are shared
    // in its own L2 and every XCD gets the same mix of query blocks (measured
    // at B=4 H=16 S=4096 D=128: 574 -> 564 us, the slowest tenth of the calls
    // 690 -> 580 us; causal unchanged)
    const int64_t hx = BH / 8;
    const int64_t slot = blockIdx.x / 8, x = blockIdx.x % 8;
    if (causal) {  // query block slowest: most keys first across the heads
      bh = x * hx + slot % hx;
      qidx = (int)(slot / hx);
    } else {  // head by head
      bh = x * hx + slot / nqb;
      qidx = (int)(slot % nqb);
    }
  } else {
    // (batch, head) fastest: consecutive workgroups (dealt to different
    // XCDs) take different heads of the same query block, so every XCD gets
    // every query block
    bh = (int64_t)blockIdx.x % BH;
    qidx = (int)((int64_t)blockIdx.x / BH);
  }
  const int qblk = causal ? nqb - 1 - qidx : qidx;  // causal: most keys first
  const int q0 = qblk * kAttnBlockM + wave * 32;
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
  // m_run: running max (base 2); m_use: the offset the exponentials take
  // (m_run, or 0 while no key was seen); l_lane: this lane's share of the
  // running sum (its 16 keys per block), the halves added at the end
  float m_run = kNegInf, m_use = 0.f, l_lane = 0.f;
  float m_lazy = kNegInf;  // m_run + kLazy

  // keys visible to the workgroup's last query
  const int q_first = qblk * kAttnBlockM;
  const int q_last = q_first + kAttnBlockM - 1;
  int kend = Sk;
  if (causal) {
    const int lim = q_last + (Sk - Sq) + 1;
    kend = lim < kend ? lim : kend;
  }
  const int nblk = kend > 0 ? (kend + BN - 1) / BN : 0;
  // key blocks starting past mask_after reach the end of the keys or, when
  // causal, the diagonal of the workgroup's first query (a scalar test per
  // block)
  int mask_after = Sk - BN;
  if (causal) {
    const int d = q_first + (Sk - Sq) - BN + 1;
    mask_after = d < mask_after ? d : mask_after;
  }
  mask_after = __builtin_amdgcn_readfirstlane(mask_after);

  // tile loads: chunk c = tid + 256 i of a tile is key c / (D/8), d0 = (c % (D/8)) * 8
  // (row order), for K and V alike
  u32x4 kreg[CPT], vreg[CPT];
  // byte offsets of this thread's chunks from the tile's first key (lane
  // constants): a full tile is read as uniform tile base + 32-bit offset
  uint32_t koff[CPT], voff[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int c = tid + 256 * i;
    koff[i] = (uint32_t)(((c / (D / 8)) * D + (c % (D / 8)) * 8) * 2);
    voff[i] = koff[i];
  }
  auto load_tile = [&](int n0) {
    if (n0 + BN <= Sk) {  // uniform: every key of the tile exists
      const char* kt = reinterpret_cast<const char*>(kb + (int64_t)n0 * D);
      const char* vtl = reinterpret_cast<const char*>(vb + (int64_t)n0 * D);
      const uint32_t z = opaque_zero();  // keeps the offsets 32-bit (SGPR base + VGPR offset)
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        kreg[i] = *reinterpret_cast<const u32x4*>(kt + (koff[i] + z));
        vreg[i] = *reinterpret_cast<const u32x4*>(vtl + (voff[i] + z));
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + 256 * i;
      const int key = n0 + c / (D / 8);
      const int d0 = (c % (D / 8)) * 8;
      const int kr = key < Sk ? key : Sk - 1;
      u32x4 a = *reinterpret_cast<const u32x4*>(kb + (int64_t)kr * D + d0);
      kreg[i] = key < Sk ? a : u32x4{0, 0, 0, 0};
      u32x4 b = *reinterpret_cast<const u32x4*>(vb + (int64_t)kr * D + d0);
      vreg[i] = key < Sk ? b : u32x4{0, 0, 0, 0};
    }
  };
  // this lane's chunk of copy i is key row tid / (D/8) + i 256 / (D/8), d
  // (tid % (D/8)) 8: one lane offset per tile, the rest immediates
  constexpr int RPI = 256 / (D / 8);
  const int kst_lane = (tid / (D / 8)) * KP + (tid % (D / 8)) * 8;
  const int vst_lane = (tid / (D / 8)) * VS + (tid % (D / 8)) * 8;
  auto store_tile = [&](int stage) {
    bf16_t* ks = ks_st[stage] + kst_lane;
    bf16_t* vt = vt_st[stage] + vst_lane;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      *reinterpret_cast<u32x4*>(ks + RPI * i * KP) = kreg[i];
      *reinterpret_cast<u32x4*>(vt + RPI * i * VS) = vreg[i];
    }
  };

  // Stage blk & 1 holds key block blk. Block blk + 1 is written to the other
  // stage after this wave's compute of block blk: every wave has finished
  // reading that stage (block blk - 1) before the barrier that ended the
  // previous iteration. One barrier per key block.
  if (nblk > 0) {
    load_tile(0);
    store_tile(0);
    if (nblk > 1) load_tile(BN);
  }
  __syncthreads();
  for (int blk = 0; blk < nblk; ++blk) {
    const int n0 = blk * BN;
    const bf16_t* ks = ks_st[blk & 1];
    const bf16_t* vt = vt_st[blk & 1];

    // S^T = K_blk * Q^T, one independent accumulator per 32-key tile
    f32x16 s[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) s[t] = f32x16{};
    // the K operands four k-steps at a time (one LDS round trip each; the
    // second batch's reads overlap the first batch's matrix work)
    mfma_prio_hi();
    {
      const uint32_t kl = lds_offset(ks + lq * KP + 8 * h);
      u32x4 a[4];
      read_k4<0>(kl, a);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a[kk]), as_bf16x8(qop[kk]), s[0], 0, 0, 0);
      if constexpr (NKK == 8) {
        u32x4 c[4];
        read_k4<128>(kl, c);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
          s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(c[kk]), as_bf16x8(qop[4 + kk]), s[0], 0,
                                                         0, 0);
      }
    }
    mfma_prio_lo();

    // online softmax for query qi over keys n0 + 32t + key(j),
    // key(j) = (j/4)*8 + 4h + j%4; t = scale_log2 * s (base-2 units)
    const bool need_mask = n0 > mask_after;
    const int klim = causal ? qi + (Sk - Sq) : Sk - 1;  // last visible key
    if (need_mask) {  // uniform; hidden scores take the identity of the max (or min)
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int key = n0 + 32 * t + (j >> 2) * 8 + 4 * h + (j & 3);
          s[t][j] = (key < Sk && key <= klim) ? s[t][j] : (scale_log2 >= 0.f ? kNegInf : -kNegInf);
        }
    }
    // block max of t: the max of s for scale >= 0, else the min; started at
    // the largest finite magnitude so that a block with every key hidden
    // gives a finite (or -inf) tmax for any scale, never -inf * 0
    float smax;
    if (scale_log2 >= 0.f) {
      smax = -kFltMax;
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int j = 0; j < 16; j += 2) smax = max3(smax, s[t][j], s[t][j + 1]);
    } else {
      smax = kFltMax;
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int j = 0; j < 16; ++j) smax = s[t][j] < smax ? s[t][j] : smax;
    }
    // this lane's half of the query's block max (its 16 keys)
    const float thalf = smax * scale_log2;
    // raise the running max only past the allowance: the query's block max
    // exceeds it iff one of its halves does, so the exchange between the
    // halves is needed only on a raise (wave-uniform decision)
    const bool raise = thalf > m_lazy;
    if (__builtin_amdgcn_ballot_w64(raise) != 0) {
      const HalfPair t2 = half_pair(thalf);
      const float tmax = __builtin_fmaxf(t2.lo, t2.hi);
      const float m_new = tmax > m_run ? tmax : m_run;
      const float alpha = m_run == kNegInf ? 0.f : exp2_hw(m_run - m_new);
      l_lane *= alpha;
#pragma unroll
      for (int b = 0; b < NDB; ++b) acc[b] *= alpha;
      m_run = m_new;
      m_use = m_new;
      m_lazy = m_new + kLazy;
    }
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int j = 0; j < 16; ++j) s[t][j] = exp2_hw(__builtin_fmaf(s[t][j], scale_log2, -m_use));
    if (need_mask) {  // hidden keys contribute exactly 0 (also when scale is 0)
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int key = n0 + 32 * t + (j >> 2) * 8 + 4 * h + (j & 3);
          s[t][j] = (key < Sk && key <= klim) ? s[t][j] : 0.f;
        }
    }
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int j = 0; j < 16; ++j) l_lane += s[t][j];

    // P^T as B operands: tile t, k-step 0 = the lane's j 0..7, k-step 1 = j 8..15
    u32x4 pb[2 * NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      pb[2 * t] = {pack_bf16x2(s[t][0], s[t][1]), pack_bf16x2(s[t][2], s[t][3]),
                   pack_bf16x2(s[t][4], s[t][5]), pack_bf16x2(s[t][6], s[t][7])};
      pb[2 * t + 1] = {pack_bf16x2(s[t][8], s[t][9]), pack_bf16x2(s[t][10], s[t][11]),
                       pack_bf16x2(s[t][12], s[t][13]), pack_bf16x2(s[t][14], s[t][15])};
    }

    // O^T += V^T * P^T. The V^T operand (row d = 32b + lane % 32, slots i of
    // lane half h = keys 4h + 0..3, 8 + 4h + 0..3 of each 16-key step, the
    // C-layout order of P^T) comes from the row-major V tile through two
    // transposing reads per MFMA: in each 16-lane group, lane t reads the 4 d
    // values 4(t % 4) + 0..3 of key t / 4 (of the group's 4 keys and 16 d),
    // and lane u receives d = u of all 4 keys.
    {
      const int g16 = lane & 15;
      const int vrow = 4 * h + (g16 >> 2);                       // key within 8
      const int vcol = 16 * ((lane >> 4) & 1) + 4 * (g16 & 3);   // d within 32
      const uint32_t vl = lds_offset(vt + vrow * VS + vcol);
      // the reads of one 32-row block b of O^T: r[2 st + x] is key step st,
      // rows 8x .. 8x + 7 of it
      constexpr int SB = 2 * VS;  // bytes per key row
      auto pv = [&](const u32x2 (&r)[4], int b) {
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const u32x4 a = {r[2 * st].x, r[2 * st].y, r[2 * st + 1].x, r[2 * st + 1].y};
          acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(pb[st]), acc[b], 0,
                                                           0, 0);
        }
      };
      // the row sum and the bf16 packing are done before any read: the
      // scores' registers are free for the operands
      __builtin_amdgcn_sched_barrier(0);
      mfma_prio_hi();
      {
        u32x2 r[4];
        read_tr4<0, 8 * SB, 16 * SB, 24 * SB>(vl, r);
        pv(r, 0);
      }
      {
        u32x2 r[4];
        read_tr4<64, 64 + 8 * SB, 64 + 16 * SB, 64 + 24 * SB>(vl, r);
        pv(r, 1);
      }
      if constexpr (NDB == 4) {
        {
          u32x2 r[4];
          read_tr4<128, 128 + 8 * SB, 128 + 16 * SB, 128 + 24 * SB>(vl, r);
          pv(r, 2);
        }
        {
          u32x2 r[4];
          read_tr4<192, 192 + 8 * SB, 192 + 16 * SB, 192 + 24 * SB>(vl, r);
          pv(r, 3);
        }
      }
      mfma_prio_lo();
    }

    if (blk + 1 < nblk) {
      store_tile((blk + 1) & 1);
      if (blk + 2 < nblk) load_tile(n0 + 2 * BN);  // in flight during the next compute
    }
    __syncthreads();
  }

  // O = O^T / l, lane (query qi) writes d = 32b + 8g + 4h + 0..3 (8 bytes)
  const HalfPair l2 = half_pair(l_lane);
  const float l_run = l2.lo + l2.hi;
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

// Key blocks of 32 (64-key blocks measured no faster: 580 -> 597 us, 239
// VGPRs and two waves per SIMD instead of three).
constexpr int kAttnBlockN = 32;

hipError_t launch_attention_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                                int64_t BH, int Sq, int Sk, int D, int causal, float scale,
                                hipStream_t s) {
  const int64_t nqb = (Sq + kAttnBlockM - 1) / kAttnBlockM;
  const dim3 grid((unsigned)(nqb * BH));
  const float sl2 = scale * kLog2e;
  const bf16_t* qp = static_cast<const bf16_t*>(q);
  const bf16_t* kp = static_cast<const bf16_t*>(k);
  const bf16_t* vp = static_cast<const bf16_t*>(v);
  bf16_t* op = static_cast<bf16_t*>(o);
  if (D == 64)
    return launch_kernel(&attention_fwd_kernel<64, kAttnBlockN>, grid, dim3(256), s, qp, kp, vp, op,
                         lse, BH, Sq, Sk, causal, sl2);
  return launch_kernel(&attention_fwd_kernel<128, kAttnBlockN>, grid, dim3(256), s, qp, kp, vp, op,
                       lse, BH, Sq, Sk, causal, sl2);
}

}  // namespace fr
