// Row softmax, one pass over memory ("Engineering a CUDA Machine Learning
// Framework from Scratch", §3.1 Online FlashSoftmax).
//
// Template shape
//   Tin/Tout  storage types (float or bf16_t); arithmetic is fp32
//   T         lanes per row: 64 = one wavefront per row (several rows per
//             workgroup, no barrier), 256/512/1024 = one workgroup per row
//   NV        128-bit chunks (or scalars when EPV == 1) per lane
//   EPV       elements per chunk: 16 / sizeof(Tin), or 1 for the scalar path
// The exponentials stay in registers between the reduction and the store:
// base-2 with a bias for bf16 outputs, compensated natural for fp32 outputs.
#include "fr_kernels.hpp"
#include "softmax_core.hpp"

namespace fr {

// bf16 outputs: exponentials with the 2^8 bias (every e_j <= 2^8) and one
// factor f = G 2^n per lane, applied with one multiply per element (the
// rounding argument is log2_scale's). Measured at 16384 x 4096 against a
// 2^64 bias with a two-step ldexp scaling: 48.1 -> 46.7 us.
template <typename Tin, typename Tout, int T, int NV, int EPV, int OCC>
__global__ __launch_bounds__(T == 64 ? 256 : T) __attribute__((amdgpu_waves_per_eu(OCC))) void softmax_kernel(const Tin* x, Tout* y,
                                                                     int64_t rows, int cols) {
  constexpr int BLOCK = T == 64 ? 256 : T;
  constexpr int RPB = BLOCK / T;  // rows per workgroup
  constexpr int NW = T / 64;      // waves per row
  constexpr bool kLog2 = sizeof(Tout) == 2;
  using Merge = MaxSumMerge<kLog2>;
  __shared__ float xw[2][NW][2];

  // wave index made provably uniform, so per-row values live in SGPRs
  const int wib = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int tid = T == 64 ? lane : (int)threadIdx.x;  // lane within the row owner
  const int sub = T == 64 ? wib : 0;                   // row slot within the block
  const int wave = T == 64 ? 0 : wib;                  // wave within the row owner
  int merges = 0;  // cross-wave merges so far: picks the LDS slot
  for (int64_t row = (int64_t)blockIdx.x * RPB + sub; row < rows;
       row += (int64_t)gridDim.x * RPB) {
    const Tin* xr = x + row * cols;
    Tout* yr = y + row * cols;
    const RowGeom<EPV> g(xr, cols);

    float v[NV][EPV];
    load_chunks<Tin, T, NV, EPV>(xr, g, tid, v, kNegInf);
    const int ec = g.extra_col(tid);
    float xe = ec >= 0 ? load1(xr + ec) : kNegInf;

    // the wave's maximum first: exponentials relative to it, plain sums
    const float m = wave_max(lane_max<NV, EPV>(v, xe));
    MaxSumState st =
        kLog2 ? lane_exp_log2<NV, EPV>(v, xe, m) : lane_exp_nat<NV, EPV>(v, xe, m);
    st.s = wave_reduce(SumState{st.s}, SumMerge{}).s;
    if constexpr (NW > 1)
      st = block_merge_tree<NW>(st, xw[merges++ & 1], wave, lane, Merge{}, MaxSumState{kNegInf, 0.f});

    if constexpr (kLog2) {
      const Log2Scale sc = log2_scale(m, st.m, st.s);
      const float f = __builtin_ldexpf(sc.g, sc.n);
#pragma unroll
      for (int i = 0; i < NV; ++i)
#pragma unroll
        for (int k = 0; k < EPV; ++k) v[i][k] *= f;
      xe *= f;
    } else {
      const float f = nat_scale(m, st.m, st.s);
#pragma unroll
      for (int i = 0; i < NV; ++i)
#pragma unroll
        for (int k = 0; k < EPV; ++k) v[i][k] *= f;
      xe *= f;
    }

    // non-temporal stores, but cached ones for bf16 in / fp32 out, whose two
    // 16-byte stores per lane each cover half of a wave's lines (st_stream)
    store_chunks<Tout, T, NV, EPV, !(sizeof(Tin) == 2 && sizeof(Tout) == 4)>(yr, g, tid, v);
    if (ec >= 0) store1(yr + ec, xe);
  }
}

template <typename Tin, typename Tout, int T, int NV, int EPV, int OCC>
static hipError_t launch_softmax(const void* x, void* y, int64_t rows, int cols, hipStream_t s) {
  constexpr int BLOCK = T == 64 ? 256 : T;
  constexpr int RPB = BLOCK / T;
  const int64_t blocks = (rows + RPB - 1) / RPB;
  const unsigned grid = (unsigned)(blocks < kMaxGrid ? blocks : kMaxGrid);
  return launch_kernel(&softmax_kernel<Tin, Tout, T, NV, EPV, OCC>, dim3(grid), dim3(BLOCK), s,
                     static_cast<const Tin*>(x), static_cast<Tout*>(y), rows, cols);
}

// Variant tables, in order of preference (the first that holds the row wins).
// OCC is the waves-per-SIMD target handed to the register allocator; the
// last column group is the scalar path (misaligned or mixed-width rows).
#define FR_SM(TI, TO, T, NV, EPV, OCC) {T, NV, EPV, &launch_softmax<TI, TO, T, NV, EPV, OCC>}
#define FR_SM_SCALAR(TI, TO)                                              \
  FR_SM(TI, TO, 64, 16, 1, 4), FR_SM(TI, TO, 256, 16, 1, 4),              \
      FR_SM(TI, TO, 1024, 16, 1, 4), FR_SM(TI, TO, 1024, 64, 1, 4)

static const SoftmaxVariant kSmF32F32[] = {
    FR_SM(float, float, 64, 1, 4, 8),     FR_SM(float, float, 64, 2, 4, 8),
    FR_SM(float, float, 64, 4, 4, 8),     FR_SM(float, float, 64, 8, 4, 6),
    FR_SM(float, float, 64, 16, 4, 4),    FR_SM(float, float, 256, 8, 4, 6),
    FR_SM(float, float, 512, 8, 4, 6),    FR_SM(float, float, 1024, 8, 4, 4),
    FR_SM(float, float, 1024, 13, 4, 4),  FR_SM(float, float, 512, 25, 4, 4),
    FR_SM(float, float, 256, 50, 4, 2),
    FR_SM(float, float, 1024, 16, 4, 4),  FR_SM_SCALAR(float, float)};
// bf16 rows of 2049-4096: two wavefronts per row, 4 chunks per lane, 8 waves
// per SIMD (16384 x 4096 with cold buffers: 45.9 us against 47.2 us for a
// wavefront per row with 8 chunks)
static const SoftmaxVariant kSmBf16Bf16[] = {
    FR_SM(bf16_t, bf16_t, 64, 1, 8, 8),   FR_SM(bf16_t, bf16_t, 64, 2, 8, 8),
    FR_SM(bf16_t, bf16_t, 64, 4, 8, 6),   FR_SM(bf16_t, bf16_t, 128, 4, 8, 8),
    FR_SM(bf16_t, bf16_t, 64, 8, 8, 4),   FR_SM(bf16_t, bf16_t, 256, 2, 8, 8),
    FR_SM(bf16_t, bf16_t, 256, 4, 8, 6),  FR_SM(bf16_t, bf16_t, 512, 4, 8, 6),
    FR_SM(bf16_t, bf16_t, 1024, 4, 8, 4), FR_SM(bf16_t, bf16_t, 1024, 8, 8, 4),
    FR_SM(bf16_t, bf16_t, 512, 1, 8, 8),  FR_SM_SCALAR(bf16_t, bf16_t)};
static const SoftmaxVariant kSmF32Bf16[] = {
    FR_SM(float, bf16_t, 64, 1, 4, 8),    FR_SM(float, bf16_t, 64, 2, 4, 8),
    FR_SM(float, bf16_t, 64, 4, 4, 8),    FR_SM(float, bf16_t, 64, 8, 4, 6),
    FR_SM(float, bf16_t, 64, 16, 4, 4),   FR_SM(float, bf16_t, 256, 8, 4, 6),
    FR_SM(float, bf16_t, 512, 8, 4, 6),   FR_SM(float, bf16_t, 1024, 8, 4, 4),
    FR_SM(float, bf16_t, 1024, 16, 4, 4), FR_SM_SCALAR(float, bf16_t)};
static const SoftmaxVariant kSmBf16F32[] = {
    FR_SM(bf16_t, float, 64, 1, 8, 8),    FR_SM(bf16_t, float, 64, 2, 8, 8),
    FR_SM(bf16_t, float, 64, 4, 8, 6),    FR_SM(bf16_t, float, 64, 8, 8, 4),
    FR_SM(bf16_t, float, 256, 4, 8, 6),   FR_SM(bf16_t, float, 512, 4, 8, 6),
    FR_SM(bf16_t, float, 1024, 4, 8, 4),  FR_SM(bf16_t, float, 1024, 8, 8, 4),
    FR_SM_SCALAR(bf16_t, float)};

VariantSpan<SoftmaxVariant> softmax_variants(int in_bf16, int out_bf16) {
  if (!in_bf16 && !out_bf16) return {kSmF32F32, sizeof(kSmF32F32) / sizeof(kSmF32F32[0])};
  if (in_bf16 && out_bf16) return {kSmBf16Bf16, sizeof(kSmBf16Bf16) / sizeof(kSmBf16Bf16[0])};
  if (!in_bf16) return {kSmF32Bf16, sizeof(kSmF32Bf16) / sizeof(kSmF32Bf16[0])};
  return {kSmBf16F32, sizeof(kSmBf16F32) / sizeof(kSmBf16F32[0])};
}

}  // namespace fr
