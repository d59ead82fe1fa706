// LayerNorm (Welford moments) and residual-add + RMSNorm, one pass over
// memory per row.
//
// LayerNorm ("Engineering a CUDA Machine Learning Framework from Scratch",
// §3.2 Welford Single-Pass Normalization): each lane computes the exact
// (count, mean, M2) of its register-resident values; the triples are merged
// pairwise (Welford / Chan update) across the wavefront with DPP and across
// waves through LDS; the row is then normalised from the same registers.
//   y_j = (x_j - mu) * rstd * gamma_j + beta_j, rstd = 1/sqrt(M2/C + eps).
//
// Residual add + RMSNorm ("NexusGrad", Core Capabilities: RMSNorm, residual
// blocks, fused kernels): h = x + residual in fp32, the updated residual is
// stored as soon as it is formed, the sum of squares is reduced, and
//   y_j = h_j * rstd * w_j, rstd = 1/sqrt(sum h^2 / C + eps)
// is written from the unrounded h held in registers.
//
// The 128-bit path here requires every row to start on a 16-byte boundary
// (the per-column vectors are then aligned with the rows); other layouts use
// the scalar path (EPV == 1).
#include "fr_kernels.hpp"
#include "fr_device.hpp"

namespace fr {

template <typename Ts, int T, int NV, int EPV, int OCC>
__global__ __launch_bounds__(T == 64 ? 256 : T) __attribute__((amdgpu_waves_per_eu(OCC)))
void layernorm_kernel(const Ts* x, const Ts* gamma, const Ts* beta, Ts* y, float* mean,
                      float* rstd, int64_t rows, int cols, float eps) {
  constexpr int BLOCK = T == 64 ? 256 : T;
  constexpr int RPB = BLOCK / T;
  constexpr int NW = T / 64;
  __shared__ float xw[2][NW][3];

  const int wib = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int tid = T == 64 ? lane : (int)threadIdx.x;
  const int sub = T == 64 ? wib : 0;
  const int wave = T == 64 ? 0 : wib;
  int merges = 0;  // cross-wave merges so far: picks the LDS slot
  for (int64_t row = (int64_t)blockIdx.x * RPB + sub; row < rows;
       row += (int64_t)gridDim.x * RPB) {
    const Ts* xr = x + row * cols;
    Ts* yr = y + row * cols;
    const RowGeom<EPV> g(xr, cols);
    const bool full = g.nvec == T * NV;

    float v[NV][EPV];
    load_chunks<Ts, T, NV, EPV>(xr, g, tid, v, 0.f);
    const int ec = g.extra_col(tid);
    const float xe = ec >= 0 ? load1(xr + ec) : 0.f;

    // lane moments, exact two-pass over the lane's registers
    int nslots = NV;
    if (!full) {
      const int rem = g.nvec - tid;  // chunks i*T + tid < nvec  <=>  i < ceil(rem / T)
      nslots = rem <= 0 ? 0 : (rem + T - 1) / T;
      nslots = nslots < NV ? nslots : NV;
    }
    const int n_l = nslots * EPV + (ec >= 0 ? 1 : 0);
    float s0 = xe, s1 = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i)
#pragma unroll
      for (int k = 0; k < EPV; ++k) {
        if (k & 1) s1 += v[i][k]; else s0 += v[i][k];
      }
    const float mu_l = n_l > 0 ? (s0 + s1) / (float)n_l : 0.f;
    float q0 = 0.f, q1 = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const bool ok = full || i < nslots;
#pragma unroll
      for (int k = 0; k < EPV; ++k) {
        const float d = ok ? v[i][k] - mu_l : 0.f;
        if (k & 1) q1 = __builtin_fmaf(d, d, q1); else q0 = __builtin_fmaf(d, d, q0);
      }
    }
    if (ec >= 0) {
      const float d = xe - mu_l;
      q0 = __builtin_fmaf(d, d, q0);
    }
    WelfordState st{(float)n_l, mu_l, q0 + q1};
    st = wave_reduce(st, WelfordMerge{});
    if constexpr (NW > 1) st = block_merge<NW>(st, xw[merges++ & 1], wave, lane, WelfordMerge{});

    const float mu = st.mu;
    const float rs = 1.f / __builtin_sqrtf(st.m2 / (float)cols + eps);
    // per-column parameters are re-read by every row: cache hits
    if (g.nvec > 0) {
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        float ga[EPV], be[EPV];
        load_param_slot<Ts, T, EPV>(gamma, g, tid, i, ga);
        load_param_slot<Ts, T, EPV>(beta, g, tid, i, be);
#pragma unroll
        for (int k = 0; k < EPV; ++k) v[i][k] = __builtin_fmaf((v[i][k] - mu) * rs, ga[k], be[k]);
      }
      store_chunks<Ts, T, NV, EPV>(yr, g, tid, v);
    }
    if (ec >= 0) store1(yr + ec, __builtin_fmaf((xe - mu) * rs, load1(gamma + ec), load1(beta + ec)));
    if (wave == 0 && lane == 0) {
      if (mean) mean[row] = mu;
      if (rstd) rstd[row] = rs;
    }
  }
}

template <typename Ts, int T, int NV, int EPV, int OCC>
__global__ __launch_bounds__(T == 64 ? 256 : T) __attribute__((amdgpu_waves_per_eu(OCC)))
void add_rmsnorm_kernel(const Ts* x, const Ts* res, const Ts* w, Ts* y, Ts* res_out, int64_t rows,
                        int cols, float eps) {
  constexpr int BLOCK = T == 64 ? 256 : T;
  constexpr int RPB = BLOCK / T;
  constexpr int NW = T / 64;
  __shared__ float xw[2][NW][1];

  const int wib = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int tid = T == 64 ? lane : (int)threadIdx.x;
  const int sub = T == 64 ? wib : 0;
  const int wave = T == 64 ? 0 : wib;
  int merges = 0;  // cross-wave merges so far: picks the LDS slot
  for (int64_t row = (int64_t)blockIdx.x * RPB + sub; row < rows;
       row += (int64_t)gridDim.x * RPB) {
    const int64_t off = row * cols;
    const RowGeom<EPV> g(x + off, cols);

    float h[NV][EPV], r[NV][EPV];
    load_chunks<Ts, T, NV, EPV>(x + off, g, tid, h, 0.f);
    load_chunks<Ts, T, NV, EPV>(res + off, g, tid, r, 0.f);
    const int ec = g.extra_col(tid);
    float he = ec >= 0 ? load1(x + off + ec) + load1(res + off + ec) : 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i)
#pragma unroll
      for (int k = 0; k < EPV; ++k) h[i][k] += r[i][k];
    if (res_out) {  // updated residual, rounded once at the store
      store_chunks<Ts, T, NV, EPV>(res_out + off, g, tid, h);
      if (ec >= 0) store1(res_out + off + ec, he);
    }

    float q0 = he * he, q1 = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i)
#pragma unroll
      for (int k = 0; k < EPV; ++k) {
        if (k & 1) q1 = __builtin_fmaf(h[i][k], h[i][k], q1);
        else q0 = __builtin_fmaf(h[i][k], h[i][k], q0);
      }
    SumState st{q0 + q1};
    st = wave_reduce(st, SumMerge{});
    if constexpr (NW > 1) st = block_merge<NW>(st, xw[merges++ & 1], wave, lane, SumMerge{});

    const float rs = 1.f / __builtin_sqrtf(st.s / (float)cols + eps);
    if (g.nvec > 0) {
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        float wt[EPV];
        load_param_slot<Ts, T, EPV>(w, g, tid, i, wt);
#pragma unroll
        for (int k = 0; k < EPV; ++k) h[i][k] = h[i][k] * rs * wt[k];
      }
      store_chunks<Ts, T, NV, EPV>(y + off, g, tid, h);
    }
    if (ec >= 0) store1(y + off + ec, he * rs * load1(w + ec));
  }
}

template <typename Ts, int T, int NV, int EPV, int OCC>
static hipError_t launch_layernorm(const void* x, const void* gamma, const void* beta, void* y,
                                   float* mean, float* rstd, int64_t rows, int cols, float eps,
                                   hipStream_t s) {
  constexpr int BLOCK = T == 64 ? 256 : T;
  constexpr int RPB = BLOCK / T;
  const int64_t blocks = (rows + RPB - 1) / RPB;
  const unsigned grid = (unsigned)(blocks < kMaxGrid ? blocks : kMaxGrid);
  return launch_kernel(&layernorm_kernel<Ts, T, NV, EPV, OCC>, dim3(grid), dim3(BLOCK), s,
                     static_cast<const Ts*>(x), static_cast<const Ts*>(gamma),
                     static_cast<const Ts*>(beta), static_cast<Ts*>(y), mean, rstd, rows, cols, eps);
}

template <typename Ts, int T, int NV, int EPV, int OCC>
static hipError_t launch_rmsnorm(const void* x, const void* res, const void* w, void* y,
                                 void* res_out, int64_t rows, int cols, float eps, hipStream_t s) {
  constexpr int BLOCK = T == 64 ? 256 : T;
  constexpr int RPB = BLOCK / T;
  const int64_t blocks = (rows + RPB - 1) / RPB;
  const unsigned grid = (unsigned)(blocks < kMaxGrid ? blocks : kMaxGrid);
  return launch_kernel(&add_rmsnorm_kernel<Ts, T, NV, EPV, OCC>, dim3(grid), dim3(BLOCK), s,
                     static_cast<const Ts*>(x), static_cast<const Ts*>(res),
                     static_cast<const Ts*>(w), static_cast<Ts*>(y), static_cast<Ts*>(res_out), rows,
                     cols, eps);
}

#define FR_LN(TS, T, NV, EPV, OCC) {T, NV, EPV, &launch_layernorm<TS, T, NV, EPV, OCC>}
#define FR_RN(TS, T, NV, EPV, OCC) {T, NV, EPV, &launch_rmsnorm<TS, T, NV, EPV, OCC>}

static const LayerNormVariant kLnF32[] = {
    FR_LN(float, 64, 1, 4, 8),   FR_LN(float, 64, 2, 4, 8),    FR_LN(float, 64, 4, 4, 6),
    FR_LN(float, 64, 8, 4, 4),   FR_LN(float, 256, 4, 4, 6),   FR_LN(float, 256, 8, 4, 4),
    FR_LN(float, 512, 8, 4, 4),  FR_LN(float, 1024, 8, 4, 4),  FR_LN(float, 1024, 16, 4, 2),
    FR_LN(float, 64, 16, 1, 4),  FR_LN(float, 256, 16, 1, 4),  FR_LN(float, 1024, 16, 1, 4),
    FR_LN(float, 1024, 64, 1, 2)};
static const LayerNormVariant kLnBf16[] = {
    FR_LN(bf16_t, 64, 1, 8, 8),  FR_LN(bf16_t, 64, 2, 8, 8),   FR_LN(bf16_t, 64, 4, 8, 4),
    FR_LN(bf16_t, 256, 2, 8, 8), FR_LN(bf16_t, 256, 4, 8, 4),  FR_LN(bf16_t, 512, 4, 8, 4),
    FR_LN(bf16_t, 1024, 4, 8, 4), FR_LN(bf16_t, 1024, 8, 8, 2), FR_LN(bf16_t, 64, 16, 1, 4),
    FR_LN(bf16_t, 256, 16, 1, 4), FR_LN(bf16_t, 1024, 16, 1, 4), FR_LN(bf16_t, 1024, 64, 1, 2)};
static const RmsNormVariant kRnF32[] = {
    FR_RN(float, 64, 1, 4, 8),   FR_RN(float, 64, 2, 4, 8),    FR_RN(float, 64, 4, 4, 8),
    FR_RN(float, 64, 8, 4, 4),   FR_RN(float, 256, 4, 4, 8),   FR_RN(float, 256, 8, 4, 4),
    FR_RN(float, 512, 8, 4, 4),  FR_RN(float, 1024, 8, 4, 4),  FR_RN(float, 1024, 16, 4, 2),
    FR_RN(float, 64, 16, 1, 4),  FR_RN(float, 256, 16, 1, 4),  FR_RN(float, 1024, 16, 1, 4),
    FR_RN(float, 1024, 64, 1, 2)};
static const RmsNormVariant kRnBf16[] = {
    FR_RN(bf16_t, 64, 1, 8, 8),  FR_RN(bf16_t, 64, 2, 8, 8),   FR_RN(bf16_t, 64, 4, 8, 4),
    FR_RN(bf16_t, 256, 2, 8, 8), FR_RN(bf16_t, 512, 2, 8, 8),  FR_RN(bf16_t, 256, 4, 8, 4),
    FR_RN(bf16_t, 512, 4, 8, 4), FR_RN(bf16_t, 1024, 1, 8, 8), FR_RN(bf16_t, 1024, 4, 8, 4),
    FR_RN(bf16_t, 1024, 8, 8, 2), FR_RN(bf16_t, 64, 16, 1, 4), FR_RN(bf16_t, 256, 16, 1, 4),
    FR_RN(bf16_t, 1024, 16, 1, 4), FR_RN(bf16_t, 1024, 64, 1, 2)};

VariantSpan<LayerNormVariant> layernorm_variants(int bf16) {
  if (bf16) return {kLnBf16, sizeof(kLnBf16) / sizeof(kLnBf16[0])};
  return {kLnF32, sizeof(kLnF32) / sizeof(kLnF32[0])};
}
VariantSpan<RmsNormVariant> rmsnorm_variants(int bf16) {
  if (bf16) return {kRnBf16, sizeof(kRnBf16) / sizeof(kRnBf16[0])};
  return {kRnF32, sizeof(kRnF32) / sizeof(kRnF32[0])};
}

}  // namespace fr
