// Softmax cross-entropy, forward and backward in one pass over memory
// ("Engineering a CUDA Machine Learning Framework from Scratch", §2.1: loss
// gradients fused into registers; "GPU Programming for Machine Learning",
// Module 3: cross-entropy loss).
//
// Per row: the online-softmax state (M, S) of the logits (as in softmax.hip,
// fp32 path, exponentials kept in registers), then
//   loss    = M + ln S - x[label]
//   grad_j  = exp(x_j - M) / S - [j == label]
//   argmax  = smallest j with x_j == M (optional)
// The lane that owns the label column reads the label logit, writes the
// loss, and overwrites its stored p with p - 1. A label outside [0, cols)
// gives a NaN loss and an unmodified softmax row.
#include "fr_kernels.hpp"
#include "softmax_core.hpp"

namespace fr {

// Lane of the row owner that holds column `c` (0 <= c < cols): a head or
// tail column sits in the extra slot of lane c or head + (c - body_end); a
// body column in chunk (c - head) / EPV, held by lane chunk % T.
template <int T, int EPV>
__device__ __forceinline__ int owner_lane(int c, const RowGeom<EPV>& g) {
  const int body_end = g.head + g.nvec * EPV;
  if (c < g.head) return c;
  if (c >= body_end) return g.head + (c - body_end);
  return ((c - g.head) / EPV) % T;
}

template <typename Tin, int T, int NV, int EPV, int OCC, bool ARGMAX>
__global__ __launch_bounds__(T == 64 ? 256 : T) __attribute__((amdgpu_waves_per_eu(OCC)))
void xent_kernel(const Tin* x, const int32_t* labels, float* loss, Tin* grad, int32_t* argmax,
                 int64_t rows, int cols) {
  constexpr int BLOCK = T == 64 ? 256 : T;
  constexpr int RPB = BLOCK / T;
  constexpr int NW = T / 64;
  using State = typename std::conditional<ARGMAX, MaxSumIdxState, MaxSumState>::type;
  using Merge = typename std::conditional<ARGMAX, MaxSumIdxMerge, MaxSumMerge<false>>::type;
  constexpr int NF = sizeof(State) / sizeof(float);
  __shared__ float xw[2][NW][NF];

  const int wib = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int tid = T == 64 ? lane : (int)threadIdx.x;
  const int sub = T == 64 ? wib : 0;
  const int wave = T == 64 ? 0 : wib;
  int it = 0;
  for (int64_t row = (int64_t)blockIdx.x * RPB + sub; row < rows;
       row += (int64_t)gridDim.x * RPB, ++it) {
    const Tin* xr = x + row * cols;
    Tin* gr = grad + row * cols;
    const RowGeom<EPV> g(xr, cols);

    float v[NV][EPV];
    load_chunks<Tin, T, NV, EPV>(xr, g, tid, v, kNegInf);
    const int ec = g.extra_col(tid);
    float xe = ec >= 0 ? load1(xr + ec) : kNegInf;

    // The label column is handled by the one lane that owns it (the lane of
    // the row owner that loads that column). It reads the label logit with
    // its own load, before any of its stores: in-place calls (grad == logits)
    // stay correct because a lane's accesses to one address keep their order.
    const int label = __builtin_amdgcn_readfirstlane(labels[row]);
    const bool valid = label >= 0 && label < cols;
    const bool label_lane = valid && owner_lane<T, EPV>(label, g) == tid;
    float x_label = 0.f;
    if (label_lane) x_label = load1(xr + label);

    const float m = lane_max<NV, EPV>(v, xe);
    State st;
    if constexpr (ARGMAX) {
      // smallest column of this lane holding its maximum
      float best = 3.0e38f;
#pragma unroll
      for (int i = 0; i < NV; ++i)
#pragma unroll
        for (int k = 0; k < EPV; ++k) {
          const float col = (float)((uint32_t)g.head + (uint32_t)(i * T + tid) * EPV + k);
          best = (v[i][k] == m && col < best) ? col : best;
        }
      if (ec >= 0 && xe == m && (float)ec < best) best = (float)ec;
      st.idx = best;
    }
    {
      const MaxSumState ms = lane_exp_nat<NV, EPV>(v, xe, m);  // e_j replaces x_j
      st.m = ms.m;
      st.s = ms.s;
    }
    st = wave_reduce(st, Merge{});
    if constexpr (NW > 1) st = block_merge<NW>(st, xw[it & 1], wave, lane, Merge{});

    const float f = nat_scale(m, st.m, st.s);
#pragma unroll
    for (int i = 0; i < NV; ++i)
#pragma unroll
      for (int k = 0; k < EPV; ++k) v[i][k] *= f;
    xe *= f;
    store_chunks<Tin, T, NV, EPV>(gr, g, tid, v);
    if (ec >= 0) store1(gr + ec, xe);

    if (label_lane) {
      // overwrite the label element with p - 1 (after this lane's own store
      // of p to the same address), and write the loss
      const float p = exp_acc(x_label - st.m) / st.s;
      store1(gr + label, p - 1.f);
      loss[row] = st.m + logf(st.s) - x_label;
    } else if (!valid && tid == 0) {
      loss[row] = __builtin_nanf("");
    }
    if constexpr (ARGMAX) {
      if (tid == 0) argmax[row] = (int32_t)st.idx;
    }
  }
}

template <typename Tin, int T, int NV, int EPV, int OCC, bool ARGMAX>
static hipError_t launch_xent(const void* x, const int32_t* labels, float* loss, void* grad,
                              int32_t* argmax, int64_t rows, int cols, hipStream_t s) {
  constexpr int BLOCK = T == 64 ? 256 : T;
  constexpr int RPB = BLOCK / T;
  const int64_t blocks = (rows + RPB - 1) / RPB;
  const unsigned grid = (unsigned)(blocks < kMaxGrid ? blocks : kMaxGrid);
  return launch_kernel(&xent_kernel<Tin, T, NV, EPV, OCC, ARGMAX>, dim3(grid), dim3(BLOCK), s,
                     static_cast<const Tin*>(x), labels, loss, static_cast<Tin*>(grad), argmax, rows,
                     cols);
}

#define FR_XE(T, NV, EPV, OCC, AM) {T, NV, EPV, &launch_xent<float, T, NV, EPV, OCC, AM>}
#define FR_XE_TABLE(AM)                                                                   \
  {FR_XE(64, 1, 4, 8, AM),     FR_XE(64, 2, 4, 8, AM),     FR_XE(64, 4, 4, 8, AM),        \
   FR_XE(64, 8, 4, 6, AM),     FR_XE(64, 16, 4, 4, AM),    FR_XE(256, 8, 4, 6, AM),       \
   FR_XE(512, 8, 4, 6, AM),    FR_XE(1024, 8, 4, 4, AM),   FR_XE(1024, 13, 4, 4, AM),     \
   FR_XE(512, 25, 4, 4, AM),   FR_XE(256, 50, 4, 2, AM),   FR_XE(1024, 16, 4, 4, AM),     \
   FR_XE(64, 16, 1, 4, AM),    FR_XE(256, 16, 1, 4, AM),   FR_XE(1024, 16, 1, 4, AM),     \
   FR_XE(1024, 64, 1, 4, AM)}

static const XentVariant kXe[] = FR_XE_TABLE(false);
static const XentVariant kXeArgmax[] = FR_XE_TABLE(true);

VariantSpan<XentVariant> xent_variants(int bf16, int with_argmax) {
  if (bf16) return {nullptr, 0};
  if (with_argmax) return {kXeArgmax, sizeof(kXeArgmax) / sizeof(kXeArgmax[0])};
  return {kXe, sizeof(kXe) / sizeof(kXe[0])};
}

}  // namespace fr
