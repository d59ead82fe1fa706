// Split-row LayerNorm and residual-add + RMSNorm: rows of any width up to
// 2^24, several workgroups per row.
//
// As the split softmax (split.hip): a row is cut into segments of `seg`
// columns (a multiple of 32: each segment keeps its row's address phase),
// workgroup (row, segment) owns one segment in registers.
//   pass 1 (norm_split_stats_kernel): the segment's partial state — the exact
//     (count, mean, M2) of its values for LayerNorm ("Engineering a CUDA
//     Machine Learning Framework from Scratch", §3.2 Welford Single-Pass
//     Normalization: partial moments merged pairwise), the sum of h^2,
//     h = x + residual in fp32, for RMSNorm — into the workspace
//     [rows][segments];
//   pass 2 (norm_split_apply_kernel): every workgroup of a row merges the
//     row's partials in segment order (the same bits in all of them), re-reads
//     its segment and writes y (and the updated residual, and the row's mean
//     and rstd from segment 0).
// The updated residual is written in pass 2, after its segment's residual has
// been re-read, so residual_out may be the residual itself. Both also have
// the one-pass form of split.hip (norm_split_coop_kernel: the states
// exchanged within one launch, the segment written from the registers).
#include "coop.hpp"
#include "fr_device.hpp"
#include "fr_kernels.hpp"

namespace fr {

namespace {

// Segment `sg` of a row: [c0, c0 + len).
struct NormSegment {
  int c0, len;
  __device__ __forceinline__ NormSegment(int sg, int seg, int cols)
      : c0(sg * seg), len(cols - sg * seg < seg ? cols - sg * seg : seg) {}
};

// Exact (count, mean, M2) of this lane's values (slots past the segment end
// hold 0 and are left out), two passes over the registers.
template <int T, int NV, int EPV, int AL>
__device__ __forceinline__ WelfordState lane_moments(const float (&v)[NV][EPV], float xe, int ec,
                                                     const RowGeom<EPV, AL>& g, int tid) {
  const bool full = g.nvec == T * NV;
  int nslots = NV;
  if (!full) {
    const int rem = g.nvec - tid;
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
  return {(float)n_l, mu_l, q0 + q1};
}

}  // namespace

// ------------------------------------------------------------------ pass 1

// (the bodies: work items w0, w0 + wstride, ... of rows * nseg)
template <typename Ts, int T, int NV, int EPV, bool RMS>
__device__ __forceinline__ void norm_split_stats_body(const Ts* x, const Ts* res, int64_t rows,
                                                      int cols, int seg, int nseg, float4* part,
                                                      int64_t w0, int64_t wstride) {
  constexpr int NW = T / 64;
  __shared__ float xw[2][NW][RMS ? 1 : 3];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int tid = threadIdx.x;
  const int64_t work = rows * nseg;
  int merges = 0;  // cross-wave merges so far: picks the LDS slot
  for (int64_t w = w0; w < work; w += wstride) {
    const int64_t row = w / nseg;
    const int sg = (int)(w - row * nseg);
    const NormSegment sgm(sg, seg, cols);
    const int64_t off = row * cols + sgm.c0;
    const RowGeom<EPV> g(x + off, sgm.len);
    const int ec = g.extra_col(tid);
    float v[NV][EPV];
    if constexpr (RMS) {
      float r[NV][EPV];
      load_chunks2<Ts, T, NV, EPV, kHeadAlign, kPass1NT>(x + off, res + off, g, tid, v, r, 0.f);
      float he = load_extra(x + off, ec, 0.f) + load_extra(res + off, ec, 0.f);
      float q0 = he * he, q1 = 0.f;
#pragma unroll
      for (int i = 0; i < NV; ++i)
#pragma unroll
        for (int k = 0; k < EPV; ++k) {
          const float h = v[i][k] + r[i][k];
          if (k & 1) q1 = __builtin_fmaf(h, h, q1); else q0 = __builtin_fmaf(h, h, q0);
        }
      SumState st{q0 + q1};
      st = wave_reduce(st, SumMerge{});
      if constexpr (NW > 1) st = block_merge<NW>(st, xw[merges++ & 1], wave, lane, SumMerge{});
      if (tid == 0) part[w] = float4{st.s, 0.f, 0.f, 0.f};
    } else {
      load_chunks<Ts, T, NV, EPV, kHeadAlign, kPass1NT>(x + off, g, tid, v, 0.f);
      const float xe = load_extra(x + off, ec, 0.f);
      WelfordState st = lane_moments<T, NV, EPV>(v, xe, ec, g, tid);
      st = wave_reduce(st, WelfordMerge{});
      if constexpr (NW > 1) st = block_merge<NW>(st, xw[merges++ & 1], wave, lane, WelfordMerge{});
      if (tid == 0) part[w] = float4{st.n, st.mu, st.m2, 0.f};
    }
  }
}

// ------------------------------------------------------------------ pass 2

// The row's merged partials: lane j merges partials j, j + T, ... in order,
// then the DPP tree and the LDS merge (a fixed order).
template <int T, typename S, typename M, typename F>
__device__ __forceinline__ S merge_partials(const float4* part, int64_t row, int nseg, S id,
                                            F from, float (*slot)[sizeof(S) / sizeof(float)],
                                            int wave, int lane, int tid, M merge) {
  constexpr int NW = T / 64;
  S st = id;
  for (int j = tid; j < nseg; j += T) st = merge(st, from(part[row * nseg + j]));
  st = wave_reduce(st, merge);
  if constexpr (NW > 1) st = block_merge<NW>(st, slot, wave, lane, merge);
  return st;
}

// LayerNorm: p1 = gamma, p2 = beta, res / res_out unused. RMSNorm: p1 = the
// weight, p2 / mean / rstd unused.
template <typename Ts, int T, int NV, int EPV, bool RMS>
__device__ __forceinline__ void norm_split_apply_body(const Ts* x, const Ts* res, const Ts* p1,
                                                      const Ts* p2, Ts* y, Ts* res_out, float* mean,
                                                      float* rstd, int64_t rows, int cols, int seg,
                                                      int nseg, const float4* part, float eps,
                                                      int64_t w0, int64_t wstride) {
  constexpr int NW = T / 64;
  __shared__ float xw[2][NW][RMS ? 1 : 3];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int tid = threadIdx.x;
  const int64_t work = rows * nseg;
  int merges = 0;  // cross-wave merges so far: picks the LDS slot
  for (int64_t w = w0; w < work; w += wstride) {
    const int64_t row = w / nseg;
    const int sg = (int)(w - row * nseg);
    const NormSegment sgm(sg, seg, cols);
    const int64_t off = row * cols + sgm.c0;
    const RowGeom<EPV> g(x + off, sgm.len);
    const int ec = g.extra_col(tid);
    const Ts* q1 = p1 + sgm.c0;
    float v[NV][EPV];
    if constexpr (RMS) {
      const SumState st = merge_partials<T>(
          part, row, nseg, SumState{0.f}, [](float4 p) { return SumState{p.x}; },
          xw[merges++ & 1], wave, lane, tid, SumMerge{});
      const float rs = 1.f / __builtin_sqrtf(st.s / (float)cols + eps);
      float r[NV][EPV];
      load_chunks2<Ts, T, NV, EPV>(x + off, res + off, g, tid, v, r, 0.f);
      float he = load_extra(x + off, ec, 0.f) + load_extra(res + off, ec, 0.f);
#pragma unroll
      for (int i = 0; i < NV; ++i)
#pragma unroll
        for (int k = 0; k < EPV; ++k) v[i][k] += r[i][k];
      if (res_out) {  // updated residual, rounded once at the store
        store_chunks<Ts, T, NV, EPV>(res_out + off, g, tid, v);
        if (ec >= 0) store1(res_out + off + ec, he);
      }
      if (g.nvec > 0) {
#pragma unroll
        for (int i = 0; i < NV; ++i) {
          float wt[EPV];
          load_param_slot<Ts, T, EPV>(q1, g, tid, i, wt);
#pragma unroll
          for (int k = 0; k < EPV; ++k) v[i][k] = v[i][k] * rs * wt[k];
        }
        store_chunks<Ts, T, NV, EPV>(y + off, g, tid, v);
      }
      if (ec >= 0) store1(y + off + ec, he * rs * load1(q1 + ec));
    } else {
      const WelfordState st = merge_partials<T>(
          part, row, nseg, WelfordState{0.f, 0.f, 0.f},
          [](float4 p) { return WelfordState{p.x, p.y, p.z}; }, xw[merges++ & 1], wave, lane, tid,
          WelfordMerge{});
      const float mu = st.mu;
      const float rs = 1.f / __builtin_sqrtf(st.m2 / (float)cols + eps);
      load_chunks<Ts, T, NV, EPV>(x + off, g, tid, v, 0.f);
      const float xe = load_extra(x + off, ec, 0.f);
      const Ts* q2 = p2 + sgm.c0;
      if (g.nvec > 0) {
#pragma unroll
        for (int i = 0; i < NV; ++i) {
          float ga[EPV], be[EPV];
          load_param_slot<Ts, T, EPV>(q1, g, tid, i, ga);
          load_param_slot<Ts, T, EPV>(q2, g, tid, i, be);
#pragma unroll
          for (int k = 0; k < EPV; ++k) v[i][k] = __builtin_fmaf((v[i][k] - mu) * rs, ga[k], be[k]);
        }
        store_chunks<Ts, T, NV, EPV>(y + off, g, tid, v);
      }
      if (ec >= 0) store1(y + off + ec, __builtin_fmaf((xe - mu) * rs, load1(q1 + ec), load1(q2 + ec)));
      if (sg == 0 && tid == 0) {
        if (mean) mean[row] = mu;
        if (rstd) rstd[row] = rs;
      }
    }
  }
}

template <typename Ts, int T, int NV, int EPV, int OCC, bool RMS>
__global__ __launch_bounds__(T) __attribute__((amdgpu_waves_per_eu(OCC)))
void norm_split_stats_kernel(const Ts* x, const Ts* res, int64_t rows, int cols, int seg,
                             int nseg, float4* part) {
  norm_split_stats_body<Ts, T, NV, EPV, RMS>(x, res, rows, cols, seg, nseg, part, blockIdx.x,
                                             gridDim.x);
}

template <typename Ts, int T, int NV, int EPV, int OCC, bool RMS>
__global__ __launch_bounds__(T) __attribute__((amdgpu_waves_per_eu(OCC)))
void norm_split_apply_kernel(const Ts* x, const Ts* res, const Ts* p1, const Ts* p2, Ts* y,
                             Ts* res_out, float* mean, float* rstd, int64_t rows, int cols,
                             int seg, int nseg, const float4* part, float eps) {
  norm_split_apply_body<Ts, T, NV, EPV, RMS>(x, res, p1, p2, y, res_out, mean, rstd, rows, cols,
                                             seg, nseg, part, eps, blockIdx.x, gridDim.x);
}

// Pass 2 of one row batch (rows ra from row r_a) and pass 1 of the next (rows
// rn from row r_n) in one launch: they touch different rows; workgroups
// [0, n_apply) take the first batch's segments, the rest the next batch's.
template <typename Ts, int T, int NV, int EPV, int OCC, bool RMS>
__global__ __launch_bounds__(T) __attribute__((amdgpu_waves_per_eu(OCC)))
void norm_split_apply_stats_kernel(const Ts* x, const Ts* res, const Ts* p1, const Ts* p2, Ts* y,
                                   Ts* res_out, float* mean, float* rstd, int cols, int seg,
                                   int nseg, float4* part, float eps, int64_t r_a, int64_t ra,
                                   int64_t r_n, int64_t rn, unsigned n_apply) {
  if (blockIdx.x < n_apply) {
    const int64_t e0 = r_a * cols;
    norm_split_apply_body<Ts, T, NV, EPV, RMS>(
        x + e0, res ? res + e0 : nullptr, p1, p2, y + e0, res_out ? res_out + e0 : nullptr,
        mean ? mean + r_a : nullptr, rstd ? rstd + r_a : nullptr, ra, cols, seg, nseg,
        part + r_a * nseg, eps, blockIdx.x, n_apply);
  } else {
    const int64_t e0 = r_n * cols;
    norm_split_stats_body<Ts, T, NV, EPV, RMS>(x + e0, res ? res + e0 : nullptr, rn, cols, seg,
                                               nseg, part + r_n * nseg, blockIdx.x - n_apply,
                                               gridDim.x - n_apply);
  }
}

// ---------------------------------------------------------- one-pass form
// One workgroup per (row, segment) work item exchanging its segment's state
// with the row's others (coop.hpp) instead of a second read: it loads its
// segment (and residual) into registers, takes the state as pass 1 does,
// posts it — LayerNorm: word 0 = {mean, count} (count >= 1: never zero),
// word 1 = {M2, 1}; RMSNorm: {sum of h^2, 1} — waits for the row's others,
// merges them in segment order (lane j holds segment j's, one DPP tree: the
// same bits in every workgroup of the row) and writes y (and the updated
// residual, and the row's mean and rstd from segment 0) from the registers.
// Each workgroup writes only its own segment, after reading it: y may be x
// and residual_out the residual.
template <typename Ts, int T, int NV, int EPV, int OCC, bool RMS>
__global__ __launch_bounds__(T) __attribute__((amdgpu_waves_per_eu(OCC)))
void norm_split_coop_kernel(const Ts* x, const Ts* res, const Ts* p1, const Ts* p2, Ts* y,
                            Ts* res_out, float* mean, float* rstd, int64_t rows, int cols, int seg,
                            int nseg, float eps, uint64_t* slots, uint32_t* ctl, int spin_limit) {
  constexpr int NW = T / 64;
  constexpr int NWD = RMS ? 1 : 2;  // words posted per segment
  __shared__ float xw[2][NW][RMS ? 1 : 3];
  __shared__ float team[kCoopMaxSegments][4];
  __shared__ uint32_t ticket;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int tid = threadIdx.x;
  const int64_t w = coop_ticket(ctl, &ticket);  // < rows * nseg: one per workgroup
  const int64_t row = w / nseg;
  const int sg = (int)(w - row * nseg);
  const NormSegment sgm(sg, seg, cols);
  const int64_t off = row * cols + sgm.c0;
  const RowGeom<EPV> g(x + off, sgm.len);
  const int ec = g.extra_col(tid);
  const Ts* q1 = p1 + sgm.c0;
  uint64_t* row_slots = slots + (size_t)row * nseg * 2;
  float v[NV][EPV];
  if constexpr (RMS) {
    float r[NV][EPV];
    load_chunks2<Ts, T, NV, EPV>(x + off, res + off, g, tid, v, r, 0.f);
    const float he = load_extra(x + off, ec, 0.f) + load_extra(res + off, ec, 0.f);
    float s0 = he * he, s1 = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i)
#pragma unroll
      for (int k = 0; k < EPV; ++k) {
        v[i][k] += r[i][k];  // h, in fp32
        if (k & 1) s1 = __builtin_fmaf(v[i][k], v[i][k], s1);
        else s0 = __builtin_fmaf(v[i][k], v[i][k], s0);
      }
    SumState st{s0 + s1};
    st = wave_reduce(st, SumMerge{});
    if constexpr (NW > 1) st = block_merge<NW>(st, xw[0], wave, lane, SumMerge{});
    coop_post<NWD>(row_slots, sg, coop_word(st.s, 1.f), 0);
    if (wave == 0) coop_wait<NWD>(row_slots, nseg, ctl + 1, spin_limit, lane, team);
    lds_barrier();
    SumState tot{0.f};
    if (lane < nseg) tot = SumState{team[lane][0]};
    tot = wave_reduce(tot, SumMerge{});
    const float rs = 1.f / __builtin_sqrtf(tot.s / (float)cols + eps);
    if (res_out) {  // updated residual, rounded once at the store
      store_chunks<Ts, T, NV, EPV>(res_out + off, g, tid, v);
      if (ec >= 0) store1(res_out + off + ec, he);
    }
    if (g.nvec > 0) {
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        float wt[EPV];
        load_param_slot<Ts, T, EPV>(q1, g, tid, i, wt);
#pragma unroll
        for (int k = 0; k < EPV; ++k) v[i][k] = v[i][k] * rs * wt[k];
      }
      store_chunks<Ts, T, NV, EPV>(y + off, g, tid, v);
    }
    if (ec >= 0) store1(y + off + ec, he * rs * load1(q1 + ec));
  } else {
    load_chunks<Ts, T, NV, EPV>(x + off, g, tid, v, 0.f);
    const float xe = load_extra(x + off, ec, 0.f);
    WelfordState st = lane_moments<T, NV, EPV>(v, xe, ec, g, tid);
    st = wave_reduce(st, WelfordMerge{});
    if constexpr (NW > 1) st = block_merge<NW>(st, xw[0], wave, lane, WelfordMerge{});
    coop_post<NWD>(row_slots, sg, coop_word(st.mu, st.n), coop_word(st.m2, 1.f));
    if (wave == 0) coop_wait<NWD>(row_slots, nseg, ctl + 1, spin_limit, lane, team);
    lds_barrier();
    WelfordState tot{0.f, 0.f, 0.f};
    if (lane < nseg) tot = WelfordState{team[lane][1], team[lane][0], team[lane][2]};
    tot = wave_reduce(tot, WelfordMerge{});
    const float mu = tot.mu;
    const float rs = 1.f / __builtin_sqrtf(tot.m2 / (float)cols + eps);
    const Ts* q2 = p2 + sgm.c0;
    if (g.nvec > 0) {
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        float ga[EPV], be[EPV];
        load_param_slot<Ts, T, EPV>(q1, g, tid, i, ga);
        load_param_slot<Ts, T, EPV>(q2, g, tid, i, be);
#pragma unroll
        for (int k = 0; k < EPV; ++k) v[i][k] = __builtin_fmaf((v[i][k] - mu) * rs, ga[k], be[k]);
      }
      store_chunks<Ts, T, NV, EPV>(y + off, g, tid, v);
    }
    if (ec >= 0) store1(y + off + ec, __builtin_fmaf((xe - mu) * rs, load1(q1 + ec), load1(q2 + ec)));
    if (sg == 0 && tid == 0) {
      if (mean) mean[row] = mu;
      if (rstd) rstd[row] = rs;
    }
  }
}

// --------------------------------------------------------------- launchers

template <typename Ts, int T, int NV, int EPV, int OCC, bool RMS>
static hipError_t launch_norm_split(const void* x, const void* res, const void* p1, const void* p2,
                                    void* y, void* res_out, float* mean, float* rstd, int64_t rows,
                                    int cols, float eps, float4* part, int64_t part_bytes,
                                    bool one_pass, hipStream_t s) {
  constexpr int SEG = T * NV * EPV;
  const int nseg = (cols + SEG - 1) / SEG;
  const Ts* xi = static_cast<const Ts*>(x);
  const Ts* ri = static_cast<const Ts*>(res);
  Ts* yo = static_cast<Ts*>(y);
  Ts* ro = static_cast<Ts*>(res_out);
  if (one_pass && coop_applies(rows, nseg, part_bytes)) {
    hipError_t e = launch_coop_clear(part, rows, nseg, s);
    if (e != hipSuccess) return e;
    return launch_kernel(&norm_split_coop_kernel<Ts, T, NV, EPV, OCC, RMS>,
                         dim3((unsigned)(rows * nseg)), dim3(T), s, xi, ri, static_cast<const Ts*>(p1),
                         static_cast<const Ts*>(p2), yo, ro, mean, rstd, rows, cols, SEG, nseg, eps,
                         reinterpret_cast<uint64_t*>(part + 1), reinterpret_cast<uint32_t*>(part),
                         coop_spin_limit());
  }
  const int64_t batch = split_batch_rows(rows, (int64_t)cols * (RMS ? 2 : 1) * sizeof(Ts));
  auto grid_of = [&](int64_t nr) {
    const int64_t work = nr * nseg;
    return (unsigned)(work < kMaxGrid ? work : kMaxGrid);
  };
  // pass 1 of the first batch; per further batch, pass 2 of the one before
  // with pass 1 of this one; then pass 2 of the last
  int64_t r0 = 0, nr = rows < batch ? rows : batch;
  hipError_t e = launch_kernel(&norm_split_stats_kernel<Ts, T, NV, EPV, OCC, RMS>, dim3(grid_of(nr)),
                               dim3(T), s, xi, ri, nr, cols, SEG, nseg, part);
  if (e != hipSuccess) return e;
  for (int64_t r1 = batch; r1 < rows; r1 += batch) {
    const int64_t n1 = rows - r1 < batch ? rows - r1 : batch;
    const unsigned na = grid_of(nr), ns = grid_of(n1);
    e = launch_kernel(&norm_split_apply_stats_kernel<Ts, T, NV, EPV, OCC, RMS>, dim3(na + ns),
                      dim3(T), s, xi, ri, static_cast<const Ts*>(p1), static_cast<const Ts*>(p2),
                      yo, ro, mean, rstd, cols, SEG, nseg, part, eps, r0, nr, r1, n1, na);
    if (e != hipSuccess) return e;
    r0 = r1;
    nr = n1;
  }
  const int64_t e0 = r0 * cols;
  return launch_kernel(&norm_split_apply_kernel<Ts, T, NV, EPV, OCC, RMS>, dim3(grid_of(nr)),
                       dim3(T), s, xi + e0, ri ? ri + e0 : nullptr, static_cast<const Ts*>(p1),
                       static_cast<const Ts*>(p2), yo + e0, ro ? ro + e0 : nullptr,
                       mean ? mean + r0 : nullptr, rstd ? rstd + r0 : nullptr, nr, cols, SEG, nseg,
                       static_cast<const float4*>(part + r0 * nseg), eps);
}

#define FR_NS(TS, T, NV, EPV, R) {T, NV, EPV, &launch_norm_split<TS, T, NV, EPV, 4, R>}
#define FR_NS2(TS, T, NV, EPV, R) {T, NV, EPV, &launch_norm_split<TS, T, NV, EPV, 2, R>}
// Segment shapes, 32 elements per lane as the split softmax: 256 lanes
// (8192 columns, the two passes' default), 512 and 1024 lanes; 512 lanes x
// 64 elements (the RMSNorm's one-pass default; built for 256 registers, two
// waves per SIMD: with 128 it spilled); the scalar path 256 x 32.
#define FR_NS_TABLE(TS, E, R)                                               \
  {FR_NS(TS, 256, 32 / E, E, R), FR_NS(TS, 512, 32 / E, E, R),              \
   FR_NS(TS, 1024, 32 / E, E, R), FR_NS2(TS, 512, 64 / E, E, R),            \
   FR_NS(TS, 256, 32, 1, R)}

static const NormSplitVariant kNsLnF32[] = FR_NS_TABLE(float, 4, false);
static const NormSplitVariant kNsLnBf16[] = FR_NS_TABLE(bf16_t, 8, false);
static const NormSplitVariant kNsRnF32[] = FR_NS_TABLE(float, 4, true);
static const NormSplitVariant kNsRnBf16[] = FR_NS_TABLE(bf16_t, 8, true);

#define FR_SPAN(a) {a, sizeof(a) / sizeof(a[0])}

VariantSpan<NormSplitVariant> norm_split_variants(int bf16, int rms) {
  if (rms) return bf16 ? VariantSpan<NormSplitVariant>FR_SPAN(kNsRnBf16)
                       : VariantSpan<NormSplitVariant>FR_SPAN(kNsRnF32);
  return bf16 ? VariantSpan<NormSplitVariant>FR_SPAN(kNsLnBf16)
              : VariantSpan<NormSplitVariant>FR_SPAN(kNsLnF32);
}

}  // namespace fr
