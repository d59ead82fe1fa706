// Split-row softmax, softmax cross-entropy and softmax backward: rows of any
// width up to 2^24, several workgroups per row.
//
// A row is cut into segments of `seg` columns (a multiple of 32, so every
// segment keeps its row's address phase); workgroup (row, segment) owns one
// segment in registers. Two forms for the softmax and cross-entropy:
//   one pass (split_coop_kernel): each workgroup takes its segment's partial
//     online-softmax state (m, s) — plus the sum of its logits t and the
//     column of its maximum when the options need them — posts it to the
//     row's slots in the workspace, waits for the row's other states, merges
//     them and writes p (or the cross-entropy gradient, loss and argmax)
//     from its registers: the logits are read once;
//   two passes: pass 1 (split_stats_kernel) writes each segment's state to
//     the workspace [rows][segments]; pass 2 (split_apply_kernel) merges a
//     row's states in segment order (the same order, hence the same bits, in
//     every workgroup of the row), re-reads its segment and writes.
// The merge is the online normaliser's ("Engineering a CUDA Machine Learning
// Framework from Scratch", §3.1) applied to segment states. In the two
// passes the logits are read twice and the outputs written once; pass 1 uses
// ordinary (cached) loads and the launcher runs both passes over one batch
// of rows at a time, so that the second read of a segment can come from the
// last-level cache: pass 1 of the first batch, then for each further batch
// one launch with pass 2 of the batch before and pass 1 of this one
// (split_apply_stats_kernel; they touch different rows), then pass 2 of the
// last. The softmax backward runs two passes (its per-row sum s = sum p dy).
#include "coop.hpp"
#include "fr_kernels.hpp"
#include "softmax_core.hpp"

namespace fr {

// (m, s, t, idx): max, sum of exp(x - m), sum of x, column of the max
// (a float, exact below 2^24; empty 3e38). Empty state (-inf, 0, 0, 3e38).
struct SplitState {
  float m, s, t, idx;
  template <int C, int M>
  static __device__ __forceinline__ SplitState move(const SplitState& a) {
    return {dpp_move<C, M>(a.m, kNegInf), dpp_move<C, M>(a.s, 0.f), dpp_move<C, M>(a.t, 0.f),
            dpp_move<C, M>(a.idx, 3.0e38f)};
  }
  __device__ __forceinline__ SplitState lane63() const {
    return {read_lane63(m), read_lane63(s), read_lane63(t), read_lane63(idx)};
  }
};
struct SplitMerge {
  __device__ __forceinline__ SplitState operator()(const SplitState& a, const SplitState& b) const {
    const MaxSumState r = MaxSumMerge<false>{}(MaxSumState{a.m, a.s}, MaxSumState{b.m, b.s});
    const float lo_idx = a.idx < b.idx ? a.idx : b.idx;
    const float idx = a.m > b.m ? a.idx : (b.m > a.m ? b.idx : lo_idx);
    return {r.m, r.s, a.t + b.t, idx};
  }
};

// Segment `sg` of a row: [c0, c0 + len).
struct Segment {
  int c0, len;
  __device__ __forceinline__ Segment(int sg, int seg, int cols)
      : c0(sg * seg), len(cols - sg * seg < seg ? cols - sg * seg : seg) {}
};

// ------------------------------------------------------------------ pass 1

// The state of the segment held in v (xe: the extra column of lanes with
// ec >= 0; c0: the segment's first column), merged over the workgroup's
// waves through the LDS slot (the alternation rule of block_merge).
// STATS bit 1: the sum of the logits (label smoothing); bit 2: the column of
// the maximum (argmax). Without them a segment costs a max, a subtraction, a
// multiply and one base-2 exponential per element: the sum of exponentials
// needs no compensated exponential (its relative error is an average of the
// terms' errors, each about |x - m| * log2e * 2^-24 for the terms that
// matter), unlike an output p_j. x - m is formed first: folding m into an fma
// with log2e would put the rounding of m * log2e (|m| * 2^-24) into every
// term.
template <int T, int NV, int EPV, int STATS, typename G>
__device__ __forceinline__ SplitState segment_state(const float (&v)[NV][EPV], float xe, int ec,
                                                    const G& g, int c0, int tid, int wave,
                                                    int lane, float (*slot)[4]) {
  constexpr int NW = T / 64;
  constexpr bool WANT_T = STATS & 1;
  constexpr bool WANT_IDX = STATS & 2;
  // the wave's maximum first: exponentials relative to it, plain sums
  const float m = wave_max(lane_max<NV, EPV>(v, xe));
  float t = 0.f, best = 3.0e38f;
  if constexpr (WANT_T) {  // masked slots hold -inf and are skipped
    const bool full = g.nvec == T * NV;
    float t0 = ec >= 0 ? xe : 0.f, t1 = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const bool ok = full || i * T + tid < g.nvec;
#pragma unroll
      for (int k = 0; k < EPV; ++k) {
        const float a = ok ? v[i][k] : 0.f;
        if (k & 1) t1 += a; else t0 += a;
      }
    }
    t = t0 + t1;
  }
  if constexpr (WANT_IDX) {
    // first slot holding the wave's max: scan backwards keeping the last
    // match; slot order is column order within a lane
    int c = -1;
#pragma unroll
    for (int i = NV - 1; i >= 0; --i)
#pragma unroll
      for (int k = EPV - 1; k >= 0; --k) c = v[i][k] == m ? i * EPV + k : c;
    if (c >= 0)
      best = (float)(c0 + g.head + ((c / EPV) * T + tid) * EPV + (c % EPV));
    if (ec >= 0 && xe == m) {
      const float ce = (float)(c0 + ec);
      best = ce < best ? ce : best;
    }
  }
  // sum of exp(x - m) with the hardware exponential
  const float mr = (m == kNegInf) ? 0.f : m;
  float s0 = 0.f, s1 = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i)
#pragma unroll
    for (int k = 0; k < EPV; ++k) {
      const float e = exp2_hw((v[i][k] - mr) * kLog2e);
      if (k & 1) s1 += e; else s0 += e;
    }
  const float se = exp2_hw((xe - mr) * kLog2e);
  const WaveSums ws = wave_reduce(WaveSums{(s0 + s1) + se, t, best}, WaveSumsMerge{});
  SplitState st{m, ws.s, ws.t, ws.idx};
  if constexpr (NW > 1)
    st = block_merge_tree<NW>(st, slot, wave, lane, SplitMerge{},
                              SplitState{kNegInf, 0.f, 0.f, 3.0e38f});
  return st;
}

// The body: work items w0, w0 + wstride, ... of rows * nseg.
template <typename Tin, int T, int NV, int EPV, int STATS>
__device__ __forceinline__ void split_stats_body(const Tin* x, int64_t rows, int cols, int seg,
                                                 int nseg, const int32_t* labels, XentOptions opt,
                                                 int skip_ignored, float4* part, int64_t w0,
                                                 int64_t wstride) {
  constexpr int NW = T / 64;
  __shared__ float xw[2][NW][4];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int tid = threadIdx.x;
  const int64_t work = rows * nseg;
  int merges = 0;  // cross-wave merges so far: picks the LDS slot
  for (int64_t w = w0; w < work; w += wstride) {
    const int64_t row = w / nseg;
    const int sg = (int)(w - row * nseg);
    const Segment sgm(sg, seg, cols);
    if (skip_ignored && labels[row] == opt.ignore_index) {  // uniform; its partial is not read
      continue;
    }
    const Tin* xs = x + row * cols + sgm.c0;
    const RowGeom<EPV> g(xs, sgm.len);
    float v[NV][EPV];
    int ec;
    float xe;
    if (whole_segment<T, NV>(g)) {  // uniform
      load_whole<Tin, T, NV, EPV, kPass1NT>(xs, tid, v);
      ec = -1;
      xe = kNegInf;
    } else {
      load_chunks<Tin, T, NV, EPV, kHeadAlign, kPass1NT>(xs, g, tid, v, kNegInf);
      ec = g.extra_col(tid);
      xe = load_extra(xs, ec, kNegInf);
    }

    const SplitState st = segment_state<T, NV, EPV, STATS>(v, xe, ec, g, sgm.c0, tid, wave, lane,
                                                           xw[merges++ & 1]);
    if (tid == 0) part[w] = float4{st.m, st.s, st.t, st.idx};
  }
}

template <typename Tin, int T, int NV, int EPV, int OCC, int STATS>
__global__ __launch_bounds__(T) __attribute__((amdgpu_waves_per_eu(OCC)))
void split_stats_kernel(const Tin* x, int64_t rows, int cols, int seg, int nseg,
                        const int32_t* labels, XentOptions opt, int skip_ignored, float4* part) {
  split_stats_body<Tin, T, NV, EPV, STATS>(x, rows, cols, seg, nseg, labels, opt, skip_ignored, part,
                                           blockIdx.x, gridDim.x);
}

// ------------------------------------------------------------------ pass 2

// The row's merged state: lane j merges partials j, j + T, ... in order, then
// the DPP tree and the LDS merge (a fixed order: every workgroup of the row
// gets the same bits).
template <int T>
__device__ __forceinline__ SplitState merge_row(const float4* part, int64_t row, int nseg,
                                                float (*slot)[4], int wave, int lane, int tid) {
  constexpr int NW = T / 64;
  SplitState st{kNegInf, 0.f, 0.f, 3.0e38f};
  for (int j = tid; j < nseg; j += T) {
    const float4 p = part[row * nseg + j];
    st = SplitMerge{}(st, SplitState{p.x, p.y, p.z, p.w});
  }
  st = wave_reduce(st, SplitMerge{});
  if constexpr (NW > 1) st = block_merge<NW>(st, slot, wave, lane, SplitMerge{});
  return st;
}

// p_j = exp(x_j - M) / S into the output type, times a scale a, minus b
// (cross-entropy: a = g, b = g eps / C; softmax: a = 1, b = 0). bf16 outputs:
// a base-2 exponential with a 2^8 bias, e_j = 2^((x_j - M) log2e + 8) <= 2^8,
// normal for every p_j that can round to a non-zero bf16 (p_j >= 2^-134 needs
// e_j >= 2^-126, as 1/S <= 1), and one fma with the factor 2^-8 a / S (a
// normal number: an exact power-of-two scaling of a/S), rounding p_j once.
template <typename Tout>
__device__ __forceinline__ float split_p(float xv, float M, float fac, float b) {
  if constexpr (sizeof(Tout) == 2) {
    const float e = exp2_hw(__builtin_fmaf(xv - M, kLog2e, 8.f));
    return __builtin_fmaf(e, fac, -b);
  } else {
    return __builtin_fmaf(exp_acc(xv - M), fac, -b);
  }
}

// Writes the segment's outputs from its logits v (and xe) and the row's
// merged state st (inv_s = 1 / st.s): p, or the cross-entropy gradient with
// the row's loss (from the lane owning the label column) and argmax (from
// segment 0).
template <typename Tin, typename Tout, int T, int NV, int EPV, bool XENT, typename G>
__device__ __forceinline__ void segment_apply(float (&v)[NV][EPV], float xe, int ec, const G& g,
                                              const Segment& sgm, const Tin* xs, Tout* ys,
                                              const SplitState& st, float inv_s, int label,
                                              float gsc, float goff, const XentOptions& opt,
                                              float* loss, int32_t* argmax, int64_t row, int sg,
                                              int cols, int tid, bool states_ok = true) {
  // label column handled by the lane of this segment that owns it
  bool label_lane = false;
  float x_label = 0.f;
  const bool valid = XENT && label >= 0 && label < cols;
  if constexpr (XENT) {
    const int lc = label - sgm.c0;
    if (valid && lc >= 0 && lc < sgm.len) {
      const int body_end = g.head + g.nvec * EPV;
      const int owner = lc < g.head ? lc
                        : lc >= body_end ? g.head + (lc - body_end)
                                         : ((lc - g.head) / EPV) % T;
      label_lane = owner == tid;
    }
    if (label_lane) x_label = load1(xs + lc);
  }

  // the factor a / S (2^-8 a / S for the biased bf16 exponentials)
  const float fac = (sizeof(Tout) == 2 ? 0x1p-8f : 1.f) * (XENT ? inv_s * gsc : inv_s);
  const float off = XENT ? goff : 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i)
#pragma unroll
    for (int k = 0; k < EPV; ++k) v[i][k] = split_p<Tout>(v[i][k], st.m, fac, off);
  xe = split_p<Tout>(xe, st.m, fac, off);
  store_chunks<Tout, T, NV, EPV>(ys, g, tid, v);
  if (ec >= 0) store1(ys + ec, xe);

  if constexpr (XENT) {
    if (label_lane) {
      const float eps = opt.smoothing;
      const float p = exp_acc(x_label - st.m) * inv_s;
      store1(ys + (label - sgm.c0), gsc * ((p - (1.f - eps)) - eps / (float)cols));
      float l = st.m + logf(st.s);
      if (eps != 1.f) l -= (1.f - eps) * x_label;
      if (eps != 0.f) l -= eps * (st.t / (float)cols);
      loss[row] = l;
    } else if (!valid && sg == 0 && tid == 0) {
      loss[row] = __builtin_nanf("");
    }
    // -1: a row of the one-pass form whose states did not all arrive
    if (argmax && sg == 0 && tid == 0) argmax[row] = states_ok ? (int32_t)st.idx : -1;
  }
}

// XENT: y is the gradient (Tout == Tin); loss, argmax, labels and opt apply.
// The body: work items w0, w0 + wstride, ... of rows * nseg.
template <typename Tin, typename Tout, int T, int NV, int EPV, bool XENT>
__device__ __forceinline__ void split_apply_body(const Tin* x, Tout* y, int64_t rows, int cols,
                                                 int seg, int nseg, const float4* part,
                                                 const int32_t* labels, float* loss,
                                                 int32_t* argmax, XentOptions opt, int64_t w0,
                                                 int64_t wstride) {
  constexpr int NW = T / 64;
  __shared__ float xw[2][NW][4];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int tid = threadIdx.x;

  float gsc = 1.f, goff = 0.f;
  if constexpr (XENT) {
    gsc = opt.grad_scale;
    if (opt.count) gsc = gsc / (float)(*opt.count);
    goff = gsc * (opt.smoothing / (float)cols);
  }

  const int64_t work = rows * nseg;
  int merges = 0;  // cross-wave merges so far: picks the LDS slot
  for (int64_t w = w0; w < work; w += wstride) {
    const int64_t row = w / nseg;
    const int sg = (int)(w - row * nseg);
    const Segment sgm(sg, seg, cols);
    const Tin* xs = x + row * cols + sgm.c0;
    Tout* ys = y + row * cols + sgm.c0;
    const RowGeom<EPV> g(xs, sgm.len);
    const int ec = g.extra_col(tid);

    int label = 0;
    bool ignored = false;
    if constexpr (XENT) {
      label = __builtin_amdgcn_readfirstlane(labels[row]);
      ignored = opt.use_ignore && label == opt.ignore_index;
    }
    if (ignored) {  // uniform: a zero gradient segment, loss 0
      float z[NV][EPV];
#pragma unroll
      for (int i = 0; i < NV; ++i)
#pragma unroll
        for (int k = 0; k < EPV; ++k) z[i][k] = 0.f;
      store_chunks<Tout, T, NV, EPV>(ys, g, tid, z);
      if (ec >= 0) store1(ys + ec, 0.f);
      if (argmax) {  // uniform: every lane takes part in the merge (it has a barrier);
                     // pass 1 wrote this row's partials because argmax is wanted
        const SplitState st = merge_row<T>(part, row, nseg, xw[merges++ & 1], wave, lane, tid);
        if (sg == 0 && tid == 0) argmax[row] = (int32_t)st.idx;
      }
      if (sg == 0 && tid == 0) loss[row] = 0.f;
      continue;
    }

    const SplitState st = merge_row<T>(part, row, nseg, xw[merges++ & 1], wave, lane, tid);
    const float inv_s = 1.f / st.s;
    float v[NV][EPV];
    load_chunks<Tin, T, NV, EPV>(xs, g, tid, v, kNegInf);
    const float xe = load_extra(xs, ec, kNegInf);
    segment_apply<Tin, Tout, T, NV, EPV, XENT>(v, xe, ec, g, sgm, xs, ys, st, inv_s, label, gsc, goff,
                                              opt, loss, argmax, row, sg, cols, tid);
  }
}

template <typename Tin, typename Tout, int T, int NV, int EPV, int OCC, bool XENT>
__global__ __launch_bounds__(T) __attribute__((amdgpu_waves_per_eu(OCC)))
void split_apply_kernel(const Tin* x, Tout* y, int64_t rows, int cols, int seg, int nseg,
                        const float4* part, const int32_t* labels, float* loss, int32_t* argmax,
                        XentOptions opt) {
  split_apply_body<Tin, Tout, T, NV, EPV, XENT>(x, y, rows, cols, seg, nseg, part, labels, loss,
                                                argmax, opt, blockIdx.x, gridDim.x);
}

// Pass 2 of one row batch and pass 1 of the next in one launch (they touch
// different rows): workgroups [0, n_apply) take the first batch's segments,
// the rest the next batch's.
struct SplitBatch {
  const void* x;
  void* y;
  int64_t rows;
  float4* part;
  const int32_t* labels;
  float* loss;
  int32_t* argmax;
};
template <typename Tin, typename Tout, int T, int NV, int EPV, int OCC, bool XENT, int STATS>
__global__ __launch_bounds__(T) __attribute__((amdgpu_waves_per_eu(OCC)))
void split_apply_stats_kernel(SplitBatch a, SplitBatch n, int cols, int seg, int nseg,
                              XentOptions opt, int skip_ignored, unsigned n_apply) {
  if (blockIdx.x < n_apply)
    split_apply_body<Tin, Tout, T, NV, EPV, XENT>(
        static_cast<const Tin*>(a.x), static_cast<Tout*>(a.y), a.rows, cols, seg, nseg, a.part,
        a.labels, a.loss, a.argmax, opt, blockIdx.x, n_apply);
  else
    split_stats_body<Tin, T, NV, EPV, STATS>(static_cast<const Tin*>(n.x), n.rows, cols, seg, nseg,
                                             n.labels, opt, skip_ignored, n.part, blockIdx.x - n_apply,
                                             gridDim.x - n_apply);
}

// ---------------------------------------------------------- one-pass form
// One workgroup per (row, segment) work item, as in the two passes, but the
// row's workgroups wait for each other (the exchange of coop.hpp): each
// loads its segment into registers and takes its state as pass 1 does,
// posts word 0 = {m, s} and, with the options that need them, word 1 =
// {t, idx + 1} (neither is ever zero: s >= 1 when m is finite, -inf and NaN
// have non-zero bits, idx + 1 >= 1), waits for the row's other states,
// merges all nseg of them in segment order (lane j holds segment j's, one
// DPP tree: every workgroup of the row gets the same bits) and writes its
// outputs from the registers as pass 2 does after its second read: the
// input is read once.

template <typename Tin, typename Tout, int T, int NV, int EPV, int OCC, bool XENT, int STATS>
__global__ __launch_bounds__(T) __attribute__((amdgpu_waves_per_eu(OCC)))
void split_coop_kernel(const Tin* x, Tout* y, int64_t rows, int cols, int seg, int nseg,
                       const int32_t* labels, float* loss, int32_t* argmax, XentOptions opt,
                       int skip_ignored, uint64_t* slots, uint32_t* ctl, int spin_limit) {
  constexpr int NW = T / 64;
  constexpr int NWD = STATS ? 2 : 1;  // words posted per segment
  __shared__ float xw[2][NW][4];
  __shared__ float team[kCoopMaxSegments][4];
  __shared__ uint32_t ticket;
  __shared__ int team_ok;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int tid = threadIdx.x;
  if constexpr (NWD == 1) {  // the fields not posted: t = 0, idx + 1 = 3e38
    team[lane][2] = 0.f;
    team[lane][3] = 3.0e38f;
  }
  const int64_t w = coop_ticket(ctl, &ticket);  // < rows * nseg: one per workgroup
  const int64_t row = w / nseg;
  const int sg = (int)(w - row * nseg);
  const Segment sgm(sg, seg, cols);
  const Tin* xs = x + row * cols + sgm.c0;
  Tout* ys = y + row * cols + sgm.c0;
  const RowGeom<EPV> g(xs, sgm.len);
  const int ec = g.extra_col(tid);

  float gsc = 1.f, goff = 0.f;
  int label = 0;
  bool ignored = false;
  if constexpr (XENT) {
    gsc = opt.grad_scale;
    if (opt.count) gsc = gsc / (float)(*opt.count);
    goff = gsc * (opt.smoothing / (float)cols);
    label = __builtin_amdgcn_readfirstlane(labels[row]);
    ignored = opt.use_ignore && label == opt.ignore_index;
  }
  if (ignored && skip_ignored) {  // uniform over the row: no post; a zero gradient, loss 0
    float z[NV][EPV];
#pragma unroll
    for (int i = 0; i < NV; ++i)
#pragma unroll
      for (int k = 0; k < EPV; ++k) z[i][k] = 0.f;
    store_chunks<Tout, T, NV, EPV>(ys, g, tid, z);
    if (ec >= 0) store1(ys + ec, 0.f);
    if (sg == 0 && tid == 0) loss[row] = 0.f;
    return;
  }

  float v[NV][EPV];
  float xe;
  if (whole_segment<T, NV>(g)) {  // uniform
    load_whole<Tin, T, NV, EPV>(xs, tid, v);
    xe = kNegInf;
  } else {
    load_chunks<Tin, T, NV, EPV>(xs, g, tid, v, kNegInf);
    xe = load_extra(xs, ec, kNegInf);
  }
  const SplitState mine = segment_state<T, NV, EPV, STATS>(v, xe, ec, g, sgm.c0, tid, wave, lane,
                                                           xw[0]);
  uint64_t* row_slots = slots + (size_t)row * nseg * 2;
  coop_post<NWD>(row_slots, sg, coop_word(mine.m, mine.s), coop_word(mine.t, mine.idx + 1.f));
  if (wave == 0) {
    const bool ok = coop_wait<NWD>(row_slots, nseg, ctl + 1, spin_limit, lane, team);
    if (lane == 0) team_ok = ok;
  }
  lds_barrier();
  const bool states_ok = __builtin_amdgcn_readfirstlane(team_ok) != 0;
  // the row's state: lane j < nseg holds segment j's, one DPP tree (the same
  // in every wave of every workgroup of the row); idx + 1 -> idx is exact
  // below 2^24
  SplitState st{kNegInf, 0.f, 0.f, 3.0e38f};
  if (lane < nseg) st = SplitState{team[lane][0], team[lane][1], team[lane][2], team[lane][3] - 1.f};
  st = wave_reduce(st, SplitMerge{});

  if (ignored) {  // with argmax: the row's argmax, a zero gradient, loss 0
#pragma unroll
    for (int i = 0; i < NV; ++i)
#pragma unroll
      for (int k = 0; k < EPV; ++k) v[i][k] = 0.f;
    store_chunks<Tout, T, NV, EPV>(ys, g, tid, v);
    if (ec >= 0) store1(ys + ec, 0.f);
    if (sg == 0 && tid == 0) {
      loss[row] = 0.f;
      argmax[row] = states_ok ? (int32_t)st.idx : -1;  // -1: states missing
    }
    return;
  }
  segment_apply<Tin, Tout, T, NV, EPV, XENT>(v, xe, ec, g, sgm, xs, ys, st, 1.f / st.s, label, gsc,
                                            goff, opt, loss, argmax, row, sg, cols, tid, states_ok);
}

// Zeroes n 16-byte words (the one-pass form's counter, abort word and slots).
__global__ __launch_bounds__(256) void coop_clear_kernel(uint4* p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = uint4{0u, 0u, 0u, 0u};
}

hipError_t launch_coop_clear(void* ws, int64_t rows, int nseg, hipStream_t s) {
  const int64_t n16 = coop_workspace_bytes(rows, nseg) / 16;
  return launch_kernel(&coop_clear_kernel, dim3((unsigned)((n16 + 255) / 256)), dim3(256), s,
                       static_cast<uint4*>(ws), n16);
}

// ------------------------------------------------ softmax backward, split
// dx = p (dy - s), s = sum_j p_j dy_j: pass 1 writes each segment's sum of
// p * dy, pass 2 adds the row's segment sums in segment order (the same bits
// in every workgroup of the row), re-reads p and dy and writes dx.

// (the bodies: work items w0, w0 + wstride, ... of rows * nseg)
template <typename Ts, int T, int NV, int EPV>
__device__ __forceinline__ void softmax_bwd_split_stats_body(const Ts* p, const Ts* dy, int64_t rows,
                                                             int cols, int seg, int nseg,
                                                             float4* part, int64_t w0,
                                                             int64_t wstride) {
  constexpr int NW = T / 64;
  __shared__ float xw[2][NW][1];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int tid = threadIdx.x;
  const int64_t work = rows * nseg;
  int merges = 0;  // cross-wave merges so far: picks the LDS slot
  for (int64_t w = w0; w < work; w += wstride) {
    const int64_t row = w / nseg;
    const Segment sgm((int)(w - row * nseg), seg, cols);
    const int64_t off = row * cols + sgm.c0;
    const RowGeom<EPV> g(p + off, sgm.len);
    const int ec = g.extra_col(tid);
    float a[NV][EPV], d[NV][EPV];
    load_chunks2<Ts, T, NV, EPV, kHeadAlign, kPass1NT>(p + off, dy + off, g, tid, a, d, 0.f);
    float s0 = load_extra(p + off, ec, 0.f) * load_extra(dy + off, ec, 0.f), s1 = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i)
#pragma unroll
      for (int k = 0; k < EPV; ++k) {
        if (k & 1) s1 = __builtin_fmaf(a[i][k], d[i][k], s1);
        else s0 = __builtin_fmaf(a[i][k], d[i][k], s0);
      }
    SumState st{s0 + s1};
    st = wave_reduce(st, SumMerge{});
    if constexpr (NW > 1) st = block_merge<NW>(st, xw[merges++ & 1], wave, lane, SumMerge{});
    if (tid == 0) part[w] = float4{st.s, 0.f, 0.f, 0.f};
  }
}

template <typename Ts, int T, int NV, int EPV>
__device__ __forceinline__ void softmax_bwd_split_apply_body(const Ts* p, const Ts* dy, Ts* dx,
                                                             int64_t rows, int cols, int seg,
                                                             int nseg, const float4* part,
                                                             int64_t w0, int64_t wstride) {
  constexpr int NW = T / 64;
  __shared__ float xw[2][NW][1];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int tid = threadIdx.x;
  const int64_t work = rows * nseg;
  int merges = 0;  // cross-wave merges so far: picks the LDS slot
  for (int64_t w = w0; w < work; w += wstride) {
    const int64_t row = w / nseg;
    const Segment sgm((int)(w - row * nseg), seg, cols);
    SumState st{0.f};
    for (int j = tid; j < nseg; j += T) st.s += part[row * nseg + j].x;
    st = wave_reduce(st, SumMerge{});
    if constexpr (NW > 1) st = block_merge<NW>(st, xw[merges++ & 1], wave, lane, SumMerge{});
    const float s = st.s;
    const int64_t off = row * cols + sgm.c0;
    const RowGeom<EPV> g(p + off, sgm.len);
    const int ec = g.extra_col(tid);
    float a[NV][EPV], d[NV][EPV];
    load_chunks2<Ts, T, NV, EPV>(p + off, dy + off, g, tid, a, d, 0.f);
    const float ae = load_extra(p + off, ec, 0.f), de = load_extra(dy + off, ec, 0.f);
#pragma unroll
    for (int i = 0; i < NV; ++i)
#pragma unroll
      for (int k = 0; k < EPV; ++k) a[i][k] = a[i][k] * (d[i][k] - s);
    store_chunks<Ts, T, NV, EPV>(dx + off, g, tid, a);
    if (ec >= 0) store1(dx + off + ec, ae * (de - s));
  }
}

template <typename Ts, int T, int NV, int EPV, int OCC>
__global__ __launch_bounds__(T) __attribute__((amdgpu_waves_per_eu(OCC)))
void softmax_bwd_split_stats_kernel(const Ts* p, const Ts* dy, int64_t rows, int cols, int seg,
                                    int nseg, float4* part) {
  softmax_bwd_split_stats_body<Ts, T, NV, EPV>(p, dy, rows, cols, seg, nseg, part, blockIdx.x,
                                               gridDim.x);
}

template <typename Ts, int T, int NV, int EPV, int OCC>
__global__ __launch_bounds__(T) __attribute__((amdgpu_waves_per_eu(OCC)))
void softmax_bwd_split_apply_kernel(const Ts* p, const Ts* dy, Ts* dx, int64_t rows, int cols,
                                    int seg, int nseg, const float4* part) {
  softmax_bwd_split_apply_body<Ts, T, NV, EPV>(p, dy, dx, rows, cols, seg, nseg, part, blockIdx.x,
                                               gridDim.x);
}

// Pass 2 of one row batch (rows ra at offset ea) and pass 1 of the next (rows
// rn at en) in one launch, as split_apply_stats_kernel.
template <typename Ts, int T, int NV, int EPV, int OCC>
__global__ __launch_bounds__(T) __attribute__((amdgpu_waves_per_eu(OCC)))
void softmax_bwd_split_apply_stats_kernel(const Ts* p, const Ts* dy, Ts* dx, int cols, int seg,
                                          int nseg, int64_t ea, int64_t ra, const float4* pa,
                                          int64_t en, int64_t rn, float4* pn, unsigned n_apply) {
  if (blockIdx.x < n_apply)
    softmax_bwd_split_apply_body<Ts, T, NV, EPV>(p + ea, dy + ea, dx + ea, ra, cols, seg, nseg, pa,
                                                 blockIdx.x, n_apply);
  else
    softmax_bwd_split_stats_body<Ts, T, NV, EPV>(p + en, dy + en, rn, cols, seg, nseg, pn,
                                                 blockIdx.x - n_apply, gridDim.x - n_apply);
}

// One-pass form of the softmax backward (the exchange of coop.hpp): each
// workgroup loads its segment of p and dy into registers, posts {sum of
// p dy over the segment, 1} (never zero), waits for the row's other sums,
// adds them in segment order (lane j holds segment j's, one DPP tree: the
// same bits in every workgroup of the row) and writes dx = p (dy - s) from
// the registers. dx may be p or dy: a workgroup writes only its own segment,
// after reading it.
template <typename Ts, int T, int NV, int EPV, int OCC>
__global__ __launch_bounds__(T) __attribute__((amdgpu_waves_per_eu(OCC)))
void softmax_bwd_split_coop_kernel(const Ts* p, const Ts* dy, Ts* dx, int64_t rows, int cols,
                                   int seg, int nseg, uint64_t* slots, uint32_t* ctl,
                                   int spin_limit) {
  constexpr int NW = T / 64;
  __shared__ float xw[2][NW][1];
  __shared__ float team[kCoopMaxSegments][4];
  __shared__ uint32_t ticket;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int tid = threadIdx.x;
  const int64_t w = coop_ticket(ctl, &ticket);  // < rows * nseg: one per workgroup
  const int64_t row = w / nseg;
  const int sg = (int)(w - row * nseg);
  const Segment sgm(sg, seg, cols);
  const int64_t off = row * cols + sgm.c0;
  const RowGeom<EPV> g(p + off, sgm.len);
  const int ec = g.extra_col(tid);
  float a[NV][EPV], d[NV][EPV];
  load_chunks2<Ts, T, NV, EPV>(p + off, dy + off, g, tid, a, d, 0.f);
  const float ae = load_extra(p + off, ec, 0.f), de = load_extra(dy + off, ec, 0.f);
  float s0 = ae * de, s1 = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i)
#pragma unroll
    for (int k = 0; k < EPV; ++k) {
      if (k & 1) s1 = __builtin_fmaf(a[i][k], d[i][k], s1);
      else s0 = __builtin_fmaf(a[i][k], d[i][k], s0);
    }
  SumState st{s0 + s1};
  st = wave_reduce(st, SumMerge{});
  if constexpr (NW > 1) st = block_merge<NW>(st, xw[0], wave, lane, SumMerge{});
  uint64_t* row_slots = slots + (size_t)row * nseg * 2;
  coop_post<1>(row_slots, sg, coop_word(st.s, 1.f), 0);
  if (wave == 0) coop_wait<1>(row_slots, nseg, ctl + 1, spin_limit, lane, team);
  lds_barrier();
  SumState tot{0.f};
  if (lane < nseg) tot = SumState{team[lane][0]};
  tot = wave_reduce(tot, SumMerge{});
  const float s = tot.s;
#pragma unroll
  for (int i = 0; i < NV; ++i)
#pragma unroll
    for (int k = 0; k < EPV; ++k) a[i][k] = a[i][k] * (d[i][k] - s);
  store_chunks<Ts, T, NV, EPV>(dx + off, g, tid, a);
  if (ec >= 0) store1(dx + off + ec, ae * (de - s));
}

// --------------------------------------------------------------- launchers

static unsigned split_grid(int64_t work) {
  return (unsigned)(work < kMaxGrid ? work : kMaxGrid);
}

// The one-pass form over rows of nseg segments: its workspace (16 bytes of
// counter and abort word, then rows * nseg * 16 bytes of slots) is zeroed,
// then one workgroup per work item.
template <typename Tin, typename Tout, typename K>
static hipError_t launch_coop(K kernel, int nseg, int T, float4* part, hipStream_t s, const Tin* x,
                              Tout* y, int64_t rows, int cols, int seg, const int32_t* labels,
                              float* loss, int32_t* argmax, XentOptions o, int skip) {
  hipError_t e = launch_coop_clear(part, rows, nseg, s);
  if (e != hipSuccess) return e;
  uint32_t* ctl = reinterpret_cast<uint32_t*>(part);
  uint64_t* slots = reinterpret_cast<uint64_t*>(part + 1);
  return launch_kernel(kernel, dim3((unsigned)(rows * nseg)), dim3(T), s, x, y, rows, cols, seg, nseg,
                       labels, loss, argmax, o, skip, slots, ctl, coop_spin_limit());
}

template <typename Tin, typename Tout, int T, int NV, int EPV, int OCC, bool XENT>
static hipError_t launch_split(const void* x, void* y, int64_t rows, int cols, const int32_t* labels,
                               float* loss, int32_t* argmax, const XentOptions* opt, float4* part,
                               int64_t part_bytes, bool one_pass, hipStream_t s) {
  constexpr int SEG = T * NV * EPV;
  const int nseg = (cols + SEG - 1) / SEG;
  const XentOptions o = opt ? *opt : XentOptions{0, 0, 0.f, 1.f, nullptr, 0, 0, nullptr, nullptr};
  const int skip = XENT && o.use_ignore && !argmax;
  const int stats = XENT ? ((o.smoothing != 0.f ? 1 : 0) | (argmax ? 2 : 0)) : 0;
  if (one_pass && coop_applies(rows, nseg, part_bytes)) {
    auto kc = stats == 0   ? &split_coop_kernel<Tin, Tout, T, NV, EPV, OCC, XENT, 0>
              : stats == 1 ? &split_coop_kernel<Tin, Tout, T, NV, EPV, OCC, XENT, XENT ? 1 : 0>
              : stats == 2 ? &split_coop_kernel<Tin, Tout, T, NV, EPV, OCC, XENT, XENT ? 2 : 0>
                           : &split_coop_kernel<Tin, Tout, T, NV, EPV, OCC, XENT, XENT ? 3 : 0>;
    return launch_coop(kc, nseg, T, part, s, static_cast<const Tin*>(x), static_cast<Tout*>(y), rows,
                       cols, SEG, labels, loss, argmax, o, skip);
  }
  auto k1 = stats == 0   ? &split_stats_kernel<Tin, T, NV, EPV, OCC, 0>
            : stats == 1 ? &split_stats_kernel<Tin, T, NV, EPV, OCC, 1>
            : stats == 2 ? &split_stats_kernel<Tin, T, NV, EPV, OCC, 2>
                         : &split_stats_kernel<Tin, T, NV, EPV, OCC, 3>;
  auto kf = !XENT || stats == 0 ? &split_apply_stats_kernel<Tin, Tout, T, NV, EPV, OCC, XENT, 0>
            : stats == 1 ? &split_apply_stats_kernel<Tin, Tout, T, NV, EPV, OCC, XENT, XENT ? 1 : 0>
            : stats == 2 ? &split_apply_stats_kernel<Tin, Tout, T, NV, EPV, OCC, XENT, XENT ? 2 : 0>
                         : &split_apply_stats_kernel<Tin, Tout, T, NV, EPV, OCC, XENT, XENT ? 3 : 0>;
  const Tin* xi = static_cast<const Tin*>(x);
  Tout* yo = static_cast<Tout*>(y);
  const int64_t batch = split_batch_rows(rows, (int64_t)cols * sizeof(Tin));
  auto view = [&](int64_t r0) {
    const int64_t nr = rows - r0 < batch ? rows - r0 : batch;
    return SplitBatch{xi + r0 * cols, yo + r0 * cols, nr, part + r0 * nseg,
                      labels ? labels + r0 : nullptr, loss ? loss + r0 : nullptr,
                      argmax ? argmax + r0 : nullptr};
  };
  // pass 1 of the first batch; then, per further batch, pass 2 of the one
  // before and pass 1 of this one in one launch; then pass 2 of the last
  SplitBatch cur = view(0);
  hipError_t e = launch_kernel(k1, dim3(split_grid(cur.rows * nseg)), dim3(T), s, xi, cur.rows, cols,
                               SEG, nseg, cur.labels, o, skip, cur.part);
  if (e != hipSuccess) return e;
  for (int64_t r0 = batch; r0 < rows; r0 += batch) {
    const SplitBatch nxt = view(r0);
    const unsigned na = split_grid(cur.rows * nseg), ns = split_grid(nxt.rows * nseg);
    e = launch_kernel(kf, dim3(na + ns), dim3(T), s, cur, nxt, cols, SEG, nseg, o, skip, na);
    if (e != hipSuccess) return e;
    cur = nxt;
  }
  return launch_kernel(&split_apply_kernel<Tin, Tout, T, NV, EPV, OCC, XENT>,
                       dim3(split_grid(cur.rows * nseg)), dim3(T), s,
                       static_cast<const Tin*>(cur.x), static_cast<Tout*>(cur.y), cur.rows, cols, SEG,
                       nseg, static_cast<const float4*>(cur.part), cur.labels, cur.loss, cur.argmax, o);
}

template <typename Ts, int T, int NV, int EPV, int OCC>
static hipError_t launch_softmax_bwd_split(const void* p, const void* dy, void* dx, int64_t rows,
                                           int cols, float4* part, int64_t part_bytes, bool one_pass,
                                           hipStream_t s) {
  constexpr int SEG = T * NV * EPV;
  const int nseg = (cols + SEG - 1) / SEG;
  const Ts* pi = static_cast<const Ts*>(p);
  const Ts* di = static_cast<const Ts*>(dy);
  Ts* xo = static_cast<Ts*>(dx);
  if (one_pass && coop_applies(rows, nseg, part_bytes)) {
    hipError_t e = launch_coop_clear(part, rows, nseg, s);
    if (e != hipSuccess) return e;
    return launch_kernel(&softmax_bwd_split_coop_kernel<Ts, T, NV, EPV, OCC>,
                         dim3((unsigned)(rows * nseg)), dim3(T), s, pi, di, xo, rows, cols, SEG, nseg,
                         reinterpret_cast<uint64_t*>(part + 1), reinterpret_cast<uint32_t*>(part),
                         coop_spin_limit());
  }
  const int64_t batch = split_batch_rows(rows, (int64_t)cols * 2 * sizeof(Ts));
  // pass 1 of the first batch; per further batch, pass 2 of the one before
  // with pass 1 of this one; then pass 2 of the last
  int64_t r0 = 0, nr = rows < batch ? rows : batch;
  hipError_t e = launch_kernel(&softmax_bwd_split_stats_kernel<Ts, T, NV, EPV, OCC>,
                               dim3(split_grid(nr * nseg)), dim3(T), s, pi, di, nr, cols, SEG, nseg,
                               part);
  if (e != hipSuccess) return e;
  for (int64_t r1 = batch; r1 < rows; r1 += batch) {
    const int64_t n1 = rows - r1 < batch ? rows - r1 : batch;
    const unsigned na = split_grid(nr * nseg), ns = split_grid(n1 * nseg);
    e = launch_kernel(&softmax_bwd_split_apply_stats_kernel<Ts, T, NV, EPV, OCC>, dim3(na + ns),
                      dim3(T), s, pi, di, xo, cols, SEG, nseg, r0 * cols, nr,
                      static_cast<const float4*>(part + r0 * nseg), r1 * cols, n1, part + r1 * nseg,
                      na);
    if (e != hipSuccess) return e;
    r0 = r1;
    nr = n1;
  }
  return launch_kernel(&softmax_bwd_split_apply_kernel<Ts, T, NV, EPV, OCC>,
                       dim3(split_grid(nr * nseg)), dim3(T), s, pi + r0 * cols, di + r0 * cols,
                       xo + r0 * cols, nr, cols, SEG, nseg,
                       static_cast<const float4*>(part + r0 * nseg));
}

#define FR_SP(TI, TO, T, NV, EPV, OCC, X) {T, NV, EPV, &launch_split<TI, TO, T, NV, EPV, OCC, X>}
// Segment shapes: 256 lanes x 8 chunks (32 KiB segments, 8192 fp32 or 16384
// bf16 columns, the two passes' default: several workgroups per CU overlap
// one segment's loads with another's arithmetic; bf16 1024 x 262144 with
// 8 KiB-column segments of 16 KiB measured 286 -> 270 us), 512 and 1024
// lanes x 32 elements, 512 lanes x 64 elements (32768 columns: the one-pass
// default, the waits fewer and each workgroup's share larger); the scalar
// path (unaligned phases) 256 lanes x 32 elements.
#define FR_SP_TABLE(TI, TO, E, X)                                                           \
  {FR_SP(TI, TO, 256, 8, E, 4, X),       FR_SP(TI, TO, 512, 32 / E, E, 4, X),                 \
   FR_SP(TI, TO, 1024, 32 / E, E, 4, X), FR_SP(TI, TO, 512, 64 / E, E, 4, X),                 \
   FR_SP(TI, TO, 256, 32, 1, 4, X)}

static const SplitVariant kSpF32F32[] = FR_SP_TABLE(float, float, 4, false);
static const SplitVariant kSpBf16Bf16[] = FR_SP_TABLE(bf16_t, bf16_t, 8, false);
static const SplitVariant kSpF32Bf16[] = FR_SP_TABLE(float, bf16_t, 4, false);
static const SplitVariant kSpBf16F32[] = FR_SP_TABLE(bf16_t, float, 8, false);
static const SplitVariant kSpXeF32[] = FR_SP_TABLE(float, float, 4, true);
static const SplitVariant kSpXeBf16[] = FR_SP_TABLE(bf16_t, bf16_t, 8, true);

// Softmax backward: as above; the 512 x 64 shape (the one-pass default)
// holds p and dy, 128 values per lane, so it is built for 256 registers
// (two waves per SIMD: with 128 it spilled).
#define FR_SB_SPLIT(TS, T, NV, EPV) {T, NV, EPV, &launch_softmax_bwd_split<TS, T, NV, EPV, 4>}
#define FR_SB_SPLIT2(TS, T, NV, EPV) {T, NV, EPV, &launch_softmax_bwd_split<TS, T, NV, EPV, 2>}
#define FR_SB_SPLIT_TABLE(TS, E)                                                      \
  {FR_SB_SPLIT(TS, 256, 32 / E, E), FR_SB_SPLIT(TS, 512, 32 / E, E),                   \
   FR_SB_SPLIT(TS, 1024, 32 / E, E), FR_SB_SPLIT2(TS, 512, 64 / E, E),                 \
   FR_SB_SPLIT(TS, 256, 32, 1)}
static const SoftmaxBwdSplitVariant kSbSpF32[] = FR_SB_SPLIT_TABLE(float, 4);
static const SoftmaxBwdSplitVariant kSbSpBf16[] = FR_SB_SPLIT_TABLE(bf16_t, 8);

#define FR_SPAN(a) {a, sizeof(a) / sizeof(a[0])}

VariantSpan<SoftmaxBwdSplitVariant> softmax_bwd_split_variants(int bf16) {
  return bf16 ? VariantSpan<SoftmaxBwdSplitVariant>FR_SPAN(kSbSpBf16)
              : VariantSpan<SoftmaxBwdSplitVariant>FR_SPAN(kSbSpF32);
}

VariantSpan<SplitVariant> split_variants(int in_bf16, int out_bf16, int xent) {
  if (xent) return in_bf16 ? VariantSpan<SplitVariant>FR_SPAN(kSpXeBf16)
                           : VariantSpan<SplitVariant>FR_SPAN(kSpXeF32);
  if (in_bf16) return out_bf16 ? VariantSpan<SplitVariant>FR_SPAN(kSpBf16Bf16)
                               : VariantSpan<SplitVariant>FR_SPAN(kSpBf16F32);
  return out_bf16 ? VariantSpan<SplitVariant>FR_SPAN(kSpF32Bf16)
                  : VariantSpan<SplitVariant>FR_SPAN(kSpF32F32);
}

}  // namespace fr
