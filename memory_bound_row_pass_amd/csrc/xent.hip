// Softmax cross-entropy, forward and backward in one pass over memory
// ("Engineering a CUDA Machine Learning Framework from Scratch", §2.1: loss
// gradients fused into registers; "GPU Programming for Machine Learning",
// Module 3: cross-entropy loss).
//
// Per row: the online-softmax state (M, S) of the logits (as in softmax.hip:
// exponentials kept in registers, natural units for fp32 logits, biased
// base 2 for bf16 logits), then
//   loss    = M + ln S - x[label]
//   grad_j  = exp(x_j - M) / S - [j == label]
//   argmax  = smallest j with x_j == M (optional)
// The lane that owns the label column reads the label logit, writes the
// loss, and overwrites its stored p with p - 1. A label outside [0, cols)
// gives a NaN loss and an unmodified softmax row.
//
// With options (OPT, the cross-entropy variants of training code): rows whose
// label is the ignore index get loss 0 and a zero gradient; label smoothing
// eps targets q_j = (1 - eps) [j == label] + eps / C, which needs the row sum
// of the logits t = sum_j x_j carried in the row state:
//   loss   = lse - (1 - eps) x[label] - eps t / C,   lse = M + ln S
//   grad_j = g (p_j - q_j),  g = grad_scale, or grad_scale / n_valid for a
//            mean over the rows that are not ignored (n_valid counted by
//            xent_count_kernel before the row pass).
// Each lane stores g p_j - g eps / C with one fma; the label lane then
// overwrites its element with g (p_label - (1 - eps) - eps / C).
#include <atomic>
#include <mutex>

#include "fr_kernels.hpp"
#include "softmax_core.hpp"

namespace fr {

// Rows whose label is not the ignore index, counted by every thread of the
// workgroup (labels tid, tid + BLOCK, ...), summed exactly per wavefront into
// one LDS word per wave (`slots`, written once and kept for the kernel's
// lifetime), then over the waves in order: the same value in every lane.
template <int BLOCK>
__device__ __forceinline__ uint32_t sum_count_slots(const uint32_t* slots) {
  uint32_t t = 0;
#pragma unroll
  for (int i = 0; i < BLOCK / 64; ++i) t += slots[i];
  return t;
}
template <int BLOCK>
__device__ __forceinline__ uint32_t count_valid_rows(const int32_t* labels, int64_t rows,
                                                     const XentOptions& opt, uint32_t* slots) {
  uint32_t c = 0;
  for (int64_t r = threadIdx.x; r < rows; r += BLOCK)
    c += (opt.use_ignore && labels[r] == opt.ignore_index) ? 0u : 1u;
  const CountState w = wave_reduce(CountState{__uint_as_float(c)}, CountMerge{});
  if ((threadIdx.x & 63) == 0) slots[threadIdx.x >> 6] = __float_as_uint(w.b);
  __syncthreads();
  return sum_count_slots<BLOCK>(slots);
}

// The per-row losses of a call with a sum or mean reduction are written with
// device-scope stores: written through to the level where all XCDs see them
// (each XCD has its own L2), without the whole-L2 write-back and invalidate
// of a device-scope fence, which measured 285 -> 3250 us when every
// workgroup did it.
__device__ __forceinline__ void store_loss(float* p, float v, bool device_scope) {
  if (device_scope) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else *p = v;
}

// The loss total of a sum or mean reduction, in the same launch: every
// workgroup, once its loss stores have completed (each wave waits for its
// own), increments the completion counter; the workgroup that takes it to
// gridDim.x (the last) reads loss[0 .. rows) with device-scope loads, adds
// them in double in a fixed order — 1024 partial sums over rows v, v + 1024,
// ..., then a halving tree — writes the sum (or the sum / n_valid) and sets
// the counter back to zero for the next call. No workgroup waits for
// another, and no float atomics: the total is bitwise reproducible and does
// not depend on the kernel shape. (n_valid is taken again here, from the
// count or the LDS count slots, so that it is not held in a register across
// the row loop.)
template <int BLOCK>
__device__ __forceinline__ void finish_total(const float* loss, int64_t rows,
                                             const XentOptions& opt, const uint32_t* count_slots,
                                             double* red, int* last) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's loss stores are complete
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t prev =
        __hip_atomic_fetch_add(opt.done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *last = prev == gridDim.x - 1;
  }
  __syncthreads();
  if (!*last) return;  // uniform
  for (int v = threadIdx.x; v < 1024; v += BLOCK) {
    double a = 0.0;
    for (int64_t r = v; r < rows; r += 1024)
      a += (double)__hip_atomic_load(loss + r, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    red[v] = a;
  }
  __syncthreads();
  for (int w = 512; w > 0; w >>= 1) {
    for (int i = threadIdx.x; i < w; i += BLOCK) red[i] += red[i + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const double t = red[0];
    const uint32_t n_valid = opt.count ? *opt.count : sum_count_slots<BLOCK>(count_slots);
    *opt.total = opt.reduction == 2 ? (float)(t / (double)n_valid) : (float)t;
    __hip_atomic_store(opt.done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// An uniform value the compiler cannot see through: computations from it in a
// branch stay in the branch instead of being hoisted out of the row loop
// (and kept live, or spilled, across it).
__device__ __forceinline__ float opaque(float v) {
  int b = __builtin_amdgcn_readfirstlane(__float_as_int(v));
  asm volatile("" : "+s"(b));
  return __int_as_float(b);
}

// A row state with the sum of the raw logits added (label smoothing).
template <typename S>
struct PlusSum {
  S st;
  float t;
  template <int C, int M>
  static __device__ __forceinline__ PlusSum move(const PlusSum& a) {
    return {S::template move<C, M>(a.st), dpp_move<C, M>(a.t, 0.f)};
  }
  __device__ __forceinline__ PlusSum lane63() const { return {st.lane63(), read_lane63(t)}; }
};
template <typename S, typename M>
struct PlusSumMerge {
  __device__ __forceinline__ PlusSum<S> operator()(const PlusSum<S>& a, const PlusSum<S>& b) const {
    return {M{}(a.st, b.st), a.t + b.t};
  }
};

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

// Exponentials and scaling: bf16 logits (bf16 gradient) take the biased
// base-2 form of the bf16 softmax (lane_exp_log2, 2^8 bias), so gradients in
// the bf16 subnormal range are computed within one ulp and the row sum, and
// with it the loss, stays accurate to ~3e-7 relative (a 2^64 bias would leave
// ~2.6e-6); fp32 logits take the natural form with the compensated
// exponential.

// LPF > 0 (one row per workgroup): the next row is staged while the current
// one is reduced and written: its first LPF slots in LDS (16 T bytes of LDS
// per slot, no VGPRs) and its head/tail element, issued right after the
// current row is in registers. The grid is then one workgroup per compute
// unit, each looping over rows. Vector memory operations retire in issue
// order: at the next row's start, a wait that leaves the current row's
// whole-slot stores outstanding has seen every copy complete, so neither the
// stores nor the next row wait for each other (bf16 4096 x 50257 with
// options 166 -> 159 us, plain 170 -> 163 us, against a full wait for the
// copies before the current row's stores).
template <typename Tin, int T, int NV, int EPV, int OCC, bool ARGMAX, bool OPT, int LPF = 0>
__global__ __launch_bounds__(T == 64 ? 256 : T) __attribute__((amdgpu_waves_per_eu(OCC)))
void xent_kernel(const Tin* x,
                 // no output overlaps the labels (the entry points reject it), so the
                 // next row's label comes through a scalar load, whose wait does not
                 // wait for this row's stores and staged copies
                 const int32_t* __restrict__ labels, float* loss, Tin* grad, int32_t* argmax,
                 int64_t rows, int cols, XentOptions opt) {
  constexpr int BLOCK = T == 64 ? 256 : T;
  constexpr int RPB = BLOCK / T;
  constexpr int NW = T / 64;
  constexpr bool LOG2 = sizeof(Tin) == 2;
  using Base = typename std::conditional<ARGMAX, MaxSumIdxState, MaxSumState>::type;
  using BaseMerge = typename std::conditional<ARGMAX, MaxSumIdxMerge, MaxSumMerge<LOG2>>::type;
  using State = typename std::conditional<OPT, PlusSum<Base>, Base>::type;
  using Merge = typename std::conditional<OPT, PlusSumMerge<Base, BaseMerge>, BaseMerge>::type;
  constexpr int NF = sizeof(State) / sizeof(float);
  __shared__ float xw[2][NW][NF];
  static_assert(LPF == 0 || (RPB == 1 && LPF <= NV), "LDS staging: one row per block");
  __shared__ __attribute__((aligned(16))) uint32_t stage[LPF > 0 ? LPF * T * 4 : 4];
  __shared__ uint32_t count_slots[OPT ? BLOCK / 64 : 1];
  // the total's partial sums: the staging buffer once the rows are done, else
  // an array of their own
  __shared__ double red_own[OPT && LPF == 0 ? 1024 : 1];
  double* const red = LPF > 0 ? reinterpret_cast<double*>(stage) : red_own;
  static_assert(LPF == 0 || LPF * T * 4 * sizeof(uint32_t) >= 1024 * sizeof(double), "total");
  __shared__ int last_wg;

  const int wib = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int tid = T == 64 ? lane : (int)threadIdx.x;
  const int sub = T == 64 ? wib : 0;
  const int wave = T == 64 ? 0 : wib;

  // The next row's label is read one row ahead, so that the scalar load's
  // latency is not paid between rows (the ignore test needs the label before
  // the row's loads are issued).
  const int64_t stride = (int64_t)gridDim.x * RPB;
  const int64_t first = (int64_t)blockIdx.x * RPB + sub;
  int label_next = first < rows ? __builtin_amdgcn_readfirstlane(labels[first]) : 0;
  static_assert(LPF == 0 || EPV * sizeof(Tin) == 16, "staging of 16-byte chunks");
  bool have_pre = false;  // uniform: the LDS stage holds this row's first slots
  // uniform (LPF): whole-slot stores issued after the latest staging; with at
  // least NV - 1 of them a wait that leaves that many operations outstanding
  // has seen every staging copy complete
  int stores_after = 0;
  // LPF: the staged row's head/tail element. Its load is issued before the
  // row's copies and converted before the current row's stores, and the
  // staged chunks are read past the compiler's LDS-copy wait, so the counted
  // wait at a row's start is the only one that waits for this row's copies
  // and none waits for the previous row's stores (bf16 4096 x 50257:
  // 162.5 -> 151.2 us). Not with argmax: that kernel spills, and the
  // longer-lived registers made it slower (195.8 -> 210.8 us), so it keeps
  // the plain forms.
  constexpr bool kLate = !ARGMAX;
  uint32_t xe_raw = kRawNegInf<Tin>;
  float xe_next = kNegInf;
  if constexpr (LPF > 0) {
    have_pre = first < rows && !(OPT && !ARGMAX && opt.use_ignore && label_next == opt.ignore_index);
    if (have_pre) {
      const Tin* x0 = x + first * cols;
      const RowGeom<EPV> g0(x0, cols);
      const int e0 = g0.extra_col(tid);
      if (e0 >= 0) xe_raw = load1_raw(x0 + e0);
      stage_row<Tin, T, LPF, EPV>(x0, g0, tid, wave, stage);
      xe_next = raw_value<Tin>(raw_here(xe_raw));
    }
  }

  // gradient scale g and the smoothing offset g * eps / C (OPT only); the
  // rows not ignored are counted after the first row's copies are issued
  // (staged kernels). Counting inside the row loop, after a one-row
  // workgroup's loads, measured slower (fp32 4096 x 50257 mean 283 -> 324
  // us: the count's state stayed live across the loop and spilled).
  float gsc = 1.f, goff = 0.f;
  if constexpr (OPT) {
    gsc = opt.grad_scale;
    if (opt.count) gsc = gsc / (float)(*opt.count);
    else if (opt.count_inline) gsc = gsc / (float)count_valid_rows<BLOCK>(labels, rows, opt, count_slots);
    goff = gsc * (opt.smoothing / (float)cols);
    // uniform: held in scalar registers (as vector registers they were
    // spilled and reloaded in every row)
    gsc = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(gsc)));
    goff = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(goff)));
  }

  int merges = 0;  // cross-wave merges so far: picks the LDS slot
  for (int64_t row = first; row < rows; row += stride) {
    const Tin* xr = x + row * cols;
    Tin* gr = grad + row * cols;
    const RowGeom<EPV> g(xr, cols);
    const int ec = g.extra_col(tid);
    const int64_t rn = row + stride;

    const int label = label_next;
    if (rn < rows) label_next = __builtin_amdgcn_readfirstlane(labels[rn]);
    const bool ignored = OPT && opt.use_ignore && label == opt.ignore_index;
    if constexpr (OPT && !ARGMAX) {
      if (ignored) {  // uniform in the row owner: no loads, a zero row
        // (zeros from an opaque value: a zero vector hoisted out of the row
        // loop was spilled and reloaded in every row)
        const float zf = opaque(0.f);
        float z[NV][EPV];
#pragma unroll
        for (int i = 0; i < NV; ++i)
#pragma unroll
          for (int k = 0; k < EPV; ++k) z[i][k] = zf;
        store_chunks<Tin, T, NV, EPV>(gr, g, tid, z);
        if (ec >= 0) store1(gr + ec, zf);
        if (tid == 0) store_loss(loss + row, 0.f, opt.reduction != 0);
        if constexpr (LPF > 0) {
          have_pre = rn < rows && !(opt.use_ignore && label_next == opt.ignore_index);
          if (have_pre) {
            const Tin* xn = x + rn * cols;
            wait_lds_reads();
            const RowGeom<EPV> gn(xn, cols);
            const int en = gn.extra_col(tid);
            xe_raw = en >= 0 ? load1_raw(xn + en) : kRawNegInf<Tin>;
            stage_row<Tin, T, LPF, EPV>(xn, gn, tid, wave, stage);
            xe_next = raw_value<Tin>(raw_here(xe_raw));
            stores_after = 0;  // staged after this row's stores
          }
        }
        continue;
      }
    }

    // The label column is handled by the one lane that owns it (the lane of
    // the row owner that loads that column). It reads the label logit with
    // its own load, before any of its stores: in-place calls (grad == logits)
    // stay correct because a lane's accesses to one address keep their order.
    const bool valid = label >= 0 && label < cols;
    const bool label_lane = valid && !ignored && owner_lane<T, EPV>(label, g) == tid;
    float v[NV][EPV];
    float xe;
    if constexpr (LPF > 0) {
      if (have_pre) {
        if (stores_after >= NV - 1) wait_vmcnt_upto<NV - 1>();
        else wait_lds_copies();
        load_staged<Tin, T, NV, LPF, EPV, kLate>(xr, g, tid, stage, v, kNegInf);
        xe = xe_next;
      } else {
        load_chunks<Tin, T, NV, EPV>(xr, g, tid, v, kNegInf);
        xe = ec >= 0 ? load1(xr + ec) : kNegInf;
      }
    } else {
      load_chunks<Tin, T, NV, EPV>(xr, g, tid, v, kNegInf);
      xe = ec >= 0 ? load1(xr + ec) : kNegInf;
    }
    uint32_t x_label_raw = 0;  // converted where it is used, after the row's reduction
    if (label_lane) x_label_raw = load1_raw(xr + label);
    if constexpr (LPF > 0) {
      // the next row's first slots (not when it is an ignored row that is
      // not read)
      have_pre = rn < rows &&
                 !(OPT && !ARGMAX && opt.use_ignore && label_next == opt.ignore_index);
      if (have_pre) {
        const Tin* xn = x + rn * cols;
        wait_lds_reads();  // this row's staged slots are in registers
        const RowGeom<EPV> gn(xn, cols);
        const int en = gn.extra_col(tid);
        if constexpr (kLate) {
          xe_raw = en >= 0 ? load1_raw(xn + en) : kRawNegInf<Tin>;  // converted before the stores
          stage_row<Tin, T, LPF, EPV>(xn, gn, tid, wave, stage);
        } else {
          stage_row<Tin, T, LPF, EPV>(xn, gn, tid, wave, stage);
          xe_next = en >= 0 ? load1(xn + en) : kNegInf;
        }
        stores_after = 0;
      }
    }

    // the wave's maximum first: exponentials relative to it, plain sums
    const float m = wave_max(lane_max<NV, EPV>(v, xe));
    Base bs;
    float tsum = 0.f;
    if constexpr (OPT) {
      // sum of this lane's logits (masked slots hold -inf and are skipped;
      // only a slot that runs past the row's end can hold any)
      float t0 = ec >= 0 ? xe : 0.f, t1 = 0.f;
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        if ((i + 1) * T <= g.nvec) {  // uniform: the whole slot lies in the row
#pragma unroll
          for (int k = 0; k < EPV; ++k) {
            if (k & 1) t1 += v[i][k]; else t0 += v[i][k];
          }
        } else {
          const bool ok = i * T + tid < g.nvec;
#pragma unroll
          for (int k = 0; k < EPV; ++k) {
            const float a = ok ? v[i][k] : 0.f;
            if (k & 1) t1 += a; else t0 += a;
          }
        }
      }
      tsum = t0 + t1;
    }
    float best = 3.0e38f;
    if constexpr (ARGMAX) {
      // smallest column of this lane holding the wave's maximum
#pragma unroll
      for (int i = 0; i < NV; ++i)
#pragma unroll
        for (int k = 0; k < EPV; ++k) {
          const float col = (float)((uint32_t)g.head + (uint32_t)(i * T + tid) * EPV + k);
          best = (v[i][k] == m && col < best) ? col : best;
        }
      if (ec >= 0 && xe == m && (float)ec < best) best = (float)ec;
    }
    {
      // e_j replaces x_j; the wave's sums and first column of its maximum
      const MaxSumState ms = LOG2 ? lane_exp_log2<NV, EPV>(v, xe, m)
                                  : lane_exp_nat<NV, EPV>(v, xe, m);
      const WaveSums ws = wave_reduce(WaveSums{ms.s, tsum, best}, WaveSumsMerge{});
      bs.m = m;
      bs.s = ws.s;
      if constexpr (ARGMAX) bs.idx = ws.idx;
      tsum = ws.t;
    }
    State st;
    if constexpr (OPT) st = State{bs, tsum};
    else st = bs;
    if constexpr (NW > 1) {
      Base eb;  // the empty state
      eb.m = kNegInf;
      eb.s = 0.f;
      if constexpr (ARGMAX) eb.idx = 3.0e38f;
      State empty;
      if constexpr (OPT) empty = State{eb, 0.f};
      else empty = eb;
      st = block_merge_tree<NW>(st, xw[merges++ & 1], wave, lane, Merge{}, empty);
    }
    Base rs;
    if constexpr (OPT) {
      rs = st.st;
      tsum = st.t;
    } else {
      rs = st;
    }
    // the row sum in natural units (the base-2 form carries the 2^kExpBias bias)
    const float s_row = LOG2 ? __builtin_ldexpf(rs.s, -kExpBias) : rs.s;

    if (OPT && ignored) {  // (argmax wanted) zero row, loss 0
#pragma unroll
      for (int i = 0; i < NV; ++i)
#pragma unroll
        for (int k = 0; k < EPV; ++k) v[i][k] = 0.f;
      xe = 0.f;
    } else if constexpr (LOG2) {
      // One factor f = g 2^n per wave and one fma per element. With the 2^8
      // bias every e_j <= 2^8, so where f is subnormal its rounding (at most
      // 2^-150) moves p_j by at most 2^-142, a 2^-9 fraction of the finest
      // bf16 step; where f is normal, f = g 2^n exactly and the fma rounds
      // p_j - offset once.
      const Log2Scale sc = log2_scale(m, rs.m, rs.s);
      const float f = __builtin_ldexpf(sc.g * gsc, sc.n);
#pragma unroll
      for (int i = 0; i < NV; ++i)
#pragma unroll
        for (int k = 0; k < EPV; ++k) v[i][k] = __builtin_fmaf(v[i][k], f, -goff);
      xe = __builtin_fmaf(xe, f, -goff);
    } else if constexpr (OPT) {
      const float f = nat_scale(m, rs.m, rs.s) * gsc;
#pragma unroll
      for (int i = 0; i < NV; ++i)
#pragma unroll
        for (int k = 0; k < EPV; ++k) v[i][k] = __builtin_fmaf(v[i][k], f, -goff);
      xe = __builtin_fmaf(xe, f, -goff);
    } else {
      const float f = nat_scale(m, rs.m, rs.s);
#pragma unroll
      for (int i = 0; i < NV; ++i)
#pragma unroll
        for (int k = 0; k < EPV; ++k) v[i][k] *= f;
      xe *= f;
    }
    // the next row's head/tail element, before this row's stores (its wait
    // leaves the next row's copies in flight)
    if constexpr (LPF > 0 && kLate) xe_next = raw_value<Tin>(raw_here(xe_raw));
    store_chunks<Tin, T, NV, EPV>(gr, g, tid, v);
    if constexpr (LPF > 0) stores_after = g.nvec / T;  // whole slots
    if (ec >= 0) store1(gr + ec, xe);

    if (label_lane) {
      // overwrite the label element (after this lane's own store of it to
      // the same address), and write the loss
      const float x_label = raw_value<Tin>(kLate ? raw_here(x_label_raw) : x_label_raw);
      const float p = exp_acc(x_label - rs.m) / s_row;
      const float lse = rs.m + logf(s_row);
      if constexpr (OPT) {
        // terms with a zero weight are left out (a -inf logit would make
        // them 0 * inf); the same reading as the definition's weighted sum.
        // The constants are formed here from opaque copies, so they are not
        // hoisted out of the row loop and held (or spilled) across it.
        const float eps = opaque(opt.smoothing);
        const float fc = (float)cols;
        store1(gr + label, opaque(gsc) * ((p - (1.f - eps)) - eps / fc));
        float l = lse;
        if (eps != 1.f) l -= (1.f - eps) * x_label;
        if (eps != 0.f) l -= eps * (tsum / fc);
        store_loss(loss + row, l, opt.reduction != 0);
      } else {
        store1(gr + label, p - 1.f);
        loss[row] = lse - x_label;
      }
    } else if (tid == 0 && (ignored || !valid)) {
      store_loss(loss + row, ignored ? 0.f : __builtin_nanf(""), OPT && opt.reduction != 0);
    }
    if constexpr (ARGMAX) {
      if (tid == 0) argmax[row] = (int32_t)rs.idx;
    }
  }
  if constexpr (OPT) {
    if (opt.reduction) finish_total<BLOCK>(loss, rows, opt, count_slots, red, &last_wg);
  }
}

// ------------------------------------------- completion counters (sum / mean)
// A pool of counters per GPU, zero at load; every call that reduces over
// rows takes the next one and its last workgroup sets it back to zero. Calls
// in flight at the same time on one GPU (on different streams) take
// different counters unless more than kXentDoneSlots of them overlap.
constexpr int kXentDoneSlots = 256;
static __device__ uint32_t xent_done[kXentDoneSlots];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_done_mu;
uint32_t* g_done_ptr[kMaxDevices] = {};
std::atomic<uint32_t> g_done_next{0};
}  // namespace

hipError_t xent_done_counter(uint32_t** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  uint32_t* base;
  {
    std::lock_guard<std::mutex> lock(g_done_mu);
    if (!g_done_ptr[dev]) {
      void* p = nullptr;
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(xent_done));
      if (e != hipSuccess) return e;
      if (!p) return hipErrorInvalidSymbol;
      g_done_ptr[dev] = static_cast<uint32_t*>(p);
    }
    base = g_done_ptr[dev];
  }
  *out = base + g_done_next.fetch_add(1, std::memory_order_relaxed) % kXentDoneSlots;
  return hipSuccess;
}

// ------------------------------------------------- reductions over rows
// Single-workgroup kernels (1024 lanes) for the row-count and the loss total:
// each lane takes rows lane, lane + 1024, ... in order, then a fixed LDS tree.

// n_valid = number of rows whose label is not the ignore index.
__global__ __launch_bounds__(1024) void xent_count_kernel(const int32_t* labels, int64_t rows,
                                                          int use_ignore, int ignore_index,
                                                          uint32_t* out) {
  __shared__ uint32_t red[1024];
  uint32_t c = 0;
  for (int64_t r = threadIdx.x; r < rows; r += 1024)
    c += (use_ignore && labels[r] == ignore_index) ? 0u : 1u;
  red[threadIdx.x] = c;
  __syncthreads();
#pragma unroll
  for (int w = 512; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) *out = red[0];
}

// total = sum of loss[r] (double accumulation), divided by *count for a mean.
// `total` may be the same 4 bytes as `count` (the count is read first).
__global__ __launch_bounds__(1024) void xent_total_kernel(const float* loss, int64_t rows,
                                                          const uint32_t* count, float* total) {
  __shared__ double red[1024];
  double sacc = 0.0;
  for (int64_t r = threadIdx.x; r < rows; r += 1024) sacc += (double)loss[r];
  red[threadIdx.x] = sacc;
  __syncthreads();
#pragma unroll
  for (int w = 512; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const double t = red[0];
    *total = count ? (float)(t / (double)*count) : (float)t;
  }
}

hipError_t launch_xent_count(const int32_t* labels, int64_t rows, int use_ignore, int ignore_index,
                             uint32_t* out, hipStream_t s) {
  return launch_kernel(&xent_count_kernel, dim3(1), dim3(1024), s, labels, rows, use_ignore,
                       ignore_index, out);
}

hipError_t launch_xent_total(const float* loss, int64_t rows, const uint32_t* count, float* total,
                             hipStream_t s) {
  return launch_kernel(&xent_total_kernel, dim3(1), dim3(1024), s, loss, rows, count, total);
}

template <typename Tin, int T, int NV, int EPV, int OCC, bool ARGMAX, bool OPT, int LPF = 0>
static hipError_t launch_xent(const void* x, const int32_t* labels, float* loss, void* grad,
                              int32_t* argmax, int64_t rows, int cols, const XentOptions* opt,
                              hipStream_t s) {
  constexpr int BLOCK = T == 64 ? 256 : T;
  constexpr int RPB = BLOCK / T;
  int64_t blocks = (rows + RPB - 1) / RPB;
  if (LPF > 0) {  // one resident workgroup per compute unit, looping over rows
    const int64_t ncu = device_cu_count();
    blocks = blocks < ncu ? blocks : ncu;
  }
  const unsigned grid = (unsigned)(blocks < kMaxGrid ? blocks : kMaxGrid);
  const XentOptions o = opt ? *opt : XentOptions{0, 0, 0.f, 1.f, nullptr, 0, 0, nullptr, nullptr};
  return launch_kernel(&xent_kernel<Tin, T, NV, EPV, OCC, ARGMAX, OPT, LPF>, dim3(grid), dim3(BLOCK), s,
                       static_cast<const Tin*>(x), labels, loss, static_cast<Tin*>(grad), argmax,
                       rows, cols, o);
}

#define FR_XE(TS, T, NV, EPV, OCC, AM, OPT) {T, NV, EPV, &launch_xent<TS, T, NV, EPV, OCC, AM, OPT>}
// LDS staging of the next row (measured at 4096 x 50257): the whole bf16 row
// (7 slots, 112 KiB) takes the options kernel from 170 to 165 us and the
// argmax kernel from 284 to 200 us (a one-slot register prefetch had taken
// the options kernel from 177 to 170 us before). fp32 rows stay unstaged:
// 9 slots in LDS measured 287 -> 295 us, 2-5 register slots 285 -> 290 us.
#define FR_XE_STAGED(TS, T, NV, EPV, OCC, AM, OPT, LPF) \
  {T, NV, EPV, &launch_xent<TS, T, NV, EPV, OCC, AM, OPT, LPF>}
#define FR_XE_F32(AM, OPT)                                                                       \
  {FR_XE(float, 64, 1, 4, 8, AM, OPT),    FR_XE(float, 64, 2, 4, 8, AM, OPT),                    \
   FR_XE(float, 64, 4, 4, 8, AM, OPT),    FR_XE(float, 64, 8, 4, 6, AM, OPT),                    \
   FR_XE(float, 64, 16, 4, 4, AM, OPT),   FR_XE(float, 256, 8, 4, 6, AM, OPT),                   \
   FR_XE(float, 512, 8, 4, 6, AM, OPT),   FR_XE(float, 1024, 8, 4, 4, AM, OPT),                  \
   FR_XE(float, 1024, 13, 4, 4, AM, OPT), FR_XE(float, 512, 25, 4, 4, AM, OPT),                  \
   FR_XE(float, 256, 50, 4, 2, AM, OPT),  FR_XE(float, 1024, 16, 4, 4, AM, OPT),                 \
   FR_XE(float, 64, 16, 1, 4, AM, OPT),   FR_XE(float, 256, 16, 1, 4, AM, OPT),                  \
   FR_XE(float, 1024, 16, 1, 4, AM, OPT), FR_XE(float, 1024, 64, 1, 4, AM, OPT)}
#define FR_XE_BF16(AM)                                                                           \
  {FR_XE(bf16_t, 64, 1, 8, 8, AM, true),    FR_XE(bf16_t, 64, 2, 8, 8, AM, true),                \
   FR_XE(bf16_t, 64, 4, 8, 6, AM, true),    FR_XE(bf16_t, 64, 8, 8, 4, AM, true),                \
   FR_XE(bf16_t, 256, 4, 8, 6, AM, true),   FR_XE(bf16_t, 512, 4, 8, 6, AM, true),               \
   FR_XE(bf16_t, 1024, 4, 8, 4, AM, true),  FR_XE_STAGED(bf16_t, 1024, 7, 8, 4, AM, true, 7),    \
   FR_XE(bf16_t, 1024, 8, 8, 4, AM, true),  FR_XE(bf16_t, 64, 16, 1, 4, AM, true),               \
   FR_XE(bf16_t, 256, 16, 1, 4, AM, true),  FR_XE(bf16_t, 1024, 16, 1, 4, AM, true),             \
   FR_XE(bf16_t, 1024, 64, 1, 4, AM, true)}

// plain (fr_softmax_xent_fwd_bwd, fp32) and with options (fr_softmax_xent_ex)
static const XentVariant kXe[] = FR_XE_F32(false, false);
static const XentVariant kXeArgmax[] = FR_XE_F32(true, false);
static const XentVariant kXeOpt[] = FR_XE_F32(false, true);
static const XentVariant kXeOptArgmax[] = FR_XE_F32(true, true);
static const XentVariant kXeBf16[] = FR_XE_BF16(false);
static const XentVariant kXeBf16Argmax[] = FR_XE_BF16(true);

#define FR_SPAN(a) {a, sizeof(a) / sizeof(a[0])}

VariantSpan<XentVariant> xent_variants(int bf16, int with_argmax) {
  if (bf16) return {nullptr, 0};
  if (with_argmax) return FR_SPAN(kXeArgmax);
  return FR_SPAN(kXe);
}

VariantSpan<XentVariant> xent_ex_variants(int bf16, int with_argmax) {
  if (bf16) return with_argmax ? VariantSpan<XentVariant>FR_SPAN(kXeBf16Argmax)
                               : VariantSpan<XentVariant>FR_SPAN(kXeBf16);
  return with_argmax ? VariantSpan<XentVariant>FR_SPAN(kXeOptArgmax)
                     : VariantSpan<XentVariant>FR_SPAN(kXeOpt);
}

}  // namespace fr
