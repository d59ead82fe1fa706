// Backward passes of the row operations, each reading its row operands once.
//
// Softmax ("NexusGrad", Verified VJP Operators: softmax): from the stored
// forward output p and the upstream gradient dy,
//   s = sum_k p_k dy_k,   dx_j = p_j (dy_j - s),
// one reduction per row and the gradient written from the same registers.
//
// Residual add + RMSNorm (same page, RMSNorm and residual blocks): from the
// stored updated residual h = x + residual, the weight w, dy and the gradient
// dres reaching h through the updated residual,
//   r = 1/sqrt(sum h^2 / C + eps),   c = r^2 sum_k dy_k w_k h_k / C,
//   dh_j = r (w_j dy_j - h_j c) + dres_j,   dw_j = sum_rows dy_j h_j r.
// LayerNorm (same page; "Engineering a CUDA Machine Learning Framework from
// Scratch", §3.2 for the saved statistics): from x, dy, gamma and the saved
// per-row mean and rstd, with n = (x - mean) rstd and g = dy gamma,
//   dx_j = rstd (g_j - mean(g) - n_j mean(g n)),
//   dgamma_j = sum_rows dy_j n_j,   dbeta_j = sum_rows dy_j.
//
// Parameter gradients are column sums over all rows. The norm kernels run a
// persistent grid of at most grid_max workgroups, each of RPB row groups of
// T lanes; every lane owns the same columns in every row it visits (rows on
// the 16-byte grid, no head peel), so it accumulates its columns' partial
// sums in registers across its rows. At the end the row groups of a
// workgroup are summed through LDS in a fixed order and the workgroup writes
// one partial row per parameter to the workspace; colsum_kernel then adds
// the partial rows in a fixed order. There are no atomics: results are
// bitwise reproducible run to run.
#include "coop.hpp"
#include "fr_device.hpp"
#include "fr_kernels.hpp"

namespace fr {

// Clamped streaming load of chunk slot i (as load_chunks, one slot).
template <typename Ts, int T, int EPV, int AL>
__device__ __forceinline__ void load_slot(const Ts* row, const RowGeom<EPV, AL>& g, int tid, int i,
                                          float* v) {
  const uint32_t last = (uint32_t)(g.nvec - 1) * EPV;
  uint32_t o = (uint32_t)(i * T * EPV) + (uint32_t)tid * EPV;
  o = o < last ? o : last;
  Vec<Ts, EPV>::load(row + g.head + o, v);
}

// Ordinary (cached) fp32 vector access for partial sums, in global memory or
// LDS: they are read back soon, unlike the streamed rows.
template <int EPV>
__device__ __forceinline__ void store_f32(float* p, const float* v) {
  if constexpr (EPV == 1) {
    *p = v[0];
  } else {
#pragma unroll
    for (int k = 0; k < EPV; k += 4)
      *reinterpret_cast<f32x4*>(p + k) = f32x4{v[k], v[k + 1], v[k + 2], v[k + 3]};
  }
}
template <int EPV>
__device__ __forceinline__ void load_f32(const float* p, float* v) {
  if constexpr (EPV == 1) {
    v[0] = *p;
  } else {
#pragma unroll
    for (int k = 0; k < EPV; k += 4) {
      const f32x4 r = *reinterpret_cast<const f32x4*>(p + k);
      v[k] = r.x; v[k + 1] = r.y; v[k + 2] = r.z; v[k + 3] = r.w;
    }
  }
}

// ---------------------------------------------------------- softmax backward

template <typename Ts, int T, int NV, int EPV, int OCC>
__global__ __launch_bounds__(T == 64 ? 256 : T) __attribute__((amdgpu_waves_per_eu(OCC)))
void softmax_bwd_kernel(const Ts* p, const Ts* dy, Ts* dx, int64_t rows, int cols) {
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
    const RowGeom<EPV> g(p + off, cols);

    const int ec = g.extra_col(tid);
    const float ae = load_extra(p + off, ec, 0.f);
    const float de = load_extra(dy + off, ec, 0.f);
    float a[NV][EPV], d[NV][EPV];
    load_chunks2<Ts, T, NV, EPV>(p + off, dy + off, g, tid, a, d, 0.f);

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
    if constexpr (NW > 1) st = block_merge<NW>(st, xw[merges++ & 1], wave, lane, SumMerge{});

    const float s = st.s;
#pragma unroll
    for (int i = 0; i < NV; ++i)
#pragma unroll
      for (int k = 0; k < EPV; ++k) a[i][k] = a[i][k] * (d[i][k] - s);
    store_chunks<Ts, T, NV, EPV>(dx + off, g, tid, a);
    if (ec >= 0) store1(dx + off + ec, ae * (de - s));
  }
}

// ------------------------------------------------- norm backward, partials

// Sum the row groups' per-lane column partials of one parameter in row-group
// order and write the workgroup's partial row (`cols` floats at wsrow).
// RPB > 1: every row group writes all its slots to buf (NV RPB T EPV floats;
// row group r's slot i of lane t at ((i RPB + r) T + t) EPV), then after one
// barrier every lane of the workgroup takes columns lid, lid + T RPB, ... and
// adds their RPB values in row-group order (the same order, and bits, as one
// row group adding them slot by slot, in one round instead of NV). The
// barrier on entry lets buf reuse LDS that the row loop read (the staging
// buffer) or that a previous call read.
template <int T, int NV, int EPV, int RPB>
__device__ __forceinline__ void flush_partials(const float (&acc)[NV][EPV], float* buf,
                                               float* wsrow, int nvec, int tid, int sub) {
  if constexpr (RPB == 1) {
#pragma unroll
    for (int i = 0; i < NV; ++i)
      if (i * T + tid < nvec) store_f32<EPV>(wsrow + (i * T + tid) * EPV, acc[i]);
  } else {
    constexpr int L = T * RPB;  // lanes of the workgroup
    constexpr int W = T * EPV;  // columns per slot
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NV; ++i) store_f32<EPV>(buf + ((i * RPB + sub) * T + tid) * EPV, acc[i]);
    __syncthreads();
    const int lid = sub * T + tid;  // threadIdx.x
    const int ncol = nvec * EPV;
#pragma unroll
    for (int j = 0; j < (NV * W + L - 1) / L; ++j) {
      const int g = lid + j * L;  // column (slot g / W, lane (g % W) / EPV)
      if (g < NV * W && g < ncol) {
        const int i = g / W;
        const float* p = buf + i * RPB * W + (g - i * W);
        float sum = p[0];
#pragma unroll
        for (int r = 1; r < RPB; ++r) sum += p[r * W];
        wsrow[g] = sum;
      }
    }
  }
}

// Column slots of a lane in the norm backward kernels. Their rows start on
// the 16-byte grid (or EPV == 1): nvec = cols / EPV >= 1 chunks, no head, no
// tail, the same columns in every row. Slot i holds chunk i*T + tid; a slot
// past the row end reads the last chunk (in bounds) and is masked. Offsets
// are 32-bit element offsets from a uniform row or parameter base.
template <int T, int NV, int EPV>
struct Slots {
  int nvec, tid;
  uint32_t last;
  __device__ __forceinline__ Slots(int cols, int tid_)
      : nvec(cols / EPV), tid(tid_), last((uint32_t)(cols / EPV - 1) * EPV) {}
  __device__ __forceinline__ uint32_t off(int i) const {
    const uint32_t o = (uint32_t)((i * T + tid) * EPV);
    return o < last ? o : last;
  }
  __device__ __forceinline__ bool ok(int i) const { return i * T + tid < nvec; }

  template <typename Ts>
  __device__ __forceinline__ void load2(const Ts* ra, const Ts* rb, float (&a)[NV][EPV],
                                        float (&b)[NV][EPV]) const {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      Vec<Ts, EPV>::load(ra + off(i), a[i]);
      Vec<Ts, EPV>::load(rb + off(i), b[i]);
    }
#pragma unroll
    for (int i = 0; i < NV; ++i)
#pragma unroll
      for (int k = 0; k < EPV; ++k) {
        a[i][k] = ok(i) ? a[i][k] : 0.f;
        b[i][k] = ok(i) ? b[i][k] : 0.f;
      }
  }
  template <typename Ts>
  __device__ __forceinline__ void load3(const Ts* ra, const Ts* rb, const Ts* rc,
                                        float (&a)[NV][EPV], float (&b)[NV][EPV],
                                        float (&c)[NV][EPV]) const {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      Vec<Ts, EPV>::load(ra + off(i), a[i]);
      Vec<Ts, EPV>::load(rb + off(i), b[i]);
      Vec<Ts, EPV>::load(rc + off(i), c[i]);
    }
#pragma unroll
    for (int i = 0; i < NV; ++i)
#pragma unroll
      for (int k = 0; k < EPV; ++k) {
        a[i][k] = ok(i) ? a[i][k] : 0.f;
        b[i][k] = ok(i) ? b[i][k] : 0.f;
        c[i][k] = ok(i) ? c[i][k] : 0.f;
      }
  }
  template <typename Ts>
  __device__ __forceinline__ void param(const Ts* par, int i, float* v) const {
    load_param<Ts, EPV>(par + off(i), v);
  }
  template <typename Ts>
  __device__ __forceinline__ void store(Ts* r, const float (&v)[NV][EPV]) const {
#pragma unroll
    for (int i = 0; i < NV; ++i)
      if (ok(i)) Vec<Ts, EPV>::store(r + off(i), v[i]);
  }
};

// The parameter pointer as a fresh uniform value in each phase of each row:
// the loads then stay in (uniform base + 32-bit lane offset) form inside the
// loop instead of being hoisted out as per-slot 64-bit addresses, and the
// second phase reloads the parameters (cache hits) instead of keeping the
// first phase's registers live across the row reduction.
// (An opaque zero is added rather than the pointer itself laundered, which
// would lose its global address space and turn the loads into flat ones.)
template <typename T>
__device__ __forceinline__ const T* fresh(const T* p) {
  int z = 0;
  asm volatile("" : "+s"(z));
  return p + z;
}

// Lane layout of the norm backward workgroup: RPB row groups of T lanes.
// The row loop runs the same number of times in every wave of the
// workgroup (block-wide barriers inside); a row group past the last row
// takes part in the barriers with no data.
template <int T, int RPB_>
struct BwdLanes {
  static constexpr int RPB = RPB_;
  static constexpr int NW = T / 64;
  int lane, sub, wave, tid;
  __device__ __forceinline__ BwdLanes() {
    const int wib = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    lane = threadIdx.x & 63;
    sub = wib / NW;
    wave = wib % NW;
    tid = wave * 64 + lane;
  }
};

// ------------------------------------------------ residual add + RMSNorm bwd

// DRES: the gradient through the updated residual is given; its loads are
// issued with those of h and dy, before the row reduction.
// STG: the row operands of the workgroup's next rows are staged in LDS
// (global_load_lds_dwordx4, 16 bytes per lane and slot, read back by the
// lane that requested them) while the current rows are reduced and written.
// Vector memory operations retire in issue order: the next iteration's wait
// leaves this iteration's whole-slot stores outstanding, and the weight is
// read from LDS, so no wait inside the row loop waits for the staging.
template <typename Ts, int T, int NV, int EPV, int RPB, int OCC, bool DRES, bool STG = false>
__global__ __launch_bounds__(T * RPB) __attribute__((amdgpu_waves_per_eu(OCC)))
void rmsnorm_bwd_kernel(const Ts* h, const Ts* dy, const Ts* dres, const Ts* w, Ts* dh, float* ws,
                        int64_t rows, int cols, float eps) {
  using L = BwdLanes<T, RPB>;
  constexpr int NW = L::NW;
  constexpr int NOP = DRES ? 3 : 2;  // staged row operands
  static_assert(!STG || EPV * sizeof(Ts) == 16, "staging: 16-byte chunks");
  __shared__ float xw[RPB][2][NW][2];
  // the partial-row buffer of flush_partials: the staging buffer when staged
  // (read for the last time before it), else its own
  __shared__ __attribute__((aligned(16))) float part[RPB > 1 && !STG ? NV * T * RPB * EPV : 4];
  __shared__ __attribute__((aligned(16))) uint32_t stage[STG ? NOP * NV * T * RPB * 4 : 4];
  static_assert(!STG || RPB == 1 || NOP * 4 >= EPV, "partials fit in the staging buffer");
  // STG: the weight's chunks of this lane's slots, loaded once (no weight
  // loads inside the row loop, whose waits would also wait for the staging)
  __shared__ __attribute__((aligned(16))) uint32_t wlds[STG ? NV * T * 4 : 4];
  const L ln;
  const Slots<T, NV, EPV> sl(cols, ln.tid);
  using Raw = typename RawChunk<Ts>::T;
  const int wib = ln.sub * NW + ln.wave;  // wave index in the workgroup
  // stage operand `op` of the row at element offset `o`: slot i of lane
  // (wib, l) lands at 16 ((op NV + i) T RPB + 64 wib + l)
  auto stage_op = [&](const Ts* src, int op) {
#pragma unroll
    for (int i = 0; i < NV; ++i)
      __builtin_amdgcn_global_load_lds(
          static_cast<const void*>(src + sl.off(i)),
          (__attribute__((address_space(3))) void*)(stage + ((op * NV + i) * T * RPB + 64 * wib) * 4),
          16, 0, kCopyNT);
  };
  auto stage_rows = [&](int64_t b) {  // the rows of iteration base b (uniform)
    const int64_t rw = b + ln.sub;
    const int64_t o = (rw < rows ? rw : rows - 1) * cols;
    stage_op(h + o, 0);
    stage_op(dy + o, 1);
    if constexpr (DRES) stage_op(dres + o, 2);
  };
  // this lane's staged operands (NOP x NV chunks), read past the compiler's
  // LDS-copy wait (the counted wait has covered them)
  auto unstage = [&](float (&v0)[NV][EPV], float (&v1)[NV][EPV], float (&v2)[DRES ? NV : 1][EPV]) {
    uint32_t a[NOP * NV];
    u32x4 r[NOP * NV];
#pragma unroll
    for (int j = 0; j < NOP * NV; ++j) a[j] = lds_offset(stage + (j * T * RPB + threadIdx.x) * 4);
    read_staged(a, r);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      RawChunk<Ts>::unpack(__builtin_bit_cast(Raw, r[i]), v0[i]);
      RawChunk<Ts>::unpack(__builtin_bit_cast(Raw, r[NV + i]), v1[i]);
      if constexpr (DRES) RawChunk<Ts>::unpack(__builtin_bit_cast(Raw, r[2 * NV + i]), v2[i]);
#pragma unroll
      for (int k = 0; k < EPV; ++k) {
        v0[i][k] = sl.ok(i) ? v0[i][k] : 0.f;
        v1[i][k] = sl.ok(i) ? v1[i][k] : 0.f;
        if constexpr (DRES) v2[i][k] = sl.ok(i) ? v2[i][k] : 0.f;
      }
    }
  };
  // the weight slot i of this lane: from LDS (STG) or from global memory
  auto wparam = [&](const Ts* wp, int i, float* wt) {
    if constexpr (STG) {
      RawChunk<Ts>::unpack(*reinterpret_cast<const Raw*>(wlds + (i * T + ln.tid) * 4), wt);
    } else {
      sl.param(wp, i, wt);
    }
  };
  bool staged = false;  // uniform in the workgroup: the next rows are being staged
  // uniform: whole-slot stores issued after the latest staging; with NV of
  // them, a wait leaving NV operations outstanding has seen the staging
  // complete (vector memory operations retire in issue order)
  int stores_after = 0;
  if constexpr (STG) {
    if (ln.sub == 0) {
#pragma unroll
      for (int i = 0; i < NV; ++i)
        *reinterpret_cast<Raw*>(wlds + (i * T + ln.tid) * 4) =
            *reinterpret_cast<const Raw*>(w + sl.off(i));
    }
    __syncthreads();
    if ((int64_t)blockIdx.x * RPB < rows) {
      stage_rows((int64_t)blockIdx.x * RPB);
      staged = true;
    }
  }

  float acc[NV][EPV];  // dw partials
#pragma unroll
  for (int i = 0; i < NV; ++i)
#pragma unroll
    for (int k = 0; k < EPV; ++k) acc[i][k] = 0.f;

  int merges = 0;  // cross-wave merges so far: picks the LDS slot
  for (int64_t base = (int64_t)blockIdx.x * RPB; base < rows;
       base += (int64_t)gridDim.x * RPB) {
    const int64_t row = base + ln.sub;
    const bool live = row < rows;  // uniform in the wave; a dead group re-reads the last row
    const int64_t off = (live ? row : rows - 1) * cols;

    float hv[NV][EPV], d[NV][EPV], dr[DRES ? NV : 1][EPV];
    if constexpr (STG) {
      if (stores_after >= NV) wait_vmcnt_upto<NV>();
      else wait_lds_copies();
      unstage(hv, d, dr);
      const int64_t nb = base + (int64_t)gridDim.x * RPB;
      staged = nb < rows;
      if (staged) {
        wait_lds_reads();  // this iteration's staged rows are in registers
        stage_rows(nb);
      }
    } else {
      if constexpr (DRES) sl.load3(h + off, dy + off, dres + off, hv, d, dr);
      else sl.load2(h + off, dy + off, hv, d);
    }
    float a0 = 0.f, a1 = 0.f, b0 = 0.f, b1 = 0.f;
    const Ts* w1 = fresh(w);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      float wt[EPV];
      wparam(w1, i, wt);
#pragma unroll
      for (int k = 0; k < EPV; ++k) {
        const float hk = hv[i][k];
        const float gk = d[i][k] * wt[k];
        if (k & 1) { a1 = __builtin_fmaf(hk, hk, a1); b1 = __builtin_fmaf(gk, hk, b1); }
        else { a0 = __builtin_fmaf(hk, hk, a0); b0 = __builtin_fmaf(gk, hk, b0); }
      }
    }
    Sum2State st{a0 + a1, b0 + b1};
    st = wave_reduce(st, Sum2Merge{});
    if constexpr (NW > 1) st = block_merge<NW>(st, xw[ln.sub][merges++ & 1], ln.wave, ln.lane, Sum2Merge{});

    if (live) {
      const float r = 1.f / __builtin_sqrtf(st.a / (float)cols + eps);
      const float c = r * r * (st.b / (float)cols);
      const Ts* w2 = fresh(w);
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        float wt[EPV];
        wparam(w2, i, wt);
#pragma unroll
        for (int k = 0; k < EPV; ++k) {
          acc[i][k] = __builtin_fmaf(d[i][k] * hv[i][k], r, acc[i][k]);
          const float t = r * __builtin_fmaf(-hv[i][k], c, wt[k] * d[i][k]);
          if constexpr (DRES) hv[i][k] = t + dr[i][k];
          else hv[i][k] = t;
        }
      }
    }
    if (live) sl.store(dh + off, hv);
    if constexpr (STG) stores_after = (staged && live && sl.nvec >= NV * T) ? NV : 0;
  }
  float* pbuf = STG ? reinterpret_cast<float*>(stage) : part;
  flush_partials<T, NV, EPV, RPB>(acc, pbuf, ws + (size_t)blockIdx.x * cols, sl.nvec, ln.tid, ln.sub);
}

// ------------------------------------------------------------ LayerNorm bwd

// STG: as the RMSNorm backward, the next rows' x and dy are staged in LDS
// (and their mean and rstd read) while the current rows are reduced and
// written, under counted waits; gamma is held in registers (loaded once), so
// no load inside the row loop waits for the staging.
template <typename Ts, int T, int NV, int EPV, int RPB, int OCC, bool STG = false>
__global__ __launch_bounds__(T * RPB) __attribute__((amdgpu_waves_per_eu(OCC)))
void layernorm_bwd_kernel(const Ts* x, const Ts* dy, const Ts* gamma,
                          // no output overlaps them (the entry points reject it), so the
                          // next rows' values come through scalar loads, which the counted
                          // wait of the staged path does not have to cover
                          const float* __restrict__ mean, const float* __restrict__ rstd, Ts* dx,
                          float* ws, int64_t rows, int cols) {
  using L = BwdLanes<T, RPB>;
  constexpr int NW = L::NW;
  static_assert(!STG || EPV * sizeof(Ts) == 16, "staging: 16-byte chunks");
  __shared__ float xw[RPB][2][NW][2];
  // the partial-row buffer of flush_partials: the staging buffer when staged
  __shared__ __attribute__((aligned(16))) float part[RPB > 1 && !STG ? NV * T * RPB * EPV : 4];
  __shared__ __attribute__((aligned(16))) uint32_t stage[STG ? 2 * NV * T * RPB * 4 : 4];
  static_assert(!STG || RPB == 1 || 8 >= EPV, "partials fit in the staging buffer");
  const L ln;
  const Slots<T, NV, EPV> sl(cols, ln.tid);
  using Raw = typename RawChunk<Ts>::T;
  const int wib = ln.sub * NW + ln.wave;  // wave index in the workgroup
  auto stage_op = [&](const Ts* src, int op) {
#pragma unroll
    for (int i = 0; i < NV; ++i)
      __builtin_amdgcn_global_load_lds(
          static_cast<const void*>(src + sl.off(i)),
          (__attribute__((address_space(3))) void*)(stage + ((op * NV + i) * T * RPB + 64 * wib) * 4),
          16, 0, kCopyNT);
  };
  // this lane's staged x and dy chunks, read past the compiler's LDS-copy
  // wait (the counted wait has covered them)
  auto unstage = [&](float (&v0)[NV][EPV], float (&v1)[NV][EPV]) {
    uint32_t a[2 * NV];
    u32x4 r[2 * NV];
#pragma unroll
    for (int j = 0; j < 2 * NV; ++j) a[j] = lds_offset(stage + (j * T * RPB + threadIdx.x) * 4);
    read_staged(a, r);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      RawChunk<Ts>::unpack(__builtin_bit_cast(Raw, r[i]), v0[i]);
      RawChunk<Ts>::unpack(__builtin_bit_cast(Raw, r[NV + i]), v1[i]);
#pragma unroll
      for (int k = 0; k < EPV; ++k) {
        v0[i][k] = sl.ok(i) ? v0[i][k] : 0.f;
        v1[i][k] = sl.ok(i) ? v1[i][k] : 0.f;
      }
    }
  };
  float gam[STG ? NV : 1][EPV];
  float mu_next = 0.f, rs_next = 0.f;
  bool staged = false;  // uniform in the workgroup: the next rows are being staged
  int stores_after = 0;  // uniform: whole-slot stores issued after the latest staging
  auto stage_rows = [&](int64_t b) {
    const int64_t rw = b + ln.sub;
    const int64_t rr = rw < rows ? rw : rows - 1;
    stage_op(x + rr * cols, 0);
    stage_op(dy + rr * cols, 1);
    mu_next = mean[rr];
    rs_next = rstd[rr];
  };
  if constexpr (STG) {
#pragma unroll
    for (int i = 0; i < NV; ++i) sl.param(gamma, i, gam[i]);
    if ((int64_t)blockIdx.x * RPB < rows) {
      stage_rows((int64_t)blockIdx.x * RPB);
      staged = true;
    }
  }

  float ag[NV][EPV], ab[NV][EPV];  // dgamma, dbeta partials
#pragma unroll
  for (int i = 0; i < NV; ++i)
#pragma unroll
    for (int k = 0; k < EPV; ++k) { ag[i][k] = 0.f; ab[i][k] = 0.f; }

  int merges = 0;  // cross-wave merges so far: picks the LDS slot
  for (int64_t base = (int64_t)blockIdx.x * RPB; base < rows;
       base += (int64_t)gridDim.x * RPB) {
    const int64_t row = base + ln.sub;
    const bool live = row < rows;
    const int64_t rr = live ? row : rows - 1;
    const int64_t off = rr * cols;
    float mu, rs;
    float n[NV][EPV], d[NV][EPV];
    if constexpr (STG) {
      if (stores_after >= NV) wait_vmcnt_upto<NV>();
      else wait_lds_copies();
      unstage(n, d);
      mu = mu_next;
      rs = rs_next;
      const int64_t nb = base + (int64_t)gridDim.x * RPB;
      staged = nb < rows;
      if (staged) {
        wait_lds_reads();  // this iteration's staged rows are in registers
        stage_rows(nb);
      }
    } else {
      mu = mean[rr];
      rs = rstd[rr];
      sl.load2(x + off, dy + off, n, d);
    }
    float a0 = 0.f, a1 = 0.f, b0 = 0.f, b1 = 0.f;
    const Ts* g1 = fresh(gamma);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      float ga[EPV];
      if constexpr (STG) {
#pragma unroll
        for (int k = 0; k < EPV; ++k) ga[k] = gam[i][k];
      } else {
        sl.param(g1, i, ga);
      }
#pragma unroll
      for (int k = 0; k < EPV; ++k) {
        n[i][k] = (n[i][k] - mu) * rs;  // masked slots have dy = 0 and add nothing
        const float gk = d[i][k] * ga[k];
        if (k & 1) { a1 += gk; b1 = __builtin_fmaf(gk, n[i][k], b1); }
        else { a0 += gk; b0 = __builtin_fmaf(gk, n[i][k], b0); }
      }
    }
    Sum2State st{a0 + a1, b0 + b1};
    st = wave_reduce(st, Sum2Merge{});
    if constexpr (NW > 1) st = block_merge<NW>(st, xw[ln.sub][merges++ & 1], ln.wave, ln.lane, Sum2Merge{});

    if (live) {
      const float mg = st.a / (float)cols;
      const float mgn = st.b / (float)cols;
      const Ts* g2 = fresh(gamma);
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        float ga[EPV];
        if constexpr (STG) {
#pragma unroll
          for (int k = 0; k < EPV; ++k) ga[k] = gam[i][k];
        } else {
          sl.param(g2, i, ga);
        }
#pragma unroll
        for (int k = 0; k < EPV; ++k) {
          ag[i][k] = __builtin_fmaf(d[i][k], n[i][k], ag[i][k]);
          ab[i][k] += d[i][k];
          n[i][k] = rs * __builtin_fmaf(-n[i][k], mgn, __builtin_fmaf(d[i][k], ga[k], -mg));
        }
      }
      sl.store(dx + off, n);
    }
    if constexpr (STG) stores_after = (staged && live && sl.nvec >= NV * T) ? NV : 0;
  }
  const size_t G = gridDim.x;
  float* pbuf = STG ? reinterpret_cast<float*>(stage) : part;
  flush_partials<T, NV, EPV, RPB>(ag, pbuf, ws + (size_t)blockIdx.x * cols, sl.nvec, ln.tid, ln.sub);
  flush_partials<T, NV, EPV, RPB>(ab, pbuf, ws + (G + blockIdx.x) * cols, sl.nvec, ln.tid, ln.sub);
}

// ------------------------------------------------- split-row norm backward
// Rows wider than one workgroup's registers: the row is cut into segments
// of kBwdSplitSeg columns (rows on the 16-byte grid or the scalar path, so a
// segment's lanes own fixed columns, as above).
//   pass 1 (norm_bwd_split_sums_kernel): each (row, segment) writes its two
//     partial row sums — sum h^2 and sum dy w h (RMSNorm), sum g and sum g n
//     (LayerNorm) — to part[row][segment];
//   pass 2 (norm_bwd_split_apply_kernel): workgroup (segment sg, row group
//     rg) takes rows rg, rg + RG, ...: per row it adds the row's partials in
//     segment order (the same bits in every workgroup of the row), writes
//     the segment's dh / dx and accumulates its columns' parameter-gradient
//     partials in registers; at the end it writes them to partial row rg of
//     the workspace [params][RG][cols];
//   colsum_kernel then adds the RG partial rows in order.

template <typename Ts, int T, int NV, int EPV, bool LN>
__global__ __launch_bounds__(T) __attribute__((amdgpu_waves_per_eu(4)))
void norm_bwd_split_sums_kernel(const Ts* xh, const Ts* dy, const Ts* w, const float* mean,
                                const float* rstd, int64_t rows, int cols, int nseg,
                                float4* part) {
  constexpr int NW = T / 64;
  constexpr int SEG = T * NV * EPV;
  __shared__ float xw[2][NW][2];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int tid = threadIdx.x;
  const int64_t work = rows * nseg;
  int merges = 0;  // cross-wave merges so far: picks the LDS slot
  for (int64_t wk = blockIdx.x; wk < work; wk += gridDim.x) {
    const int64_t row = wk / nseg;
    const int c0 = (int)(wk - row * nseg) * SEG;
    const int len = cols - c0 < SEG ? cols - c0 : SEG;
    const Slots<T, NV, EPV> sl(len, tid);
    const int64_t off = row * cols + c0;
    float a[NV][EPV], d[NV][EPV];
    sl.load2(xh + off, dy + off, a, d);
    float mu = 0.f, rs = 1.f;
    if constexpr (LN) {
      mu = mean[row];
      rs = rstd[row];
    }
    const Ts* w1 = fresh(w) + c0;
    float a0 = 0.f, a1 = 0.f, b0 = 0.f, b1 = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      float wt[EPV];
      sl.param(w1, i, wt);
#pragma unroll
      for (int k = 0; k < EPV; ++k) {
        const float gk = d[i][k] * wt[k];
        if constexpr (LN) {
          const float nk = sl.ok(i) ? (a[i][k] - mu) * rs : 0.f;
          if (k & 1) { a1 += gk; b1 = __builtin_fmaf(gk, nk, b1); }
          else { a0 += gk; b0 = __builtin_fmaf(gk, nk, b0); }
        } else {
          const float hk = a[i][k];
          if (k & 1) { a1 = __builtin_fmaf(hk, hk, a1); b1 = __builtin_fmaf(gk, hk, b1); }
          else { a0 = __builtin_fmaf(hk, hk, a0); b0 = __builtin_fmaf(gk, hk, b0); }
        }
      }
    }
    Sum2State st{a0 + a1, b0 + b1};
    st = wave_reduce(st, Sum2Merge{});
    if constexpr (NW > 1) st = block_merge<NW>(st, xw[merges++ & 1], wave, lane, Sum2Merge{});
    if (tid == 0) part[wk] = float4{st.a, st.b, 0.f, 0.f};
  }
}

// xh: h (RMSNorm) or x (LayerNorm); w: weight or gamma; dres: RMSNorm only
// (may be NULL); out: dh or dx; ws: [params][RG][cols].
template <typename Ts, int T, int NV, int EPV, bool LN, bool DRES>
__global__ __launch_bounds__(T) __attribute__((amdgpu_waves_per_eu(4)))
void norm_bwd_split_apply_kernel(const Ts* xh, const Ts* dy, const Ts* dres, const Ts* w,
                                 const float* mean, const float* rstd, Ts* out, float* ws,
                                 int64_t rows, int cols, int nseg, int RG, const float4* part,
                                 float eps) {
  constexpr int NW = T / 64;
  constexpr int SEG = T * NV * EPV;
  __shared__ float xw[2][NW][2];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int tid = threadIdx.x;
  const int sg = (int)(blockIdx.x % (unsigned)nseg);
  const int rg = (int)(blockIdx.x / (unsigned)nseg);
  const int c0 = sg * SEG;
  const int len = cols - c0 < SEG ? cols - c0 : SEG;
  const Slots<T, NV, EPV> sl(len, tid);

  float acc[NV][EPV], acc2[LN ? NV : 1][EPV];  // dw (dgamma) and dbeta partials
#pragma unroll
  for (int i = 0; i < NV; ++i)
#pragma unroll
    for (int k = 0; k < EPV; ++k) acc[i][k] = 0.f;
#pragma unroll
  for (int i = 0; i < (LN ? NV : 1); ++i)
#pragma unroll
    for (int k = 0; k < EPV; ++k) acc2[i][k] = 0.f;

  // the weight (gamma) of this workgroup's columns, the same in every row:
  // held in registers on the vector path (the scalar path, 16 values per
  // lane, re-reads it per row instead of spilling)
  constexpr bool WREG = EPV > 1;
  float wv[WREG ? NV : 1][EPV];
  if constexpr (WREG) {
#pragma unroll
    for (int i = 0; i < NV; ++i) sl.param(w + c0, i, wv[i]);
  }
  auto weight = [&](const Ts* wp, int i, float* t) {
    if constexpr (WREG) {
#pragma unroll
      for (int k = 0; k < EPV; ++k) t[k] = wv[i][k];
    } else {
      sl.param(wp, i, t);
    }
  };

  int merges = 0;  // cross-wave merges so far: picks the LDS slot
  for (int64_t row = rg; row < rows; row += RG) {
    // the segment's row operands first: they do not depend on the row sums,
    // so their loads are in flight while the partials are merged (the merge's
    // barrier would otherwise keep them behind it)
    const int64_t off = row * cols + c0;
    float a[NV][EPV], d[NV][EPV], dr[DRES ? NV : 1][EPV];
    if constexpr (DRES) sl.load3(xh + off, dy + off, dres + off, a, d, dr);
    else sl.load2(xh + off, dy + off, a, d);

    Sum2State st{0.f, 0.f};
    for (int j = tid; j < nseg; j += T) {
      const float4 p = part[row * nseg + j];
      st = Sum2Merge{}(st, Sum2State{p.x, p.y});
    }
    st = wave_reduce(st, Sum2Merge{});
    if constexpr (NW > 1) st = block_merge<NW>(st, xw[merges++ & 1], wave, lane, Sum2Merge{});

    const Ts* w1 = fresh(w) + c0;
    if constexpr (LN) {
      const float mu = mean[row], rs = rstd[row];
      const float mg = st.a / (float)cols, mgn = st.b / (float)cols;
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        float ga[EPV];
        weight(w1, i, ga);
#pragma unroll
        for (int k = 0; k < EPV; ++k) {
          const float nk = (a[i][k] - mu) * rs;
          acc[i][k] = __builtin_fmaf(d[i][k], nk, acc[i][k]);
          acc2[i][k] += d[i][k];
          a[i][k] = rs * __builtin_fmaf(-nk, mgn, __builtin_fmaf(d[i][k], ga[k], -mg));
        }
      }
    } else {
      const float r = 1.f / __builtin_sqrtf(st.a / (float)cols + eps);
      const float c = r * r * (st.b / (float)cols);
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        float wt[EPV];
        weight(w1, i, wt);
#pragma unroll
        for (int k = 0; k < EPV; ++k) {
          acc[i][k] = __builtin_fmaf(d[i][k] * a[i][k], r, acc[i][k]);
          const float t = r * __builtin_fmaf(-a[i][k], c, wt[k] * d[i][k]);
          if constexpr (DRES) a[i][k] = t + dr[i][k];
          else a[i][k] = t;
        }
      }
    }
    sl.store(out + off, a);
  }
  // this workgroup's partial row segment (slots past the segment end hold 0
  // and are not written)
  float* w0 = ws + (size_t)rg * cols + c0;
#pragma unroll
  for (int i = 0; i < NV; ++i)
    if (sl.ok(i)) store_f32<EPV>(w0 + (i * T + tid) * EPV, acc[i]);
  if constexpr (LN) {
    float* w1 = ws + ((size_t)RG + rg) * cols + c0;
#pragma unroll
    for (int i = 0; i < NV; ++i)
      if (sl.ok(i)) store_f32<EPV>(w1 + (i * T + tid) * EPV, acc2[i]);
  }
}

// One-pass form (the exchange of coop.hpp), h, dy (and dres) read once:
// teams of nseg workgroups — row group rg's segments, handed out in start
// order (ticket w: rg = w / nseg, segment w % nseg) — walk rows rg, rg + RG,
// ... together. Per row each member loads its segment, takes its two sums as
// pass 1 does, posts {sum a, 1} and {sum b, 1} (never zero) into the row's
// slots, waits for the row's other segments, adds them in segment order
// (lane j holds segment j's, one DPP tree: the same bits in every workgroup
// of the row), then writes the segment's dh / dx and accumulates its
// columns' parameter-gradient partials as pass 2 does; at the end it writes
// them to partial row rg, and colsum_kernel adds the partial rows. A team
// waits only for its own members, on the same rows in the same order, and
// lower tickets are lower teams: the lowest unfinished team needs room for
// its own workgroups only.
template <typename Ts, int T, int NV, int EPV, bool LN, bool DRES>
__global__ __launch_bounds__(T) __attribute__((amdgpu_waves_per_eu(4)))
void norm_bwd_split_coop_kernel(const Ts* xh, const Ts* dy, const Ts* dres, const Ts* w,
                                const float* mean, const float* rstd, Ts* out, float* ws,
                                int64_t rows, int cols, int nseg, int RG, float eps,
                                uint64_t* slots, uint32_t* ctl, int spin_limit) {
  constexpr int NW = T / 64;
  constexpr int SEG = T * NV * EPV;
  __shared__ float xw[2][NW][2];
  __shared__ float team[kCoopMaxSegments][4];
  __shared__ uint32_t ticket;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int tid = threadIdx.x;
  const int64_t tk = coop_ticket(ctl, &ticket);  // < RG * nseg: one per workgroup
  const int rg = (int)(tk / nseg);
  const int sg = (int)(tk - (int64_t)rg * nseg);
  const int c0 = sg * SEG;
  const int len = cols - c0 < SEG ? cols - c0 : SEG;
  const Slots<T, NV, EPV> sl(len, tid);

  float acc[NV][EPV], acc2[LN ? NV : 1][EPV];  // dw (dgamma) and dbeta partials
#pragma unroll
  for (int i = 0; i < NV; ++i)
#pragma unroll
    for (int k = 0; k < EPV; ++k) acc[i][k] = 0.f;
#pragma unroll
  for (int i = 0; i < (LN ? NV : 1); ++i)
#pragma unroll
    for (int k = 0; k < EPV; ++k) acc2[i][k] = 0.f;
  constexpr bool WREG = EPV > 1;  // the weight in registers on the vector path
  float wv[WREG ? NV : 1][EPV];
  if constexpr (WREG) {
#pragma unroll
    for (int i = 0; i < NV; ++i) sl.param(w + c0, i, wv[i]);
  }
  auto weight = [&](const Ts* wp, int i, float* t) {
    if constexpr (WREG) {
#pragma unroll
      for (int k = 0; k < EPV; ++k) t[k] = wv[i][k];
    } else {
      sl.param(wp, i, t);
    }
  };

  int merges = 0;  // cross-wave merges so far: picks the LDS slot
  for (int64_t row = rg; row < rows; row += RG) {
    const int64_t off = row * cols + c0;
    float a[NV][EPV], d[NV][EPV], dr[DRES ? NV : 1][EPV];
    if constexpr (DRES) sl.load3(xh + off, dy + off, dres + off, a, d, dr);
    else sl.load2(xh + off, dy + off, a, d);
    // slot i's operands (0 past the row end)
    auto operands = [&](int i, float (&va)[EPV], float (&vd)[EPV], float (&vr)[EPV]) {
#pragma unroll
      for (int k = 0; k < EPV; ++k) {
        va[k] = a[i][k];
        vd[k] = d[i][k];
        if constexpr (DRES) vr[k] = dr[i][k];
      }
    };
    float mu = 0.f, rs = 1.f;
    if constexpr (LN) {
      mu = mean[row];
      rs = rstd[row];
    }
    const Ts* w1 = fresh(w) + c0;
    float a0 = 0.f, a1 = 0.f, b0 = 0.f, b1 = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      float wt[EPV], va[EPV], vd[EPV], vr[EPV];
      weight(w1, i, wt);
      operands(i, va, vd, vr);
#pragma unroll
      for (int k = 0; k < EPV; ++k) {
        const float gk = vd[k] * wt[k];
        if constexpr (LN) {
          const float nk = sl.ok(i) ? (va[k] - mu) * rs : 0.f;
          if (k & 1) { a1 += gk; b1 = __builtin_fmaf(gk, nk, b1); }
          else { a0 += gk; b0 = __builtin_fmaf(gk, nk, b0); }
        } else {
          const float hk = va[k];
          if (k & 1) { a1 = __builtin_fmaf(hk, hk, a1); b1 = __builtin_fmaf(gk, hk, b1); }
          else { a0 = __builtin_fmaf(hk, hk, a0); b0 = __builtin_fmaf(gk, hk, b0); }
        }
      }
    }
    Sum2State mine{a0 + a1, b0 + b1};
    mine = wave_reduce(mine, Sum2Merge{});
    if constexpr (NW > 1) mine = block_merge<NW>(mine, xw[merges++ & 1], wave, lane, Sum2Merge{});
    uint64_t* row_slots = slots + (size_t)row * nseg * 2;
    coop_post<2>(row_slots, sg, coop_word(mine.a, 1.f), coop_word(mine.b, 1.f));
    if (wave == 0) coop_wait<2>(row_slots, nseg, ctl + 1, spin_limit, lane, team);
    lds_barrier();
    Sum2State st{0.f, 0.f};
    if (lane < nseg) st = Sum2State{team[lane][0], team[lane][2]};
    st = wave_reduce(st, Sum2Merge{});

    const float mg = st.a / (float)cols, mgn = st.b / (float)cols;  // LayerNorm
    const float r = LN ? 0.f : 1.f / __builtin_sqrtf(st.a / (float)cols + eps);  // RMSNorm
    const float c = r * r * (st.b / (float)cols);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      float wt[EPV], va[EPV], vd[EPV], vr[EPV], o[EPV];
      weight(w1, i, wt);
      operands(i, va, vd, vr);
#pragma unroll
      for (int k = 0; k < EPV; ++k) {
        if constexpr (LN) {
          const float nk = (va[k] - mu) * rs;
          acc[i][k] = __builtin_fmaf(vd[k], nk, acc[i][k]);
          acc2[i][k] += vd[k];
          o[k] = rs * __builtin_fmaf(-nk, mgn, __builtin_fmaf(vd[k], wt[k], -mg));
        } else {
          acc[i][k] = __builtin_fmaf(vd[k] * va[k], r, acc[i][k]);
          const float t = r * __builtin_fmaf(-va[k], c, wt[k] * vd[k]);
          if constexpr (DRES) o[k] = t + vr[k];
          else o[k] = t;
        }
      }
      if (sl.ok(i)) Vec<Ts, EPV>::store(out + off + sl.off(i), o);
    }
  }
  float* w0 = ws + (size_t)rg * cols + c0;
#pragma unroll
  for (int i = 0; i < NV; ++i)
    if (sl.ok(i)) store_f32<EPV>(w0 + (i * T + tid) * EPV, acc[i]);
  if constexpr (LN) {
    float* w1 = ws + ((size_t)RG + rg) * cols + c0;
#pragma unroll
    for (int i = 0; i < NV; ++i)
      if (sl.ok(i)) store_f32<EPV>(w1 + (i * T + tid) * EPV, acc2[i]);
  }
}

// ------------------------------------------------------------ column sums
// out_p[c] = sum over the partial rows b = 0 .. partials-1 of ws[p][b][c],
// parameter p = blockIdx.y. A workgroup takes a 32-column tile (one 128-byte
// line per partial row) and 32 row groups: lane group ty sums rows ty,
// ty+32, ... in order, then the 32 group sums are added in order of ty.
constexpr int kColTile = 32;
constexpr int kColGroups = 32;

__global__ __launch_bounds__(kColTile * kColGroups) void colsum_kernel(const float* ws, int partials,
                                                                       int cols, float* out0,
                                                                       float* out1) {
  __shared__ float red[kColGroups][kColTile + 1];
  const int tx = threadIdx.x % kColTile;
  const int ty = threadIdx.x / kColTile;
  const int c = blockIdx.x * kColTile + tx;
  const float* src = ws + (size_t)blockIdx.y * partials * cols;
  float s = 0.f;
  if (c < cols) {
    // partials <= kBwdGridMax: all of a group's loads issued before the first add
    float v[kBwdGridMax / kColGroups];
#pragma unroll
    for (int j = 0; j < kBwdGridMax / kColGroups; ++j) {
      const int b = ty + kColGroups * j;
      v[j] = b < partials ? src[(size_t)b * cols + c] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < kBwdGridMax / kColGroups; ++j) s += v[j];
  }
  red[ty][tx] = s;
  __syncthreads();
  if (ty == 0 && c < cols) {
    float t = red[0][tx];
#pragma unroll
    for (int r = 1; r < kColGroups; ++r) t += red[r][tx];
    (blockIdx.y == 0 ? out0 : out1)[c] = t;
  }
}

hipError_t launch_colsum(const float* ws, int partials, int cols, float* out0, float* out1,
                         hipStream_t s) {
  const unsigned tiles = (unsigned)((cols + kColTile - 1) / kColTile);
  return launch_kernel(&colsum_kernel, dim3(tiles, out1 ? 2 : 1), dim3(kColTile * kColGroups), s, ws,
                       partials, cols, out0, out1);
}

// ------------------------------------------------------------- launchers

template <typename Ts, int T, int NV, int EPV, int OCC>
static hipError_t launch_softmax_bwd(const void* p, const void* dy, void* dx, int64_t rows, int cols,
                                     hipStream_t s) {
  constexpr int BLOCK = T == 64 ? 256 : T;
  constexpr int RPB = BLOCK / T;
  const int64_t blocks = (rows + RPB - 1) / RPB;
  const unsigned grid = (unsigned)(blocks < kMaxGrid ? blocks : kMaxGrid);
  return launch_kernel(&softmax_bwd_kernel<Ts, T, NV, EPV, OCC>, dim3(grid), dim3(BLOCK), s,
                       static_cast<const Ts*>(p), static_cast<const Ts*>(dy), static_cast<Ts*>(dx),
                       rows, cols);
}

template <typename Ts, int T, int NV, int EPV, int RPB, int OCC, bool STG = false>
static hipError_t launch_rmsnorm_bwd(const void* h, const void* dy, const void* dres, const void* w,
                                     void* dh, float* ws, int grid, int64_t rows, int cols,
                                     float eps, hipStream_t s) {
  // staged with dres as well (three operands, 96 KiB): measured at 8192^2
  // (weight in LDS, counted waits) with dres 100.1 -> 96.2 us, without
  // 89.9 -> 80.2 us
  auto k = dres ? &rmsnorm_bwd_kernel<Ts, T, NV, EPV, RPB, OCC, true, STG>
                : &rmsnorm_bwd_kernel<Ts, T, NV, EPV, RPB, OCC, false, STG>;
  return launch_kernel(k, dim3(grid), dim3(T * RPB), s, static_cast<const Ts*>(h),
                       static_cast<const Ts*>(dy), static_cast<const Ts*>(dres),
                       static_cast<const Ts*>(w), static_cast<Ts*>(dh), ws, rows, cols, eps);
}

// Staging of the LayerNorm backward rows (x, dy: 2 NV 16 T RPB bytes of LDS)
// on the 16-byte vector path, below 1024 lanes per row (the 1024-lane shapes
// spill with gamma held in registers). Measured: bf16 16384 x 4096
// 89.6 -> 74.0 us; fp32 16384 x 4096 150.8 -> 145.7 us, 8192 x 8192
// 154.2 -> 148.9 us, 16384 x 1024 43.4 -> 42.4 us, 4096 x 1024 18.1 -> 17.8 us.
template <typename Ts, int T, int NV, int EPV, int RPB, int OCC>
static hipError_t launch_layernorm_bwd(const void* x, const void* dy, const void* gamma,
                                       const float* mean, const float* rstd, void* dx, float* ws,
                                       int grid, int64_t rows, int cols, hipStream_t s) {
  constexpr bool STG =
      T < 1024 && EPV * sizeof(Ts) == 16 && 2 * NV * T * RPB * 16 <= 128 * 1024;
  return launch_kernel(&layernorm_bwd_kernel<Ts, T, NV, EPV, RPB, OCC, STG>, dim3(grid), dim3(T * RPB), s,
                       static_cast<const Ts*>(x), static_cast<const Ts*>(dy),
                       static_cast<const Ts*>(gamma), mean, rstd, static_cast<Ts*>(dx), ws, rows,
                       cols);
}

template <typename Ts, int NV, int EPV, bool LN>
static hipError_t launch_norm_bwd_split_t(const void* xh, const void* dy, const void* dres,
                                          const void* w, const float* mean, const float* rstd,
                                          void* out, float* dw0, float* dw1, void* workspace,
                                          int64_t rows, int cols, float eps, bool one_pass,
                                          hipStream_t s) {
  constexpr int T = 512;
  static_assert(T * NV * EPV == kBwdSplitSeg, "segment");
  const int nseg = (cols + kBwdSplitSeg - 1) / kBwdSplitSeg;
  const int RG = norm_bwd_split_groups(rows, nseg);
  float4* part = static_cast<float4*>(workspace);
  float* ws = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                       norm_bwd_split_part_bytes(rows, cols));
  if (one_pass && nseg <= kCoopMaxSegments) {
    hipError_t e = launch_coop_clear(part, rows, nseg, s);
    if (e != hipSuccess) return e;
    auto kc = (!LN && dres) ? &norm_bwd_split_coop_kernel<Ts, T, NV, EPV, LN, true>
                            : &norm_bwd_split_coop_kernel<Ts, T, NV, EPV, LN, false>;
    e = launch_kernel(kc, dim3((unsigned)(nseg * RG)), dim3(T), s, static_cast<const Ts*>(xh),
                      static_cast<const Ts*>(dy), static_cast<const Ts*>(dres),
                      static_cast<const Ts*>(w), mean, rstd, static_cast<Ts*>(out), ws, rows, cols,
                      nseg, RG, eps, reinterpret_cast<uint64_t*>(part + 1),
                      reinterpret_cast<uint32_t*>(part), coop_spin_limit());
    if (e != hipSuccess) return e;
    return launch_colsum(ws, RG, cols, dw0, dw1, s);
  }
  const int64_t work = rows * nseg;
  const unsigned g1 = (unsigned)(work < kMaxGrid ? work : kMaxGrid);
  hipError_t e = launch_kernel(&norm_bwd_split_sums_kernel<Ts, T, NV, EPV, LN>, dim3(g1), dim3(T), s,
                               static_cast<const Ts*>(xh), static_cast<const Ts*>(dy),
                               static_cast<const Ts*>(w), mean, rstd, rows, cols, nseg, part);
  if (e != hipSuccess) return e;
  auto k2 = (!LN && dres) ? &norm_bwd_split_apply_kernel<Ts, T, NV, EPV, LN, true>
                          : &norm_bwd_split_apply_kernel<Ts, T, NV, EPV, LN, false>;
  e = launch_kernel(k2, dim3((unsigned)(nseg * RG)), dim3(T), s, static_cast<const Ts*>(xh),
                    static_cast<const Ts*>(dy), static_cast<const Ts*>(dres),
                    static_cast<const Ts*>(w), mean, rstd, static_cast<Ts*>(out), ws, rows, cols,
                    nseg, RG, static_cast<const float4*>(part), eps);
  if (e != hipSuccess) return e;
  return launch_colsum(ws, RG, cols, dw0, dw1, s);
}

hipError_t launch_norm_bwd_split(int layernorm, int bf16, int vec, const void* xh, const void* dy,
                                 const void* dres, const void* w, const float* mean,
                                 const float* rstd, void* out, float* dw0, float* dw1,
                                 void* workspace, int64_t rows, int cols, float eps,
                                 bool one_pass, hipStream_t s) {
  auto go = [&](auto launch) {
    return launch(xh, dy, dres, w, mean, rstd, out, dw0, dw1, workspace, rows, cols, eps, one_pass,
                  s);
  };
  if (layernorm) {
    if (bf16)
      return vec ? go(&launch_norm_bwd_split_t<bf16_t, 2, 8, true>)
                 : go(&launch_norm_bwd_split_t<bf16_t, 16, 1, true>);
    return vec ? go(&launch_norm_bwd_split_t<float, 4, 4, true>)
               : go(&launch_norm_bwd_split_t<float, 16, 1, true>);
  }
  if (bf16)
    return vec ? go(&launch_norm_bwd_split_t<bf16_t, 2, 8, false>)
               : go(&launch_norm_bwd_split_t<bf16_t, 16, 1, false>);
  return vec ? go(&launch_norm_bwd_split_t<float, 4, 4, false>)
             : go(&launch_norm_bwd_split_t<float, 16, 1, false>);
}

// Norm backward shapes: (T, NV, EPV, RPB, OCC, grid_max). The default
// workgroup is 1024 lanes (RPB = 1024 / T) with one workgroup per CU
// (grid_max 256, OCC 4: at most 128 VGPRs).
#define FR_RB(TS, T, NV, EPV, RPB, OCC, G) {T, NV, EPV, RPB, G, &launch_rmsnorm_bwd<TS, T, NV, EPV, RPB, OCC>}
// The 8192-column bf16 shape stages its next rows (h, dy and dres) in LDS.
#define FR_RBS(TS, T, NV, EPV, RPB, OCC, G) \
  {T, NV, EPV, RPB, G, &launch_rmsnorm_bwd<TS, T, NV, EPV, RPB, OCC, true>}
#define FR_LB(TS, T, NV, EPV, RPB, OCC, G) {T, NV, EPV, RPB, G, &launch_layernorm_bwd<TS, T, NV, EPV, RPB, OCC>}
#define FR_SB(TS, T, NV, EPV, OCC) {T, NV, EPV, &launch_softmax_bwd<TS, T, NV, EPV, OCC>}

static const SoftmaxBwdVariant kSbF32[] = {
    FR_SB(float, 64, 1, 4, 8),    FR_SB(float, 64, 2, 4, 8),    FR_SB(float, 64, 4, 4, 6),
    FR_SB(float, 64, 8, 4, 4),    FR_SB(float, 256, 4, 4, 6),   FR_SB(float, 256, 8, 4, 4),
    FR_SB(float, 512, 8, 4, 4),   FR_SB(float, 64, 16, 1, 4),   FR_SB(float, 256, 16, 1, 4),
    FR_SB(float, 1024, 16, 1, 4)};
static const SoftmaxBwdVariant kSbBf16[] = {
    FR_SB(bf16_t, 64, 1, 8, 8),   FR_SB(bf16_t, 64, 2, 8, 6),   FR_SB(bf16_t, 64, 4, 8, 4),
    FR_SB(bf16_t, 256, 2, 8, 6),  FR_SB(bf16_t, 256, 4, 8, 4),  FR_SB(bf16_t, 512, 4, 8, 4),
    FR_SB(bf16_t, 64, 16, 1, 4),  FR_SB(bf16_t, 256, 16, 1, 4), FR_SB(bf16_t, 1024, 16, 1, 4)};

static const RmsNormBwdVariant kRbF32[] = {
    FR_RB(float, 64, 1, 4, 16, 4, 256),   FR_RB(float, 64, 2, 4, 16, 4, 256),
    FR_RB(float, 64, 4, 4, 16, 4, 256),   FR_RB(float, 256, 2, 4, 4, 4, 256),
    FR_RB(float, 256, 4, 4, 4, 4, 256),   FR_RB(float, 512, 4, 4, 2, 4, 256),
    FR_RB(float, 1024, 4, 4, 1, 4, 256),  FR_RB(float, 64, 16, 1, 16, 4, 256),
    FR_RB(float, 256, 16, 1, 4, 4, 256),  FR_RB(float, 1024, 16, 1, 1, 4, 256)};
static const RmsNormBwdVariant kRbBf16[] = {
    FR_RB(bf16_t, 64, 1, 8, 16, 4, 256),  FR_RB(bf16_t, 64, 2, 8, 16, 4, 256),
    FR_RB(bf16_t, 256, 1, 8, 4, 4, 256),  FR_RB(bf16_t, 256, 2, 8, 4, 4, 256),
    FR_RBS(bf16_t, 512, 2, 8, 2, 4, 256), FR_RB(bf16_t, 1024, 2, 8, 1, 4, 256),
    FR_RB(bf16_t, 64, 16, 1, 16, 4, 256), FR_RB(bf16_t, 256, 16, 1, 4, 4, 256),
    FR_RB(bf16_t, 1024, 16, 1, 1, 4, 256)};

static const LayerNormBwdVariant kLbF32[] = {
    FR_LB(float, 64, 1, 4, 16, 4, 256),   FR_LB(float, 64, 2, 4, 16, 4, 256),
    FR_LB(float, 64, 4, 4, 16, 4, 256),   FR_LB(float, 256, 2, 4, 4, 4, 256),
    FR_LB(float, 256, 4, 4, 4, 4, 256),   FR_LB(float, 512, 4, 4, 2, 4, 256),
    FR_LB(float, 1024, 4, 4, 1, 4, 256),  FR_LB(float, 64, 16, 1, 16, 4, 256),
    FR_LB(float, 256, 16, 1, 4, 4, 256),  FR_LB(float, 1024, 16, 1, 1, 4, 256)};
static const LayerNormBwdVariant kLbBf16[] = {
    FR_LB(bf16_t, 64, 1, 8, 16, 4, 256),  FR_LB(bf16_t, 64, 2, 8, 16, 4, 256),
    FR_LB(bf16_t, 256, 1, 8, 4, 4, 256),  FR_LB(bf16_t, 256, 2, 8, 4, 4, 256),
    FR_LB(bf16_t, 512, 2, 8, 2, 4, 256),  FR_LB(bf16_t, 1024, 2, 8, 1, 4, 256),
    FR_LB(bf16_t, 64, 16, 1, 16, 4, 256), FR_LB(bf16_t, 256, 16, 1, 4, 4, 256),
    FR_LB(bf16_t, 1024, 16, 1, 1, 4, 256)};

#define FR_SPAN(a) {a, sizeof(a) / sizeof(a[0])}

VariantSpan<SoftmaxBwdVariant> softmax_bwd_variants(int bf16) {
  if (bf16) return FR_SPAN(kSbBf16);
  return FR_SPAN(kSbF32);
}
VariantSpan<RmsNormBwdVariant> rmsnorm_bwd_variants(int bf16) {
  if (bf16) return FR_SPAN(kRbBf16);
  return FR_SPAN(kRbF32);
}
VariantSpan<LayerNormBwdVariant> layernorm_bwd_variants(int bf16) {
  if (bf16) return FR_SPAN(kLbBf16);
  return FR_SPAN(kLbF32);
}

}  // namespace fr
