// Device building blocks shared by the fused row kernels (gfx950 / CDNA4).
//
// Row ownership: one wavefront (64 lanes) or one workgroup owns a whole row,
// so every reduction stays inside the owner and no cross-row exchange exists
// ("ML Compiler Lab", Own a complete row tile; Check the graph before
// selecting a schedule: cross-row reductions are rejected). Each lane keeps
// its share of the row in VGPRs from the load to the store.
//
// Memory access: 128-bit loads/stores (global_load_dwordx4 /
// global_store_dwordx4), consecutive lanes on consecutive 16-byte chunks
// ("Engineering a CUDA Machine Learning Framework from Scratch", §2.3 128-Bit
// Memory Vectorization and Register Warp Reductions). The in-wave reduction
// uses DPP lane moves instead of shuffles through LDS.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fr {

// bf16 storage (raw bits); arithmetic is always fp32.
struct bf16_t {
  uint16_t u;
};

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr float kNegInf = -__builtin_inff();
// log2(e), and ln(2) split in two so that t - y*ln2 is formed to ~2^-48.
constexpr double kLog2eD = 1.4426950408889634073599;
constexpr double kLn2D = 0.6931471805599453094172;
constexpr float kLog2e = (float)kLog2eD;
constexpr float kLn2 = (float)kLn2D;
constexpr float kLn2Lo = (float)(kLn2D - (double)(float)kLn2D);

// ---------------------------------------------------------------- bf16 <-> f32

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two fp32 -> packed bf16 pair, round to nearest even (one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}
__device__ __forceinline__ uint16_t to_bf16(float a) {
  return __builtin_bit_cast(uint16_t, (__bf16)a);
}

// ------------------------------------------------------------------ arithmetic

// max of three, straight to v_max3_f32. Written as inline asm so that the
// compiler does not quiet each loaded operand first (IEEE mode); a quiet NaN
// operand is ignored here and reaches the result through the exponential sum.
__device__ __forceinline__ float max3(float a, float b, float c) {
  float r;
  asm volatile("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// 2^y with the hardware v_exp_f32 (results below 2^-126 flush to zero).
__device__ __forceinline__ float exp2_hw(float y) { return __builtin_amdgcn_exp2f(y); }

// e^t for fp32 outputs: y = fl(t*log2e); rho = t - y*ln2 (two fmas, exact to
// ~2^-48 relative); e^t = 2^y * e^rho ~= 2^y + 2^y*rho. Removes the rounding
// of t*log2e from the result; what remains is v_exp_f32's own error.
// t = -inf gives 0 (rho would be inf - inf; clamping it to -1 keeps 0 * rho
// finite), t = NaN gives NaN (through 2^y).
__device__ __forceinline__ float exp_acc(float t) {
  float y = t * kLog2e;
  float rho = __builtin_fmaf(-y, kLn2, t);
  rho = __builtin_fmaf(-y, kLn2Lo, rho);
  rho = __builtin_fmaxf(rho, -1.f);
  float e = exp2_hw(y);
  return __builtin_fmaf(e, rho, e);
}

// --------------------------------------------------------------- global access
// Inputs are streamed once with non-temporal loads (measured on MI355X: the
// fastest load policy for every row kernel; the read-only probe reaches
// 6.9-7.3 TB/s with them against 6.0-6.7 TB/s with cached loads).
// ld_stream<false> is an ordinary cached load, for data that is read again
// soon (the first pass of a two-pass kernel).
// Stores are non-temporal too, except where a kernel asks otherwise
// (st_stream<false>). Measured on MI355X with cold buffers (rotating sets
// of >= 1.5 GB, so that neither inputs nor outputs survive in the 256 MB
// memory-side cache between uses, as in a real sequence of kernels): cached
// stores were 2-9% slower for every row kernel and 8-24% slower for the
// cross-entropy and the split-row passes; the one exception is a softmax
// with bf16 input and fp32 output, whose lanes write their 32 bytes as two
// 16-byte stores, so each store instruction covers every other 16 bytes of
// its lines: cached stores let the cache merge the halves (112 -> 83 us at
// 16384 x 4096). (Timed with the same buffers call after call, an output of
// up to 256 MB stays dirty in that cache and cached stores look faster.)
template <bool NT = true, typename V>
__device__ __forceinline__ V ld_stream(const V* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}
template <bool NT = true, typename V>
__device__ __forceinline__ void st_stream(V v, V* p) {
  if constexpr (NT) __builtin_nontemporal_store(v, p);
  else *p = v;
}
// Cache-policy bits of global_load_lds for streamed data: the non-temporal
// hint, as ld_stream.
constexpr int kCopyNT = 2;

template <typename T, int EPV>
struct Vec;  // load/store EPV consecutive elements as fp32

template <>
struct Vec<float, 4> {
  template <bool NT = true>
  static __device__ __forceinline__ void load(const float* p, float* v) {
    f32x4 r = ld_stream<NT>(reinterpret_cast<const f32x4*>(p));
    v[0] = r.x; v[1] = r.y; v[2] = r.z; v[3] = r.w;
  }
  template <bool NT = true>
  static __device__ __forceinline__ void store(float* p, const float* v) {
    f32x4 r = {v[0], v[1], v[2], v[3]};
    st_stream<NT>(r, reinterpret_cast<f32x4*>(p));
  }
};

template <>
struct Vec<float, 8> {  // output side of bf16 -> f32 (two 16-byte stores)
  template <bool NT = true>
  static __device__ __forceinline__ void load(const float* p, float* v) {
    Vec<float, 4>::load<NT>(p, v);
    Vec<float, 4>::load<NT>(p + 4, v + 4);
  }
  template <bool NT = true>
  static __device__ __forceinline__ void store(float* p, const float* v) {
    Vec<float, 4>::store<NT>(p, v);
    Vec<float, 4>::store<NT>(p + 4, v + 4);
  }
};

template <>
struct Vec<bf16_t, 8> {
  template <bool NT = true>
  static __device__ __forceinline__ void load(const bf16_t* p, float* v) {
    u32x4 r = ld_stream<NT>(reinterpret_cast<const u32x4*>(p));
    v[0] = bf16_lo(r.x); v[1] = bf16_hi(r.x);
    v[2] = bf16_lo(r.y); v[3] = bf16_hi(r.y);
    v[4] = bf16_lo(r.z); v[5] = bf16_hi(r.z);
    v[6] = bf16_lo(r.w); v[7] = bf16_hi(r.w);
  }
  template <bool NT = true>
  static __device__ __forceinline__ void store(bf16_t* p, const float* v) {
    u32x4 r = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
               pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])};
    st_stream<NT>(r, reinterpret_cast<u32x4*>(p));
  }
};

template <>
struct Vec<bf16_t, 4> {  // output side of f32 -> bf16 (one 8-byte store)
  template <bool NT = true>
  static __device__ __forceinline__ void load(const bf16_t* p, float* v) {
    u32x2 r = ld_stream<NT>(reinterpret_cast<const u32x2*>(p));
    v[0] = bf16_lo(r.x); v[1] = bf16_hi(r.x);
    v[2] = bf16_lo(r.y); v[3] = bf16_hi(r.y);
  }
  template <bool NT = true>
  static __device__ __forceinline__ void store(bf16_t* p, const float* v) {
    u32x2 r = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    st_stream<NT>(r, reinterpret_cast<u32x2*>(p));
  }
};

template <>
struct Vec<float, 1> {
  template <bool NT = true>
  static __device__ __forceinline__ void load(const float* p, float* v) {
    v[0] = ld_stream<NT>(p);
  }
  template <bool NT = true>
  static __device__ __forceinline__ void store(float* p, const float* v) {
    st_stream<NT>(v[0], p);
  }
};

template <>
struct Vec<bf16_t, 1> {
  template <bool NT = true>
  static __device__ __forceinline__ void load(const bf16_t* p, float* v) {
    uint16_t u = ld_stream<NT>(reinterpret_cast<const uint16_t*>(p));
    v[0] = __uint_as_float((uint32_t)u << 16);
  }
  template <bool NT = true>
  static __device__ __forceinline__ void store(bf16_t* p, const float* v) {
    st_stream<NT>(to_bf16(v[0]), reinterpret_cast<uint16_t*>(p));
  }
};

// Per-column parameters (gamma, beta, weight) are re-read by every row and
// stay cache resident: ordinary loads.
template <typename T, int EPV>
__device__ __forceinline__ void load_param(const T* p, float* v);
template <>
__device__ __forceinline__ void load_param<float, 4>(const float* p, float* v) {
  f32x4 r = *reinterpret_cast<const f32x4*>(p);
  v[0] = r.x; v[1] = r.y; v[2] = r.z; v[3] = r.w;
}
template <>
__device__ __forceinline__ void load_param<bf16_t, 8>(const bf16_t* p, float* v) {
  u32x4 r = *reinterpret_cast<const u32x4*>(p);
  v[0] = bf16_lo(r.x); v[1] = bf16_hi(r.x);
  v[2] = bf16_lo(r.y); v[3] = bf16_hi(r.y);
  v[4] = bf16_lo(r.z); v[5] = bf16_hi(r.z);
  v[6] = bf16_lo(r.w); v[7] = bf16_hi(r.w);
}
template <>
__device__ __forceinline__ void load_param<float, 1>(const float* p, float* v) { v[0] = *p; }
template <>
__device__ __forceinline__ void load_param<bf16_t, 1>(const bf16_t* p, float* v) {
  v[0] = __uint_as_float((uint32_t)p->u << 16);
}

// Single element of any storage type (head/tail slots, label logit).
__device__ __forceinline__ float load1(const float* p) { return *p; }
__device__ __forceinline__ float load1(const bf16_t* p) { return __uint_as_float((uint32_t)p->u << 16); }
// One element as its storage bits, converted later (raw_value): a value
// converted right after its load makes the compiler wait for the load there,
// and that wait (vmcnt) also waits for every vector memory operation issued
// before it — stores, staged copies — where the value is only needed later.
__device__ __forceinline__ uint32_t load1_raw(const float* p) { return __float_as_uint(*p); }
__device__ __forceinline__ uint32_t load1_raw(const bf16_t* p) { return (uint32_t)p->u; }
template <typename Ts>
__device__ __forceinline__ float raw_value(uint32_t r) {
  return sizeof(Ts) == 2 ? __uint_as_float(r << 16) : __uint_as_float(r);
}
template <typename Ts>
constexpr uint32_t kRawNegInf = sizeof(Ts) == 2 ? 0xff80u : 0xff800000u;
// The raw value at this point of the program: the conversion after it cannot
// be moved up to the load, and the memory clobber keeps it behind the
// memory operations before it (the compiler's wait for the load lands here).
__device__ __forceinline__ uint32_t raw_here(uint32_t r) {
  asm volatile("" : "+v"(r) : : "memory");
  return r;
}
__device__ __forceinline__ void store1(float* p, float v) { *p = v; }
__device__ __forceinline__ void store1(bf16_t* p, float v) { p->u = to_bf16(v); }

// ----------------------------------------------------------------- row layout
// A row of `cols` elements starting at `row_ptr` is cut into
//   head: the elements before the first kHeadAlign-element boundary
//         (EPV > 1 only; 128 bytes for fp32, 64 for bf16),
//   body: nvec chunks of EPV elements (16 bytes), starting on that boundary,
//   tail: what is left (< EPV elements).
// Starting the body on a cache-line boundary makes every wavefront access
// whole lines; rows of odd width would otherwise split a line between
// neighbouring wavefronts on every access.
// Lane t of a row-owner of T lanes holds body chunks t, t+T, t+2T, ...
// (slot i -> chunk i*T + t) and at most one head/tail element in its extra
// slot: lanes [0, head) take the head, lanes [head, head+tail) the tail
// (head + tail <= 31 + 7 < 64 <= T).
constexpr int kHeadAlign = 32;  // elements

// ALIGN is the element boundary the body starts on (kHeadAlign by default;
// EPV keeps the head at 0 for rows on the 16-byte grid, so a lane owns the
// same columns in every row — what per-column gradient sums need).
template <int EPV, int ALIGN = kHeadAlign>
struct RowGeom {
  int head, nvec, tail;
  template <typename T>
  __device__ __forceinline__ RowGeom(const T* row_ptr, int cols) {
    if constexpr (EPV == 1) {
      head = 0; nvec = cols; tail = 0;
    } else {
      const uint32_t mis =
          (uint32_t)(reinterpret_cast<uintptr_t>(row_ptr) / sizeof(T)) & (ALIGN - 1);
      const int h = (int)((ALIGN - mis) & (ALIGN - 1));
      head = h < cols ? h : cols;
      nvec = (cols - head) / EPV;
      tail = cols - head - nvec * EPV;
    }
  }
  // column of this lane's extra element, or -1
  __device__ __forceinline__ int extra_col(int lane) const {
    if (lane < head) return lane;
    if (lane < head + tail) return head + nvec * EPV + (lane - head);
    return -1;
  }
  __device__ __forceinline__ int chunk_col(int chunk) const { return head + chunk * EPV; }
};

// ------------------------------------------------------- row chunk load/store
// Slot i of lane t holds chunk i*T + t. Every load is issued: a slot past
// the end of the row re-reads the row's last chunk (always in bounds) and is
// then overwritten with `fill`; stores of such slots are masked off. A single
// code path keeps the register allocation tight (rows that fill every slot
// simply never mask).
//
// The lane offset is re-formed in every call from an opaque zero: otherwise
// the compiler hoists the NV per-slot offsets out of a row loop, and when
// they do not fit in registers it spills them and reloads each one right
// before its load; a scratch reload waits on the same counter as the row's
// loads, which then issue one at a time.
__device__ __forceinline__ uint32_t opaque_zero() {
  uint32_t z = 0;
  asm volatile("" : "+s"(z));
  return z;
}

// A whole row segment (no head or tail element, every slot in it):
// unconditional loads, no clamps, masks or fill. The general loader's fill
// stores for a row without whole chunks are placed by the compiler ahead of
// its branch, so they run on every row; the split-row first passes, whose
// segments are whole but for a row's last, take this path instead (bf16
// cross-entropy [1024, 262144]: 263.0 -> 252.7 us per call). Used in the
// shared loaders themselves it measured slower on the one-pass kernels, and
// in the other split first passes (norms, softmax backward) within noise.
template <typename Ts, int T, int NV, int EPV, bool NT = true>
__device__ __forceinline__ void load_whole(const Ts* row, int tid, float (&v)[NV][EPV]) {
  const uint32_t lo = (uint32_t)tid * EPV + opaque_zero();
#pragma unroll
  for (int i = 0; i < NV; ++i) Vec<Ts, EPV>::template load<NT>(row + (uint32_t)(i * T * EPV) + lo, v[i]);
}
template <int T, int NV, int EPV, int AL>
__device__ __forceinline__ bool whole_segment(const RowGeom<EPV, AL>& g) {
  return g.nvec == T * NV && g.head == 0 && g.tail == 0;
}

template <typename Ts, int T, int NV, int EPV, int AL, bool NT = true>
__device__ __forceinline__ void load_chunks(const Ts* row, const RowGeom<EPV, AL>& g, int tid,
                                            float (&v)[NV][EPV], float fill) {
  if (g.nvec > 0) {
    const Ts* base = row + g.head;                  // uniform
    const uint32_t lo = (uint32_t)tid * EPV + opaque_zero();  // lane offset, elements
    const uint32_t last = (uint32_t)(g.nvec - 1) * EPV;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      uint32_t o = (uint32_t)(i * T * EPV) + lo;
      o = o < last ? o : last;
      Vec<Ts, EPV>::template load<NT>(base + o, v[i]);
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      if ((i + 1) * T <= g.nvec) continue;  // uniform: the whole slot lies in the row
      const bool ok = i * T + tid < g.nvec;
#pragma unroll
      for (int k = 0; k < EPV; ++k) v[i][k] = ok ? v[i][k] : fill;
    }
  } else {
#pragma unroll
    for (int i = 0; i < NV; ++i)
#pragma unroll
      for (int k = 0; k < EPV; ++k) v[i][k] = fill;
  }
}

// A 16-byte chunk as loaded (raw), and its unpacking into fp32 values.
template <typename Ts>
struct RawChunk;
template <>
struct RawChunk<float> {
  using T = f32x4;
  static __device__ __forceinline__ void unpack(const T& r, float* v) {
    v[0] = r.x; v[1] = r.y; v[2] = r.z; v[3] = r.w;
  }
};
template <>
struct RawChunk<bf16_t> {
  using T = u32x4;
  static __device__ __forceinline__ void unpack(const T& r, float* v) {
    v[0] = bf16_lo(r.x); v[1] = bf16_hi(r.x);
    v[2] = bf16_lo(r.y); v[3] = bf16_hi(r.y);
    v[4] = bf16_lo(r.z); v[5] = bf16_hi(r.z);
    v[6] = bf16_lo(r.w); v[7] = bf16_hi(r.w);
  }
};

// Next-row staging in LDS: slot i < LPF of lane t is copied from global
// memory straight into LDS by global_load_lds_dwordx4, which holds no VGPRs
// while in flight and writes lane l of a wave at that wave's LDS base + 16 l
// (checked on gfx950 for both cache policies); with the base of wave w at
// slot i set to 16 (i T + 64 w), lane t's chunk lands at 16 (i T + t) and is
// read back by lane t itself, so no barrier is needed.
// The compiler does not order these copies against LDS reads:
// wait_lds_copies() (or a counted wait) precedes reading staged data, and
// wait_lds_reads() precedes staging over data that was read.
__device__ __forceinline__ void wait_lds_copies() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// All but the K most recently issued vector memory operations of this wave
// have completed (they retire in issue order).
template <int K>
__device__ __forceinline__ void wait_vmcnt_upto() {
  static_assert(K >= 0 && K < 64, "vmcnt");
  asm volatile("s_waitcnt vmcnt(%0)" ::"I"(K) : "memory");
}
__device__ __forceinline__ void wait_lds_reads() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Reads of staged chunks back from LDS, out of the compiler's sight: it
// cannot tell which LDS bytes an outstanding global_load_lds writes, so it
// puts a full vmcnt(0) before every read of a staging buffer — which also
// waits for earlier stores and for copies staged further ahead, defeating
// the counted waits. The caller has waited for the copies these reads
// return; the reads complete inside the asm (lgkmcnt(0)), so no output
// register is still in flight when it ends. Addresses: LDS byte offsets.
__device__ __forceinline__ uint32_t lds_offset(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p;
}
__device__ __forceinline__ void read_staged4(const uint32_t* a, u32x4* r) {
  asm volatile(
      "ds_read_b128 %0, %4\n\t"
      "ds_read_b128 %1, %5\n\t"
      "ds_read_b128 %2, %6\n\t"
      "ds_read_b128 %3, %7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3])
      : "memory");
}
__device__ __forceinline__ void read_staged2(const uint32_t* a, u32x4* r) {
  asm volatile(
      "ds_read_b128 %0, %2\n\t"
      "ds_read_b128 %1, %3\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1])
      : "v"(a[0]), "v"(a[1])
      : "memory");
}
__device__ __forceinline__ void read_staged1(const uint32_t* a, u32x4* r) {
  asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(r[0]) : "v"(a[0]) : "memory");
}
template <int N>
__device__ __forceinline__ void read_staged(const uint32_t (&a)[N], u32x4 (&r)[N]) {
#pragma unroll
  for (int i = 0; i < N / 4; ++i) read_staged4(a + 4 * i, r + 4 * i);
  if constexpr (N % 4 >= 2) read_staged2(a + N / 4 * 4, r + N / 4 * 4);
  if constexpr (N % 2 == 1) read_staged1(a + N - 1, r + N - 1);
}

template <typename Ts, int T, int LPF, int EPV, int AL>
__device__ __forceinline__ void stage_row(const Ts* row, const RowGeom<EPV, AL>& g, int tid,
                                          int wave, uint32_t* stage) {
  static_assert(EPV * sizeof(Ts) == 16, "16-byte chunks");
  if (g.nvec > 0) {
    const Ts* base = row + g.head;
    const uint32_t lo = (uint32_t)tid * EPV + opaque_zero();
    const uint32_t last = (uint32_t)(g.nvec - 1) * EPV;
#pragma unroll
    for (int i = 0; i < LPF; ++i) {
      uint32_t o = (uint32_t)(i * T * EPV) + lo;
      o = o < last ? o : last;
      __builtin_amdgcn_global_load_lds(
          static_cast<const void*>(base + o),
          (__attribute__((address_space(3))) void*)(stage + (i * T + wave * 64) * 4), 16, 0,
          kCopyNT);
    }
  }
}

// The row into registers when its first LPF slots were staged by stage_row
// and the caller has waited for the copies: the remaining slots are loaded
// from global memory, the staged ones taken from LDS; all are masked as in
// load_chunks.
template <typename Ts, int T, int NV, int LPF, int EPV, bool HIDDEN, int AL>
__device__ __forceinline__ void load_staged(const Ts* row, const RowGeom<EPV, AL>& g, int tid,
                                            const uint32_t* stage, float (&v)[NV][EPV],
                                            float fill) {
  static_assert(LPF <= NV, "staged slots");
  if (g.nvec > 0) {
    const Ts* base = row + g.head;
    const uint32_t lo = (uint32_t)tid * EPV + opaque_zero();
    const uint32_t last = (uint32_t)(g.nvec - 1) * EPV;
#pragma unroll
    for (int i = LPF; i < NV; ++i) {
      uint32_t o = (uint32_t)(i * T * EPV) + lo;
      o = o < last ? o : last;
      Vec<Ts, EPV>::load(base + o, v[i]);
    }
    // HIDDEN: read past the compiler's LDS-copy wait (read_staged), two
    // chunks at a time, each pair unpacked at once; the lane's LDS offset is
    // formed anew in every row (opaque zero), so no per-slot address is kept
    // — and spilled — across the row loop. Else plain reads (the compiler
    // waits for all outstanding copies and stores first).
    const uint32_t sb = lds_offset(stage) + (uint32_t)tid * 16u + opaque_zero();
#pragma unroll
    for (int i = 0; i < (HIDDEN ? LPF : 0); i += 2) {
      uint32_t a[2];
      u32x4 r[2];
      a[0] = sb + (uint32_t)(i * T * 16);
      if (i + 1 < LPF) {
        a[1] = sb + (uint32_t)((i + 1) * T * 16);
        read_staged2(a, r);
        RawChunk<Ts>::unpack(__builtin_bit_cast(typename RawChunk<Ts>::T, r[1]), v[i + 1]);
      } else {
        read_staged1(a, r);
      }
      RawChunk<Ts>::unpack(__builtin_bit_cast(typename RawChunk<Ts>::T, r[0]), v[i]);
    }
#pragma unroll
    for (int i = 0; i < (HIDDEN ? 0 : LPF); ++i) {
      const typename RawChunk<Ts>::T r =
          *reinterpret_cast<const typename RawChunk<Ts>::T*>(stage + (i * T + tid) * 4);
      RawChunk<Ts>::unpack(r, v[i]);
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      if ((i + 1) * T <= g.nvec) continue;  // uniform: the whole slot lies in the row
      const bool ok = i * T + tid < g.nvec;
#pragma unroll
      for (int k = 0; k < EPV; ++k) v[i][k] = ok ? v[i][k] : fill;
    }
  } else {
#pragma unroll
    for (int i = 0; i < NV; ++i)
#pragma unroll
      for (int k = 0; k < EPV; ++k) v[i][k] = fill;
  }
}

// Two row operands of the same geometry in one branch, so that the second
// operand's loads are issued before the first operand's data is waited for.
template <typename Ts, int T, int NV, int EPV, int AL, bool NT = true>
__device__ __forceinline__ void load_chunks2(const Ts* ra, const Ts* rb, const RowGeom<EPV, AL>& g,
                                             int tid, float (&a)[NV][EPV], float (&b)[NV][EPV],
                                             float fill) {
  if (g.nvec > 0) {
    const uint32_t lo = (uint32_t)tid * EPV;
    const uint32_t last = (uint32_t)(g.nvec - 1) * EPV;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      uint32_t o = (uint32_t)(i * T * EPV) + lo;
      o = o < last ? o : last;
      Vec<Ts, EPV>::template load<NT>(ra + g.head + o, a[i]);
      Vec<Ts, EPV>::template load<NT>(rb + g.head + o, b[i]);
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      if ((i + 1) * T <= g.nvec) continue;  // uniform: the whole slot lies in the row
      const bool ok = i * T + tid < g.nvec;
#pragma unroll
      for (int k = 0; k < EPV; ++k) {
        a[i][k] = ok ? a[i][k] : fill;
        b[i][k] = ok ? b[i][k] : fill;
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < NV; ++i)
#pragma unroll
      for (int k = 0; k < EPV; ++k) { a[i][k] = fill; b[i][k] = fill; }
  }
}

// The head/tail element of this lane (column `ec`, or -1: none) without a
// divergent branch: lanes with none re-read column 0 and take `fill`.
template <typename Ts>
__device__ __forceinline__ float load_extra(const Ts* row, int ec, float fill) {
  const float v = load1(row + (ec >= 0 ? ec : 0));
  return ec >= 0 ? v : fill;
}

// NTS: non-temporal stores (the kernel's store policy, see st_stream).
template <typename Ts, int T, int NV, int EPV, bool NTS = true, int AL>
__device__ __forceinline__ void store_chunks(Ts* row, const RowGeom<EPV, AL>& g, int tid,
                                             const float (&v)[NV][EPV]) {
  Ts* base = row + g.head;
  const uint32_t lo = (uint32_t)tid * EPV + opaque_zero();
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    Ts* p = base + ((uint32_t)(i * T * EPV) + lo);
    if ((i + 1) * T <= g.nvec) Vec<Ts, EPV>::template store<NTS>(p, v[i]);  // uniform: whole slot
    else if (i * T + tid < g.nvec) Vec<Ts, EPV>::template store<NTS>(p, v[i]);
  }
}

// Per-column parameters of chunk slot i of this lane (rows on the 128-bit
// path share their phase with the parameter vectors, so chunk columns map
// to aligned parameter chunks). Only valid when g.nvec > 0 (callers test it
// once, uniformly); slots past the row end read the last chunk.
template <typename Ts, int T, int EPV, int AL>
__device__ __forceinline__ void load_param_slot(const Ts* par, const RowGeom<EPV, AL>& g, int tid, int i,
                                                float* w) {
  const uint32_t last = (uint32_t)(g.nvec - 1) * EPV;
  uint32_t o = (uint32_t)(i * T * EPV) + (uint32_t)tid * EPV;
  o = o < last ? o : last;
  load_param<Ts, EPV>((par + g.head) + o, w);
}

// ------------------------------------------------------- wavefront reduction
// Reduce a state held by all 64 lanes to lane 63 with six DPP steps
//   quad_perm [1,0,3,2], quad_perm [2,3,0,1]   -> 4-lane totals
//   row_half_mirror, row_mirror                 -> 16-lane (row) totals
//   row_bcast:15 (rows 1,3), row_bcast:31 (rows 2,3) -> wave total in lane 63
// then broadcast it with v_readlane. Lanes outside a row_bcast row mask read
// the identity. Only lane 63's value is used, so the result is the same on
// every lane and bitwise reproducible.

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_move(float src, float identity) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
      __builtin_bit_cast(int, identity), __builtin_bit_cast(int, src), CTRL, ROW_MASK, 0xF, false));
}

__device__ __forceinline__ float read_lane63(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

template <typename S, typename Merge>
__device__ __forceinline__ S wave_reduce(S v, Merge merge) {
  v = merge(v, S::template move<0xB1, 0xF>(v));   // quad_perm [1,0,3,2]
  v = merge(v, S::template move<0x4E, 0xF>(v));   // quad_perm [2,3,0,1]
  v = merge(v, S::template move<0x141, 0xF>(v));  // row_half_mirror
  v = merge(v, S::template move<0x140, 0xF>(v));  // row_mirror
  v = merge(v, S::template move<0x142, 0xA>(v));  // row_bcast:15
  v = merge(v, S::template move<0x143, 0xC>(v));  // row_bcast:31
  return v.lane63();
}

// Sum state (RMSNorm).
struct SumState {
  float s;
  template <int C, int M>
  static __device__ __forceinline__ SumState move(const SumState& a) { return {dpp_move<C, M>(a.s, 0.f)}; }
  __device__ __forceinline__ SumState lane63() const { return {read_lane63(s)}; }
};
struct SumMerge {
  __device__ __forceinline__ SumState operator()(const SumState& a, const SumState& b) const {
    return {a.s + b.s};
  }
};

// Two independent sums (backward kernels: e.g. sum h^2 and sum dy*w*h).
struct Sum2State {
  float a, b;
  template <int C, int M>
  static __device__ __forceinline__ Sum2State move(const Sum2State& v) {
    return {dpp_move<C, M>(v.a, 0.f), dpp_move<C, M>(v.b, 0.f)};
  }
  __device__ __forceinline__ Sum2State lane63() const { return {read_lane63(a), read_lane63(b)}; }
};
struct Sum2Merge {
  __device__ __forceinline__ Sum2State operator()(const Sum2State& x, const Sum2State& y) const {
    return {x.a + y.a, x.b + y.b};
  }
};

// Exact unsigned integer sum (counts): the words travel as float bit
// patterns through the DPP moves, unchanged, and are added as integers.
struct CountState {
  float b;
  template <int C, int M>
  static __device__ __forceinline__ CountState move(const CountState& a) { return {dpp_move<C, M>(a.b, 0.f)}; }
  __device__ __forceinline__ CountState lane63() const { return {read_lane63(b)}; }
};
struct CountMerge {
  __device__ __forceinline__ CountState operator()(const CountState& a, const CountState& b) const {
    return {__uint_as_float(__float_as_uint(a.b) + __float_as_uint(b.b))};
  }
};

// Maximum over a wavefront (the DPP tree above with max): no exponential,
// one move and one max per step. -inf is the identity; a NaN lane value is
// passed over here and reaches the result through the exponential sums.
struct MaxState {
  float m;
  template <int C, int M>
  static __device__ __forceinline__ MaxState move(const MaxState& a) { return {dpp_move<C, M>(a.m, kNegInf)}; }
  __device__ __forceinline__ MaxState lane63() const { return {read_lane63(m)}; }
};
struct MaxMerge {
  __device__ __forceinline__ MaxState operator()(const MaxState& a, const MaxState& b) const {
    return {__builtin_fmaxf(a.m, b.m)};
  }
};
__device__ __forceinline__ float wave_max(float v) { return wave_reduce(MaxState{v}, MaxMerge{}).m; }

// Two sums and a minimum over a wavefront, in one DPP tree: the row sums of a
// softmax lane state taken relative to the wave's maximum (exponentials s,
// logits t) and the smallest column holding that maximum (idx, a float;
// empty 3e38). Fields a kernel does not read cost nothing (dead moves are
// dropped).
struct WaveSums {
  float s, t, idx;
  template <int C, int M>
  static __device__ __forceinline__ WaveSums move(const WaveSums& a) {
    return {dpp_move<C, M>(a.s, 0.f), dpp_move<C, M>(a.t, 0.f), dpp_move<C, M>(a.idx, 3.0e38f)};
  }
  __device__ __forceinline__ WaveSums lane63() const {
    return {read_lane63(s), read_lane63(t), read_lane63(idx)};
  }
};
struct WaveSumsMerge {
  __device__ __forceinline__ WaveSums operator()(const WaveSums& a, const WaveSums& b) const {
    return {a.s + b.s, a.t + b.t, __builtin_fminf(a.idx, b.idx)};
  }
};

// Softmax state: running max m and the sum s of exponentials taken relative
// to m ("Online FlashSoftmax" recurrence). Empty state (-inf, 0).
struct MaxSumState {
  float m, s;
  template <int C, int M>
  static __device__ __forceinline__ MaxSumState move(const MaxSumState& a) {
    return {dpp_move<C, M>(a.m, kNegInf), dpp_move<C, M>(a.s, 0.f)};
  }
  __device__ __forceinline__ MaxSumState lane63() const { return {read_lane63(m), read_lane63(s)}; }
};

// (ma, sa) (+) (mb, sb) = (M, s_hi + s_lo * e^(lo - M)), M = max, lo = min.
// The larger side is never rescaled; an empty side (or two empty sides)
// contributes nothing. States are in natural units; LOG2 selects the plain
// hardware exponential for the rescale (bf16 outputs), otherwise the
// compensated one.
template <bool LOG2>
struct MaxSumMerge {
  __device__ __forceinline__ MaxSumState operator()(const MaxSumState& a, const MaxSumState& b) const {
    const bool a_hi = a.m >= b.m;
    const float M = a_hi ? a.m : b.m;
    const float lo = a_hi ? b.m : a.m;
    const float s_hi = a_hi ? a.s : b.s;
    const float s_lo = a_hi ? b.s : a.s;
    float f;
    if constexpr (LOG2) f = exp2_hw((lo - M) * kLog2e);
    else f = exp_acc(lo - M);
    f = (lo == M) ? 1.f : f;  // equal maxima (including two empty states)
    return {M, __builtin_fmaf(s_lo, f, s_hi)};
  }
};

// Softmax state with the position of the maximum (cross-entropy argmax).
// idx is a column index held as a float (exact below 2^24); empty state
// (-inf, 0, +huge). Ties keep the smaller index.
struct MaxSumIdxState {
  float m, s, idx;
  template <int C, int M>
  static __device__ __forceinline__ MaxSumIdxState move(const MaxSumIdxState& a) {
    return {dpp_move<C, M>(a.m, kNegInf), dpp_move<C, M>(a.s, 0.f), dpp_move<C, M>(a.idx, 3.0e38f)};
  }
  __device__ __forceinline__ MaxSumIdxState lane63() const {
    return {read_lane63(m), read_lane63(s), read_lane63(idx)};
  }
};
struct MaxSumIdxMerge {
  __device__ __forceinline__ MaxSumIdxState operator()(const MaxSumIdxState& a,
                                                       const MaxSumIdxState& b) const {
    const MaxSumState r = MaxSumMerge<false>{}(MaxSumState{a.m, a.s}, MaxSumState{b.m, b.s});
    const float lo_idx = a.idx < b.idx ? a.idx : b.idx;
    const float idx = a.m > b.m ? a.idx : (b.m > a.m ? b.idx : lo_idx);
    return {r.m, r.s, idx};
  }
};

// Welford state: count n, mean mu, sum of squared deviations M2. Empty (0,0,0).
struct WelfordState {
  float n, mu, m2;
  template <int C, int M>
  static __device__ __forceinline__ WelfordState move(const WelfordState& a) {
    return {dpp_move<C, M>(a.n, 0.f), dpp_move<C, M>(a.mu, 0.f), dpp_move<C, M>(a.m2, 0.f)};
  }
  __device__ __forceinline__ WelfordState lane63() const {
    return {read_lane63(n), read_lane63(mu), read_lane63(m2)};
  }
};
// Pairwise (Chan et al.) merge: n = na + nb, d = mub - mua,
// mu = mua + d * nb/n, M2 = M2a + M2b + d^2 * na * nb/n.
struct WelfordMerge {
  __device__ __forceinline__ WelfordState operator()(const WelfordState& a, const WelfordState& b) const {
    const float n = a.n + b.n;
    const float wb = n > 0.f ? b.n / n : 0.f;
    const float d = b.mu - a.mu;
    return {n, __builtin_fmaf(d, wb, a.mu), a.m2 + b.m2 + d * d * (a.n * wb)};
  }
};

// -------------------------------------------------------- cross-wave merge
// Row-per-workgroup kernels: lane 0 of each wave puts the wave's state in
// LDS, one barrier, then every lane merges the NW states in wave order, so
// all waves see bitwise the same row state. A kernel that merges more than
// once passes the two slot buffers alternately, switching with every merge
// it performs (a counter of merges, not of rows: a row that skips its merge
// must not switch). Each merge has one barrier, so a buffer is written again
// only after the barrier of the merge in between, which every wave reaches
// after its reads of that buffer have completed (the barrier waits for the
// wave's LDS reads): no wave overwrites a state a slower wave still reads.
template <int NW, typename S, int NF>
struct XWave {
  float slot[2][NW][NF];
};

// The barrier of the cross-wave merge orders LDS only: the slots are LDS,
// and no wave reads global memory, or LDS copied from it by another wave,
// through this barrier. (__syncthreads() is a workgroup fence as well, which
// here waits for every outstanding vector memory operation of the wave: the
// previous row's stores and the next row's staged copies, which would then
// stop overlapping the rest of the row.)
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int NW, typename S, typename Merge>
__device__ __forceinline__ S block_merge(S wave_state, float (*slot)[sizeof(S) / sizeof(float)],
                                         int wave, int lane, Merge merge) {
  constexpr int NF = sizeof(S) / sizeof(float);
  if (lane == 0) {
    const float* f = reinterpret_cast<const float*>(&wave_state);
#pragma unroll
    for (int k = 0; k < NF; ++k) slot[wave][k] = f[k];
  }
  lds_barrier();
  S acc;
  {
    float* f = reinterpret_cast<float*>(&acc);
#pragma unroll
    for (int k = 0; k < NF; ++k) f[k] = slot[0][k];
  }
#pragma unroll
  for (int w = 1; w < NW; ++w) {
    S o;
    float* f = reinterpret_cast<float*>(&o);
#pragma unroll
    for (int k = 0; k < NF; ++k) f[k] = slot[w][k];
    acc = merge(acc, o);
  }
  return acc;
}

// Row-per-workgroup kernels, merged through a DPP tree: lane 0 of each wave
// puts the wave's state in LDS, one barrier, then lane j < NW of every
// 16-lane row loads wave j's state (the other lanes hold `empty`) and
// log2(NW) DPP steps (quad_perm [1,0,3,2], [2,3,0,1], row_half_mirror,
// row_mirror) leave the merge of all NW states in lane 0: NW - 1 merges on
// a fixed tree of depth log2(NW) instead of a chain of NW - 1. Every wave runs
// the same steps on the same values, so all of them get bitwise the same
// state; it is read from lane 0 into scalar registers. NW is a power of two
// up to 16. The LDS slots follow block_merge's alternation rule.
template <typename S>
__device__ __forceinline__ S read_lane0(const S& v) {
  constexpr int NF = sizeof(S) / sizeof(float);
  S r;
  const float* a = reinterpret_cast<const float*>(&v);
  float* b = reinterpret_cast<float*>(&r);
#pragma unroll
  for (int k = 0; k < NF; ++k)
    b[k] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, a[k]), 0));
  return r;
}

template <int NW, typename S, typename Merge>
__device__ __forceinline__ S block_merge_tree(S wave_state, float (*slot)[sizeof(S) / sizeof(float)],
                                              int wave, int lane, Merge merge, const S& empty) {
  static_assert(NW >= 2 && NW <= 16 && (NW & (NW - 1)) == 0, "2 to 16 waves, a power of two");
  constexpr int NF = sizeof(S) / sizeof(float);
  if (lane == 0) {
    const float* f = reinterpret_cast<const float*>(&wave_state);
#pragma unroll
    for (int k = 0; k < NF; ++k) slot[wave][k] = f[k];
  }
  lds_barrier();
  const int j = lane & 15;
  S acc = empty;
  if (j < NW) {
    float* f = reinterpret_cast<float*>(&acc);
#pragma unroll
    for (int k = 0; k < NF; ++k) f[k] = slot[j][k];
  }
  acc = merge(acc, S::template move<0xB1, 0xF>(acc));                         // pairs
  if constexpr (NW > 2) acc = merge(acc, S::template move<0x4E, 0xF>(acc));   // quads
  if constexpr (NW > 4) acc = merge(acc, S::template move<0x141, 0xF>(acc));  // 8 lanes
  if constexpr (NW > 8) acc = merge(acc, S::template move<0x140, 0xF>(acc));  // 16 lanes
  return read_lane0(acc);
}

}  // namespace fr
