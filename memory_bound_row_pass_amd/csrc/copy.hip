// Memory-system probes: what HBM sustains for a read-only, a write-only and a
// copy pattern, with the access pattern of the row kernels and nothing else
// (no arithmetic). They are the ceilings the row kernels' bandwidth is
// compared with ("Engineering a CUDA Machine Learning Framework from
// Scratch", §2.1 The Memory Bandwidth Bottleneck: the row operations are
// bound by memory traffic, not arithmetic), and the known-size references
// for scaling the hardware byte counters.
//
// Access pattern: a workgroup of T lanes owns a contiguous "row" of up to
// T * NV 16-byte chunks (rows follow each other without gaps); lane t holds
// chunks t, t + T, ..., so consecutive lanes touch consecutive chunks (one
// wave instruction covers 1 KiB). A copy issues all loads of its row, waits
// for all of them and for the workgroup barrier, then stores: the dependency
// of a row kernel, whose stores need the whole row's reduction. T == 64 runs
// four rows per 256-lane workgroup (one per wavefront), as the wave-per-row
// kernels do. One workgroup per row group; the dispatcher hands them out.
#include "fusedrow.h"

#include "fr_device.hpp"
#include "fr_kernels.hpp"

namespace fr {

template <bool NT>
__device__ __forceinline__ u32x4 probe_load(const u32x4* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}
template <bool NT>
__device__ __forceinline__ void probe_store(u32x4 v, u32x4* p) {
  if constexpr (NT) __builtin_nontemporal_store(v, p);
  else *p = v;
}

// XOR of a 32-bit word over a wavefront (the DPP tree of the row kernels;
// the words travel as float bit patterns, moved unchanged).
struct XorState {
  float b;
  template <int C, int M>
  static __device__ __forceinline__ XorState move(const XorState& a) { return {dpp_move<C, M>(a.b, 0.f)}; }
  __device__ __forceinline__ XorState lane63() const { return {read_lane63(b)}; }
};
struct XorMerge {
  __device__ __forceinline__ XorState operator()(const XorState& a, const XorState& b) const {
    return {__uint_as_float(__float_as_uint(a.b) ^ __float_as_uint(b.b))};
  }
};

// MODE: 0 read (each row's XOR of its words goes to sink[row]), 1 write
// (every 32-bit word set to `value`), 2 copy. n16: 16-byte chunks in the
// buffer(s); rc: chunks per row (<= T * NV); the last row may be partial
// (lanes past the end of the row or buffer neither load nor store). Every
// wave reaches the barriers.
// POL bit 0: non-temporal loads; bit 1: non-temporal stores (else ordinary
// cached accesses).
template <int MODE, int T, int NV, int POL>
__global__ __launch_bounds__(T == 64 ? 256 : T) void stream_probe_kernel(
    const u32x4* __restrict__ src, u32x4* __restrict__ dst, int64_t n16, int rc, uint32_t value,
    uint32_t* __restrict__ sink) {
  constexpr int RPB = T == 64 ? 4 : 1;
  const int sub = T == 64 ? (int)(threadIdx.x >> 6) : 0;
  const int tid = T == 64 ? (int)(threadIdx.x & 63) : (int)threadIdx.x;
  const int64_t row = (int64_t)blockIdx.x * RPB + sub;
  const int64_t c0 = row * rc;
  const int64_t end = c0 + rc < n16 ? c0 + rc : n16;  // the row's end (chunks)
  const bool whole = rc == T * NV && c0 + T * NV <= n16;  // uniform in the row owner
  u32x4 v[NV];
  if constexpr (MODE != 1) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int64_t c = c0 + i * T + tid;
      v[i] = (whole || c < end) ? probe_load<(POL & 1) != 0>(src + c) : u32x4{0, 0, 0, 0};
    }
  } else {
#pragma unroll
    for (int i = 0; i < NV; ++i) v[i] = u32x4{value, value, value, value};
  }
  if constexpr (MODE == 0) {
    uint32_t x = 0;
#pragma unroll
    for (int i = 0; i < NV; ++i) x ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
    const XorState w = wave_reduce(XorState{__uint_as_float(x)}, XorMerge{});
    __shared__ uint32_t acc[RPB];
    if (tid == 0) acc[sub] = 0;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) atomicXor(&acc[sub], __float_as_uint(w.b));  // one per wave
    __syncthreads();
    if (tid == 0 && c0 < n16) sink[row] = acc[sub];
  } else {
    if constexpr (MODE == 2) {  // every load of the row has arrived, in every wave
      if constexpr (T == 64) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int64_t c = c0 + i * T + tid;
      if (whole || c < end) probe_store<(POL & 2) != 0>(v[i], dst + c);
    }
  }
}

__global__ __launch_bounds__(256) void byte_copy_kernel(const uint8_t* src, uint8_t* dst, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) dst[i] = src[i];
}


namespace {

typedef void (*ProbeKernel)(const u32x4*, u32x4*, int64_t, int, uint32_t, uint32_t*);

struct ProbeShape {
  int threads, vecs;
  ProbeKernel k[3][4];  // [mode][policy]
};

#define FR_PROBE_MODE(M, T, NV)                                                      \
  {&stream_probe_kernel<M, T, NV, 0>, &stream_probe_kernel<M, T, NV, 1>,               \
   &stream_probe_kernel<M, T, NV, 2>, &stream_probe_kernel<M, T, NV, 3>}
#define FR_PROBE_SHAPE(T, NV) \
  {T, NV, {FR_PROBE_MODE(0, T, NV), FR_PROBE_MODE(1, T, NV), FR_PROBE_MODE(2, T, NV)}}

// The shapes of the row kernels: 64 x 8 and 128 x 4 (bf16 16384 x 4096),
// 512 x 2 (add + RMSNorm 8192^2, per operand), 1024 x 13 and 1024 x 7
// (cross-entropy 4096 x 50257, fp32 and bf16), and neighbours.
const ProbeShape kProbeShapes[] = {
    FR_PROBE_SHAPE(64, 2),    FR_PROBE_SHAPE(64, 4),    FR_PROBE_SHAPE(64, 8),
    FR_PROBE_SHAPE(64, 16),   FR_PROBE_SHAPE(128, 4),   FR_PROBE_SHAPE(256, 1),
    FR_PROBE_SHAPE(256, 2),
    FR_PROBE_SHAPE(256, 4),   FR_PROBE_SHAPE(256, 8),   FR_PROBE_SHAPE(256, 16),
    FR_PROBE_SHAPE(512, 1),   FR_PROBE_SHAPE(512, 2),   FR_PROBE_SHAPE(512, 4),
    FR_PROBE_SHAPE(512, 8),   FR_PROBE_SHAPE(1024, 1),  FR_PROBE_SHAPE(1024, 2),
    FR_PROBE_SHAPE(1024, 4),  FR_PROBE_SHAPE(1024, 7),  FR_PROBE_SHAPE(1024, 8),
    FR_PROBE_SHAPE(1024, 13), FR_PROBE_SHAPE(1024, 16)};

const ProbeShape* find_shape(int threads, int vecs) {
  for (const ProbeShape& s : kProbeShapes)
    if (s.threads == threads && s.vecs == vecs) return &s;
  return nullptr;
}

}  // namespace

bool stream_probe_shape_exists(int threads, int vecs) { return find_shape(threads, vecs) != nullptr; }

int64_t stream_probe_rows(int64_t bytes, int64_t row_bytes) {
  return (bytes + row_bytes - 1) / row_bytes;
}

hipError_t launch_stream_probe(int mode, const void* src, void* dst, int64_t bytes,
                               int64_t row_bytes, int threads, int vecs, int policy,
                               uint32_t value, uint32_t* sink, hipStream_t s) {
  const ProbeShape* sh = find_shape(threads, vecs);
  if (!sh || mode < 0 || mode > 2 || row_bytes < 16 || row_bytes % 16 != 0 ||
      row_bytes > (int64_t)threads * vecs * 16)
    return hipErrorInvalidValue;
  const int64_t rows = stream_probe_rows(bytes, row_bytes);
  const int64_t rpb = threads == 64 ? 4 : 1;
  const int64_t blocks = (rows + rpb - 1) / rpb;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  return launch_kernel(sh->k[mode][policy & 3], dim3((unsigned)blocks),
                       dim3(threads == 64 ? 256 : threads), s, static_cast<const u32x4*>(src),
                       static_cast<u32x4*>(dst), bytes / 16, (int)(row_bytes / 16), value, sink);
}

hipError_t launch_stream_copy(const void* src, void* dst, int64_t bytes, hipStream_t s) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(src), b = reinterpret_cast<uintptr_t>(dst);
  if (a % 16 == 0 && b % 16 == 0 && bytes % 16 == 0)
    return launch_stream_probe(2, src, dst, bytes, FR_STREAM_THREADS * FR_STREAM_VECS * 16,
                               FR_STREAM_THREADS, FR_STREAM_VECS, FR_STREAM_POLICY, 0, nullptr, s);
  int64_t blocks = (bytes + 255) / 256;
  blocks = blocks < 4096 ? blocks : 4096;
  return launch_kernel(&byte_copy_kernel, dim3((unsigned)blocks), dim3(256), s,
                       static_cast<const uint8_t*>(src), static_cast<uint8_t*>(dst), bytes);
}

}  // namespace fr
