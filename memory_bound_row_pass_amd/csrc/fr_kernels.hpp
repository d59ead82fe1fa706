// Internal interface between the C-ABI front end (api.cpp) and the kernel
// translation units: per-op variant tables of typed launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fr {

// Records the HIP error of a failed launch for fr_debug_last_launch_error.
void note_launch_error(hipError_t e);

// Largest grid used; row loops stride by the grid beyond it.
constexpr int64_t kMaxGrid = int64_t(1) << 30;

// Two-pass (split-row) launches run both passes over one batch of rows before
// the next batch, so that the second pass re-reads input the first pass has
// just brought through the memory-side last-level cache (256 MB on MI355X)
// instead of from HBM. The batch holds at most split_batch_bytes() of input
// (0: one batch of all rows); kSplitBatchBytes is the default, measured best
// among 32 MB .. 512 MB and unbatched.
constexpr int64_t kSplitBatchBytes = int64_t(256) << 20;
int64_t split_batch_bytes();  // the current setting (fr_debug_set_split_batch_bytes)
int device_cu_count();        // compute units of the current device (cached per device)
// Pass-1 loads of the two-pass kernels are ordinary cached loads, so that the
// row batch stays in the last-level cache for pass 2 (with the row batches,
// fp32 cross-entropy [2048, 131072]: 541 -> 504 us per call).
constexpr bool kPass1NT = false;
// The one-pass form of the split-row softmax and cross-entropy: a row's
// segment workgroups exchange their partial states through device-scope
// atomics in the workspace and write their outputs from the registers, so
// the input is read once (split_one_pass(): 0 never, 1 where it applies
// and the rows are many enough, the default; 2 wherever it applies).
int split_one_pass();
// Polls a workgroup makes for its row's other states before it gives up (its
// outputs for the row are then NaN): a bound on every wait, so the kernel
// always ends (fr_debug_set_coop_spin_limit).
constexpr int kCoopSpinLimit = 1 << 18;
int coop_spin_limit();
// Most segments in one row of the one-pass form: the row's states are merged
// by one wavefront's DPP tree, one state per lane.
constexpr int kCoopMaxSegments = 64;
// Workspace of the one-pass form: 16 bytes of ticket counter and abort word,
// then two 64-bit words per (row, segment).
inline int64_t coop_workspace_bytes(int64_t rows, int nseg) { return 16 + rows * nseg * 16; }
// Bytes of the split workspace for [rows, cols] (fr_split_workspace_bytes):
// one 16-byte state per segment of the smallest segment shape, and 16 bytes
// more — room for the one-pass form of every segment shape.
constexpr int kSplitMinSegment = 8192;
inline int64_t split_part_bytes(int64_t rows, int64_t cols) {
  return rows > 0 ? rows * ((cols + kSplitMinSegment - 1) / kSplitMinSegment) * 16 + 16 : 0;
}
inline bool coop_applies(int64_t rows, int nseg, int64_t part_bytes) {
  return nseg <= kCoopMaxSegments && rows * nseg < (int64_t(1) << 31) &&
         coop_workspace_bytes(rows, nseg) <= part_bytes;
}

inline int64_t split_batch_rows(int64_t rows, int64_t input_bytes_per_row) {
  const int64_t bytes = split_batch_bytes();
  if (bytes <= 0) return rows;
  int64_t b = bytes / input_bytes_per_row;
  b = b < 1 ? 1 : b;
  return b < rows ? b : rows;
}

// A compiled kernel shape: `threads` lanes own one row, each holding `nv`
// chunks of `epv` elements (epv == 1: scalar path).
template <typename F>
struct Variant {
  int threads, nv, epv;
  F launch;
};

template <typename V>
struct VariantSpan {
  const V* v;
  size_t n;
};

typedef hipError_t (*SoftmaxLaunch)(const void* x, void* y, int64_t rows, int cols, hipStream_t s);
typedef hipError_t (*LayerNormLaunch)(const void* x, const void* gamma, const void* beta, void* y,
                                      float* mean, float* rstd, int64_t rows, int cols, float eps,
                                      hipStream_t s);
typedef hipError_t (*RmsNormLaunch)(const void* x, const void* res, const void* w, void* y,
                                    void* res_out, int64_t rows, int cols, float eps, hipStream_t s);
// Cross-entropy options (kernel argument, by value).
//   count: device pointer to the number of rows not ignored, counted by
//          xent_count_kernel before the row pass (mean reduction), or NULL;
//   count_inline: instead, every workgroup counts the rows not ignored itself
//          (mean reduction over few enough rows, kXentInlineCountRows);
//   reduction: 1 sum, 2 mean: the last workgroup to finish (completion
//          counter `done`, zero on entry and left zero) adds the per-row
//          losses in a fixed order and writes `total` (one-pass kernels;
//          the split-row path keeps xent_total_kernel).
struct XentOptions {
  int use_ignore;
  int ignore_index;
  float smoothing;
  float grad_scale;
  const uint32_t* count;
  int count_inline;
  int reduction;
  uint32_t* done;
  float* total;
};
// Rows up to which a mean's row count is taken inside the row kernel (each
// workgroup reads all labels once: at most 32 KiB).
constexpr int64_t kXentInlineCountRows = 8192;
// A completion counter of the library's per-device pool (zero when idle;
// successive calls take successive counters).
hipError_t xent_done_counter(uint32_t** out);
typedef hipError_t (*XentLaunch)(const void* logits, const int32_t* labels, float* loss, void* grad,
                                 int32_t* argmax, int64_t rows, int cols, const XentOptions* opt,
                                 hipStream_t s);

// Backward launchers. The norm backward kernels run `grid` workgroups of
// kBwdBlock lanes and leave one fp32 partial row per workgroup and parameter
// gradient in ws ([nparams][grid][cols]); launch_colsum reduces them.
typedef hipError_t (*SoftmaxBwdLaunch)(const void* p, const void* dy, void* dx, int64_t rows,
                                       int cols, hipStream_t s);
typedef hipError_t (*RmsNormBwdLaunch)(const void* h, const void* dy, const void* dres,
                                       const void* w, void* dh, float* ws, int grid, int64_t rows,
                                       int cols, float eps, hipStream_t s);
typedef hipError_t (*LayerNormBwdLaunch)(const void* x, const void* dy, const void* gamma,
                                         const float* mean, const float* rstd, void* dx, float* ws,
                                         int grid, int64_t rows, int cols, hipStream_t s);

// Most workgroups (= partial rows in the workspace) of a norm backward launch.
constexpr int kBwdGridMax = 512;

// A compiled norm-backward shape: row groups of `threads` lanes, `rpb` row
// groups per workgroup, at most `grid_max` workgroups (a fixed number, not
// derived from the device, so the reduction order and the results do not
// depend on it).
template <typename F>
struct BwdVariant {
  int threads, nv, epv, rpb, grid_max;
  F launch;
};

template <typename V>
inline int bwd_grid(const V& v, int64_t rows) {
  const int64_t g = (rows + v.rpb - 1) / v.rpb;
  return (int)(g < v.grid_max ? g : v.grid_max);
}

// Split-row launch: pass 1 (segment partials into `part`, 16 bytes per
// (row, segment)) then pass 2, both on `s`. Segment = threads * nv * epv
// columns. labels / loss / argmax / opt: cross-entropy only (NULL otherwise).
typedef hipError_t (*SplitLaunch)(const void* x, void* y, int64_t rows, int cols,
                                  const int32_t* labels, float* loss, int32_t* argmax,
                                  const XentOptions* opt, float4* part, int64_t part_bytes,
                                  bool one_pass, hipStream_t s);

// Split-row LayerNorm / residual-add + RMSNorm (pass 1 partials into
// `part`, then pass 2). LayerNorm: p1 = gamma, p2 = beta, res and res_out
// NULL. RMSNorm: p1 = weight; p2, mean and rstd NULL.
typedef hipError_t (*NormSplitLaunch)(const void* x, const void* res, const void* p1,
                                      const void* p2, void* y, void* res_out, float* mean,
                                      float* rstd, int64_t rows, int cols, float eps, float4* part,
                                      int64_t part_bytes, bool one_pass, hipStream_t s);

// Split-row softmax backward (pass 1 segment sums of p * dy into `part`).
typedef hipError_t (*SoftmaxBwdSplitLaunch)(const void* p, const void* dy, void* dx, int64_t rows,
                                            int cols, float4* part, int64_t part_bytes,
                                            bool one_pass, hipStream_t s);

typedef Variant<SoftmaxLaunch> SoftmaxVariant;
typedef Variant<LayerNormLaunch> LayerNormVariant;
typedef Variant<RmsNormLaunch> RmsNormVariant;
typedef Variant<XentLaunch> XentVariant;
typedef Variant<SoftmaxBwdLaunch> SoftmaxBwdVariant;
typedef Variant<SplitLaunch> SplitVariant;
typedef Variant<NormSplitLaunch> NormSplitVariant;
typedef Variant<SoftmaxBwdSplitLaunch> SoftmaxBwdSplitVariant;
typedef BwdVariant<RmsNormBwdLaunch> RmsNormBwdVariant;
typedef BwdVariant<LayerNormBwdLaunch> LayerNormBwdVariant;

VariantSpan<SoftmaxVariant> softmax_variants(int in_bf16, int out_bf16);
VariantSpan<LayerNormVariant> layernorm_variants(int bf16);
VariantSpan<RmsNormVariant> rmsnorm_variants(int bf16);
VariantSpan<XentVariant> xent_variants(int bf16, int with_argmax);
VariantSpan<XentVariant> xent_ex_variants(int bf16, int with_argmax);
VariantSpan<SplitVariant> split_variants(int in_bf16, int out_bf16, int xent);
VariantSpan<NormSplitVariant> norm_split_variants(int bf16, int rms);
VariantSpan<SoftmaxBwdSplitVariant> softmax_bwd_split_variants(int bf16);
hipError_t launch_xent_count(const int32_t* labels, int64_t rows, int use_ignore, int ignore_index,
                             uint32_t* out, hipStream_t s);
hipError_t launch_xent_total(const float* loss, int64_t rows, const uint32_t* count, float* total,
                             hipStream_t s);
VariantSpan<SoftmaxBwdVariant> softmax_bwd_variants(int bf16);
VariantSpan<RmsNormBwdVariant> rmsnorm_bwd_variants(int bf16);
VariantSpan<LayerNormBwdVariant> layernorm_bwd_variants(int bf16);

// Split-row norm backward (rows wider than FR_BWD_MAX_COLS): segments of
// kBwdSplitSeg columns; workspace = the row-sum partials (16 bytes per row
// segment, padded to 256 bytes) then [params][RG][cols] fp32 partial rows,
// RG = norm_bwd_split_groups(rows, segments) <= kBwdGridMax.
constexpr int kBwdSplitSeg = 8192;
inline int norm_bwd_split_groups(int64_t rows, int nseg) {
  int g = 1024 / nseg;
  g = g < 1 ? 1 : (g > kBwdGridMax ? kBwdGridMax : g);
  return (int)(rows < g ? rows : g);
}
// The per-(row, segment) sums of the two passes, or the one-pass form's
// counter, abort word and slots (16 bytes more).
inline int64_t norm_bwd_split_part_bytes(int64_t rows, int64_t cols) {
  const int64_t nseg = (cols + kBwdSplitSeg - 1) / kBwdSplitSeg;
  return rows > 0 ? (rows * nseg * 16 + 16 + 255) / 256 * 256 : 0;
}
hipError_t launch_norm_bwd_split(int layernorm, int bf16, int vec, const void* xh, const void* dy,
                                 const void* dres, const void* w, const float* mean,
                                 const float* rstd, void* out, float* dw0, float* dw1,
                                 void* workspace, int64_t rows, int cols, float eps, bool one_pass,
                                 hipStream_t s);

// Allocation-free RMSNorm backward (noalloc.hip): the partial rows go to a
// library-held device array of kNoallocScratchBytes per GPU.
constexpr int64_t kNoallocScratchBytes = int64_t(8) << 20;
hipError_t launch_rmsnorm_bwd_noalloc(const RmsNormBwdVariant* v, const void* h, const void* dy,
                                      const void* dres, const void* w, void* dh, float* dweight,
                                      int64_t rows, int cols, float eps, hipStream_t s);

// out0[c] (and out1[c] when out1 != NULL) = sum over b < partials of
// ws[p][b][c], in order of b; partials == 0 writes zeros.
hipError_t launch_colsum(const float* ws, int partials, int cols, float* out0, float* out1,
                         hipStream_t s);

hipError_t launch_stream_copy(const void* src, void* dst, int64_t bytes, hipStream_t s);
// Memory-system probes (copy.hip): mode 0 read, 1 write, 2 copy; rows of
// row_bytes (a multiple of 16, at most threads * vecs * 16) on a compiled
// (threads, vecs) shape; policy bit 0: non-temporal loads, bit 1:
// non-temporal stores.
bool stream_probe_shape_exists(int threads, int vecs);
int64_t stream_probe_rows(int64_t bytes, int64_t row_bytes);
hipError_t launch_stream_probe(int mode, const void* src, void* dst, int64_t bytes,
                               int64_t row_bytes, int threads, int vecs, int policy,
                               uint32_t value, uint32_t* sink, hipStream_t s);

// Matrix-core probe (mfma_probe.hip): `workgroups` workgroups of 256 lanes,
// each wavefront `iters` rounds of 8 bf16 32x32x16 matrix instructions on
// operands of `pattern` (0 constant, 1 pseudo-random); sink: workgroups * 256
// floats.
hipError_t launch_mfma_probe(int workgroups, int iters, int pattern, float* sink, hipStream_t s);

// Attention forward, bf16, head dim D in {64, 128}; BH = batch * heads.
hipError_t launch_attention_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                                int64_t BH, int Sq, int Sk, int D, int causal, float scale,
                                hipStream_t s);

// Launch `kernel` and return the status of this launch alone (not an error
// left behind by an earlier runtime call, as hipGetLastError would).
// Arguments must have exactly the kernel's parameter types.
template <typename... Params, typename... Args>
hipError_t launch_kernel(void (*kernel)(Params...), dim3 grid, dim3 block, hipStream_t s,
                         Args... args) {
  static_assert(sizeof...(Params) == sizeof...(Args), "argument count");
  void* argv[] = {static_cast<void*>(&args)...};
  const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, argv, 0, s);
  if (e != hipSuccess) note_launch_error(e);
  return e;
}

}  // namespace fr
