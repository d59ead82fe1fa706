// C-ABI front end of libfusedrow: argument validation (before any HIP call),
// aliasing and alignment rules, kernel-variant selection and launch.
// The contract of each entry point is documented in include/fusedrow.h.
#include "fusedrow.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>

#include "fr_kernels.hpp"

namespace {

using fr::VariantSpan;

// ------------------------------------------------------------ forced variant
struct Forced {
  std::atomic<int> threads{0};
  std::atomic<int> vecs{0};
};
Forced g_forced[FR_OP_SOFTMAX_BWD_SPLIT + 1];

// ------------------------------------------------------------------- buffers
struct Buf {
  uintptr_t lo = 0, hi = 0;  // [lo, hi)
  bool row_data = false;     // [rows, cols] buffer (may be aliased in place)
  int esize = 0;
  bool output = false;
  bool present = false;
};

Buf make_buf(const void* p, int64_t bytes, bool row_data, int esize, bool output) {
  Buf b;
  if (!p) return b;
  b.present = true;
  b.lo = reinterpret_cast<uintptr_t>(p);
  b.hi = b.lo + static_cast<uintptr_t>(bytes);
  b.row_data = row_data;
  b.esize = esize;
  b.output = output;
  return b;
}

// Outputs may not overlap anything, except that an output row buffer may be
// exactly the same range as an input row buffer of the same element size.
fr_status_t check_alias(const Buf* bufs, int n) {
  for (int i = 0; i < n; ++i) {
    if (!bufs[i].present) continue;
    for (int j = i + 1; j < n; ++j) {
      if (!bufs[j].present) continue;
      const Buf& a = bufs[i];
      const Buf& b = bufs[j];
      if (!a.output && !b.output) continue;
      const bool overlap = a.lo < b.hi && b.lo < a.hi;
      if (!overlap) continue;
      const bool in_place = a.output != b.output && a.row_data && b.row_data && a.lo == b.lo &&
                            a.hi == b.hi && a.esize == b.esize;
      if (!in_place) return FR_E_ALIAS;
    }
  }
  return FR_OK;
}

bool aligned(const void* p, int a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
int esize(fr_dtype_t d) { return d == FR_BF16 ? 2 : 4; }
bool dtype_ok(fr_dtype_t d) { return d == FR_F32 || d == FR_BF16; }

// rows >= 0, 1 <= cols <= FR_MAX_COLS, rows*cols*8 fits in int64.
fr_status_t check_shape(int64_t rows, int64_t cols) {
  if (rows < 0 || cols < 1 || cols > FR_MAX_COLS) return FR_E_SHAPE;
  if (rows > INT64_MAX / 8 / cols) return FR_E_SHAPE;
  return FR_OK;
}

// Pick the first variant of `sp` on the requested path (epv == vector width,
// or 1 for the scalar path) whose lanes can hold `cols` elements; honour a
// forced (threads, vecs) pair when one is set for `op`.
template <typename V>
const V* select_variant(VariantSpan<V> sp, int op, int64_t cols, int epv) {
  const int ft = g_forced[op].threads.load(std::memory_order_relaxed);
  const int fv = g_forced[op].vecs.load(std::memory_order_relaxed);
  for (size_t i = 0; i < sp.n; ++i) {
    const V& v = sp.v[i];
    if (v.epv != epv) continue;
    if (ft && (v.threads != ft || v.nv != fv)) continue;
    if ((int64_t)v.threads * v.nv * v.epv >= cols) return &v;
    if (ft) return nullptr;
  }
  return nullptr;
}

fr_status_t launch_status(hipError_t e) { return e == hipSuccess ? FR_OK : FR_E_LAUNCH; }

// Rows that fill the chip once but not twice (ncu < rows <= 2 ncu, such as
// one GPU's share of a row-sharded batch): where the width-chosen shape is a
// 1024-lane one (one resident row per CU: two rounds), a 256-lane shape that
// holds the row keeps two rows per CU resident and runs them all in one
// round. Measured, cross-entropy fp32 [512, 50257]: 38.8 -> 34.3 us (at 256
// and at 1024+ rows the 1024-lane shape stays faster). Not with a forced
// variant. Queries the device's CU count (a HIP call), so only after the
// argument checks.
template <typename V>
const V* few_rows_variant(VariantSpan<V> sp, int op, int64_t rows, int64_t cols, int epv,
                          const V* dflt) {
  if (!dflt || dflt->threads != 1024 || g_forced[op].threads.load(std::memory_order_relaxed))
    return dflt;
  const int64_t ncu = fr::device_cu_count();
  if (rows <= ncu || rows > 2 * ncu) return dflt;
  for (size_t i = 0; i < sp.n; ++i) {
    const V& v = sp.v[i];
    if (v.epv == epv && v.threads == 256 && (int64_t)v.threads * v.nv * v.epv >= cols) return &v;
  }
  return dflt;
}

// Split-row shape: a forced (threads, vecs), else the table's first shape on
// the requested path (the smallest segment: measured fastest on MI355X).
template <typename V>
const V* select_split(VariantSpan<V> sp, int op, int epv) {
  const int ft = g_forced[op].threads.load(std::memory_order_relaxed);
  const int fv = g_forced[op].vecs.load(std::memory_order_relaxed);
  for (size_t i = 0; i < sp.n; ++i) {
    const V& v = sp.v[i];
    if (v.epv != epv) continue;
    if (!ft || (v.threads == ft && v.nv == fv)) return &v;
  }
  return nullptr;
}

// Split-row shape and form. A forced (threads, vecs) keeps its shape and
// takes the one-pass form wherever that applies (setting != 0). Otherwise
// the op's one-pass shape (512 lanes x `elems` elements) in the one-pass
// form, for rows of at most 64 such segments, when (setting 1) the rows
// give at least 4 work items per compute unit — below that, two passes over
// the table's first (smallest) segments measured faster (cross-entropy fp32
// [96, 131072] 39.1 against 36.9 us; [288, 131072] 77.8 against 81.1 us) —
// or (setting 2) always; else the table's first shape, in two passes.
// rows < 0: a single row.
template <typename V>
struct SplitChoice {
  const V* v;
  bool one_pass;
};
template <typename V>
SplitChoice<V> choose_split(VariantSpan<V> sp, int op, int epv, int64_t rows, int64_t cols,
                            int elems) {
  const int mode = fr::split_one_pass();
  if (g_forced[op].threads.load(std::memory_order_relaxed)) return {select_split(sp, op, epv), mode != 0};
  if (mode != 0 && elems > 0) {
    const int64_t nseg = (cols + 512 * elems - 1) / (512 * elems);
    const int64_t r = rows < 0 ? 1 : rows;
    if (nseg <= fr::kCoopMaxSegments && (mode == 2 || r * nseg >= 4 * fr::device_cu_count()))
      for (size_t i = 0; i < sp.n; ++i) {
        const V& v = sp.v[i];
        if (v.epv == epv && v.threads == 512 && v.nv * v.epv == elems) return {&v, true};
      }
  }
  return {select_split(sp, op, epv), mode == 2};
}
// Elements per lane of the one-pass shape of the softmax, cross-entropy,
// residual-add + RMSNorm and softmax backward (measured against 32 at 512
// lanes: RMSNorm bf16 [256, 262144] 110 against 118 us, softmax backward
// bf16 [256, 131072] 52 against 56 us). The LayerNorm's apply step reads
// gamma and beta for every row segment: in fp32 one pass at 512 x 32 pays
// (per call against the two passes: [512, 131072] 126.9 against 131.1 us,
// [2048, 32768] 118.1 against 129.6; 512 x 64 129 us, 1024 x 32 131-135),
// in bf16 no shape does (512 x 32: 86-89 against 81 us), so none (0).
constexpr int kOnePassElems = 64;
inline int one_pass_elems_ln(fr_dtype_t dtype) { return dtype == FR_F32 ? 32 : 0; }

thread_local int t_last_launch_error = 0;

int vec_epv(int esz) { return 16 / esz; }

}  // namespace

namespace {
std::atomic<int64_t> g_split_batch_bytes{fr::kSplitBatchBytes};
std::atomic<int> g_split_one_pass{1};
std::atomic<int> g_coop_spin_limit{fr::kCoopSpinLimit};
}  // namespace

namespace fr {
void note_launch_error(hipError_t e) { t_last_launch_error = static_cast<int>(e); }
int64_t split_batch_bytes() { return g_split_batch_bytes.load(std::memory_order_relaxed); }
int split_one_pass() { return g_split_one_pass.load(std::memory_order_relaxed); }
int coop_spin_limit() { return g_coop_spin_limit.load(std::memory_order_relaxed); }
int device_cu_count() {
  static std::atomic<int> cache[64];  // 0: not yet queried
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}
}  // namespace fr

extern "C" {

int fr_debug_last_launch_error(void) { return t_last_launch_error; }

int64_t fr_debug_set_split_batch_bytes(int64_t bytes) {
  const int64_t prev = g_split_batch_bytes.load();
  g_split_batch_bytes.store(bytes < 0 ? fr::kSplitBatchBytes : bytes);
  return prev;
}

int fr_debug_set_split_one_pass(int mode) {
  return g_split_one_pass.exchange(mode < 0 || mode > 2 ? 1 : mode);
}

int fr_debug_set_coop_spin_limit(int polls) {
  return g_coop_spin_limit.exchange(polls < 0 ? fr::kCoopSpinLimit : polls);
}


const char* fr_status_str(fr_status_t s) {
  switch (s) {
    case FR_OK: return "FR_OK";
    case FR_E_NULL: return "FR_E_NULL: a required pointer is NULL";
    case FR_E_SHAPE: return "FR_E_SHAPE: rows/cols out of range";
    case FR_E_DTYPE: return "FR_E_DTYPE: unsupported dtype combination";
    case FR_E_ALIAS: return "FR_E_ALIAS: an output overlaps another buffer";
    case FR_E_LAUNCH: return "FR_E_LAUNCH: kernel launch failed";
    case FR_E_ALIGN: return "FR_E_ALIGN: pointer not aligned to its element size";
    case FR_E_VALUE: return "FR_E_VALUE: invalid scalar argument";
    case FR_E_VARIANT: return "FR_E_VARIANT: forced kernel variant unavailable for this row";
  }
  return "unknown fr_status_t";
}

const char* fr_version(void) { return "fusedrow 0.1.0 (gfx950)"; }

fr_status_t fr_debug_force_variant(fr_op_t op, int threads, int vecs) {
  if (op < FR_OP_SOFTMAX || op > FR_OP_SOFTMAX_BWD_SPLIT) return FR_E_VALUE;
  if (threads < 0 || vecs < 0) return FR_E_VALUE;
  g_forced[op].vecs.store(threads ? vecs : 0);
  g_forced[op].threads.store(threads);
  return FR_OK;
}

namespace {
// rows < 0: the width-only choice (fr_debug_select_variant)
fr_status_t describe_variant(fr_op_t op, int64_t rows, int64_t cols, fr_dtype_t in_dtype,
                             fr_dtype_t out_dtype, int vector_path, int* threads, int* vecs,
                             int* elems_per_vec) {
  if (!threads || !vecs || !elems_per_vec) return FR_E_NULL;
  if (!dtype_ok(in_dtype) || !dtype_ok(out_dtype)) return FR_E_DTYPE;
  const bool split = op == FR_OP_SOFTMAX_SPLIT || op == FR_OP_XENT_SPLIT ||
                     op == FR_OP_LAYERNORM_SPLIT || op == FR_OP_RMSNORM_SPLIT ||
                     op == FR_OP_SOFTMAX_BWD_SPLIT;
  const int64_t maxc = split ? FR_SPLIT_MAX_COLS : FR_MAX_COLS;
  if (cols < 1 || cols > maxc) return FR_E_SHAPE;
  const int epv = vector_path ? vec_epv(esize(in_dtype)) : 1;
  int t = 0, n = 0, e = 0;
  switch (op) {
    case FR_OP_SOFTMAX: {
      auto v = select_variant(fr::softmax_variants(in_dtype == FR_BF16, out_dtype == FR_BF16), op,
                              cols, epv);
      if (v) { t = v->threads; n = v->nv; e = v->epv; }
      break;
    }
    case FR_OP_LAYERNORM: {
      auto v = select_variant(fr::layernorm_variants(in_dtype == FR_BF16), op, cols, epv);
      if (v) { t = v->threads; n = v->nv; e = v->epv; }
      break;
    }
    case FR_OP_RMSNORM: {
      auto v = select_variant(fr::rmsnorm_variants(in_dtype == FR_BF16), op, cols, epv);
      if (v) { t = v->threads; n = v->nv; e = v->epv; }
      break;
    }
    case FR_OP_XENT: {
      // fp32: the plain table (the options table has the same shapes); bf16
      // logits exist only with options
      const auto sp = in_dtype == FR_BF16 ? fr::xent_ex_variants(1, 0) : fr::xent_variants(0, 0);
      auto v = select_variant(sp, op, cols, epv);
      if (rows >= 0) v = few_rows_variant(sp, op, rows, cols, epv, v);
      if (v) { t = v->threads; n = v->nv; e = v->epv; }
      break;
    }
    case FR_OP_SOFTMAX_BWD: {
      if (cols > FR_BWD_MAX_COLS) return FR_E_SHAPE;
      auto v = select_variant(fr::softmax_bwd_variants(in_dtype == FR_BF16), op, cols, epv);
      if (v) { t = v->threads; n = v->nv; e = v->epv; }
      break;
    }
    case FR_OP_RMSNORM_BWD: {
      if (cols > FR_BWD_MAX_COLS) return FR_E_SHAPE;
      auto v = select_variant(fr::rmsnorm_bwd_variants(in_dtype == FR_BF16), op, cols, epv);
      if (v) { t = v->threads; n = v->nv; e = v->epv; }
      break;
    }
    case FR_OP_LAYERNORM_BWD: {
      if (cols > FR_BWD_MAX_COLS) return FR_E_SHAPE;
      auto v = select_variant(fr::layernorm_bwd_variants(in_dtype == FR_BF16), op, cols, epv);
      if (v) { t = v->threads; n = v->nv; e = v->epv; }
      break;
    }
    case FR_OP_SOFTMAX_SPLIT:
    case FR_OP_XENT_SPLIT: {
      auto v = choose_split(fr::split_variants(in_dtype == FR_BF16, out_dtype == FR_BF16,
                                               op == FR_OP_XENT_SPLIT),
                            op, epv, rows, cols, kOnePassElems).v;
      if (v) { t = v->threads; n = v->nv; e = v->epv; }
      break;
    }
    case FR_OP_SOFTMAX_BWD_SPLIT: {
      auto v = choose_split(fr::softmax_bwd_split_variants(in_dtype == FR_BF16), op, epv, rows, cols,
                            kOnePassElems).v;
      if (v) { t = v->threads; n = v->nv; e = v->epv; }
      break;
    }
    case FR_OP_LAYERNORM_SPLIT:
    case FR_OP_RMSNORM_SPLIT: {
      auto v = choose_split(fr::norm_split_variants(in_dtype == FR_BF16, op == FR_OP_RMSNORM_SPLIT),
                            op, epv, rows, cols,
                            op == FR_OP_RMSNORM_SPLIT ? kOnePassElems : one_pass_elems_ln(in_dtype)).v;
      if (v) { t = v->threads; n = v->nv; e = v->epv; }
      break;
    }
    default: return FR_E_VALUE;
  }
  if (!t) return FR_E_VARIANT;
  *threads = t; *vecs = n; *elems_per_vec = e;
  return FR_OK;
}
}  // namespace

fr_status_t fr_debug_select_variant(fr_op_t op, int64_t cols, fr_dtype_t in_dtype,
                                    fr_dtype_t out_dtype, int vector_path, int* threads, int* vecs,
                                    int* elems_per_vec) {
  return describe_variant(op, -1, cols, in_dtype, out_dtype, vector_path, threads, vecs,
                          elems_per_vec);
}

fr_status_t fr_debug_select_variant_for(fr_op_t op, int64_t rows, int64_t cols, fr_dtype_t in_dtype,
                                        fr_dtype_t out_dtype, int vector_path, int* threads,
                                        int* vecs, int* elems_per_vec) {
  if (rows < 0) return FR_E_SHAPE;
  return describe_variant(op, rows, cols, in_dtype, out_dtype, vector_path, threads, vecs,
                          elems_per_vec);
}

fr_status_t fr_softmax_fwd(const void* x, void* y, int64_t rows, int64_t cols, fr_dtype_t x_dtype,
                           fr_dtype_t y_dtype, void* stream) {
  if (fr_status_t s = check_shape(rows, cols)) return s;
  if (!dtype_ok(x_dtype) || !dtype_ok(y_dtype)) return FR_E_DTYPE;
  if (rows == 0) return FR_OK;
  if (!x || !y) return FR_E_NULL;
  const int xs = esize(x_dtype), ys = esize(y_dtype);
  if (!aligned(x, xs) || !aligned(y, ys)) return FR_E_ALIGN;
  const Buf bufs[] = {make_buf(x, rows * cols * xs, true, xs, false),
                      make_buf(y, rows * cols * ys, true, ys, true)};
  if (fr_status_t s = check_alias(bufs, 2)) return s;

  // 128-bit path: same-width rows sharing their address phase (per-row
  // head/tail split), or mixed widths with every row 16-byte aligned.
  const int ve = vec_epv(xs);
  bool vec;
  if (xs == ys) vec = (reinterpret_cast<uintptr_t>(x) % 16) == (reinterpret_cast<uintptr_t>(y) % 16);
  else vec = aligned(x, 16) && aligned(y, 16) && cols % ve == 0;
  auto sp = fr::softmax_variants(x_dtype == FR_BF16, y_dtype == FR_BF16);
  const fr::SoftmaxVariant* v = select_variant(sp, FR_OP_SOFTMAX, cols, vec ? ve : 1);
  if (!v) return g_forced[FR_OP_SOFTMAX].threads.load() ? FR_E_VARIANT : FR_E_SHAPE;
  return launch_status(v->launch(x, y, rows, (int)cols, static_cast<hipStream_t>(stream)));
}

fr_status_t fr_layernorm_fwd(const void* x, const void* gamma, const void* beta, void* y,
                             float* mean, float* rstd, int64_t rows, int64_t cols, float eps,
                             fr_dtype_t dtype, void* stream) {
  if (fr_status_t s = check_shape(rows, cols)) return s;
  if (!dtype_ok(dtype)) return FR_E_DTYPE;
  if (!std::isfinite(eps) || eps < 0.f) return FR_E_VALUE;
  if (rows == 0) return FR_OK;
  if (!x || !gamma || !beta || !y) return FR_E_NULL;
  const int es = esize(dtype);
  if (!aligned(x, es) || !aligned(y, es) || !aligned(gamma, es) || !aligned(beta, es) ||
      (mean && !aligned(mean, 4)) || (rstd && !aligned(rstd, 4)))
    return FR_E_ALIGN;
  const Buf bufs[] = {make_buf(x, rows * cols * es, true, es, false),
                      make_buf(gamma, cols * es, false, es, false),
                      make_buf(beta, cols * es, false, es, false),
                      make_buf(y, rows * cols * es, true, es, true),
                      make_buf(mean, rows * 4, false, 4, true),
                      make_buf(rstd, rows * 4, false, 4, true)};
  if (fr_status_t s = check_alias(bufs, 6)) return s;
  const bool vec = aligned(x, 16) && aligned(y, 16) && aligned(gamma, 16) && aligned(beta, 16) &&
                   (cols * es) % 16 == 0;
  const fr::LayerNormVariant* v =
      select_variant(fr::layernorm_variants(dtype == FR_BF16), FR_OP_LAYERNORM, cols, vec ? vec_epv(es) : 1);
  if (!v) return g_forced[FR_OP_LAYERNORM].threads.load() ? FR_E_VARIANT : FR_E_SHAPE;
  return launch_status(v->launch(x, gamma, beta, y, mean, rstd, rows, (int)cols, eps,
                                 static_cast<hipStream_t>(stream)));
}

fr_status_t fr_add_rmsnorm_fwd(const void* x, const void* residual, const void* weight, void* y,
                               void* residual_out, int64_t rows, int64_t cols, float eps,
                               fr_dtype_t dtype, void* stream) {
  if (fr_status_t s = check_shape(rows, cols)) return s;
  if (!dtype_ok(dtype)) return FR_E_DTYPE;
  if (!std::isfinite(eps) || eps < 0.f) return FR_E_VALUE;
  if (rows == 0) return FR_OK;
  if (!x || !residual || !weight || !y) return FR_E_NULL;
  const int es = esize(dtype);
  if (!aligned(x, es) || !aligned(residual, es) || !aligned(weight, es) || !aligned(y, es) ||
      (residual_out && !aligned(residual_out, es)))
    return FR_E_ALIGN;
  const Buf bufs[] = {make_buf(x, rows * cols * es, true, es, false),
                      make_buf(residual, rows * cols * es, true, es, false),
                      make_buf(weight, cols * es, false, es, false),
                      make_buf(y, rows * cols * es, true, es, true),
                      make_buf(residual_out, rows * cols * es, true, es, true)};
  if (fr_status_t s = check_alias(bufs, 5)) return s;
  const bool vec = aligned(x, 16) && aligned(residual, 16) && aligned(weight, 16) &&
                   aligned(y, 16) && (!residual_out || aligned(residual_out, 16)) &&
                   (cols * es) % 16 == 0;
  const fr::RmsNormVariant* v =
      select_variant(fr::rmsnorm_variants(dtype == FR_BF16), FR_OP_RMSNORM, cols, vec ? vec_epv(es) : 1);
  if (!v) return g_forced[FR_OP_RMSNORM].threads.load() ? FR_E_VARIANT : FR_E_SHAPE;
  return launch_status(v->launch(x, residual, weight, y, residual_out, rows, (int)cols, eps,
                                 static_cast<hipStream_t>(stream)));
}

fr_status_t fr_softmax_xent_fwd_bwd(const float* logits, const int32_t* labels, float* loss,
                                    float* grad, int32_t* argmax, int64_t rows, int64_t cols,
                                    void* stream) {
  if (fr_status_t s = check_shape(rows, cols)) return s;
  if (rows == 0) return FR_OK;
  if (!logits || !labels || !loss || !grad) return FR_E_NULL;
  const int es = 4;
  if (!aligned(logits, es) || !aligned(grad, es) || !aligned(labels, 4) || !aligned(loss, 4) ||
      (argmax && !aligned(argmax, 4)))
    return FR_E_ALIGN;
  const Buf bufs[] = {make_buf(logits, rows * cols * es, true, es, false),
                      make_buf(labels, rows * 4, false, 4, false),
                      make_buf(loss, rows * 4, false, 4, true),
                      make_buf(grad, rows * cols * es, true, es, true),
                      make_buf(argmax, rows * 4, false, 4, true)};
  if (fr_status_t s = check_alias(bufs, 5)) return s;
  const bool vec =
      (reinterpret_cast<uintptr_t>(logits) % 16) == (reinterpret_cast<uintptr_t>(grad) % 16);
  const auto sp = fr::xent_variants(0, argmax != nullptr);
  const int epv = vec ? vec_epv(es) : 1;
  const fr::XentVariant* v =
      few_rows_variant(sp, FR_OP_XENT, rows, cols, epv, select_variant(sp, FR_OP_XENT, cols, epv));
  if (!v) return g_forced[FR_OP_XENT].threads.load() ? FR_E_VARIANT : FR_E_SHAPE;
  return launch_status(v->launch(logits, labels, loss, grad, argmax, rows, (int)cols, nullptr,
                                 static_cast<hipStream_t>(stream)));
}

fr_status_t fr_softmax_xent_ex(const void* logits, const int32_t* labels, float* loss, void* grad,
                               int32_t* argmax, float* loss_total, int64_t rows, int64_t cols,
                               fr_dtype_t dtype, const fr_xent_options_t* options, void* stream) {
  if (fr_status_t s = check_shape(rows, cols)) return s;
  if (!dtype_ok(dtype)) return FR_E_DTYPE;
  fr_xent_options_t o = {0, 0, 0.f, 1.f, FR_REDUCE_NONE};
  if (options) o = *options;
  if (!std::isfinite(o.label_smoothing) || o.label_smoothing < 0.f || o.label_smoothing > 1.f ||
      !std::isfinite(o.grad_scale) ||
      (o.reduction != FR_REDUCE_NONE && o.reduction != FR_REDUCE_SUM &&
       o.reduction != FR_REDUCE_MEAN))
    return FR_E_VALUE;
  if (o.reduction == FR_REDUCE_MEAN && rows > (int64_t)UINT32_MAX) return FR_E_SHAPE;
  const bool reduce = o.reduction != FR_REDUCE_NONE;
  if (reduce && !loss_total) return FR_E_NULL;
  if (loss_total && !aligned(loss_total, 4)) return FR_E_ALIGN;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool mean = o.reduction == FR_REDUCE_MEAN;
  if (rows == 0) {
    if (!reduce) return FR_OK;
    uint32_t* count = mean ? reinterpret_cast<uint32_t*>(loss_total) : nullptr;
    if (count)
      if (fr_status_t s = launch_status(fr::launch_xent_count(labels, 0, 0, 0, count, st))) return s;
    return launch_status(fr::launch_xent_total(loss, 0, count, loss_total, st));
  }
  if (!logits || !labels || !loss || !grad) return FR_E_NULL;
  const int es = esize(dtype);
  if (!aligned(logits, es) || !aligned(grad, es) || !aligned(labels, 4) || !aligned(loss, 4) ||
      (argmax && !aligned(argmax, 4)))
    return FR_E_ALIGN;
  const Buf bufs[] = {make_buf(logits, rows * cols * es, true, es, false),
                      make_buf(labels, rows * 4, false, 4, false),
                      make_buf(loss, rows * 4, false, 4, true),
                      make_buf(grad, rows * cols * es, true, es, true),
                      make_buf(argmax, rows * 4, false, 4, true),
                      make_buf(reduce ? loss_total : nullptr, 4, false, 4, true)};
  if (fr_status_t s = check_alias(bufs, 6)) return s;
  const bool vec =
      (reinterpret_cast<uintptr_t>(logits) % 16) == (reinterpret_cast<uintptr_t>(grad) % 16);
  const auto sp = fr::xent_ex_variants(dtype == FR_BF16, argmax != nullptr);
  const int epv = vec ? vec_epv(es) : 1;
  const fr::XentVariant* v =
      few_rows_variant(sp, FR_OP_XENT, rows, cols, epv, select_variant(sp, FR_OP_XENT, cols, epv));
  if (!v) return g_forced[FR_OP_XENT].threads.load() ? FR_E_VARIANT : FR_E_SHAPE;
  // A mean needs the rows not ignored before any gradient is scaled: the row
  // kernel's workgroups count them themselves over few rows, a count kernel
  // writes them to loss_total first over many. The total itself is added up
  // by the row kernel's last workgroup (a completion counter of the pool).
  const bool count_inline = mean && rows <= fr::kXentInlineCountRows;
  uint32_t* count = mean && !count_inline ? reinterpret_cast<uint32_t*>(loss_total) : nullptr;
  uint32_t* done = nullptr;
  if (reduce)
    if (fr_status_t s = launch_status(fr::xent_done_counter(&done))) return s;
  if (count)
    if (fr_status_t s = launch_status(
            fr::launch_xent_count(labels, rows, o.use_ignore_index != 0, o.ignore_index, count, st)))
      return s;
  const fr::XentOptions ko = {o.use_ignore_index != 0, o.ignore_index, o.label_smoothing,
                              o.grad_scale, count, count_inline ? 1 : 0, (int)o.reduction, done,
                              reduce ? loss_total : nullptr};
  return launch_status(v->launch(logits, labels, loss, grad, argmax, rows, (int)cols, &ko, st));
}

fr_status_t fr_softmax_bwd(const void* p, const void* dy, void* dx, int64_t rows, int64_t cols,
                           fr_dtype_t dtype, void* stream) {
  if (fr_status_t s = check_shape(rows, cols)) return s;
  if (cols > FR_BWD_MAX_COLS) return FR_E_SHAPE;
  if (!dtype_ok(dtype)) return FR_E_DTYPE;
  if (rows == 0) return FR_OK;
  if (!p || !dy || !dx) return FR_E_NULL;
  const int es = esize(dtype);
  if (!aligned(p, es) || !aligned(dy, es) || !aligned(dx, es)) return FR_E_ALIGN;
  const int64_t nb = rows * cols * es;
  const Buf bufs[] = {make_buf(p, nb, true, es, false), make_buf(dy, nb, true, es, false),
                      make_buf(dx, nb, true, es, true)};
  if (fr_status_t s = check_alias(bufs, 3)) return s;
  const uintptr_t ph = reinterpret_cast<uintptr_t>(p) % 16;
  const bool vec = reinterpret_cast<uintptr_t>(dy) % 16 == ph &&
                   reinterpret_cast<uintptr_t>(dx) % 16 == ph;
  const fr::SoftmaxBwdVariant* v = select_variant(fr::softmax_bwd_variants(dtype == FR_BF16),
                                                  FR_OP_SOFTMAX_BWD, cols, vec ? vec_epv(es) : 1);
  if (!v) return g_forced[FR_OP_SOFTMAX_BWD].threads.load() ? FR_E_VARIANT : FR_E_SHAPE;
  return launch_status(v->launch(p, dy, dx, rows, (int)cols, static_cast<hipStream_t>(stream)));
}

int64_t fr_norm_bwd_workspace_bytes(fr_op_t op, int64_t rows, int64_t cols) {
  if (op != FR_OP_RMSNORM_BWD && op != FR_OP_LAYERNORM_BWD) return -1;
  if (check_shape(rows, cols) != FR_OK || cols > FR_BWD_MAX_COLS) return -1;
  const int64_t np = op == FR_OP_LAYERNORM_BWD ? 2 : 1;
  const int64_t parts = rows < FR_BWD_PARTIALS ? rows : FR_BWD_PARTIALS;
  return parts * cols * 4 * np;
}

fr_status_t fr_add_rmsnorm_bwd(const void* h, const void* dy, const void* dres, const void* weight,
                               void* dh, float* dweight, void* workspace, int64_t workspace_bytes,
                               int64_t rows, int64_t cols, float eps, fr_dtype_t dtype,
                               void* stream) {
  if (fr_status_t s = check_shape(rows, cols)) return s;
  if (cols > FR_BWD_MAX_COLS) return FR_E_SHAPE;
  if (!dtype_ok(dtype)) return FR_E_DTYPE;
  if (!std::isfinite(eps) || eps < 0.f) return FR_E_VALUE;
  const int64_t need = fr_norm_bwd_workspace_bytes(FR_OP_RMSNORM_BWD, rows, cols);
  if (workspace_bytes < need) return FR_E_SHAPE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (!dweight) return FR_E_NULL;
  if (!aligned(dweight, 4)) return FR_E_ALIGN;
  if (rows == 0) return launch_status(fr::launch_colsum(nullptr, 0, (int)cols, dweight, nullptr, st));
  if (!h || !dy || !weight || !dh || !workspace) return FR_E_NULL;
  const int es = esize(dtype);
  if (!aligned(h, es) || !aligned(dy, es) || !aligned(weight, es) || !aligned(dh, es) ||
      (dres && !aligned(dres, es)) || !aligned(workspace, 16))
    return FR_E_ALIGN;
  const int64_t nb = rows * cols * es;
  const Buf bufs[] = {make_buf(h, nb, true, es, false),
                      make_buf(dy, nb, true, es, false),
                      make_buf(dres, nb, true, es, false),
                      make_buf(weight, cols * es, false, es, false),
                      make_buf(dh, nb, true, es, true),
                      make_buf(dweight, cols * 4, false, 4, true),
                      make_buf(workspace, need, false, 1, true)};
  if (fr_status_t s = check_alias(bufs, 7)) return s;
  const bool vec = aligned(h, 16) && aligned(dy, 16) && (!dres || aligned(dres, 16)) &&
                   aligned(weight, 16) && aligned(dh, 16) && (cols * es) % 16 == 0;
  const fr::RmsNormBwdVariant* v = select_variant(fr::rmsnorm_bwd_variants(dtype == FR_BF16),
                                                  FR_OP_RMSNORM_BWD, cols, vec ? vec_epv(es) : 1);
  if (!v) return g_forced[FR_OP_RMSNORM_BWD].threads.load() ? FR_E_VARIANT : FR_E_SHAPE;
  const int grid = fr::bwd_grid(*v, rows);
  float* ws = static_cast<float*>(workspace);
  if (fr_status_t s = launch_status(v->launch(h, dy, dres, weight, dh, ws, grid, rows, (int)cols,
                                              eps, st)))
    return s;
  return launch_status(fr::launch_colsum(ws, grid, (int)cols, dweight, nullptr, st));
}

fr_status_t fr_add_rmsnorm_bwd_noalloc(const void* h, const void* dy, const void* dres,
                                       const void* weight, void* dh, float* dweight, int64_t rows,
                                       int64_t cols, float eps, fr_dtype_t dtype, void* stream) {
  static_assert(FR_NOALLOC_SCRATCH_BYTES == fr::kNoallocScratchBytes, "scratch size");
  if (fr_status_t s = check_shape(rows, cols)) return s;
  if (cols > FR_BWD_MAX_COLS) return FR_E_SHAPE;
  if (!dtype_ok(dtype)) return FR_E_DTYPE;
  if (!std::isfinite(eps) || eps < 0.f) return FR_E_VALUE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (!dweight) return FR_E_NULL;
  if (!aligned(dweight, 4)) return FR_E_ALIGN;
  if (rows == 0) return launch_status(fr::launch_colsum(nullptr, 0, (int)cols, dweight, nullptr, st));
  if (!h || !dy || !weight || !dh) return FR_E_NULL;
  const int es = esize(dtype);
  if (!aligned(h, es) || !aligned(dy, es) || !aligned(weight, es) || !aligned(dh, es) ||
      (dres && !aligned(dres, es)))
    return FR_E_ALIGN;
  const int64_t nb = rows * cols * es;
  const Buf bufs[] = {make_buf(h, nb, true, es, false),
                      make_buf(dy, nb, true, es, false),
                      make_buf(dres, nb, true, es, false),
                      make_buf(weight, cols * es, false, es, false),
                      make_buf(dh, nb, true, es, true),
                      make_buf(dweight, cols * 4, false, 4, true)};
  if (fr_status_t s = check_alias(bufs, 6)) return s;
  const bool vec = aligned(h, 16) && aligned(dy, 16) && (!dres || aligned(dres, 16)) &&
                   aligned(weight, 16) && aligned(dh, 16) && (cols * es) % 16 == 0;
  const fr::RmsNormBwdVariant* v = select_variant(fr::rmsnorm_bwd_variants(dtype == FR_BF16),
                                                  FR_OP_RMSNORM_BWD, cols, vec ? vec_epv(es) : 1);
  if (!v) return g_forced[FR_OP_RMSNORM_BWD].threads.load() ? FR_E_VARIANT : FR_E_SHAPE;
  // the partial rows must fit the library's array (checked before any HIP call)
  if ((int64_t)fr::bwd_grid(*v, rows) * cols * 4 > fr::kNoallocScratchBytes) return FR_E_SHAPE;
  return launch_status(fr::launch_rmsnorm_bwd_noalloc(v, h, dy, dres, weight, dh, dweight, rows,
                                                      (int)cols, eps, st));
}

namespace {
// The split norm backward in one pass with setting 2, or with setting 1 for
// fp32 when the teams give at least 4 workgroups per compute unit; else two.
// A team waits once per row, and a bf16 row segment carries half the bytes
// per wait: measured (per call, one pass against two) fp32 [1024, 65536]
// RMSNorm with dres 243 against 281 us, LayerNorm 205 against 245; bf16
// [2048, 32768] RMSNorm with dres 156 against 149, without 129 against 130,
// LayerNorm 142 against 140; few rows ([256, 32768] bf16) 52 against 46.
bool norm_bwd_one_pass(int64_t rows, int64_t cols, fr_dtype_t dtype) {
  const int mode = fr::split_one_pass();
  const int nseg = (int)((cols + fr::kBwdSplitSeg - 1) / fr::kBwdSplitSeg);
  if (mode == 0 || nseg > fr::kCoopMaxSegments) return false;
  return mode == 2 || (dtype == FR_F32 && (int64_t)fr::norm_bwd_split_groups(rows, nseg) * nseg >=
                                              4 * fr::device_cu_count());
}
}  // namespace

int64_t fr_norm_bwd_split_workspace_bytes(fr_op_t op, int64_t rows, int64_t cols) {
  if (op != FR_OP_RMSNORM_BWD && op != FR_OP_LAYERNORM_BWD) return -1;
  if (rows < 0 || cols < 1 || cols > FR_SPLIT_MAX_COLS || rows > INT64_MAX / 8 / cols) return -1;
  const int nseg = (int)((cols + fr::kBwdSplitSeg - 1) / fr::kBwdSplitSeg);
  const int64_t np = op == FR_OP_LAYERNORM_BWD ? 2 : 1;
  return fr::norm_bwd_split_part_bytes(rows, cols) +
         (int64_t)fr::norm_bwd_split_groups(rows, nseg) * cols * 4 * np;
}

fr_status_t fr_add_rmsnorm_bwd_split(const void* h, const void* dy, const void* dres,
                                     const void* weight, void* dh, float* dweight, void* workspace,
                                     int64_t workspace_bytes, int64_t rows, int64_t cols, float eps,
                                     fr_dtype_t dtype, void* stream) {
  const int64_t need = fr_norm_bwd_split_workspace_bytes(FR_OP_RMSNORM_BWD, rows, cols);
  if (need < 0) return FR_E_SHAPE;
  if (!dtype_ok(dtype)) return FR_E_DTYPE;
  if (!std::isfinite(eps) || eps < 0.f) return FR_E_VALUE;
  if (workspace_bytes < need) return FR_E_SHAPE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (!dweight) return FR_E_NULL;
  if (!aligned(dweight, 4)) return FR_E_ALIGN;
  if (rows == 0) return launch_status(fr::launch_colsum(nullptr, 0, (int)cols, dweight, nullptr, st));
  if (!h || !dy || !weight || !dh || !workspace) return FR_E_NULL;
  const int es = esize(dtype);
  if (!aligned(h, es) || !aligned(dy, es) || !aligned(weight, es) || !aligned(dh, es) ||
      (dres && !aligned(dres, es)) || !aligned(workspace, 16))
    return FR_E_ALIGN;
  const int64_t nb = rows * cols * es;
  const Buf bufs[] = {make_buf(h, nb, true, es, false),
                      make_buf(dy, nb, true, es, false),
                      make_buf(dres, nb, true, es, false),
                      make_buf(weight, cols * es, false, es, false),
                      make_buf(dh, nb, true, es, true),
                      make_buf(dweight, cols * 4, false, 4, true),
                      make_buf(workspace, need, false, 1, true)};
  if (fr_status_t s = check_alias(bufs, 7)) return s;
  const bool vec = aligned(h, 16) && aligned(dy, 16) && (!dres || aligned(dres, 16)) &&
                   aligned(weight, 16) && aligned(dh, 16) && (cols * es) % 16 == 0;
  return launch_status(fr::launch_norm_bwd_split(0, dtype == FR_BF16, vec, h, dy, dres, weight,
                                                 nullptr, nullptr, dh, dweight, nullptr, workspace,
                                                 rows, (int)cols, eps,
                                                 norm_bwd_one_pass(rows, cols, dtype), st));
}

fr_status_t fr_layernorm_bwd_split(const void* x, const void* dy, const void* gamma,
                                   const float* mean, const float* rstd, void* dx, float* dgamma,
                                   float* dbeta, void* workspace, int64_t workspace_bytes,
                                   int64_t rows, int64_t cols, fr_dtype_t dtype, void* stream) {
  const int64_t need = fr_norm_bwd_split_workspace_bytes(FR_OP_LAYERNORM_BWD, rows, cols);
  if (need < 0) return FR_E_SHAPE;
  if (!dtype_ok(dtype)) return FR_E_DTYPE;
  if (workspace_bytes < need) return FR_E_SHAPE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (!dgamma || !dbeta) return FR_E_NULL;
  if (!aligned(dgamma, 4) || !aligned(dbeta, 4)) return FR_E_ALIGN;
  if (rows == 0) {
    const Buf pb[] = {make_buf(dgamma, cols * 4, false, 4, true),
                      make_buf(dbeta, cols * 4, false, 4, true)};
    if (fr_status_t s = check_alias(pb, 2)) return s;
    return launch_status(fr::launch_colsum(nullptr, 0, (int)cols, dgamma, dbeta, st));
  }
  if (!x || !dy || !gamma || !mean || !rstd || !dx || !workspace) return FR_E_NULL;
  const int es = esize(dtype);
  if (!aligned(x, es) || !aligned(dy, es) || !aligned(gamma, es) || !aligned(dx, es) ||
      !aligned(mean, 4) || !aligned(rstd, 4) || !aligned(workspace, 16))
    return FR_E_ALIGN;
  const int64_t nb = rows * cols * es;
  const Buf bufs[] = {make_buf(x, nb, true, es, false),
                      make_buf(dy, nb, true, es, false),
                      make_buf(gamma, cols * es, false, es, false),
                      make_buf(mean, rows * 4, false, 4, false),
                      make_buf(rstd, rows * 4, false, 4, false),
                      make_buf(dx, nb, true, es, true),
                      make_buf(dgamma, cols * 4, false, 4, true),
                      make_buf(dbeta, cols * 4, false, 4, true),
                      make_buf(workspace, need, false, 1, true)};
  if (fr_status_t s = check_alias(bufs, 9)) return s;
  const bool vec = aligned(x, 16) && aligned(dy, 16) && aligned(gamma, 16) && aligned(dx, 16) &&
                   (cols * es) % 16 == 0;
  return launch_status(fr::launch_norm_bwd_split(1, dtype == FR_BF16, vec, x, dy, nullptr, gamma,
                                                 mean, rstd, dx, dgamma, dbeta, workspace, rows,
                                                 (int)cols, 0.f, norm_bwd_one_pass(rows, cols, dtype),
                                                 st));
}

fr_status_t fr_layernorm_bwd(const void* x, const void* dy, const void* gamma, const float* mean,
                             const float* rstd, void* dx, float* dgamma, float* dbeta,
                             void* workspace, int64_t workspace_bytes, int64_t rows, int64_t cols,
                             fr_dtype_t dtype, void* stream) {
  if (fr_status_t s = check_shape(rows, cols)) return s;
  if (cols > FR_BWD_MAX_COLS) return FR_E_SHAPE;
  if (!dtype_ok(dtype)) return FR_E_DTYPE;
  const int64_t need = fr_norm_bwd_workspace_bytes(FR_OP_LAYERNORM_BWD, rows, cols);
  if (workspace_bytes < need) return FR_E_SHAPE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (!dgamma || !dbeta) return FR_E_NULL;
  if (!aligned(dgamma, 4) || !aligned(dbeta, 4)) return FR_E_ALIGN;
  if (rows == 0) {
    const Buf pb[] = {make_buf(dgamma, cols * 4, false, 4, true),
                      make_buf(dbeta, cols * 4, false, 4, true)};
    if (fr_status_t s = check_alias(pb, 2)) return s;
    return launch_status(fr::launch_colsum(nullptr, 0, (int)cols, dgamma, dbeta, st));
  }
  if (!x || !dy || !gamma || !mean || !rstd || !dx || !workspace) return FR_E_NULL;
  const int es = esize(dtype);
  if (!aligned(x, es) || !aligned(dy, es) || !aligned(gamma, es) || !aligned(dx, es) ||
      !aligned(mean, 4) || !aligned(rstd, 4) || !aligned(workspace, 16))
    return FR_E_ALIGN;
  const int64_t nb = rows * cols * es;
  const Buf bufs[] = {make_buf(x, nb, true, es, false),
                      make_buf(dy, nb, true, es, false),
                      make_buf(gamma, cols * es, false, es, false),
                      make_buf(mean, rows * 4, false, 4, false),
                      make_buf(rstd, rows * 4, false, 4, false),
                      make_buf(dx, nb, true, es, true),
                      make_buf(dgamma, cols * 4, false, 4, true),
                      make_buf(dbeta, cols * 4, false, 4, true),
                      make_buf(workspace, need, false, 1, true)};
  if (fr_status_t s = check_alias(bufs, 9)) return s;
  const bool vec = aligned(x, 16) && aligned(dy, 16) && aligned(gamma, 16) && aligned(dx, 16) &&
                   (cols * es) % 16 == 0;
  const fr::LayerNormBwdVariant* v = select_variant(fr::layernorm_bwd_variants(dtype == FR_BF16),
                                                    FR_OP_LAYERNORM_BWD, cols, vec ? vec_epv(es) : 1);
  if (!v) return g_forced[FR_OP_LAYERNORM_BWD].threads.load() ? FR_E_VARIANT : FR_E_SHAPE;
  const int grid = fr::bwd_grid(*v, rows);
  float* ws = static_cast<float*>(workspace);
  if (fr_status_t s = launch_status(v->launch(x, dy, gamma, mean, rstd, dx, ws, grid, rows,
                                              (int)cols, st)))
    return s;
  return launch_status(fr::launch_colsum(ws, grid, (int)cols, dgamma, dbeta, st));
}

int64_t fr_split_workspace_bytes(int64_t rows, int64_t cols) {
  if (rows < 0 || cols < 1 || cols > FR_SPLIT_MAX_COLS) return -1;
  if (rows > INT64_MAX / 8 / cols) return -1;
  static_assert(FR_SPLIT_MIN_SEGMENT == fr::kSplitMinSegment, "workspace bound");
  return fr::split_part_bytes(rows, cols);
}

namespace {
// Shared argument checks of the split entry points (rows, cols, workspace).
fr_status_t check_split(int64_t rows, int64_t cols, const void* workspace, int64_t workspace_bytes) {
  if (rows < 0 || cols < 1 || cols > FR_SPLIT_MAX_COLS) return FR_E_SHAPE;
  if (rows > INT64_MAX / 8 / cols) return FR_E_SHAPE;
  if (rows == 0) return FR_OK;
  if (workspace_bytes < fr_split_workspace_bytes(rows, cols)) return FR_E_SHAPE;
  if (!workspace) return FR_E_NULL;
  if (!aligned(workspace, 16)) return FR_E_ALIGN;
  return FR_OK;
}
}  // namespace

fr_status_t fr_softmax_fwd_split(const void* x, void* y, int64_t rows, int64_t cols,
                                 fr_dtype_t x_dtype, fr_dtype_t y_dtype, void* workspace,
                                 int64_t workspace_bytes, void* stream) {
  if (fr_status_t s = check_split(rows, cols, workspace, workspace_bytes)) return s;
  if (!dtype_ok(x_dtype) || !dtype_ok(y_dtype)) return FR_E_DTYPE;
  if (rows == 0) return FR_OK;
  if (!x || !y) return FR_E_NULL;
  const int xs = esize(x_dtype), ys = esize(y_dtype);
  if (!aligned(x, xs) || !aligned(y, ys)) return FR_E_ALIGN;
  const Buf bufs[] = {make_buf(x, rows * cols * xs, true, xs, false),
                      make_buf(y, rows * cols * ys, true, ys, true),
                      make_buf(workspace, fr_split_workspace_bytes(rows, cols), false, 1, true)};
  if (fr_status_t s = check_alias(bufs, 3)) return s;
  const int ve = vec_epv(xs);
  bool vec;
  if (xs == ys) vec = (reinterpret_cast<uintptr_t>(x) % 16) == (reinterpret_cast<uintptr_t>(y) % 16);
  else vec = aligned(x, 16) && aligned(y, 16) && cols % ve == 0;
  const auto c = choose_split(fr::split_variants(x_dtype == FR_BF16, y_dtype == FR_BF16, 0),
                              FR_OP_SOFTMAX_SPLIT, vec ? ve : 1, rows, cols, kOnePassElems);
  if (!c.v) return FR_E_VARIANT;
  return launch_status(c.v->launch(x, y, rows, (int)cols, nullptr, nullptr, nullptr, nullptr,
                                   static_cast<float4*>(workspace),
                                   fr_split_workspace_bytes(rows, cols), c.one_pass,
                                   static_cast<hipStream_t>(stream)));
}

fr_status_t fr_softmax_xent_split(const void* logits, const int32_t* labels, float* loss,
                                  void* grad, int32_t* argmax, float* loss_total, int64_t rows,
                                  int64_t cols, fr_dtype_t dtype, const fr_xent_options_t* options,
                                  void* workspace, int64_t workspace_bytes, void* stream) {
  if (fr_status_t s = check_split(rows, cols, workspace, workspace_bytes)) return s;
  if (!dtype_ok(dtype)) return FR_E_DTYPE;
  fr_xent_options_t o = {0, 0, 0.f, 1.f, FR_REDUCE_NONE};
  if (options) o = *options;
  if (!std::isfinite(o.label_smoothing) || o.label_smoothing < 0.f || o.label_smoothing > 1.f ||
      !std::isfinite(o.grad_scale) ||
      (o.reduction != FR_REDUCE_NONE && o.reduction != FR_REDUCE_SUM &&
       o.reduction != FR_REDUCE_MEAN))
    return FR_E_VALUE;
  if (o.reduction == FR_REDUCE_MEAN && rows > (int64_t)UINT32_MAX) return FR_E_SHAPE;
  const bool reduce = o.reduction != FR_REDUCE_NONE;
  if (reduce && !loss_total) return FR_E_NULL;
  if (loss_total && !aligned(loss_total, 4)) return FR_E_ALIGN;
  hipStream_t st = static_cast<hipStream_t>(stream);
  uint32_t* count = o.reduction == FR_REDUCE_MEAN ? reinterpret_cast<uint32_t*>(loss_total) : nullptr;
  if (rows == 0) {
    if (!reduce) return FR_OK;
    if (count)
      if (fr_status_t s = launch_status(fr::launch_xent_count(labels, 0, 0, 0, count, st))) return s;
    return launch_status(fr::launch_xent_total(loss, 0, count, loss_total, st));
  }
  if (!logits || !labels || !loss || !grad) return FR_E_NULL;
  const int es = esize(dtype);
  if (!aligned(logits, es) || !aligned(grad, es) || !aligned(labels, 4) || !aligned(loss, 4) ||
      (argmax && !aligned(argmax, 4)))
    return FR_E_ALIGN;
  const Buf bufs[] = {make_buf(logits, rows * cols * es, true, es, false),
                      make_buf(labels, rows * 4, false, 4, false),
                      make_buf(loss, rows * 4, false, 4, true),
                      make_buf(grad, rows * cols * es, true, es, true),
                      make_buf(argmax, rows * 4, false, 4, true),
                      make_buf(reduce ? loss_total : nullptr, 4, false, 4, true),
                      make_buf(workspace, fr_split_workspace_bytes(rows, cols), false, 1, true)};
  if (fr_status_t s = check_alias(bufs, 7)) return s;
  const bool vec =
      (reinterpret_cast<uintptr_t>(logits) % 16) == (reinterpret_cast<uintptr_t>(grad) % 16);
  const auto c = choose_split(fr::split_variants(dtype == FR_BF16, dtype == FR_BF16, 1),
                              FR_OP_XENT_SPLIT, vec ? vec_epv(es) : 1, rows, cols, kOnePassElems);
  if (!c.v) return FR_E_VARIANT;
  if (count)
    if (fr_status_t s = launch_status(
            fr::launch_xent_count(labels, rows, o.use_ignore_index != 0, o.ignore_index, count, st)))
      return s;
  const fr::XentOptions ko = {o.use_ignore_index != 0, o.ignore_index, o.label_smoothing,
                              o.grad_scale, count, 0, 0, nullptr, nullptr};
  if (fr_status_t s = launch_status(c.v->launch(logits, grad, rows, (int)cols, labels, loss, argmax,
                                                &ko, static_cast<float4*>(workspace),
                                                fr_split_workspace_bytes(rows, cols), c.one_pass,
                                                st)))
    return s;
  if (!reduce) return FR_OK;
  return launch_status(fr::launch_xent_total(loss, rows, count, loss_total, st));
}

fr_status_t fr_layernorm_fwd_split(const void* x, const void* gamma, const void* beta, void* y,
                                   float* mean, float* rstd, int64_t rows, int64_t cols, float eps,
                                   fr_dtype_t dtype, void* workspace, int64_t workspace_bytes,
                                   void* stream) {
  if (fr_status_t s = check_split(rows, cols, workspace, workspace_bytes)) return s;
  if (!dtype_ok(dtype)) return FR_E_DTYPE;
  if (!std::isfinite(eps) || eps < 0.f) return FR_E_VALUE;
  if (rows == 0) return FR_OK;
  if (!x || !gamma || !beta || !y) return FR_E_NULL;
  const int es = esize(dtype);
  if (!aligned(x, es) || !aligned(y, es) || !aligned(gamma, es) || !aligned(beta, es) ||
      (mean && !aligned(mean, 4)) || (rstd && !aligned(rstd, 4)))
    return FR_E_ALIGN;
  const Buf bufs[] = {make_buf(x, rows * cols * es, true, es, false),
                      make_buf(gamma, cols * es, false, es, false),
                      make_buf(beta, cols * es, false, es, false),
                      make_buf(y, rows * cols * es, true, es, true),
                      make_buf(mean, rows * 4, false, 4, true),
                      make_buf(rstd, rows * 4, false, 4, true),
                      make_buf(workspace, fr_split_workspace_bytes(rows, cols), false, 1, true)};
  if (fr_status_t s = check_alias(bufs, 7)) return s;
  const bool vec = aligned(x, 16) && aligned(y, 16) && aligned(gamma, 16) && aligned(beta, 16) &&
                   (cols * es) % 16 == 0;
  const auto c = choose_split(fr::norm_split_variants(dtype == FR_BF16, 0), FR_OP_LAYERNORM_SPLIT,
                              vec ? vec_epv(es) : 1, rows, cols, one_pass_elems_ln(dtype));
  if (!c.v) return FR_E_VARIANT;
  return launch_status(c.v->launch(x, nullptr, gamma, beta, y, nullptr, mean, rstd, rows, (int)cols,
                                   eps, static_cast<float4*>(workspace),
                                   fr_split_workspace_bytes(rows, cols), c.one_pass,
                                   static_cast<hipStream_t>(stream)));
}

fr_status_t fr_add_rmsnorm_fwd_split(const void* x, const void* residual, const void* weight,
                                     void* y, void* residual_out, int64_t rows, int64_t cols,
                                     float eps, fr_dtype_t dtype, void* workspace,
                                     int64_t workspace_bytes, void* stream) {
  if (fr_status_t s = check_split(rows, cols, workspace, workspace_bytes)) return s;
  if (!dtype_ok(dtype)) return FR_E_DTYPE;
  if (!std::isfinite(eps) || eps < 0.f) return FR_E_VALUE;
  if (rows == 0) return FR_OK;
  if (!x || !residual || !weight || !y) return FR_E_NULL;
  const int es = esize(dtype);
  if (!aligned(x, es) || !aligned(residual, es) || !aligned(weight, es) || !aligned(y, es) ||
      (residual_out && !aligned(residual_out, es)))
    return FR_E_ALIGN;
  const Buf bufs[] = {make_buf(x, rows * cols * es, true, es, false),
                      make_buf(residual, rows * cols * es, true, es, false),
                      make_buf(weight, cols * es, false, es, false),
                      make_buf(y, rows * cols * es, true, es, true),
                      make_buf(residual_out, rows * cols * es, true, es, true),
                      make_buf(workspace, fr_split_workspace_bytes(rows, cols), false, 1, true)};
  if (fr_status_t s = check_alias(bufs, 6)) return s;
  const bool vec = aligned(x, 16) && aligned(residual, 16) && aligned(weight, 16) &&
                   aligned(y, 16) && (!residual_out || aligned(residual_out, 16)) &&
                   (cols * es) % 16 == 0;
  const auto c = choose_split(fr::norm_split_variants(dtype == FR_BF16, 1), FR_OP_RMSNORM_SPLIT,
                              vec ? vec_epv(es) : 1, rows, cols, kOnePassElems);
  if (!c.v) return FR_E_VARIANT;
  return launch_status(c.v->launch(x, residual, weight, nullptr, y, residual_out, nullptr, nullptr,
                                   rows, (int)cols, eps, static_cast<float4*>(workspace),
                                   fr_split_workspace_bytes(rows, cols), c.one_pass,
                                   static_cast<hipStream_t>(stream)));
}

fr_status_t fr_softmax_bwd_split(const void* p, const void* dy, void* dx, int64_t rows,
                                 int64_t cols, fr_dtype_t dtype, void* workspace,
                                 int64_t workspace_bytes, void* stream) {
  if (fr_status_t s = check_split(rows, cols, workspace, workspace_bytes)) return s;
  if (!dtype_ok(dtype)) return FR_E_DTYPE;
  if (rows == 0) return FR_OK;
  if (!p || !dy || !dx) return FR_E_NULL;
  const int es = esize(dtype);
  if (!aligned(p, es) || !aligned(dy, es) || !aligned(dx, es)) return FR_E_ALIGN;
  const int64_t nb = rows * cols * es;
  const Buf bufs[] = {make_buf(p, nb, true, es, false), make_buf(dy, nb, true, es, false),
                      make_buf(dx, nb, true, es, true),
                      make_buf(workspace, fr_split_workspace_bytes(rows, cols), false, 1, true)};
  if (fr_status_t s = check_alias(bufs, 4)) return s;
  const uintptr_t ph = reinterpret_cast<uintptr_t>(p) % 16;
  const bool vec = reinterpret_cast<uintptr_t>(dy) % 16 == ph &&
                   reinterpret_cast<uintptr_t>(dx) % 16 == ph;
  const auto c = choose_split(fr::softmax_bwd_split_variants(dtype == FR_BF16),
                              FR_OP_SOFTMAX_BWD_SPLIT, vec ? vec_epv(es) : 1, rows, cols,
                              kOnePassElems);
  if (!c.v) return FR_E_VARIANT;
  return launch_status(c.v->launch(p, dy, dx, rows, (int)cols, static_cast<float4*>(workspace),
                                   fr_split_workspace_bytes(rows, cols), c.one_pass,
                                   static_cast<hipStream_t>(stream)));
}

fr_status_t fr_attention_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                             int64_t batch, int64_t heads, int64_t seq_q, int64_t seq_k,
                             int64_t head_dim, int causal, float scale, fr_dtype_t dtype,
                             void* stream) {
  if (batch < 0 || heads < 0 || seq_q < 0 || seq_k < 0) return FR_E_SHAPE;
  if (head_dim != 64 && head_dim != 128) return FR_E_SHAPE;
  if (seq_q > INT32_MAX / 2 || seq_k > INT32_MAX / 2) return FR_E_SHAPE;
  if (heads > 0 && batch > INT64_MAX / heads) return FR_E_SHAPE;  // before the product
  const int64_t bh = batch * heads;
  if (bh > 65535 || bh * ((seq_q + 127) / 128) > INT32_MAX) return FR_E_SHAPE;
  if (dtype != FR_BF16) return FR_E_DTYPE;
  if (!std::isfinite(scale)) return FR_E_VALUE;
  if (bh == 0 || seq_q == 0) return FR_OK;
  if (!q || !o || (seq_k > 0 && (!k || !v))) return FR_E_NULL;
  if (!aligned(q, 16) || !aligned(o, 16) || (k && !aligned(k, 16)) || (v && !aligned(v, 16)) ||
      (lse && !aligned(lse, 4)))
    return FR_E_ALIGN;
  const int64_t qbytes = bh * seq_q * head_dim * 2, kbytes = bh * seq_k * head_dim * 2;
  // o may be exactly q (each workgroup reads its own queries before writing
  // them); it may not overlap k or v, which every workgroup of a head reads
  const Buf bufs[] = {make_buf(q, qbytes, true, 2, false),
                      make_buf(seq_k > 0 ? k : nullptr, kbytes, false, 2, false),
                      make_buf(seq_k > 0 ? v : nullptr, kbytes, false, 2, false),
                      make_buf(o, qbytes, true, 2, true),
                      make_buf(lse, bh * seq_q * 4, false, 4, true)};
  if (fr_status_t s = check_alias(bufs, 5)) return s;
  return launch_status(fr::launch_attention_fwd(q, k, v, o, lse, bh, (int)seq_q, (int)seq_k,
                                                (int)head_dim, causal ? 1 : 0, scale,
                                                static_cast<hipStream_t>(stream)));
}

fr_status_t fr_stream_copy(const void* src, void* dst, int64_t bytes, void* stream) {
  if (bytes < 0) return FR_E_SHAPE;
  if (bytes == 0) return FR_OK;
  if (!src || !dst) return FR_E_NULL;
  const Buf bufs[] = {make_buf(src, bytes, false, 1, false), make_buf(dst, bytes, false, 1, true)};
  if (fr_status_t s = check_alias(bufs, 2)) return s;
  return launch_status(fr::launch_stream_copy(src, dst, bytes, static_cast<hipStream_t>(stream)));
}

int64_t fr_stream_probe_rows(int64_t bytes, int64_t row_bytes) {
  if (bytes < 0 || row_bytes < 16 || row_bytes % 16 != 0) return -1;
  return fr::stream_probe_rows(bytes, row_bytes);
}

fr_status_t fr_stream_probe(fr_probe_t kind, const void* src, void* dst, int64_t bytes,
                            int64_t row_bytes, uint32_t value, uint32_t* sink, int threads,
                            int vecs, int policy, void* stream) {
  if (kind != FR_PROBE_READ && kind != FR_PROBE_WRITE && kind != FR_PROBE_COPY) return FR_E_VALUE;
  if (!fr::stream_probe_shape_exists(threads, vecs)) return FR_E_VARIANT;
  if (policy < 0 || policy > (FR_PROBE_NT_LOADS | FR_PROBE_NT_STORES)) return FR_E_VALUE;
  if (bytes < 0 || bytes % 16 != 0) return FR_E_SHAPE;
  if (row_bytes == 0) row_bytes = (int64_t)threads * vecs * 16;
  if (row_bytes < 16 || row_bytes % 16 != 0 || row_bytes > (int64_t)threads * vecs * 16)
    return FR_E_SHAPE;
  if (bytes == 0) return FR_OK;
  const bool reads = kind != FR_PROBE_WRITE, writes = kind != FR_PROBE_READ;
  if ((reads && !src) || (writes && !dst) || (kind == FR_PROBE_READ && !sink)) return FR_E_NULL;
  if ((reads && !aligned(src, 16)) || (writes && !aligned(dst, 16)) ||
      (kind == FR_PROBE_READ && !aligned(sink, 4)))
    return FR_E_ALIGN;
  const int64_t rows = fr::stream_probe_rows(bytes, row_bytes);
  const Buf bufs[] = {make_buf(reads ? src : nullptr, bytes, false, 1, false),
                      make_buf(writes ? dst : nullptr, bytes, false, 1, true),
                      make_buf(kind == FR_PROBE_READ ? sink : nullptr, rows * 4, false, 4, true)};
  if (fr_status_t s = check_alias(bufs, 3)) return s;
  return launch_status(fr::launch_stream_probe((int)kind, reads ? src : nullptr,
                                               writes ? dst : nullptr, bytes, row_bytes, threads,
                                               vecs, policy, value,
                                               kind == FR_PROBE_READ ? sink : nullptr,
                                               static_cast<hipStream_t>(stream)));
}

fr_status_t fr_stream_read(const void* src, int64_t bytes, uint32_t* sink, void* stream) {
  return fr_stream_probe(FR_PROBE_READ, src, nullptr, bytes, 0, 0, sink, FR_STREAM_THREADS,
                         FR_STREAM_VECS, FR_STREAM_POLICY, stream);
}

fr_status_t fr_mfma_probe(int workgroups, int iters, int pattern, float* sink, void* stream) {
  if (workgroups < 1 || workgroups > (1 << 20) || iters < 1 || iters > (1 << 19)) return FR_E_SHAPE;
  if (pattern != 0 && pattern != 1) return FR_E_VALUE;
  if (!sink) return FR_E_NULL;
  if (!aligned(sink, 4)) return FR_E_ALIGN;
  return launch_status(
      fr::launch_mfma_probe(workgroups, iters, pattern, sink, static_cast<hipStream_t>(stream)));
}

fr_status_t fr_stream_write(void* dst, int64_t bytes, uint32_t value, void* stream) {
  return fr_stream_probe(FR_PROBE_WRITE, nullptr, dst, bytes, 0, value, nullptr,
                         FR_STREAM_THREADS, FR_STREAM_VECS, FR_STREAM_POLICY, stream);
}

}  // extern "C"
