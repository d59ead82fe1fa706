"""Python binding of libfusedrow (fused single-pass row kernels for MI355X).

Argument marshalling only: every step of every operation runs in the HIP
kernels behind the C ABI declared in include/fusedrow.h. torch supplies the
device memory (caller-visible tensors) and the current stream; nothing here
computes on tensor values. There is no fallback: if libfusedrow.so is missing
or a call fails, an exception is raised.

The fr_* functions mirror the C entry points one to one and take torch CUDA
tensors; softmax / layernorm / add_rmsnorm / softmax_xent and the *_bwd
conveniences allocate the outputs (and the backward workspace) and call them.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "F32", "BF16", "FR_MAX_COLS", "FusedRowError", "lib", "status_str", "version",
    "fr_softmax_fwd", "fr_layernorm_fwd", "fr_add_rmsnorm_fwd", "fr_softmax_xent_fwd_bwd",
    "fr_stream_copy", "fr_stream_read", "fr_stream_write", "fr_stream_probe", "fr_mfma_probe",
    "fr_stream_probe_rows", "PROBE_READ", "PROBE_WRITE", "PROBE_COPY", "PROBE_NT_LOADS",
    "PROBE_NT_STORES", "fr_debug_force_variant", "fr_debug_select_variant",
    "fr_debug_select_variant_for",
    "fr_debug_set_split_batch_bytes", "split_batch_bytes", "fr_debug_set_split_one_pass",
    "split_one_pass", "fr_debug_set_coop_spin_limit", "coop_spin_limit",
    "fr_softmax_bwd", "fr_add_rmsnorm_bwd", "fr_layernorm_bwd", "fr_norm_bwd_workspace_bytes",
    "fr_add_rmsnorm_bwd_noalloc", "FR_NOALLOC_SCRATCH_BYTES",
    "fr_softmax_xent_ex", "XentOptions", "REDUCE_NONE", "REDUCE_SUM", "REDUCE_MEAN",
    "fr_softmax_fwd_split", "fr_softmax_xent_split", "fr_split_workspace_bytes",
    "OP_SOFTMAX_SPLIT", "OP_XENT_SPLIT", "FR_SPLIT_MAX_COLS", "fr_attention_fwd", "attention",
    "fr_layernorm_fwd_split", "fr_add_rmsnorm_fwd_split", "OP_LAYERNORM_SPLIT", "OP_RMSNORM_SPLIT",
    "fr_softmax_bwd_split", "OP_SOFTMAX_BWD_SPLIT", "fr_add_rmsnorm_bwd_split",
    "fr_layernorm_bwd_split", "fr_norm_bwd_split_workspace_bytes",
    "softmax", "layernorm", "add_rmsnorm", "softmax_xent", "forced_variant",
    "softmax_bwd", "add_rmsnorm_bwd", "layernorm_bwd",
    "OP_SOFTMAX", "OP_LAYERNORM", "OP_RMSNORM", "OP_XENT",
    "OP_SOFTMAX_BWD", "OP_RMSNORM_BWD", "OP_LAYERNORM_BWD", "FR_BWD_MAX_COLS", "FR_BWD_PARTIALS",
]

F32, BF16 = 0, 1
OP_SOFTMAX, OP_LAYERNORM, OP_RMSNORM, OP_XENT = 0, 1, 2, 3
OP_SOFTMAX_BWD, OP_RMSNORM_BWD, OP_LAYERNORM_BWD = 4, 5, 6
OP_SOFTMAX_SPLIT, OP_XENT_SPLIT = 7, 8
OP_LAYERNORM_SPLIT, OP_RMSNORM_SPLIT, OP_SOFTMAX_BWD_SPLIT = 9, 10, 11
FR_SPLIT_MAX_COLS = 1 << 24
FR_MAX_COLS = 65536
FR_BWD_MAX_COLS = 16384
FR_BWD_PARTIALS = 512
REDUCE_NONE, REDUCE_SUM, REDUCE_MEAN = 0, 1, 2
_REDUCTIONS = {"none": REDUCE_NONE, "sum": REDUCE_SUM, "mean": REDUCE_MEAN}


class XentOptions(ctypes.Structure):
    """fr_xent_options_t."""
    _fields_ = [("use_ignore_index", ctypes.c_int32), ("ignore_index", ctypes.c_int32),
                ("label_smoothing", ctypes.c_float), ("grad_scale", ctypes.c_float),
                ("reduction", ctypes.c_int32)]
# FUSEDROW_LIB may name an alternative build of the same library (A/B runs).
LIB_PATH = os.environ.get("FUSEDROW_LIB") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libfusedrow.so")


class FusedRowError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        extra = ""
        if status == 5:  # FR_E_LAUNCH: name the HIP error
            extra = f", hipError_t {lib.fr_debug_last_launch_error()}"
        super().__init__(f"{where}: {status_str(status)} (status {status}{extra})")


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run __graft_entry__.build() or "
            "python memory_bound_row_pass_amd/_build.py (hipcc, gfx950)")
    # torch bundles its own HIP runtime (same SONAME as /opt/rocm's). Loading
    # torch first makes libfusedrow bind to that one runtime; loading the
    # library first would put a second runtime in the process, which then
    # reports no device to whichever side did not initialise it.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    L = ctypes.CDLL(LIB_PATH)
    P, I64, I32, F = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
    IP = ctypes.POINTER(ctypes.c_int)
    sig = {
        "fr_softmax_fwd": [P, P, I64, I64, I32, I32, P],
        "fr_layernorm_fwd": [P, P, P, P, P, P, I64, I64, F, I32, P],
        "fr_add_rmsnorm_fwd": [P, P, P, P, P, I64, I64, F, I32, P],
        "fr_softmax_xent_fwd_bwd": [P, P, P, P, P, I64, I64, P],
        "fr_stream_copy": [P, P, I64, P],
        "fr_stream_read": [P, I64, P, P],
        "fr_stream_write": [P, I64, ctypes.c_uint32, P],
        "fr_mfma_probe": [I32, I32, I32, P, P],
        "fr_stream_probe": [I32, P, P, I64, I64, ctypes.c_uint32, P, I32, I32, I32, P],
        "fr_softmax_bwd": [P, P, P, I64, I64, I32, P],
        "fr_softmax_xent_ex": [P, P, P, P, P, P, I64, I64, I32, ctypes.POINTER(XentOptions), P],
        "fr_softmax_fwd_split": [P, P, I64, I64, I32, I32, P, I64, P],
        "fr_layernorm_fwd_split": [P, P, P, P, P, P, I64, I64, F, I32, P, I64, P],
        "fr_add_rmsnorm_fwd_split": [P, P, P, P, P, I64, I64, F, I32, P, I64, P],
        "fr_softmax_bwd_split": [P, P, P, I64, I64, I32, P, I64, P],
        "fr_add_rmsnorm_bwd_split": [P, P, P, P, P, P, P, I64, I64, I64, F, I32, P],
        "fr_layernorm_bwd_split": [P, P, P, P, P, P, P, P, P, I64, I64, I64, I32, P],
        "fr_attention_fwd": [P, P, P, P, P, I64, I64, I64, I64, I64, I32, F, I32, P],
        "fr_softmax_xent_split": [P, P, P, P, P, P, I64, I64, I32, ctypes.POINTER(XentOptions), P,
                                  I64, P],
        "fr_add_rmsnorm_bwd": [P, P, P, P, P, P, P, I64, I64, I64, F, I32, P],
        "fr_layernorm_bwd": [P, P, P, P, P, P, P, P, P, I64, I64, I64, I32, P],
        "fr_add_rmsnorm_bwd_noalloc": [P, P, P, P, P, P, I64, I64, F, I32, P],
        "fr_debug_force_variant": [I32, I32, I32],
        "fr_debug_select_variant": [I32, I64, I32, I32, I32, IP, IP, IP],
        "fr_debug_select_variant_for": [I32, I64, I64, I32, I32, I32, IP, IP, IP],
    }
    for name, args in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    L.fr_stream_probe_rows.argtypes = [I64, I64]
    L.fr_stream_probe_rows.restype = ctypes.c_int64
    L.fr_split_workspace_bytes.argtypes = [I64, I64]
    L.fr_split_workspace_bytes.restype = ctypes.c_int64
    L.fr_norm_bwd_workspace_bytes.argtypes = [I32, I64, I64]
    L.fr_norm_bwd_workspace_bytes.restype = ctypes.c_int64
    L.fr_norm_bwd_split_workspace_bytes.argtypes = [I32, I64, I64]
    L.fr_norm_bwd_split_workspace_bytes.restype = ctypes.c_int64
    L.fr_status_str.argtypes = [ctypes.c_int]
    L.fr_status_str.restype = ctypes.c_char_p
    L.fr_version.argtypes = []
    L.fr_version.restype = ctypes.c_char_p
    L.fr_debug_set_split_batch_bytes.argtypes = [I64]
    L.fr_debug_set_split_batch_bytes.restype = ctypes.c_int64
    L.fr_debug_set_split_one_pass.argtypes = [ctypes.c_int]
    L.fr_debug_set_split_one_pass.restype = ctypes.c_int
    L.fr_debug_set_coop_spin_limit.argtypes = [ctypes.c_int]
    L.fr_debug_set_coop_spin_limit.restype = ctypes.c_int
    L.fr_debug_last_launch_error.argtypes = []
    L.fr_debug_last_launch_error.restype = ctypes.c_int
    return L


lib = _load()


def status_str(s: int) -> str:
    return lib.fr_status_str(int(s)).decode()


def version() -> str:
    return lib.fr_version().decode()


def _check(status: int, where: str) -> None:
    if status != 0:
        raise FusedRowError(status, where)


# ------------------------------------------------------------- marshalling

def _torch():
    import torch  # imported lazily: the ABI can be loaded without torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t.dtype}; fusedrow takes float32 or bfloat16")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _rows_cols(t):
    if t.dim() != 2:
        raise ValueError(f"expected a 2-D [rows, cols] tensor, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError("row buffers must be contiguous (row-major)")
    return int(t.shape[0]), int(t.shape[1])


def _stream(stream, t):
    if stream is not None:
        return ctypes.c_void_p(int(stream))
    torch = _torch()
    if t is not None and t.is_cuda:
        return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)
    return ctypes.c_void_p(0)


def _need_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("fusedrow operates on device (CUDA/HIP) tensors only")


def _check_vec(t, cols, name):
    if t.dim() != 1 or int(t.shape[0]) != cols or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous [cols] vector")


def _check_rows(t, rows, name, dtype):
    if t.dim() != 1 or int(t.shape[0]) != rows or not t.is_contiguous() or t.dtype != dtype:
        raise ValueError(f"{name} must be a contiguous [rows] {dtype} vector")


# ------------------------------------------------------- C entry points

def fr_softmax_fwd(x, y, stream=None) -> None:
    """y = softmax(x) over each row (C: fr_softmax_fwd)."""
    _need_cuda(x, y)
    R, C = _rows_cols(x)
    if tuple(y.shape) != (R, C) or not y.is_contiguous():
        raise ValueError("y must be a contiguous tensor of x's shape")
    _check(lib.fr_softmax_fwd(_ptr(x), _ptr(y), R, C, _dtype_code(x), _dtype_code(y),
                              _stream(stream, x)), "fr_softmax_fwd")


def fr_layernorm_fwd(x, gamma, beta, y, mean=None, rstd=None, eps: float = 1e-5, stream=None) -> None:
    """LayerNorm of each row (C: fr_layernorm_fwd); mean/rstd optional fp32 [rows]."""
    torch = _torch()
    _need_cuda(x, gamma, beta, y, mean, rstd)
    R, C = _rows_cols(x)
    _check_vec(gamma, C, "gamma")
    _check_vec(beta, C, "beta")
    if tuple(y.shape) != (R, C) or not y.is_contiguous() or y.dtype != x.dtype:
        raise ValueError("y must be a contiguous tensor of x's shape and dtype")
    if gamma.dtype != x.dtype or beta.dtype != x.dtype:
        raise TypeError("gamma and beta must have x's dtype")
    for t, n in ((mean, "mean"), (rstd, "rstd")):
        if t is not None:
            _check_rows(t, R, n, torch.float32)
    _check(lib.fr_layernorm_fwd(_ptr(x), _ptr(gamma), _ptr(beta), _ptr(y), _ptr(mean), _ptr(rstd),
                                R, C, float(eps), _dtype_code(x), _stream(stream, x)),
           "fr_layernorm_fwd")


def fr_add_rmsnorm_fwd(x, residual, weight, y, residual_out=None, eps: float = 1e-6,
                       stream=None) -> None:
    """h = x + residual; residual_out = h; y = RMSNorm(h) * weight (C: fr_add_rmsnorm_fwd)."""
    _need_cuda(x, residual, weight, y, residual_out)
    R, C = _rows_cols(x)
    for t, n in ((residual, "residual"), (y, "y"), (residual_out, "residual_out")):
        if t is not None and (tuple(t.shape) != (R, C) or not t.is_contiguous() or t.dtype != x.dtype):
            raise ValueError(f"{n} must be a contiguous tensor of x's shape and dtype")
    _check_vec(weight, C, "weight")
    if weight.dtype != x.dtype:
        raise TypeError("weight must have x's dtype")
    _check(lib.fr_add_rmsnorm_fwd(_ptr(x), _ptr(residual), _ptr(weight), _ptr(y), _ptr(residual_out),
                                  R, C, float(eps), _dtype_code(x), _stream(stream, x)),
           "fr_add_rmsnorm_fwd")


def fr_softmax_xent_fwd_bwd(logits, labels, loss, grad, argmax=None, stream=None) -> None:
    """Per-row cross-entropy loss and its gradient (C: fr_softmax_xent_fwd_bwd)."""
    torch = _torch()
    _need_cuda(logits, labels, loss, grad, argmax)
    R, C = _rows_cols(logits)
    _check_rows(labels, R, "labels", torch.int32)
    _check_rows(loss, R, "loss", torch.float32)
    if argmax is not None:
        _check_rows(argmax, R, "argmax", torch.int32)
    if logits.dtype != torch.float32:
        raise TypeError("fr_softmax_xent_fwd_bwd takes float32 logits "
                        "(bf16 logits: fr_softmax_xent_ex)")
    if tuple(grad.shape) != (R, C) or not grad.is_contiguous() or grad.dtype != logits.dtype:
        raise ValueError("grad must be a contiguous tensor of logits' shape and dtype")
    _check(lib.fr_softmax_xent_fwd_bwd(_ptr(logits), _ptr(labels), _ptr(loss), _ptr(grad),
                                       _ptr(argmax), R, C, _stream(stream, logits)),
           "fr_softmax_xent_fwd_bwd")


def fr_softmax_xent_ex(logits, labels, loss, grad, argmax=None, loss_total=None,
                       ignore_index=None, label_smoothing: float = 0.0, grad_scale: float = 1.0,
                       reduction: str = "none", stream=None) -> None:
    """Cross-entropy with ignore_index / label smoothing / reduction / gradient
    scale (C: fr_softmax_xent_ex); fp32 or bf16 logits, grad in their dtype."""
    torch = _torch()
    _need_cuda(logits, labels, loss, grad, argmax, loss_total)
    R, C = _rows_cols(logits)
    _check_rows(labels, R, "labels", torch.int32)
    _check_rows(loss, R, "loss", torch.float32)
    if argmax is not None:
        _check_rows(argmax, R, "argmax", torch.int32)
    if loss_total is not None and (loss_total.numel() < 1 or loss_total.dtype != torch.float32):
        raise ValueError("loss_total must be a float32 tensor of at least one element")
    if tuple(grad.shape) != (R, C) or not grad.is_contiguous() or grad.dtype != logits.dtype:
        raise ValueError("grad must be a contiguous tensor of logits' shape and dtype")
    opts = XentOptions(int(ignore_index is not None), int(ignore_index or 0), float(label_smoothing),
                       float(grad_scale), _REDUCTIONS[reduction])
    _check(lib.fr_softmax_xent_ex(_ptr(logits), _ptr(labels), _ptr(loss), _ptr(grad), _ptr(argmax),
                                  _ptr(loss_total), R, C, _dtype_code(logits), ctypes.byref(opts),
                                  _stream(stream, logits)),
           "fr_softmax_xent_ex")


def fr_split_workspace_bytes(rows: int, cols: int) -> int:
    """Workspace bytes of the split-row entry points (C: same name)."""
    n = int(lib.fr_split_workspace_bytes(int(rows), int(cols)))
    if n < 0:
        raise ValueError(f"no split workspace size for [{rows}, {cols}]")
    return n


def fr_softmax_fwd_split(x, y, workspace, stream=None) -> None:
    """Row softmax of any width, several workgroups per row (C: fr_softmax_fwd_split)."""
    _need_cuda(x, y)
    R, C = _rows_cols(x)
    if tuple(y.shape) != (R, C) or not y.is_contiguous():
        raise ValueError("y must be a contiguous tensor of x's shape")
    wp, wn = _workspace_arg(workspace)
    _check(lib.fr_softmax_fwd_split(_ptr(x), _ptr(y), R, C, _dtype_code(x), _dtype_code(y), wp, wn,
                                    _stream(stream, x)), "fr_softmax_fwd_split")


def fr_layernorm_fwd_split(x, gamma, beta, y, workspace, mean=None, rstd=None, eps: float = 1e-5,
                           stream=None) -> None:
    """LayerNorm of rows of any width, several workgroups per row
    (C: fr_layernorm_fwd_split); arguments as fr_layernorm_fwd plus the
    workspace."""
    torch = _torch()
    _need_cuda(x, gamma, beta, y, mean, rstd)
    R, C = _rows_cols(x)
    _check_vec(gamma, C, "gamma")
    _check_vec(beta, C, "beta")
    if tuple(y.shape) != (R, C) or not y.is_contiguous() or y.dtype != x.dtype:
        raise ValueError("y must be a contiguous tensor of x's shape and dtype")
    if gamma.dtype != x.dtype or beta.dtype != x.dtype:
        raise TypeError("gamma and beta must have x's dtype")
    for t, n in ((mean, "mean"), (rstd, "rstd")):
        if t is not None:
            _check_rows(t, R, n, torch.float32)
    wp, wn = _workspace_arg(workspace)
    _check(lib.fr_layernorm_fwd_split(_ptr(x), _ptr(gamma), _ptr(beta), _ptr(y), _ptr(mean),
                                      _ptr(rstd), R, C, float(eps), _dtype_code(x), wp, wn,
                                      _stream(stream, x)), "fr_layernorm_fwd_split")


def fr_add_rmsnorm_fwd_split(x, residual, weight, y, workspace, residual_out=None,
                             eps: float = 1e-6, stream=None) -> None:
    """Residual add + RMSNorm of rows of any width, several workgroups per row
    (C: fr_add_rmsnorm_fwd_split); arguments as fr_add_rmsnorm_fwd plus the
    workspace."""
    _need_cuda(x, residual, weight, y, residual_out)
    R, C = _rows_cols(x)
    for t, n in ((residual, "residual"), (y, "y"), (residual_out, "residual_out")):
        if t is not None and (tuple(t.shape) != (R, C) or not t.is_contiguous() or t.dtype != x.dtype):
            raise ValueError(f"{n} must be a contiguous tensor of x's shape and dtype")
    _check_vec(weight, C, "weight")
    if weight.dtype != x.dtype:
        raise TypeError("weight must have x's dtype")
    wp, wn = _workspace_arg(workspace)
    _check(lib.fr_add_rmsnorm_fwd_split(_ptr(x), _ptr(residual), _ptr(weight), _ptr(y),
                                        _ptr(residual_out), R, C, float(eps), _dtype_code(x), wp, wn,
                                        _stream(stream, x)), "fr_add_rmsnorm_fwd_split")


def fr_softmax_bwd_split(p, dy, dx, workspace, stream=None) -> None:
    """Softmax backward for rows of any width, several workgroups per row
    (C: fr_softmax_bwd_split)."""
    _need_cuda(p, dy, dx)
    R, C = _rows_cols(p)
    for t, n in ((dy, "dy"), (dx, "dx")):
        if tuple(t.shape) != (R, C) or not t.is_contiguous() or t.dtype != p.dtype:
            raise ValueError(f"{n} must be a contiguous tensor of p's shape and dtype")
    wp, wn = _workspace_arg(workspace)
    _check(lib.fr_softmax_bwd_split(_ptr(p), _ptr(dy), _ptr(dx), R, C, _dtype_code(p), wp, wn,
                                    _stream(stream, p)), "fr_softmax_bwd_split")


def fr_softmax_xent_split(logits, labels, loss, grad, workspace, argmax=None, loss_total=None,
                          ignore_index=None, label_smoothing: float = 0.0, grad_scale: float = 1.0,
                          reduction: str = "none", stream=None) -> None:
    """Cross-entropy with options for rows of any width (C: fr_softmax_xent_split)."""
    torch = _torch()
    _need_cuda(logits, labels, loss, grad, argmax, loss_total)
    R, C = _rows_cols(logits)
    _check_rows(labels, R, "labels", torch.int32)
    _check_rows(loss, R, "loss", torch.float32)
    if argmax is not None:
        _check_rows(argmax, R, "argmax", torch.int32)
    if loss_total is not None and (loss_total.numel() < 1 or loss_total.dtype != torch.float32):
        raise ValueError("loss_total must be a float32 tensor of at least one element")
    if tuple(grad.shape) != (R, C) or not grad.is_contiguous() or grad.dtype != logits.dtype:
        raise ValueError("grad must be a contiguous tensor of logits' shape and dtype")
    opts = XentOptions(int(ignore_index is not None), int(ignore_index or 0), float(label_smoothing),
                       float(grad_scale), _REDUCTIONS[reduction])
    wp, wn = _workspace_arg(workspace)
    _check(lib.fr_softmax_xent_split(_ptr(logits), _ptr(labels), _ptr(loss), _ptr(grad),
                                     _ptr(argmax), _ptr(loss_total), R, C, _dtype_code(logits),
                                     ctypes.byref(opts), wp, wn, _stream(stream, logits)),
           "fr_softmax_xent_split")


def _split_workspace(R, C, device):
    torch = _torch()
    return torch.empty(max(fr_split_workspace_bytes(R, C), 16), dtype=torch.uint8, device=device)


def fr_attention_fwd(q, k, v, o, lse=None, causal: bool = False, scale=None, stream=None) -> None:
    """Attention forward with the online softmax fused in (C: fr_attention_fwd).
    q, o [B, H, Sq, D], k, v [B, H, Sk, D] bf16; lse [B, H, Sq] fp32 or None."""
    torch = _torch()
    _need_cuda(q, k, v, o, lse)
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o")):
        if t.dim() != 4 or not t.is_contiguous() or t.dtype != torch.bfloat16:
            raise ValueError(f"{n} must be a contiguous 4-D bfloat16 tensor")
    B, H, Sq, D = (int(x) for x in q.shape)
    Sk = int(k.shape[2])
    if tuple(k.shape) != (B, H, Sk, D) or tuple(v.shape) != (B, H, Sk, D) or \
            tuple(o.shape) != (B, H, Sq, D):
        raise ValueError("shapes: q, o [B, H, Sq, D]; k, v [B, H, Sk, D]")
    if lse is not None and (tuple(lse.shape) != (B, H, Sq) or lse.dtype != torch.float32
                            or not lse.is_contiguous()):
        raise ValueError("lse must be a contiguous float32 [B, H, Sq] tensor")
    sc = (1.0 / D ** 0.5) if scale is None else float(scale)
    _check(lib.fr_attention_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Sq, Sk, D,
                                int(bool(causal)), sc, BF16, _stream(stream, q)),
           "fr_attention_fwd")


def _check_like(t, ref, name):
    if t is not None and (tuple(t.shape) != tuple(ref.shape) or not t.is_contiguous()
                          or t.dtype != ref.dtype):
        raise ValueError(f"{name} must be a contiguous tensor of the row input's shape and dtype")


def _check_f32_vec(t, cols, name):
    torch = _torch()
    _check_vec(t, cols, name)
    if t.dtype != torch.float32:
        raise TypeError(f"{name} must be float32")


def _workspace_arg(ws):
    if ws is None:
        return None, 0
    _need_cuda(ws)
    if not ws.is_contiguous():
        raise ValueError("workspace must be contiguous")
    return _ptr(ws), ws.numel() * ws.element_size()


def fr_softmax_bwd(p, dy, dx, stream=None) -> None:
    """dx = p * (dy - <p, dy>) per row, from the forward output p (C: fr_softmax_bwd)."""
    _need_cuda(p, dy, dx)
    R, C = _rows_cols(p)
    _check_like(dy, p, "dy")
    _check_like(dx, p, "dx")
    _check(lib.fr_softmax_bwd(_ptr(p), _ptr(dy), _ptr(dx), R, C, _dtype_code(p), _stream(stream, p)),
           "fr_softmax_bwd")


def fr_norm_bwd_workspace_bytes(op: int, rows: int, cols: int) -> int:
    """Workspace bytes fr_add_rmsnorm_bwd / fr_layernorm_bwd need (C: same name)."""
    n = int(lib.fr_norm_bwd_workspace_bytes(int(op), int(rows), int(cols)))
    if n < 0:
        raise ValueError(f"no workspace size for op {op} at [{rows}, {cols}]")
    return n


def fr_norm_bwd_split_workspace_bytes(op: int, rows: int, cols: int) -> int:
    """Workspace bytes of the split-row norm backward (C: same name)."""
    n = int(lib.fr_norm_bwd_split_workspace_bytes(int(op), int(rows), int(cols)))
    if n < 0:
        raise ValueError(f"no split workspace size for op {op} at [{rows}, {cols}]")
    return n


def fr_add_rmsnorm_bwd_split(h, dy, weight, dh, dweight, workspace, dres=None, eps: float = 1e-6,
                             stream=None) -> None:
    """fr_add_rmsnorm_bwd for rows of any width (C: fr_add_rmsnorm_bwd_split)."""
    fr_add_rmsnorm_bwd(h, dy, weight, dh, dweight, workspace, dres, eps, stream, _split=True)


def fr_layernorm_bwd_split(x, dy, gamma, mean, rstd, dx, dgamma, dbeta, workspace,
                           stream=None) -> None:
    """fr_layernorm_bwd for rows of any width (C: fr_layernorm_bwd_split)."""
    fr_layernorm_bwd(x, dy, gamma, mean, rstd, dx, dgamma, dbeta, workspace, stream, _split=True)


def fr_add_rmsnorm_bwd(h, dy, weight, dh, dweight, workspace, dres=None, eps: float = 1e-6,
                       stream=None, _split: bool = False) -> None:
    """Backward of residual add + RMSNorm from the stored h = x + residual
    (C: fr_add_rmsnorm_bwd); dweight fp32 [cols] is overwritten."""
    _need_cuda(h, dy, weight, dh, dweight, dres)
    R, C = _rows_cols(h)
    for t, n in ((dy, "dy"), (dh, "dh"), (dres, "dres")):
        _check_like(t, h, n)
    _check_vec(weight, C, "weight")
    if weight.dtype != h.dtype:
        raise TypeError("weight must have h's dtype")
    _check_f32_vec(dweight, C, "dweight")
    wp, wn = _workspace_arg(workspace)
    fn = lib.fr_add_rmsnorm_bwd_split if _split else lib.fr_add_rmsnorm_bwd
    _check(fn(_ptr(h), _ptr(dy), _ptr(dres), _ptr(weight), _ptr(dh), _ptr(dweight), wp, wn, R, C,
              float(eps), _dtype_code(h), _stream(stream, h)),
           "fr_add_rmsnorm_bwd_split" if _split else "fr_add_rmsnorm_bwd")


FR_NOALLOC_SCRATCH_BYTES = 8 << 20


def fr_add_rmsnorm_bwd_noalloc(h, dy, weight, dh, dweight, dres=None, eps: float = 1e-6,
                               stream=None) -> None:
    """fr_add_rmsnorm_bwd with the library's own device array in place of a
    workspace (C: fr_add_rmsnorm_bwd_noalloc): allocates nothing; calls that
    overlap in time on one GPU race."""
    _need_cuda(h, dy, weight, dh, dweight, dres)
    R, C = _rows_cols(h)
    for t, n in ((dy, "dy"), (dh, "dh"), (dres, "dres")):
        _check_like(t, h, n)
    _check_vec(weight, C, "weight")
    if weight.dtype != h.dtype:
        raise TypeError("weight must have h's dtype")
    _check_f32_vec(dweight, C, "dweight")
    _check(lib.fr_add_rmsnorm_bwd_noalloc(_ptr(h), _ptr(dy), _ptr(dres), _ptr(weight), _ptr(dh),
                                          _ptr(dweight), R, C, float(eps), _dtype_code(h),
                                          _stream(stream, h)), "fr_add_rmsnorm_bwd_noalloc")


def fr_layernorm_bwd(x, dy, gamma, mean, rstd, dx, dgamma, dbeta, workspace, stream=None,
                     _split: bool = False) -> None:
    """Backward of LayerNorm at the saved mean / rstd (C: fr_layernorm_bwd);
    dgamma, dbeta fp32 [cols] are overwritten."""
    torch = _torch()
    _need_cuda(x, dy, gamma, mean, rstd, dx, dgamma, dbeta)
    R, C = _rows_cols(x)
    _check_like(dy, x, "dy")
    _check_like(dx, x, "dx")
    _check_vec(gamma, C, "gamma")
    if gamma.dtype != x.dtype:
        raise TypeError("gamma must have x's dtype")
    _check_rows(mean, R, "mean", torch.float32)
    _check_rows(rstd, R, "rstd", torch.float32)
    _check_f32_vec(dgamma, C, "dgamma")
    _check_f32_vec(dbeta, C, "dbeta")
    wp, wn = _workspace_arg(workspace)
    fn = lib.fr_layernorm_bwd_split if _split else lib.fr_layernorm_bwd
    _check(fn(_ptr(x), _ptr(dy), _ptr(gamma), _ptr(mean), _ptr(rstd), _ptr(dx), _ptr(dgamma),
              _ptr(dbeta), wp, wn, R, C, _dtype_code(x), _stream(stream, x)),
           "fr_layernorm_bwd_split" if _split else "fr_layernorm_bwd")


def fr_stream_copy(src, dst, nbytes: int | None = None, stream=None) -> None:
    """Plain device copy of nbytes (default: all of src) — bandwidth reference."""
    _need_cuda(src, dst)
    n = src.numel() * src.element_size() if nbytes is None else int(nbytes)
    if n > dst.numel() * dst.element_size() or n > src.numel() * src.element_size():
        raise ValueError("copy larger than a buffer")
    _check(lib.fr_stream_copy(_ptr(src), _ptr(dst), n, _stream(stream, src)), "fr_stream_copy")


PROBE_READ, PROBE_WRITE, PROBE_COPY = 0, 1, 2
PROBE_NT_LOADS, PROBE_NT_STORES = 1, 2
STREAM_THREADS, STREAM_VECS, STREAM_POLICY = 256, 8, 3


def fr_stream_probe_rows(nbytes: int, row_bytes: int = STREAM_THREADS * STREAM_VECS * 16) -> int:
    """Rows of row_bytes over nbytes (the sink words of a read probe)."""
    n = lib.fr_stream_probe_rows(int(nbytes), int(row_bytes))
    if n < 0:
        raise ValueError(f"bad probe row length {row_bytes}")
    return n


def fr_stream_probe(kind: int, src=None, dst=None, nbytes: int | None = None, value: int = 0,
                    sink=None, threads: int = STREAM_THREADS, vecs: int = STREAM_VECS,
                    policy: int = STREAM_POLICY, row_bytes: int = 0, stream=None) -> None:
    """Memory-system probe (C: fr_stream_probe): PROBE_READ reads src into the
    per-row XOR words of sink (uint32 viewed as int32), PROBE_WRITE fills dst
    with `value`, PROBE_COPY copies src to dst. policy: a mask of
    PROBE_NT_LOADS and PROBE_NT_STORES; row_bytes: the row length (0: the
    shape's threads * vecs * 16)."""
    _need_cuda(src, dst, sink)
    ref = src if src is not None else dst
    n = ref.numel() * ref.element_size() if nbytes is None else int(nbytes)
    for t in (src, dst):
        if t is not None and n > t.numel() * t.element_size():
            raise ValueError("probe larger than a buffer")
    rb = int(row_bytes) or threads * vecs * 16
    if sink is not None and sink.numel() * sink.element_size() < 4 * fr_stream_probe_rows(n, rb):
        raise ValueError("sink smaller than one word per row")
    _check(lib.fr_stream_probe(int(kind), _ptr(src), _ptr(dst), n, int(row_bytes),
                               ctypes.c_uint32(value & 0xFFFFFFFF),
                               _ptr(sink), int(threads), int(vecs), int(policy),
                               _stream(stream, ref)), "fr_stream_probe")


def fr_stream_read(src, sink, nbytes: int | None = None, stream=None) -> None:
    """Read-only probe in the default shape (C: fr_stream_read)."""
    _need_cuda(src, sink)
    n = src.numel() * src.element_size() if nbytes is None else int(nbytes)
    if n > src.numel() * src.element_size():
        raise ValueError("read larger than the buffer")
    if sink.numel() * sink.element_size() < 4 * fr_stream_probe_rows(n):
        raise ValueError("sink smaller than one word per row")
    _check(lib.fr_stream_read(_ptr(src), n, _ptr(sink), _stream(stream, src)), "fr_stream_read")


def fr_stream_write(dst, value: int, nbytes: int | None = None, stream=None) -> None:
    """Write-only probe in the default shape (C: fr_stream_write)."""
    _need_cuda(dst)
    n = dst.numel() * dst.element_size() if nbytes is None else int(nbytes)
    if n > dst.numel() * dst.element_size():
        raise ValueError("write larger than the buffer")
    _check(lib.fr_stream_write(_ptr(dst), n, ctypes.c_uint32(value & 0xFFFFFFFF),
                               _stream(stream, dst)), "fr_stream_write")


def fr_mfma_probe(workgroups: int, iters: int, sink, pattern: int = 0, stream=None) -> None:
    """Matrix-core probe (C: fr_mfma_probe): `workgroups` x 256 lanes, each
    wavefront `iters` rounds of 8 bf16 32x32x16 matrix instructions on
    constant (pattern 0: every sink element 32 * iters) or pseudo-random
    (pattern 1) operands; sink is a float32 device tensor of at least
    workgroups * 256 elements."""
    _need_cuda(sink)
    if sink.dtype != _torch().float32 or sink.numel() < int(workgroups) * 256:
        raise ValueError("sink: float32, at least workgroups * 256 elements")
    _check(lib.fr_mfma_probe(int(workgroups), int(iters), int(pattern), _ptr(sink),
                             _stream(stream, sink)), "fr_mfma_probe")


def fr_debug_force_variant(op: int, threads: int = 0, vecs: int = 0) -> None:
    _check(lib.fr_debug_force_variant(int(op), int(threads), int(vecs)), "fr_debug_force_variant")


def fr_debug_select_variant(op: int, cols: int, in_dtype: int = F32, out_dtype: int | None = None,
                            vector_path: bool = True):
    t, v, e = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    od = in_dtype if out_dtype is None else out_dtype
    _check(lib.fr_debug_select_variant(int(op), int(cols), int(in_dtype), int(od), int(vector_path),
                                       ctypes.byref(t), ctypes.byref(v), ctypes.byref(e)),
           "fr_debug_select_variant")
    return t.value, v.value, e.value


def fr_debug_select_variant_for(op: int, rows: int, cols: int, in_dtype: int = F32,
                                out_dtype: int | None = None, vector_path: bool = True):
    """C: fr_debug_select_variant_for (the shape a call over `rows` rows takes;
    queries the current device's compute-unit count)."""
    t, v, e = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    od = in_dtype if out_dtype is None else out_dtype
    _check(lib.fr_debug_select_variant_for(int(op), int(rows), int(cols), int(in_dtype), int(od),
                                           int(vector_path), ctypes.byref(t), ctypes.byref(v),
                                           ctypes.byref(e)),
           "fr_debug_select_variant_for")
    return t.value, v.value, e.value


class forced_variant:
    """Context manager: force (threads, vecs) for op, restore automatic selection after."""

    def __init__(self, op: int, threads: int, vecs: int):
        self.op, self.threads, self.vecs = op, threads, vecs

    def __enter__(self):
        fr_debug_force_variant(self.op, self.threads, self.vecs)
        return self

    def __exit__(self, *exc):
        fr_debug_force_variant(self.op, 0, 0)
        return False


def fr_debug_set_split_batch_bytes(nbytes: int) -> int:
    """C: fr_debug_set_split_batch_bytes; returns the previous setting."""
    return int(lib.fr_debug_set_split_batch_bytes(int(nbytes)))


class split_batch_bytes:
    """Context manager: set the split entry points' row-batch bound (bytes of
    input per batch; 0 = unbatched), restore the previous setting after."""

    def __init__(self, nbytes: int):
        self.nbytes = nbytes

    def __enter__(self):
        self.prev = fr_debug_set_split_batch_bytes(self.nbytes)
        return self

    def __exit__(self, *exc):
        fr_debug_set_split_batch_bytes(self.prev)
        return False


def fr_debug_set_split_one_pass(mode: int) -> int:
    """C: fr_debug_set_split_one_pass; returns the previous setting."""
    return int(lib.fr_debug_set_split_one_pass(int(mode)))


class split_one_pass:
    """Context manager: the one-pass form of the split softmax and
    cross-entropy never (0), where the rows are many enough (1, the default)
    or wherever it applies (2); restore the previous setting after."""

    def __init__(self, mode: int):
        self.mode = mode

    def __enter__(self):
        self.prev = fr_debug_set_split_one_pass(self.mode)
        return self

    def __exit__(self, *exc):
        fr_debug_set_split_one_pass(self.prev)
        return False


def fr_debug_set_coop_spin_limit(polls: int) -> int:
    """C: fr_debug_set_coop_spin_limit; returns the previous setting."""
    return int(lib.fr_debug_set_coop_spin_limit(int(polls)))


class coop_spin_limit:
    """Context manager: bound the one-pass split form's polls per wait
    (< 0: the default); restore the previous setting after."""

    def __init__(self, polls: int):
        self.polls = polls

    def __enter__(self):
        self.prev = fr_debug_set_coop_spin_limit(self.polls)
        return self

    def __exit__(self, *exc):
        fr_debug_set_coop_spin_limit(self.prev)
        return False


# ------------------------------------------------- allocating conveniences

def softmax(x, out_dtype=None, out=None):
    """Row softmax; rows wider than FR_MAX_COLS take the split-row path."""
    torch = _torch()
    y = out if out is not None else torch.empty(x.shape, dtype=out_dtype or x.dtype, device=x.device)
    if x.shape[1] > FR_MAX_COLS:
        fr_softmax_fwd_split(x, y, _split_workspace(x.shape[0], x.shape[1], x.device))
    else:
        fr_softmax_fwd(x, y)
    return y


def layernorm(x, gamma, beta, eps: float = 1e-5):
    """Returns (y, mean, rstd); rows wider than FR_MAX_COLS take the split-row path."""
    torch = _torch()
    R = x.shape[0]
    y = torch.empty_like(x)
    mean = torch.empty(R, dtype=torch.float32, device=x.device)
    rstd = torch.empty(R, dtype=torch.float32, device=x.device)
    if x.shape[1] > FR_MAX_COLS:
        fr_layernorm_fwd_split(x, gamma, beta, y, _split_workspace(R, x.shape[1], x.device), mean,
                               rstd, eps)
    else:
        fr_layernorm_fwd(x, gamma, beta, y, mean, rstd, eps)
    return y, mean, rstd


def add_rmsnorm(x, residual, weight, eps: float = 1e-6, inplace: bool = False):
    """Returns (y, residual_out); rows wider than FR_MAX_COLS take the split-row path."""
    torch = _torch()
    y = torch.empty_like(x)
    res_out = residual if inplace else torch.empty_like(residual)
    if x.shape[1] > FR_MAX_COLS:
        fr_add_rmsnorm_fwd_split(x, residual, weight, y, _split_workspace(x.shape[0], x.shape[1],
                                                                          x.device), res_out, eps)
    else:
        fr_add_rmsnorm_fwd(x, residual, weight, y, res_out, eps)
    return y, res_out


def softmax_xent(logits, labels, return_argmax: bool = False, ignore_index=None,
                 label_smoothing: float = 0.0, reduction: str = "none", grad_scale: float = 1.0):
    """Returns (loss, grad[, argmax]); loss is the per-row loss [rows] for
    reduction "none", else the scalar total (a 1-element tensor)."""
    torch = _torch()
    R = logits.shape[0]
    loss = torch.empty(R, dtype=torch.float32, device=logits.device)
    grad = torch.empty_like(logits)
    am = torch.empty(R, dtype=torch.int32, device=logits.device) if return_argmax else None
    plain = (logits.dtype == torch.float32 and ignore_index is None and label_smoothing == 0.0
             and reduction == "none" and grad_scale == 1.0)
    if logits.shape[1] > FR_MAX_COLS:
        total = torch.empty(1, dtype=torch.float32, device=logits.device)
        fr_softmax_xent_split(logits, labels, loss, grad, _split_workspace(R, logits.shape[1],
                              logits.device), am, total, ignore_index, label_smoothing, grad_scale,
                              reduction)
        out = loss if reduction == "none" else total
    elif plain:
        fr_softmax_xent_fwd_bwd(logits, labels, loss, grad, am)
        out = loss
    else:
        total = torch.empty(1, dtype=torch.float32, device=logits.device)
        fr_softmax_xent_ex(logits, labels, loss, grad, am, total, ignore_index, label_smoothing,
                           grad_scale, reduction)
        out = loss if reduction == "none" else total
    return (out, grad, am) if return_argmax else (out, grad)


def _workspace(op, rows, cols, device, split=False):
    torch = _torch()
    n = (fr_norm_bwd_split_workspace_bytes if split else fr_norm_bwd_workspace_bytes)(op, rows, cols)
    return torch.empty(max(n, 16), dtype=torch.uint8, device=device)


def softmax_bwd(p, dy, out=None):
    """dx = p (dy - sum(p dy)); rows wider than FR_BWD_MAX_COLS take the split-row path."""
    torch = _torch()
    dx = out if out is not None else torch.empty_like(p)
    if p.shape[1] > FR_BWD_MAX_COLS:
        fr_softmax_bwd_split(p, dy, dx, _split_workspace(p.shape[0], p.shape[1], p.device))
    else:
        fr_softmax_bwd(p, dy, dx)
    return dx


def add_rmsnorm_bwd(h, dy, weight, eps: float = 1e-6, dres=None):
    """Returns (dh, dweight); dh is the gradient of both x and residual. Rows
    wider than FR_BWD_MAX_COLS take the split-row path."""
    torch = _torch()
    R, C = h.shape
    dh = torch.empty_like(h)
    dw = torch.empty(C, dtype=torch.float32, device=h.device)
    split = C > FR_BWD_MAX_COLS
    ws = _workspace(OP_RMSNORM_BWD, R, C, h.device, split)
    fr_add_rmsnorm_bwd(h, dy, weight, dh, dw, ws, dres=dres, eps=eps, _split=split)
    return dh, dw


def layernorm_bwd(x, dy, gamma, mean, rstd):
    """Returns (dx, dgamma, dbeta); rows wider than FR_BWD_MAX_COLS take the split-row path."""
    torch = _torch()
    R, C = x.shape
    dx = torch.empty_like(x)
    dg = torch.empty(C, dtype=torch.float32, device=x.device)
    db = torch.empty(C, dtype=torch.float32, device=x.device)
    split = C > FR_BWD_MAX_COLS
    ws = _workspace(OP_LAYERNORM_BWD, R, C, x.device, split)
    fr_layernorm_bwd(x, dy, gamma, mean, rstd, dx, dg, db, ws, _split=split)
    return dx, dg, db


def attention(q, k, v, causal: bool = False, scale=None, return_lse: bool = False):
    """Returns o (and lse) of scaled dot-product attention (bf16)."""
    torch = _torch()
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device) if return_lse else None
    fr_attention_fwd(q, k, v, o, lse, causal, scale)
    return (o, lse) if return_lse else o
