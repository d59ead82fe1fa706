"""Python front end of the double-precision CPU oracle (oracle/liboracle.so).

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check and by the
benchmark's CPU-baseline leg. The product library never imports it, and it
imports nothing from the product library.

All functions take numpy arrays in the stored input dtypes (float32, or bf16
as uint16 bit patterns) and return float64 results computed by the plain
definitions in oracle.c.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

F32, BF16, F64 = 0, 1, 2

_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_build.LIB):
        _build.build()
    lib = ctypes.CDLL(_build.LIB)
    P, I64, I32, D, F = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_double, ctypes.c_float
    DP = ctypes.POINTER(ctypes.c_double)
    sig = {
        "oracle_threads": ([], I32),
        "oracle_set_threads": ([I32], None),
        "oracle_round_bf16": ([D], ctypes.c_uint16),
        "oracle_round_bf16_array": ([P, P, I64], None),
        "oracle_decode": ([P, I32, P, I64], None),
        "oracle_softmax": ([P, I32, I64, I64, P], None),
        "oracle_layernorm": ([P, P, P, I32, I64, I64, F, P, P, P], None),
        "oracle_add_rmsnorm": ([P, P, P, I32, I64, I64, F, P, P, P], None),
        "oracle_softmax_xent": ([P, I32, P, I64, I64, P, P, P], None),
        "oracle_softmax_bwd": ([P, P, I32, I64, I64, P], None),
        "oracle_softmax_xent_ex": ([P, I32, P, I64, I64, I32, I32, D, I32, D, P, P, P, P], None),
        "oracle_attention": ([P, P, P, I32, I64, I64, I64, I64, I64, I32, D, P, P], None),
        "oracle_rmsnorm_bwd": ([P, P, P, P, I32, I64, I64, F, P, P], None),
        "oracle_layernorm_bwd": ([P, P, P, P, P, I32, I64, I64, P, P, P], None),
        "oracle_online_softmax_stats": ([P, I64, DP, DP], None),
        "oracle_softmax_stats_merge": ([D, D, D, D, DP, DP], None),
        "oracle_welford": ([P, I64, DP, DP, DP], None),
        "oracle_chan_merge": ([D, D, D, D, D, D, DP, DP, DP], None),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.float64:
        return F64
    raise TypeError(f"oracle input must be float32, bf16 bits (uint16) or float64, got {a.dtype}")


def _c(a, dtype=None):
    return np.ascontiguousarray(a if dtype is None else a.astype(dtype, copy=False))


def threads() -> int:
    return _load().oracle_threads()


def set_threads(n: int) -> None:
    _load().oracle_set_threads(int(n))


def round_bf16(v) -> np.ndarray:
    """double -> bf16 bits, round to nearest even, directly from double."""
    a = _c(np.asarray(v, dtype=np.float64))
    out = np.empty(a.shape, dtype=np.uint16)
    _load().oracle_round_bf16_array(_ptr(a), _ptr(out), a.size)
    return out


def round_bf16_scalar(v: float) -> int:
    return int(_load().oracle_round_bf16(float(v)))


def decode(a: np.ndarray) -> np.ndarray:
    """Stored input (float32 or bf16 bits) -> exact float64."""
    a = _c(a)
    out = np.empty(a.shape, dtype=np.float64)
    _load().oracle_decode(_ptr(a), _dtype_code(a), _ptr(out), a.size)
    return out


def softmax(x: np.ndarray) -> np.ndarray:
    x = _c(x)
    R, C = x.shape
    p = np.empty((R, C), dtype=np.float64)
    _load().oracle_softmax(_ptr(x), _dtype_code(x), R, C, _ptr(p))
    return p


def layernorm(x, gamma, beta, eps: float):
    x, gamma, beta = _c(x), _c(gamma), _c(beta)
    if not (x.dtype == gamma.dtype == beta.dtype):
        raise TypeError("x, gamma and beta share one dtype")
    R, C = x.shape
    y = np.empty((R, C), dtype=np.float64)
    mean = np.empty(R, dtype=np.float64)
    rstd = np.empty(R, dtype=np.float64)
    _load().oracle_layernorm(_ptr(x), _ptr(gamma), _ptr(beta), _dtype_code(x), R, C,
                             float(eps), _ptr(y), _ptr(mean), _ptr(rstd))
    return y, mean, rstd


def add_rmsnorm(x, residual, weight, eps: float):
    """Returns (y, h, rstd) in float64; h = x + residual exactly."""
    x, residual, weight = _c(x), _c(residual), _c(weight)
    if not (x.dtype == residual.dtype == weight.dtype):
        raise TypeError("x, residual and weight share one dtype")
    R, C = x.shape
    y = np.empty((R, C), dtype=np.float64)
    h = np.empty((R, C), dtype=np.float64)
    rstd = np.empty(R, dtype=np.float64)
    _load().oracle_add_rmsnorm(_ptr(x), _ptr(residual), _ptr(weight), _dtype_code(x), R, C,
                               float(eps), _ptr(y), _ptr(h), _ptr(rstd))
    return y, h, rstd


def softmax_xent(logits, labels):
    """Returns (loss[R], grad[R, C], argmax[R]) in float64 / int32."""
    logits = _c(logits)
    labels = _c(labels, np.int32)
    R, C = logits.shape
    loss = np.empty(R, dtype=np.float64)
    grad = np.empty((R, C), dtype=np.float64)
    am = np.empty(R, dtype=np.int32)
    _load().oracle_softmax_xent(_ptr(logits), _dtype_code(logits), _ptr(labels), R, C,
                                _ptr(loss), _ptr(grad), _ptr(am))
    return loss, grad, am


REDUCTIONS = {"none": 0, "sum": 1, "mean": 2}


def softmax_xent_ex(logits, labels, ignore_index=None, label_smoothing=0.0, reduction="none",
                    grad_scale=1.0):
    """Cross-entropy with options. Returns (loss[R], grad[R, C], argmax[R],
    total) in float64 / int32; total is None for reduction "none".
    ignore_index None: no row is ignored. label_smoothing and grad_scale are
    used as given (pass fp32 values to match an fp32 caller)."""
    logits = _c(logits)
    labels = _c(labels, np.int32)
    R, C = logits.shape
    loss = np.empty(R, dtype=np.float64)
    grad = np.empty((R, C), dtype=np.float64)
    am = np.empty(R, dtype=np.int32)
    tot = ctypes.c_double(np.nan)
    red = REDUCTIONS[reduction]
    _load().oracle_softmax_xent_ex(
        _ptr(logits), _dtype_code(logits), _ptr(labels), R, C, int(ignore_index is not None),
        int(ignore_index or 0), float(label_smoothing), red, float(grad_scale), _ptr(loss),
        _ptr(grad), _ptr(am), ctypes.byref(tot))
    return loss, grad, am, (tot.value if red else None)


def attention(q, k, v, causal: bool = False, scale=None):
    """Scaled dot-product attention. q [B, H, Sq, D], k and v [B, H, Sk, D]
    (one dtype). Returns (o [B, H, Sq, D], lse [B, H, Sq]) in float64.
    scale defaults to 1/sqrt(D) (pass the fp32 value an fp32 caller uses)."""
    q, k, v = _c(q), _c(k), _c(v)
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k and v share one dtype")
    B, H, Sq, D = q.shape
    Sk = k.shape[2]
    if k.shape != (B, H, Sk, D) or v.shape != (B, H, Sk, D):
        raise ValueError("k and v must be [B, H, Sk, D]")
    sc = float(np.float32(1.0 / np.sqrt(D))) if scale is None else float(scale)
    o = np.empty((B, H, Sq, D), dtype=np.float64)
    lse = np.empty((B, H, Sq), dtype=np.float64)
    _load().oracle_attention(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q), B, H, Sq, Sk, D,
                             int(causal), sc, _ptr(o), _ptr(lse))
    return o, lse


def softmax_bwd(p, dy):
    """dx = p * (dy - <dy, p>) per row, from the stored forward output p."""
    p, dy = _c(p), _c(dy)
    if p.dtype != dy.dtype or p.shape != dy.shape:
        raise TypeError("p and dy share dtype and shape")
    R, C = p.shape
    dx = np.empty((R, C), dtype=np.float64)
    _load().oracle_softmax_bwd(_ptr(p), _ptr(dy), _dtype_code(p), R, C, _ptr(dx))
    return dx


def rmsnorm_bwd(h, dy, weight, eps: float, dres=None):
    """Returns (dh[R, C], dw[C]) for y = h * rstd * w (rstd recomputed from h);
    dres, the gradient reaching h through the updated residual, adds to dh."""
    h, dy, weight = _c(h), _c(dy), _c(weight)
    if not (h.dtype == dy.dtype == weight.dtype):
        raise TypeError("h, dy and weight share one dtype")
    if dres is not None:
        dres = _c(dres)
        if dres.dtype != h.dtype or dres.shape != h.shape:
            raise TypeError("dres shares h's dtype and shape")
    R, C = h.shape
    dh = np.empty((R, C), dtype=np.float64)
    dw = np.empty(C, dtype=np.float64)
    _load().oracle_rmsnorm_bwd(_ptr(h), _ptr(dy), None if dres is None else _ptr(dres),
                               _ptr(weight), _dtype_code(h), R, C, float(eps), _ptr(dh), _ptr(dw))
    return dh, dw


def layernorm_bwd(x, dy, gamma, mean, rstd):
    """Returns (dx[R, C], dgamma[C], dbeta[C]) at the given per-row mean / rstd."""
    x, dy, gamma = _c(x), _c(dy), _c(gamma)
    mean, rstd = _c(mean, np.float64), _c(rstd, np.float64)
    if not (x.dtype == dy.dtype == gamma.dtype):
        raise TypeError("x, dy and gamma share one dtype")
    R, C = x.shape
    dx = np.empty((R, C), dtype=np.float64)
    dg = np.empty(C, dtype=np.float64)
    db = np.empty(C, dtype=np.float64)
    _load().oracle_layernorm_bwd(_ptr(x), _ptr(dy), _ptr(gamma), _ptr(mean), _ptr(rstd),
                                 _dtype_code(x), R, C, _ptr(dx), _ptr(dg), _ptr(db))
    return dx, dg, db


def online_softmax_stats(x: np.ndarray):
    x = _c(x, np.float64)
    m, d = ctypes.c_double(), ctypes.c_double()
    _load().oracle_online_softmax_stats(_ptr(x), x.size, ctypes.byref(m), ctypes.byref(d))
    return m.value, d.value


def softmax_stats_merge(a, b):
    m, d = ctypes.c_double(), ctypes.c_double()
    _load().oracle_softmax_stats_merge(a[0], a[1], b[0], b[1], ctypes.byref(m), ctypes.byref(d))
    return m.value, d.value


def welford(x: np.ndarray):
    x = _c(x, np.float64)
    n, mu, m2 = ctypes.c_double(), ctypes.c_double(), ctypes.c_double()
    _load().oracle_welford(_ptr(x), x.size, ctypes.byref(n), ctypes.byref(mu), ctypes.byref(m2))
    return n.value, mu.value, m2.value


def chan_merge(a, b):
    n, mu, m2 = ctypes.c_double(), ctypes.c_double(), ctypes.c_double()
    _load().oracle_chan_merge(a[0], a[1], a[2], b[0], b[1], b[2],
                              ctypes.byref(n), ctypes.byref(mu), ctypes.byref(m2))
    return n.value, mu.value, m2.value
