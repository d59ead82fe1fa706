"""Seeded synthetic inputs for the fused row kernels.

This module only draws random numbers and stores them in the input dtypes.
It holds none of the arithmetic of the row operations; both the GPU tests /
benchmark and the CPU oracle read the buffers it returns.

Recipe (every workload):
  * generator: numpy ``Generator(PCG64(seed))``;
  * draws are made in float64, one array at a time, in the order the fields
    are listed below, row-major;
  * float64 -> float32 uses numpy's round-to-nearest-even cast;
  * bf16 inputs are then rounded float32 -> bf16 (round to nearest, ties to
    even, on the bit pattern) and kept as raw ``uint16`` bit patterns.

The five standard workloads (shapes and distributions of the row-reduction
workloads the method is exercised on; the second argument of N(.,.) is the
variance, so N(0, 4^2) has standard deviation 4):

  softmax_f32      x ~ N(0, 4^2), fp32 [64, 1000]                      seed 1001
  layernorm_f32    x ~ N(3, 2^2), fp32 [4096, 1024];                   seed 1002
                   gamma ~ U(0.5, 1.5), beta ~ N(0, 0.1) fp32 [1024]; eps 1e-5
  softmax_bf16     z ~ N(0, 1) [16384, 4096], per-row scale s ~ U(1, 60),
                   x = bf16(s * z)                                     seed 1003
  add_rmsnorm_bf16 x, r ~ N(0, 1) bf16 [8192, 8192]; w ~ U(0.8, 1.2)
                   bf16 [8192]; eps 1e-6                               seed 1004
  xent_f32         logits ~ N(0, 2^2) fp32 [4096, 50257];
                   labels ~ U{0, ..., 50256} int32 [4096]              seed 1005

Backward workloads, at the forward workloads' shapes (the per-row forward
statistics they consume, p = softmax(x) and LayerNorm's mean / rstd, are not
drawn here: the tests take them from the oracle, the benchmark from the
forward kernels):

  softmax_bwd_bf16    x ~ as softmax_bf16 [16384, 4096]; dy ~ N(0, 1)  seed 1006
  layernorm_bwd_f32   x ~ N(3, 2^2) [4096, 1024]; gamma ~ U(0.5, 1.5)
                      [1024]; dy ~ N(0, 1); eps 1e-5 (of the forward)  seed 1007
  add_rmsnorm_bwd_bf16 h ~ N(0, 2) (the updated residual x + r of two
                      N(0, 1) draws) [8192, 8192]; w ~ U(0.8, 1.2) [8192];
                      dy, dres ~ N(0, 1); eps 1e-6                     seed 1008

Attention (the online softmax inside attention):

  attention_bf16      q, k, v ~ N(0, 1) bf16 [B=4, H=16, S=4096, D=128],
                      scale 1/sqrt(128); rows = B*H*S, cols = D        seed 1009

``make(name, rows=None, cols=None)`` builds a workload with the standard
distributions at any shape (used for edge-shape and small parity cases); the
seed stays the workload's own unless ``seed`` is given.
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass, field

import numpy as np

__all__ = ["WORKLOADS", "Workload", "make", "f32_to_bf16_bits", "sha256"]


@dataclass(frozen=True)
class Spec:
    name: str
    op: str
    rows: int
    cols: int
    seed: int
    dtype: str            # storage dtype of the row data: "f32" or "bf16"
    eps: float | None = None
    desc: str = ""


WORKLOADS = {
    "softmax_f32": Spec("softmax_f32", "softmax", 64, 1000, 1001, "f32",
                        desc="fp32 row softmax, 64 x 1000, x ~ N(0, 4^2)"),
    "layernorm_f32": Spec("layernorm_f32", "layernorm", 4096, 1024, 1002, "f32", eps=1e-5,
                          desc="fp32 LayerNorm, 4096 x 1024, x ~ N(3, 2^2), "
                               "gamma ~ U(0.5,1.5), beta ~ N(0,0.1), eps 1e-5"),
    "softmax_bf16": Spec("softmax_bf16", "softmax", 16384, 4096, 1003, "bf16",
                         desc="bf16 row softmax, 16384 x 4096, x = bf16(U(1,60)_row * N(0,1))"),
    "add_rmsnorm_bf16": Spec("add_rmsnorm_bf16", "add_rmsnorm", 8192, 8192, 1004, "bf16", eps=1e-6,
                             desc="bf16 residual-add + RMSNorm, 8192 x 8192, x,r ~ N(0,1), "
                                  "w ~ U(0.8,1.2), eps 1e-6"),
    "xent_f32": Spec("xent_f32", "xent", 4096, 50257, 1005, "f32",
                     desc="fp32 softmax cross-entropy fwd+bwd, 4096 x 50257, "
                          "logits ~ N(0, 2^2), labels ~ U{0..50256}"),
    "softmax_bwd_bf16": Spec("softmax_bwd_bf16", "softmax_bwd", 16384, 4096, 1006, "bf16",
                             desc="bf16 softmax backward, 16384 x 4096, p = softmax(x) of the "
                                  "softmax_bf16 recipe, dy ~ N(0,1)"),
    "layernorm_bwd_f32": Spec("layernorm_bwd_f32", "layernorm_bwd", 4096, 1024, 1007, "f32",
                              eps=1e-5,
                              desc="fp32 LayerNorm backward, 4096 x 1024, x ~ N(3, 2^2), "
                                   "gamma ~ U(0.5,1.5), dy ~ N(0,1)"),
    "attention_bf16": Spec("attention_bf16", "attention", 4 * 16 * 4096, 128, 1009, "bf16",
                           desc="bf16 attention forward, B=4 H=16 S=4096 D=128, q,k,v ~ N(0,1)"),
    "add_rmsnorm_bwd_bf16": Spec("add_rmsnorm_bwd_bf16", "add_rmsnorm_bwd", 8192, 8192, 1008,
                                 "bf16", eps=1e-6,
                                 desc="bf16 residual-add + RMSNorm backward, 8192 x 8192, "
                                      "h ~ N(0, 2), w ~ U(0.8,1.2), dy, dres ~ N(0,1)"),
}


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return uint16 bits.

    Inputs here are finite draws, so the NaN case is not needed; it is still
    mapped to a quiet NaN so the function is total.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        r[nan] = 0x7FC0
    return r


def sha256(*arrays: np.ndarray) -> str:
    h = hashlib.sha256()
    for a in arrays:
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


@dataclass
class Workload:
    spec: Spec
    rows: int
    cols: int
    seed: int
    arrays: dict = field(default_factory=dict)

    def __getitem__(self, k):
        return self.arrays[k]

    @property
    def eps(self):
        return self.spec.eps

    def digest(self) -> str:
        return sha256(*[self.arrays[k] for k in sorted(self.arrays)])


def _store(a64: np.ndarray, dtype: str) -> np.ndarray:
    a32 = a64.astype(np.float32)
    if dtype == "f32":
        return a32
    if dtype == "bf16":
        return f32_to_bf16_bits(a32)
    raise ValueError(dtype)


def make(name: str, rows: int | None = None, cols: int | None = None,
         seed: int | None = None, dtype: str | None = None) -> Workload:
    """Draw one workload. Field order fixes the random stream (see module doc)."""
    spec = WORKLOADS[name]
    R = spec.rows if rows is None else int(rows)
    C = spec.cols if cols is None else int(cols)
    s = spec.seed if seed is None else int(seed)
    dt = spec.dtype if dtype is None else dtype
    rng = np.random.Generator(np.random.PCG64(s))
    arr = {}
    if name == "softmax_f32":
        arr["x"] = _store(rng.normal(0.0, 4.0, size=(R, C)), dt)
    elif name == "layernorm_f32":
        arr["x"] = _store(rng.normal(3.0, 2.0, size=(R, C)), dt)
        arr["gamma"] = _store(rng.uniform(0.5, 1.5, size=C), dt)
        arr["beta"] = _store(rng.normal(0.0, np.sqrt(0.1), size=C), dt)
    elif name == "softmax_bf16":
        z = rng.normal(0.0, 1.0, size=(R, C))
        scale = rng.uniform(1.0, 60.0, size=(R, 1))
        z *= scale
        arr["x"] = _store(z, dt)
        arr["row_scale"] = scale.reshape(R)
    elif name == "add_rmsnorm_bf16":
        arr["x"] = _store(rng.normal(0.0, 1.0, size=(R, C)), dt)
        arr["residual"] = _store(rng.normal(0.0, 1.0, size=(R, C)), dt)
        arr["weight"] = _store(rng.uniform(0.8, 1.2, size=C), dt)
    elif name == "xent_f32":
        arr["logits"] = _store(rng.normal(0.0, 2.0, size=(R, C)), dt)
        arr["labels"] = rng.integers(0, C, size=R, dtype=np.int64).astype(np.int32)
    elif name == "softmax_bwd_bf16":
        z = rng.normal(0.0, 1.0, size=(R, C))
        z *= rng.uniform(1.0, 60.0, size=(R, 1))
        arr["x"] = _store(z, dt)
        arr["dy"] = _store(rng.normal(0.0, 1.0, size=(R, C)), dt)
    elif name == "layernorm_bwd_f32":
        arr["x"] = _store(rng.normal(3.0, 2.0, size=(R, C)), dt)
        arr["gamma"] = _store(rng.uniform(0.5, 1.5, size=C), dt)
        arr["dy"] = _store(rng.normal(0.0, 1.0, size=(R, C)), dt)
    elif name == "add_rmsnorm_bwd_bf16":
        arr["h"] = _store(rng.normal(0.0, np.sqrt(2.0), size=(R, C)), dt)
        arr["weight"] = _store(rng.uniform(0.8, 1.2, size=C), dt)
        arr["dy"] = _store(rng.normal(0.0, 1.0, size=(R, C)), dt)
        arr["dres"] = _store(rng.normal(0.0, 1.0, size=(R, C)), dt)
    elif name == "attention_bf16":
        raise KeyError("attention_bf16: use make_attention(B, H, Sq, Sk, D)")
    else:
        raise KeyError(name)
    return Workload(spec=spec, rows=R, cols=C, seed=s, arrays=arr)


def make_attention(B=4, H=16, Sq=4096, Sk=None, D=128, seed=1009, dtype="bf16") -> Workload:
    """q [B, H, Sq, D], k and v [B, H, Sk, D] (Sk defaults to Sq), N(0, 1)."""
    Sk = Sq if Sk is None else Sk
    rng = np.random.Generator(np.random.PCG64(seed))
    arr = {"q": _store(rng.normal(0.0, 1.0, size=(B, H, Sq, D)), dtype),
           "k": _store(rng.normal(0.0, 1.0, size=(B, H, Sk, D)), dtype),
           "v": _store(rng.normal(0.0, 1.0, size=(B, H, Sk, D)), dtype)}
    return Workload(spec=WORKLOADS["attention_bf16"], rows=B * H * Sq, cols=D, seed=seed,
                    arrays=arr)
