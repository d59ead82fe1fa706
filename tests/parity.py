"""Comparison rules between the GPU results and the double-precision oracle.

fp32 outputs: |g - o| <= 1e-5 * scale + 2^-126, where scale is |o| unless a
  relative bound is ill-posed for that output:
    * LayerNorm y crosses zero: scale = max(|o|, 1);
    * LayerNorm mean: scale = max(|o|, row standard deviation) (the error of a
      sum scales with the spread of its terms, not with the mean);
    * cross-entropy grad at the label, p - 1: scale = max(|o|, p) (the
      subtraction of 1 cannot add error beyond p's own);
    * cross-entropy loss: scale = max(|o|, 1).
  2^-126 is the fp32 normal threshold: below it fp32 carries no relative
  precision, so no implementation can meet a relative bound there.
bf16 outputs: bit patterns mapped to ordered integers; pass iff within one
  bf16 ulp of the oracle value rounded to nearest even. LayerNorm y, which
  crosses zero by cancellation, may instead be within 1e-5 * max(|o|, 1)
  (the same floor as its fp32 rule); the ulp histogram is still reported.
  Backward outputs formed by cancellation (dx = p (dy - s) and the like) may
  instead meet the fp32 rule at a condition-aware scale, plus the final
  rounding to bf16.
int32 outputs: exact.
"""
import numpy as np
import torch

FLT_MIN = 2.0 ** -126
REL = 1e-5


def to_dev(a, dev="cuda:0"):
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def bf16_bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def ordered(b):
    b = np.asarray(b).astype(np.int64)
    return np.where(b & 0x8000, 0x8000 - (b & 0x7FFF), 0x8000 + b)


def check_f32(got, ref, scale=None, what=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got) == np.isfinite(ref)), f"{what}: finiteness differs"
    fin = np.isfinite(ref)
    s = np.abs(ref) if scale is None else np.asarray(scale, dtype=np.float64)
    s = np.broadcast_to(s, ref.shape)
    err = np.abs(got[fin] - ref[fin])
    bound = REL * s[fin] + FLT_MIN
    bad = err > bound
    rel = err / np.maximum(s[fin], FLT_MIN)
    stats = {"max_abs": float(err.max(initial=0.0)), "max_rel": float(rel.max(initial=0.0))}
    if bad.any():
        i = np.argmax(err - bound)
        raise AssertionError(f"{what}: {int(bad.sum())} elements beyond 1e-5 "
                             f"(worst got {got[fin][i]!r} ref {ref[fin][i]!r}); {stats}")
    return stats


def bf16_value(bits):
    return (np.asarray(bits).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def check_bf16(got_bits, ref_bits, what="", max_ulp=1, abs_floor=None, cond=None):
    """Within max_ulp bf16 ulps of the rounded oracle. With abs_floor, an
    element also passes if |g - o| <= abs_floor * max(|o|, 1) (outputs formed
    by cancellation; the histogram still reports their ulp distance).
    With cond = (ref, scale), the oracle's unrounded values and the magnitude
    its fp32 error scales with, an element also passes if
    |g - ref| <= 1e-5 * scale + 2^-8 * max(|g|, |ref|): the fp32 rule, plus
    the one rounding to bf16 of the result."""
    d = np.abs(ordered(got_bits) - ordered(ref_bits))
    hist = {"0": int((d == 0).sum()), "1": int((d == 1).sum()), ">1": int((d > 1).sum())}
    if abs_floor is not None and hist[">1"]:
        g, o = bf16_value(got_bits), bf16_value(ref_bits)
        near = np.abs(g - o) <= abs_floor * np.maximum(np.abs(o), 1.0)
        d = np.where(near, 0, d)
    if cond is not None and hist[">1"]:
        ref, scale = (np.asarray(a, dtype=np.float64) for a in cond)
        g = bf16_value(got_bits)
        near = np.abs(g - ref) <= REL * scale + 2.0 ** -8 * np.maximum(np.abs(g), np.abs(ref))
        d = np.where(near, 0, d)
    if d.max(initial=0) > max_ulp:
        i = int(np.argmax(d))
        raise AssertionError(f"{what}: max ulp {int(d.max())} at flat index {i} "
                             f"(got {int(got_bits.reshape(-1)[i]):#06x} ref {int(ref_bits.reshape(-1)[i]):#06x}); {hist}")
    return hist
