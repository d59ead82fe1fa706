"""Seeded input generators: determinism, shapes, dtypes and distributions."""
import numpy as np
import pytest

import workloads


@pytest.mark.parametrize("name", [n for n in workloads.WORKLOADS if n != "attention_bf16"])
def test_deterministic_and_shaped(name):
    a = workloads.make(name, rows=8, cols=300)
    b = workloads.make(name, rows=8, cols=300)
    assert a.digest() == b.digest()
    c = workloads.make(name, rows=8, cols=300, seed=a.seed + 1)
    assert c.digest() != a.digest()
    first = next(iter(a.arrays.values()))
    assert first.shape == (8, 300)
    assert first.dtype == (np.float32 if a.spec.dtype == "f32" else np.uint16)
    assert first.flags.c_contiguous


def test_distributions():
    w = workloads.make("softmax_f32", rows=64, cols=1000)
    assert abs(w["x"].std() - 4.0) < 0.05 and abs(w["x"].mean()) < 0.05
    w = workloads.make("layernorm_f32", rows=256, cols=1024)
    assert abs(w["x"].mean() - 3.0) < 0.02 and abs(w["x"].std() - 2.0) < 0.02
    assert w["gamma"].min() >= 0.5 and w["gamma"].max() <= 1.5
    assert abs(w["beta"].var() - 0.1) < 0.02
    w = workloads.make("xent_f32", rows=64, cols=50257)
    assert abs(w["logits"].std() - 2.0) < 0.01
    assert w["labels"].dtype == np.int32 and w["labels"].min() >= 0 and w["labels"].max() < 50257
    w = workloads.make("softmax_bf16", rows=64, cols=4096)
    s = w["row_scale"]
    assert s.min() >= 1.0 and s.max() <= 60.0
    w = workloads.make("add_rmsnorm_bf16", rows=4, cols=8192)
    wt = (w["weight"].astype(np.uint32) << 16).view(np.float32)
    assert wt.min() >= 0.79 and wt.max() <= 1.21


def test_backward_distributions():
    def f(b):
        return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    w = workloads.make("add_rmsnorm_bwd_bf16", rows=64, cols=4096)
    assert abs(f(w["h"]).var() - 2.0) < 0.03
    assert abs(f(w["dy"]).std() - 1.0) < 0.01 and abs(f(w["dres"]).std() - 1.0) < 0.01
    w = workloads.make("layernorm_bwd_f32", rows=64, cols=1024)
    assert abs(w["x"].mean() - 3.0) < 0.03 and abs(w["dy"].std() - 1.0) < 0.01
    w = workloads.make("softmax_bwd_bf16", rows=64, cols=4096)
    assert set(w.arrays) == {"x", "dy"}


def test_bf16_storage_rounding():
    v = np.array([1.0, 1 + 2**-8, 1 + 3 * 2**-8, -2.5, 3.0e38], dtype=np.float32)
    assert list(workloads.f32_to_bf16_bits(v)) == [0x3F80, 0x3F80, 0x3F82, 0xC020, 0x7F62]


def test_attention_inputs():
    a = workloads.make_attention(2, 3, 5, 7, 64, seed=1)
    b = workloads.make_attention(2, 3, 5, 7, 64, seed=1)
    assert a.digest() == b.digest()
    assert a["q"].shape == (2, 3, 5, 64) and a["k"].shape == (2, 3, 7, 64) and a["q"].dtype == np.uint16
