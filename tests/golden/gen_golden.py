"""Write the frozen oracle outputs in tests/golden/*.txt.

The pages print no worked example for these operations (the benchmark table
of "Engineering a CUDA Machine Learning Framework from Scratch" §5 did not
survive), so no stored value comes from the pages. These fixtures are a
regression guard on the oracle itself: tiny seeded inputs and the oracle's
float64 outputs, written by this script, which calls only oracle/ and the
seeded input generators. They are not pins; the pins are in
tests/test_oracle_pins.py.

Run: python tests/golden/gen_golden.py
"""
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
import workloads  # noqa: E402


def cases():
    w = workloads.make("softmax_f32", rows=3, cols=7, seed=11)
    yield "softmax_f32_3x7", {"x": w["x"]}, {"p": oracle.softmax(w["x"])}
    w = workloads.make("softmax_bf16", rows=2, cols=9, seed=12)
    p = oracle.softmax(w["x"])
    yield "softmax_bf16_2x9", {"x": w["x"]}, {"p": p, "p_bf16": oracle.round_bf16(p)}
    w = workloads.make("layernorm_f32", rows=3, cols=5, seed=13)
    y, mean, rstd = oracle.layernorm(w["x"], w["gamma"], w["beta"], w.eps)
    yield "layernorm_f32_3x5", {"x": w["x"], "gamma": w["gamma"], "beta": w["beta"],
                                "eps": np.float32(w.eps)}, {"y": y, "mean": mean, "rstd": rstd}
    w = workloads.make("add_rmsnorm_bf16", rows=2, cols=6, seed=14)
    y, h, rstd = oracle.add_rmsnorm(w["x"], w["residual"], w["weight"], w.eps)
    yield "add_rmsnorm_bf16_2x6", {"x": w["x"], "residual": w["residual"], "weight": w["weight"],
                                   "eps": np.float32(w.eps)}, \
        {"y": y, "h": h, "y_bf16": oracle.round_bf16(y), "h_bf16": oracle.round_bf16(h)}
    w = workloads.make("xent_f32", rows=3, cols=5, seed=15)
    loss, grad, am = oracle.softmax_xent(w["logits"], w["labels"])
    yield "xent_f32_3x5", {"logits": w["logits"], "labels": w["labels"]}, \
        {"loss": loss, "grad": grad, "argmax": am}


def fmt(a):
    a = np.asarray(a)
    shape = "x".join(str(s) for s in a.shape) or "scalar"
    if a.dtype == np.float64:
        vals = [float(v).hex() for v in a.reshape(-1)]
    elif a.dtype == np.float32:
        vals = [float(v).hex() for v in a.astype(np.float64).reshape(-1)]
    else:
        vals = [str(int(v)) for v in a.reshape(-1)]
    return f"{a.dtype.name} {shape} " + " ".join(vals)


def main():
    for name, inputs, outputs in cases():
        path = os.path.join(HERE, name + ".txt")
        with open(path, "w") as f:
            f.write(f"# {name}: frozen oracle output (written by tests/golden/gen_golden.py;\n")
            f.write("# regression guard for the oracle, not a pin). Floats in C99 hex.\n")
            for k, v in inputs.items():
                f.write(f"in {k} {fmt(v)}\n")
            for k, v in outputs.items():
                f.write(f"out {k} {fmt(v)}\n")
        print(path)


if __name__ == "__main__":
    main()
