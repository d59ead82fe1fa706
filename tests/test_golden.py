"""The oracle still reproduces its frozen outputs in tests/golden/ (a regression
guard on the oracle's arithmetic; the pins live in test_oracle_pins.py)."""
import glob
import os

import numpy as np

import oracle

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _parse(path):
    ins, outs = {}, {}
    for line in open(path):
        if line.startswith("#") or not line.strip():
            continue
        kind, key, dtype, shape, *vals = line.split()
        shp = () if shape == "scalar" else tuple(int(s) for s in shape.split("x"))
        if dtype in ("float64", "float32"):
            a = np.array([float.fromhex(v) for v in vals], dtype=np.float64).astype(dtype)
        else:
            a = np.array([int(v) for v in vals], dtype=dtype)
        (ins if kind == "in" else outs)[key] = a.reshape(shp)
    return ins, outs


def _run(name, ins):
    if name.startswith("softmax_"):
        p = oracle.softmax(ins["x"])
        return {"p": p, "p_bf16": oracle.round_bf16(p)}
    if name.startswith("layernorm"):
        y, m, r = oracle.layernorm(ins["x"], ins["gamma"], ins["beta"], float(ins["eps"]))
        return {"y": y, "mean": m, "rstd": r}
    if name.startswith("add_rmsnorm"):
        y, h, _ = oracle.add_rmsnorm(ins["x"], ins["residual"], ins["weight"], float(ins["eps"]))
        return {"y": y, "h": h, "y_bf16": oracle.round_bf16(y), "h_bf16": oracle.round_bf16(h)}
    if name.startswith("xent"):
        loss, grad, am = oracle.softmax_xent(ins["logits"], ins["labels"])
        return {"loss": loss, "grad": grad, "argmax": am}
    raise KeyError(name)


def test_golden_files_reproduce():
    files = sorted(glob.glob(os.path.join(HERE, "*.txt")))
    assert len(files) >= 5
    for path in files:
        name = os.path.basename(path)[:-4]
        ins, outs = _parse(path)
        got = _run(name, ins)
        for k, ref in outs.items():
            g = np.asarray(got[k])
            if ref.dtype == np.float64:
                assert np.max(np.abs(g - ref) / np.maximum(np.abs(ref), 1e-300)) <= 1e-15, (name, k)
            else:
                assert np.array_equal(g.astype(ref.dtype), ref), (name, k)
