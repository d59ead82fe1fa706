"""Benchmark of the fused row kernels on one MI355X.

One step is one pass of the whole hot path over one batch of each workload:
five launches on the current stream, in this order
  softmax fp32 [64, 1000]; LayerNorm fp32 [4096, 1024]; softmax bf16
  [16384, 4096]; residual-add + RMSNorm bf16 [8192, 8192]; softmax
  cross-entropy fwd+bwd fp32 [4096, 50257].
Inputs are seeded synthetic data resident in HBM before timing starts. One
step moves 2.49 GB, so by the time a workload's buffers come round again the
256 MB last-level cache has been swept: every launch reads HBM.

value = algorithmic bytes of one step (each input element read once, each
output element written once) / wall time of one step, in GB/s; per-launch
durations come from a second pass with HIP events recorded around each launch
on the stream the kernels run on. With --graph the timed steps replay one
captured HIP graph of the five launches.

Printed: ONE JSON line (rank 0), with per-workload figures, the roofline of
the dominant kernel (the cross-entropy launch), the memory ceilings measured
in the same run with the library's probes (the best read-only, write-only and
copy patterns, and for each large workload the copy of its own row geometry),
and the CPU oracle timed on the host cores as a baseline.

The backward entry points are measured after the step, per call, at the
forward workloads' shapes (softmax bf16 [16384, 4096], LayerNorm fp32
[4096, 1024], residual-add + RMSNorm bf16 [8192, 8192] with the residual's
gradient and the plain RMSNorm backward without it), and so are the
cross-entropy variants (fr_softmax_xent_ex at [4096, 50257], fp32 and bf16
logits, every 9th row ignored, label smoothing 0.1, mean reduction) and the
split-row cross-entropy at vocabulary widths beyond one workgroup (fp32
[2048, 131072], bf16 [1024, 262144]), the split-row norms (LayerNorm fp32
[512, 131072], residual-add + RMSNorm bf16 [256, 262144]), the split-row
softmax backward (bf16 [1024, 131072]), one GPU's share of an 8-way
row-sharded cross-entropy step (fp32 [512, 50257], the row kernel and the
split-row path) and the split-row residual-add +
RMSNorm backward (bf16 [2048, 32768], hidden size beyond the one-pass
backward); they are
reported under "backward" and "variants" and are not part of `value`; so is the
attention forward (bf16 B=4 H=16 S=4096 D=128, causal and not), reported
under "attention" in matrix TFLOP/s against the bf16 peak and against the
matrix-core probe's rate measured in the same run. Their per-row inputs from the
forward (p, mean, rstd) are produced by the forward kernels before timing.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                      [--no-backward] [--graph]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0  # MI355X HBM3E, published peak
METRIC = "achieved HBM GB/s (% of MI355X peak) and rows/s, fused row softmax/norm"
DOMINANT = "xent_f32"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "xent_f32_4096x50257_traffic.json")
KERNEL_SOURCES = ["xent.hip", "softmax_core.hpp", "fr_device.hpp"]


def algo_bytes(name, R, C):
    """Each input element read once, each output element written once."""
    if name == "softmax_f32":
        return R * C * 4 * 2
    if name == "layernorm_f32":
        return R * C * 4 * 2 + 2 * C * 4 + 2 * R * 4          # x, y; gamma, beta; mean, rstd
    if name == "softmax_bf16":
        return R * C * 2 * 2
    if name == "add_rmsnorm_bf16":
        return 4 * R * C * 2 + C * 2                           # x, r, y, r_out; w
    if name == "xent_f32":
        return 2 * R * C * 4 + R * 4 + R * 4                   # logits, grad; labels, loss
    raise KeyError(name)


def bwd_algo_bytes(name, R, C):
    """Backward: each row operand and parameter read once, each gradient
    written once (the partial sums in the workspace are not counted)."""
    if name == "softmax_bwd_bf16":
        return 3 * R * C * 2                                   # p, dy; dx
    if name == "layernorm_bwd_f32":
        return 3 * R * C * 4 + C * 4 + 2 * R * 4 + 2 * C * 4   # x, dy, dx; gamma; mean, rstd; dg, db
    if name == "add_rmsnorm_bwd_bf16":
        return 4 * R * C * 2 + C * 2 + C * 4                   # h, dy, dres, dh; w; dw
    if name == "rmsnorm_bwd_bf16":
        return 3 * R * C * 2 + C * 2 + C * 4                   # h, dy, dh; w; dw
    if name in ("xent_shard_f32", "xent_shard_split_f32"):
        return 2 * R * C * 4 + 2 * R * 4                       # logits, grad; labels, loss
    if name in ("xent_split_f32", "xent_split_bf16"):
        # one read of the logits and one write of the gradient (the split path's
        # one-pass form moves these bytes, its two passes 1.5x); labels, loss
        es = 4 if name == "xent_split_f32" else 2
        return 2 * R * C * es + 2 * R * 4
    if name == "add_rmsnorm_bwd_split_bf16":
        return 4 * R * C * 2 + C * 2 + C * 4                   # h, dy, dres, dh; w; dw
    if name == "softmax_bwd_split_bf16":
        return 3 * R * C * 2                                   # p, dy; dx (two passes read p, dy twice)
    if name == "layernorm_split_f32":
        # x, y; gamma, beta; mean, rstd (two passes read x twice)
        return 2 * R * C * 4 + 2 * C * 4 + 2 * R * 4
    if name == "add_rmsnorm_split_bf16":
        # x, r, y, r_out; w (two passes read x and r twice)
        return 4 * R * C * 2 + C * 2
    if name in ("xent_ex_f32", "xent_ex_bf16"):
        # logits of the rows not ignored (every 9th row is), grad of all rows;
        # labels, loss; total
        es = 4 if name == "xent_ex_f32" else 2
        read_rows = R - len(range(0, R, 9))
        return read_rows * C * es + R * C * es + 2 * R * 4 + 4
    raise KeyError(name)


class BwdWorkload:
    def __init__(self, name, w, dev, torch, fr):
        import numpy as np
        self.name, self.w = name, w
        self.R, self.C = w.rows, w.cols
        self.bytes = bwd_algo_bytes(name, self.R, self.C)

        def d(a):
            if a.dtype == np.uint16:
                return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
            return torch.from_numpy(a).to(dev)

        def ws(op):
            n = fr.fr_norm_bwd_workspace_bytes(op, self.R, self.C)
            return torch.empty(max(n, 16), dtype=torch.uint8, device=dev)

        if name == "softmax_bwd_bf16":
            self.p = fr.softmax(d(w["x"]))
            self.dy = d(w["dy"])
            self.dx = torch.empty_like(self.p)
            self.run = lambda: fr.fr_softmax_bwd(self.p, self.dy, self.dx)
            self.op, self.code = fr.OP_SOFTMAX_BWD, fr.BF16
        elif name == "layernorm_bwd_f32":
            self.x, self.g, self.dy = d(w["x"]), d(w["gamma"]), d(w["dy"])
            _, self.mean, self.rstd = fr.layernorm(self.x, self.g, torch.zeros_like(self.g), w.eps)
            self.dx = torch.empty_like(self.x)
            self.dg = torch.empty(self.C, device=dev)
            self.db = torch.empty(self.C, device=dev)
            self.ws = ws(fr.OP_LAYERNORM_BWD)
            self.run = lambda: fr.fr_layernorm_bwd(self.x, self.dy, self.g, self.mean, self.rstd,
                                                   self.dx, self.dg, self.db, self.ws)
            self.op, self.code = fr.OP_LAYERNORM_BWD, fr.F32
        elif name in ("xent_ex_f32", "xent_ex_bf16"):
            # cross-entropy with options at the cross-entropy shape: every 9th
            # row ignored, label smoothing 0.1, mean reduction
            self.x, lab = d(w["logits"]), w["labels"].copy()
            lab[::9] = -100
            self.lab = d(lab)
            self.loss = torch.empty(self.R, device=dev)
            self.grad = torch.empty_like(self.x)
            self.tot = torch.empty(1, device=dev)
            self.run = lambda: fr.fr_softmax_xent_ex(self.x, self.lab, self.loss, self.grad, None,
                                                     self.tot, ignore_index=-100,
                                                     label_smoothing=0.1, reduction="mean")
            self.op = fr.OP_XENT
            self.code = fr.BF16 if name == "xent_ex_bf16" else fr.F32
        elif name == "xent_shard_f32":
            # one GPU's share of an 8-way row-sharded cross-entropy step
            self.x, self.lab = d(w["logits"]), d(w["labels"])
            self.loss = torch.empty(self.R, device=dev)
            self.grad = torch.empty_like(self.x)
            self.run = lambda: fr.fr_softmax_xent_fwd_bwd(self.x, self.lab, self.loss, self.grad)
            self.op, self.code = fr.OP_XENT, fr.F32
        elif name in ("xent_split_f32", "xent_split_bf16", "xent_shard_split_f32"):
            # wide vocabularies through the split-row path, no options
            self.x, self.lab = d(w["logits"]), d(w["labels"])
            self.loss = torch.empty(self.R, device=dev)
            self.grad = torch.empty_like(self.x)
            self.ws = torch.empty(fr.fr_split_workspace_bytes(self.R, self.C), dtype=torch.uint8,
                                  device=dev)
            self.run = lambda: fr.fr_softmax_xent_split(self.x, self.lab, self.loss, self.grad,
                                                        self.ws)
            self.op = fr.OP_XENT_SPLIT
            self.code = fr.BF16 if name == "xent_split_bf16" else fr.F32
        elif name == "add_rmsnorm_bwd_split_bf16":
            # hidden size beyond the one-pass backward: the split-row path
            self.h, self.dy, self.dres = d(w["h"]), d(w["dy"]), d(w["dres"])
            self.wt = d(w["weight"])
            self.dh = torch.empty_like(self.h)
            self.dw = torch.empty(self.C, device=dev)
            self.ws = torch.empty(fr.fr_norm_bwd_split_workspace_bytes(fr.OP_RMSNORM_BWD, self.R,
                                                                       self.C),
                                  dtype=torch.uint8, device=dev)
            self.run = lambda: fr.fr_add_rmsnorm_bwd_split(self.h, self.dy, self.wt, self.dh,
                                                           self.dw, self.ws, dres=self.dres,
                                                           eps=w.eps)
            # one fixed shape (no variant table): 512 lanes x 2 x 8 per segment
            self.op, self.code, self.variant = None, fr.BF16, (512, 2, 8)
        elif name == "softmax_bwd_split_bf16":
            # wide softmax backward rows through the split-row path
            self.p = fr.softmax(d(w["x"]))
            self.dy = d(w["dy"])
            self.dx = torch.empty_like(self.p)
            self.ws = torch.empty(fr.fr_split_workspace_bytes(self.R, self.C), dtype=torch.uint8,
                                  device=dev)
            self.run = lambda: fr.fr_softmax_bwd_split(self.p, self.dy, self.dx, self.ws)
            self.op, self.code = fr.OP_SOFTMAX_BWD_SPLIT, fr.BF16
        elif name == "layernorm_split_f32":
            # wide LayerNorm rows through the split-row path
            self.x, self.g, self.b = d(w["x"]), d(w["gamma"]), d(w["beta"])
            self.y = torch.empty_like(self.x)
            self.mean = torch.empty(self.R, device=dev)
            self.rstd = torch.empty(self.R, device=dev)
            self.ws = torch.empty(fr.fr_split_workspace_bytes(self.R, self.C), dtype=torch.uint8,
                                  device=dev)
            self.run = lambda: fr.fr_layernorm_fwd_split(self.x, self.g, self.b, self.y, self.ws,
                                                         self.mean, self.rstd, w.eps)
            self.op, self.code = fr.OP_LAYERNORM_SPLIT, fr.F32
        elif name == "add_rmsnorm_split_bf16":
            self.x, self.r, self.wt = d(w["x"]), d(w["residual"]), d(w["weight"])
            self.y = torch.empty_like(self.x)
            self.ro = torch.empty_like(self.x)
            self.ws = torch.empty(fr.fr_split_workspace_bytes(self.R, self.C), dtype=torch.uint8,
                                  device=dev)
            self.run = lambda: fr.fr_add_rmsnorm_fwd_split(self.x, self.r, self.wt, self.y, self.ws,
                                                           self.ro, w.eps)
            self.op, self.code = fr.OP_RMSNORM_SPLIT, fr.BF16
        elif name in ("add_rmsnorm_bwd_bf16", "rmsnorm_bwd_bf16"):
            # with the gradient through the updated residual (dres), and the
            # plain RMSNorm backward without it
            self.h, self.dy, self.dres = d(w["h"]), d(w["dy"]), d(w["dres"])
            self.wt = d(w["weight"])
            self.dh = torch.empty_like(self.h)
            self.dw = torch.empty(self.C, device=dev)
            self.ws = ws(fr.OP_RMSNORM_BWD)
            dres = self.dres if name == "add_rmsnorm_bwd_bf16" else None
            self.run = lambda: fr.fr_add_rmsnorm_bwd(self.h, self.dy, self.wt, self.dh, self.dw,
                                                     self.ws, dres=dres, eps=w.eps)
            self.op, self.code = fr.OP_RMSNORM_BWD, fr.BF16
        if self.op is not None:
            self.variant = fr.fr_debug_select_variant_for(self.op, self.R, self.C, self.code)


def time_calls(torch, np, runs, K):
    """Per-call durations (us) of each callable, HIP events around each call
    on the current stream, K rounds of all of them in turn."""
    evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in runs] for _ in range(K)]
    for k in range(K):
        for run, (a, b) in zip(runs, evs[k]):
            a.record()
            run()
            b.record()
    torch.cuda.synchronize()
    return [np.array([evs[k][i][0].elapsed_time(evs[k][i][1]) * 1e3 for k in range(K)])
            for i in range(len(runs))]


def launch_stats(w, us):
    import numpy as np
    med, mean = float(np.median(us)), float(us.mean())
    return {
        "rows": w.R, "cols": w.C, "algo_bytes": w.bytes,
        "variant": {"threads": w.variant[0], "vecs": w.variant[1], "elems_per_vec": w.variant[2]},
        "median_us": round(med, 3), "mean_us": round(mean, 3),
        "p10_us": round(float(np.percentile(us, 10)), 3),
        "p90_us": round(float(np.percentile(us, 90)), 3),
        "gbps": round(w.bytes / (med * 1e-6) / 1e9, 1),
        "pct_peak": round(100 * w.bytes / (med * 1e-6) / 1e9 / PEAK_HBM_GBPS, 2),
        "rows_per_s": round(w.R / (med * 1e-6), 1),
        "dtype": "bf16" if w.code == 1 else "f32",
        "seed": w.w.seed,
        "input_sha256": w.w.digest()[:16],
    }


PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak, published


MFMA_PROBE_ITERS = 2048


def mfma_ceiling(torch, np, fr, dev, K):
    """The matrix-core probe (fr_mfma_probe): bf16 32x32x16 matrix
    instructions with no operand traffic and no vector work, three workgroups
    of four wavefronts per compute unit (three wavefronts per SIMD, as the
    attention kernel runs); TFLOP/s from the median of K event-timed calls,
    with pseudo-random operands (full mantissas, as real data: the ceiling)
    and with constant ones (less switching, a higher clock held)."""
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    wg = 3 * cus
    sink = torch.empty(wg * 256, device=dev)
    runs = [lambda: fr.fr_mfma_probe(wg, MFMA_PROBE_ITERS, sink, pattern=1),
            lambda: fr.fr_mfma_probe(wg, MFMA_PROBE_ITERS, sink, pattern=0)]
    for r in runs:
        for _ in range(3):
            r()
    torch.cuda.synchronize()
    us = [float(np.median(u)) for u in time_calls(torch, np, runs, max(5, min(K, 20)))]
    flops = wg * 4.0 * MFMA_PROBE_ITERS * 8 * 32768
    tf = [flops / (u * 1e-6) / 1e12 for u in us]
    return {"tflops": round(tf[0], 1), "median_us": round(us[0], 2),
            "frac_of_bf16_peak": round(tf[0] / PEAK_BF16_TFLOPS, 4),
            "constant_operands_tflops": round(tf[1], 1),
            "constant_operands_frac_of_bf16_peak": round(tf[1] / PEAK_BF16_TFLOPS, 4),
            "workgroups": wg, "iters": MFMA_PROBE_ITERS, "flops": flops}


def attention_stats(torch, np, fr, workloads, dev, K):
    """Attention forward, bf16, B=4 H=16 S=4096 D=128, causal and not: per
    call duration (HIP events) and matrix TFLOP/s against the bf16 peak and
    against the matrix-core probe's rate measured in the same run.
    Flops: 4 B H Sq Sk D (two products), half of that when causal."""
    w = workloads.make_attention(4, 16, 4096, 4096, 128)

    def d(a):
        return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)

    q, k, v = d(w["q"]), d(w["k"]), d(w["v"])
    o = torch.empty_like(q)
    lse = torch.empty(4, 16, 4096, device=dev)
    runs = [lambda: fr.fr_attention_fwd(q, k, v, o, lse, False),
            lambda: fr.fr_attention_fwd(q, k, v, o, lse, True)]
    for r in runs:
        for _ in range(3):
            r()
    torch.cuda.synchronize()
    us = time_calls(torch, np, runs, max(5, min(K, 20)))
    ceil = mfma_ceiling(torch, np, fr, dev, K)
    out = {"mfma_ceiling": ceil}
    flops = 4.0 * 64 * 4096 * 4096 * 128
    for name, u, f in (("attention_bf16_b4h16s4096d128", us[0], flops),
                       ("attention_bf16_b4h16s4096d128_causal", us[1], flops / 2)):
        med = float(np.median(u))
        tf = f / (med * 1e-6) / 1e12
        out[name] = {"median_us": round(med, 2), "tflops": round(tf, 1),
                     "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                     "frac_of_mfma_ceiling": round(tf / ceil["tflops"], 4), "flops": f,
                     "input_sha256": w.digest()[:16]}
    return out


def kernel_source_digest():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "memory_bound_row_pass_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per cross-entropy launch from the committed counter summary,
    or None when there is none or the kernel source changed since."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256") != kernel_source_digest():
        return None
    return t.get("bytes_per_launch")


class Workload:
    def __init__(self, name, w, dev, torch, fr):
        import numpy as np
        self.name, self.w = name, w
        self.R, self.C = w.rows, w.cols
        self.bytes = algo_bytes(name, self.R, self.C)

        def d(a):
            if a.dtype == np.uint16:
                return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
            return torch.from_numpy(a).to(dev)

        self.torch, self.fr = torch, fr
        if name in ("softmax_f32", "softmax_bf16"):
            self.x = d(w["x"])
            self.y = torch.empty_like(self.x)
            self.run = lambda: fr.fr_softmax_fwd(self.x, self.y)
            self.op, self.code = fr.OP_SOFTMAX, (fr.BF16 if name == "softmax_bf16" else fr.F32)
        elif name == "layernorm_f32":
            self.x, self.g, self.b = d(w["x"]), d(w["gamma"]), d(w["beta"])
            self.y = torch.empty_like(self.x)
            self.mean = torch.empty(self.R, device=dev)
            self.rstd = torch.empty(self.R, device=dev)
            self.run = lambda: fr.fr_layernorm_fwd(self.x, self.g, self.b, self.y, self.mean,
                                                   self.rstd, w.eps)
            self.op, self.code = fr.OP_LAYERNORM, fr.F32
        elif name == "add_rmsnorm_bf16":
            self.x, self.r, self.wt = d(w["x"]), d(w["residual"]), d(w["weight"])
            self.y = torch.empty_like(self.x)
            self.ro = torch.empty_like(self.x)
            self.run = lambda: fr.fr_add_rmsnorm_fwd(self.x, self.r, self.wt, self.y, self.ro, w.eps)
            self.op, self.code = fr.OP_RMSNORM, fr.BF16
        elif name == "xent_f32":
            self.x, self.lab = d(w["logits"]), d(w["labels"])
            self.loss = torch.empty(self.R, device=dev)
            self.grad = torch.empty_like(self.x)
            self.run = lambda: fr.fr_softmax_xent_fwd_bwd(self.x, self.lab, self.loss, self.grad)
            self.op, self.code = fr.OP_XENT, fr.F32
        self.variant = fr.fr_debug_select_variant_for(self.op, self.R, self.C, self.code)


# Memory ceilings, from the library's probes (fr_stream_probe: the row
# kernels' access pattern with no arithmetic; a copy waits for a row's loads
# before its stores, as a row kernel's reduction does). General patterns over
# 2 GiB: the best read-only, write-only and copy (read + write) rates among
# the shapes and cache policies swept on MI355X. (threads, vecs, policy):
# policy 1 = non-temporal loads and cached stores, 3 = both non-temporal,
# 0 = cached.
GENERAL_PROBES = {
    "copy": [(256, 1, 1), (256, 1, 3), (512, 1, 1), (64, 4, 3)],
    "read": [(512, 2, 1), (256, 2, 1)],
    "write": [(256, 1, 0), (512, 1, 0)],
}
# Each large workload's own row geometry and cache policy (non-temporal loads
# and stores, as the kernels use): (threads, vecs, policy, row bytes, bytes
# copied). The residual-add + RMSNorm row has two inputs and two outputs:
# twice the rows of one 16 KiB operand. The cross-entropy rows of 201,028 B
# (fp32) and 100,514 B (bf16, the options variant) are probed at 201,040 B
# and 100,512 B (whole 16-byte chunks).
PATTERN_PROBES = {
    "layernorm_f32": (64, 4, 3, 4096, 4096 * 4096),
    "softmax_bf16": (128, 4, 3, 8192, 16384 * 8192),
    "add_rmsnorm_bf16": (512, 2, 3, 16384, 2 * 8192 * 16384),
    "xent_f32": (1024, 13, 3, 201040, 4096 * 201040),
    "xent_ex_bf16": (1024, 7, 3, 100512, 4096 * 100512),
}


def memory_ceilings(torch, np, fr, dev, K):
    """GB/s of the general probe patterns (best of each kind) and of each
    workload's same-geometry copy: median per-launch time over K rounds of all
    probes in turn (each probe's buffers are cold, as the workloads' are)."""
    nb = 2 << 30
    src = torch.empty(nb // 4, dtype=torch.int32, device=dev).fill_(1)
    dst = torch.empty_like(src)
    sink = torch.empty(nb // 4096 + 16, dtype=torch.int32, device=dev)
    runs, names, nbytes = [], [], []

    def add(name, mode, t, v, pol, n, row_bytes=0):
        runs.append(lambda: fr.fr_stream_probe(mode, src=src if mode != fr.PROBE_WRITE else None,
                                               dst=dst if mode != fr.PROBE_READ else None,
                                               nbytes=n, value=1,
                                               sink=sink if mode == fr.PROBE_READ else None,
                                               threads=t, vecs=v, policy=pol,
                                               row_bytes=row_bytes))
        names.append(name)
        nbytes.append(2 * n if mode == fr.PROBE_COPY else n)

    modes = {"copy": fr.PROBE_COPY, "read": fr.PROBE_READ, "write": fr.PROBE_WRITE}
    for kind, shapes in GENERAL_PROBES.items():
        for (t, v, pol) in shapes:
            add(f"{kind} {t}x{v} policy {pol}", modes[kind], t, v, pol, nb)
    for wl, (t, v, pol, rb, n) in PATTERN_PROBES.items():
        add(f"pattern {wl}", fr.PROBE_COPY, t, v, pol, n, rb)
    for r in runs:
        r()
    torch.cuda.synchronize()
    us = time_calls(torch, np, runs, max(5, min(K, 20)))
    rates = {n: b / (float(np.median(u)) * 1e-6) / 1e9 for n, u, b in zip(names, us, nbytes)}
    del src, dst, sink
    best = {}
    for kind in GENERAL_PROBES:
        name = max((n for n in rates if n.startswith(kind + " ")), key=rates.get)
        best[kind] = {"gbps": round(rates[name], 1), "probe": name + " (2 GiB)"}
    pattern = {wl: round(rates[f"pattern {wl}"], 1) for wl in PATTERN_PROBES}
    return best, pattern, {n: round(r, 1) for n, r in rates.items()}


def cpu_baseline(wls, budget_s=15.0):
    """The oracle (plain double-precision C, OpenMP over rows) on the host
    cores over the same inputs: full steps, repeated while within budget;
    then the two small workloads (softmax fp32 64x1000, LayerNorm fp32
    4096x1024) again on one thread. Returns the baseline record and the last
    step's oracle outputs."""
    import oracle
    oracle.set_threads(int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1)))
    threads = oracle.threads()
    total_bytes = sum(w.bytes for w in wls)

    per_ms = {w.name: [] for w in wls}

    def one_step():
        out = {}
        for w in wls:
            a = w.w
            t1 = time.perf_counter()
            if w.name in ("softmax_f32", "softmax_bf16"):
                out[w.name] = (oracle.softmax(a["x"]),)
            elif w.name == "layernorm_f32":
                out[w.name] = oracle.layernorm(a["x"], a["gamma"], a["beta"], a.eps)
            elif w.name == "add_rmsnorm_bf16":
                y, h, _ = oracle.add_rmsnorm(a["x"], a["residual"], a["weight"], a.eps)
                out[w.name] = (oracle.round_bf16(y), oracle.round_bf16(h))
            elif w.name == "xent_f32":
                out[w.name] = oracle.softmax_xent(a["logits"], a["labels"])[:2]
            per_ms[w.name].append((time.perf_counter() - t1) * 1e3)
        return out

    t0 = time.perf_counter()
    n = 0
    while True:
        outs = one_step()
        n += 1
        el = time.perf_counter() - t0
        if el > budget_s / 2 or n >= 3:
            break
    per_step = el / n
    per_workload = {}
    for w in wls:
        ms = sorted(per_ms[w.name])[len(per_ms[w.name]) // 2]
        per_workload[w.name] = {"oracle_ms": round(ms, 2), "threads": threads,
                                "gbps": round(w.bytes / (ms * 1e-3) / 1e9, 2),
                                "rows_per_s": round(w.R / (ms * 1e-3), 1)}
    # one thread, the small workloads: median of 3 runs
    oracle.set_threads(1)
    for w in wls:
        if w.name not in ("softmax_f32", "layernorm_f32"):
            continue
        a, ts = w.w, []
        for _ in range(3):
            t1 = time.perf_counter()
            if w.name == "softmax_f32":
                oracle.softmax(a["x"])
            else:
                oracle.layernorm(a["x"], a["gamma"], a["beta"], a.eps)
            ts.append((time.perf_counter() - t1) * 1e3)
        ms = sorted(ts)[1]
        per_workload[w.name]["one_thread"] = {
            "oracle_ms": round(ms, 3), "threads": 1,
            "gbps": round(w.bytes / (ms * 1e-3) / 1e9, 3),
            "rows_per_s": round(w.R / (ms * 1e-3), 1)}
    oracle.set_threads(threads)
    return ({"value": total_bytes / per_step / 1e9, "unit": "GB/s", "cores": threads,
             "kind": "oracle",
             "sample": f"{n} full step(s): all rows of the five workloads, "
                       f"{per_step:.2f} s per step, double precision, {threads} OpenMP threads",
             "host_cpu": host_cpu(), "nproc": os.cpu_count(),
             "per_workload": per_workload},
            outs)


def host_cpu():
    """CPU model name of the host (from /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def parity_report(wls, outs):
    """The timed step's GPU outputs (every element) against the oracle's, by
    the tests' rules: fp32 |g - o| <= 1e-5 * scale + 2^-126 (scale |o|, or
    max(|o|, 1) for LayerNorm y and the losses, max(|o|, row sd) for the mean,
    max(|o|, p) at the label), bf16 within one ulp of the rounded oracle."""
    import numpy as np
    tiny = 2.0 ** -126

    def f32(g, o, scale=None):
        g = g.astype(np.float64)
        sc = np.abs(o) if scale is None else scale
        err = np.abs(g - o)
        return {"max_abs": float(err.max()), "max_rel": float((err / np.maximum(sc, tiny)).max()),
                "pass": bool(np.all(err <= 1e-5 * sc + tiny))}

    def ordered(b):
        b = b.astype(np.int64)
        return np.where(b & 0x8000, 0x8000 - (b & 0x7FFF), 0x8000 + b)

    def bf16(g_t, o_bits):
        import torch
        gb = g_t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        d = np.abs(ordered(gb) - ordered(o_bits))
        return {"ulp_hist": {"0": int((d == 0).sum()), "1": int((d == 1).sum()),
                             ">1": int((d > 1).sum())}, "pass": bool(d.max() <= 1)}

    import oracle
    rep = {}
    for w in wls:
        o = outs[w.name]
        a = w.w
        if w.name == "softmax_f32":
            r = f32(w.y.cpu().numpy(), o[0])
            r["denormal_count"] = int(((o[0] > 0) & (o[0] < tiny)).sum())
        elif w.name == "softmax_bf16":
            r = bf16(w.y, oracle.round_bf16(o[0]))
            r["denormal_count"] = int(((o[0] > 0) & (o[0] < tiny)).sum())
        elif w.name == "layernorm_f32":
            yo, mo, ro = o
            sd = np.sqrt(oracle.decode(a["x"]).var(axis=1))
            r = {"y": f32(w.y.cpu().numpy(), yo, np.maximum(np.abs(yo), 1.0)),
                 "mean": f32(w.mean.cpu().numpy(), mo, np.maximum(np.abs(mo), sd)),
                 "rstd": f32(w.rstd.cpu().numpy(), ro)}
            r["pass"] = all(v["pass"] for v in r.values())
        elif w.name == "add_rmsnorm_bf16":
            r = {"y": bf16(w.y, o[0]), "residual_out": bf16(w.ro, o[1])}
            r["pass"] = all(v["pass"] for v in r.values())
        elif w.name == "xent_f32":
            lo, go = o
            lab = a["labels"].astype(np.int64)
            rows = np.arange(len(lab))
            sc = np.abs(go)
            sc[rows, lab] = np.maximum(sc[rows, lab], go[rows, lab] + 1.0)
            r = {"loss": f32(w.loss.cpu().numpy(), lo, np.maximum(np.abs(lo), 1.0)),
                 "grad": f32(w.grad.cpu().numpy(), go, sc)}
            r["pass"] = all(v["pass"] for v in r.values())
        rep[w.name] = r
    return rep


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward measurements")
    ap.add_argument("--graph", action="store_true",
                    help="replay the step as one captured HIP graph (the launches are capture-safe)")
    ap.add_argument("--quiet", action="store_true", help="no progress lines on stderr")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the row kernels own whole rows and need no "
              "collective; multi-GPU runs are not part of this benchmark (use --gpus 1).",
              file=sys.stderr)
        sys.exit(2)

    def log(msg):
        if not args.quiet:
            print(f"[bench] {msg}", file=sys.stderr, flush=True)

    import numpy as np  # noqa: F401
    import torch
    import memory_bound_row_pass_amd as fr
    import workloads

    dev = torch.device("cuda:0")
    names = ["softmax_f32", "layernorm_f32", "softmax_bf16", "add_rmsnorm_bf16", "xent_f32"]
    wls = []
    for n in names:
        t0 = time.perf_counter()
        wls.append(Workload(n, workloads.make(n), dev, torch, fr))
        log(f"generated {n} in {time.perf_counter() - t0:.1f} s")
    step_bytes = sum(w.bytes for w in wls)
    step_rows = sum(w.R for w in wls)

    def step():
        for w in wls:
            w.run()

    graph = None
    if args.graph:
        # the five launches of one step captured once and replayed
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        run_step = graph.replay
    else:
        run_step = step

    for _ in range(args.warmup):
        run_step()
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} steps done ({'graph replay' if graph else 'eager launches'})")

    # timed region: exactly K steps, nothing else on the stream
    K = args.steps
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(K):
        run_step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / K
    log(f"timed {K} steps: {ms_per_step:.3f} ms/step")

    # per-launch durations: a second pass with HIP events around each launch
    per = {w.name: launch_stats(w, us)
           for w, us in zip(wls, time_calls(torch, np, [w.run for w in wls], K))}

    backward, variants, attention = {}, {}, {}
    if not args.no_backward:
        bws = []
        for n in ("softmax_bwd_bf16", "layernorm_bwd_f32", "add_rmsnorm_bwd_bf16"):
            t0 = time.perf_counter()
            bws.append(BwdWorkload(n, workloads.make(n), dev, torch, fr))
            log(f"generated {n} in {time.perf_counter() - t0:.1f} s")
            if n == "add_rmsnorm_bwd_bf16":  # the same inputs, no dres
                bws.append(BwdWorkload("rmsnorm_bwd_bf16", bws[-1].w, dev, torch, fr))
        nb = len(bws)
        for n, dt in (("xent_ex_f32", "f32"), ("xent_ex_bf16", "bf16")):
            bws.append(BwdWorkload(n, workloads.make("xent_f32", dtype=dt), dev, torch, fr))
            log(f"generated {n}")
        for n, dt, R, C in (("xent_split_f32", "f32", 2048, 131072),
                            ("xent_split_bf16", "bf16", 1024, 262144),
                            ("xent_shard_f32", "f32", 512, 50257),
                            ("xent_shard_split_f32", "f32", 512, 50257)):
            bws.append(BwdWorkload(n, workloads.make("xent_f32", rows=R, cols=C, dtype=dt), dev,
                                   torch, fr))
            log(f"generated {n}")
        for n, base, dt, R, C in (("layernorm_split_f32", "layernorm_f32", "f32", 512, 131072),
                                  ("add_rmsnorm_split_bf16", "add_rmsnorm_bf16", "bf16", 256, 262144),
                                  ("softmax_bwd_split_bf16", "softmax_bwd_bf16", "bf16", 1024, 131072),
                                  ("add_rmsnorm_bwd_split_bf16", "add_rmsnorm_bwd_bf16", "bf16", 2048,
                                   32768)):
            bws.append(BwdWorkload(n, workloads.make(base, rows=R, cols=C, dtype=dt), dev, torch, fr))
            log(f"generated {n}")
        for _ in range(max(3, args.warmup)):
            for b in bws:
                b.run()
        torch.cuda.synchronize()
        timed = {b.name: launch_stats(b, us)
                 for b, us in zip(bws, time_calls(torch, np, [b.run for b in bws], K))}
        backward = {b.name: timed[b.name] for b in bws[:nb]}
        variants = {b.name: timed[b.name] for b in bws[nb:]}
        log("backward and variant calls timed")
        del bws
        attention = attention_stats(torch, np, fr, workloads, dev, K)
        log("attention timed")

    best, pattern, probes = memory_ceilings(torch, np, fr, dev, K)
    ceiling = best["copy"]["gbps"]
    log(f"memory ceilings: read {best['read']['gbps']:.0f}, write {best['write']['gbps']:.0f}, "
        f"copy {ceiling:.0f} GB/s")
    for name, v in list(per.items()) + list((variants or {}).items()):
        v["pct_copy_ceiling"] = round(100 * v["gbps"] / ceiling, 1)
        if name in pattern:
            v["pattern_ceiling_gbps"] = pattern[name]
            v["pct_pattern_ceiling"] = round(100 * v["gbps"] / pattern[name], 1)
    props = torch.cuda.get_device_properties(0)
    device = {"name": props.name, "arch": getattr(props, "gcnArchName", ""),
              "compute_units": props.multi_processor_count,
              "memory_gib": round(props.total_memory / 2 ** 30, 1)}
    dom = per[DOMINANT]
    achieved = dom["algo_bytes"] / (dom["mean_us"] * 1e-6) / 1e9
    traffic = measured_traffic()
    result = {
        "metric": METRIC,
        "value": round(step_bytes / (ms_per_step * 1e-3) / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "one launch of each row-reduction workload per step: softmax fp32 64x1000, "
                        "LayerNorm fp32 4096x1024, softmax bf16 16384x4096, residual-add+RMSNorm "
                        "bf16 8192x8192, softmax cross-entropy fwd+bwd fp32 4096x50257",
            "bytes_per_step": step_bytes,
            "rows_per_step": step_rows,
            "rows_per_s": round(step_rows / (ms_per_step * 1e-3), 1),
            "pct_of_hbm_peak": round(100 * step_bytes / (ms_per_step * 1e-3) / 1e9 / PEAK_HBM_GBPS, 2),
            "copy_ceiling_gbps": round(ceiling, 1),
            "read_ceiling_gbps": best["read"]["gbps"],
            "write_ceiling_gbps": best["write"]["gbps"],
            "ceilings": {"best": best, "probes_gbps": probes,
                         "note": "fr_stream_probe rates; copy = best mixed read+write pattern; "
                                 "per_workload pattern_ceiling_gbps = the copy of that "
                                 "workload's own row geometry and cache policy"},
            "device": device,
            "storage": "fp32 and bf16 as listed; arithmetic fp32",
            "seeds": [w.w.seed for w in wls],
            "launch": "hip graph replay of the five launches" if graph else "eager launches",
        },
        "per_workload": per,
        "backward": backward,
        "variants": variants,
        "attention": attention,
        "roofline": {
            "bound": "hbm",
            "kernel": f"xent_kernel<float,{dom['variant']['threads']},{dom['variant']['vecs']},"
                      f"{dom['variant']['elems_per_vec']}> (softmax cross-entropy 4096x50257)",
            "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBPS, 4),
            "traffic": traffic,
        },
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        result["cpu_baseline"], outs = cpu_baseline(wls)
        log("comparing the timed step's outputs with the oracle's")
        result["parity"] = parity_report(wls, outs)
        del outs
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
