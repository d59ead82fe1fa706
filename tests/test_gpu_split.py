"""GPU parity of the split-row kernels (fr_softmax_fwd_split,
fr_softmax_xent_split) against the double-precision oracle, through the C
ABI: widths from 1 to 2^20 (beyond the single-workgroup limit of 65,536),
few-row shapes, every segment shape on the vector and scalar paths, mixed
dtypes, in place, and bitwise reproducibility. The tolerances are the
forward ones (softmax: 1e-5 relative / one bf16 ulp; cross-entropy: the rules
of test_gpu_xent_ex)."""
import numpy as np
import pytest
import torch

import memory_bound_row_pass_amd as fr
import oracle
import workloads
from gpu_buffers import DEV, TDT, Guarded, host, upload
from parity import check_bf16, check_f32
from test_gpu_xent_ex import expect as expect_xent
from test_gpu_xent_ex import inputs as xent_inputs

pytestmark = pytest.mark.gpu


def setup_module(module):
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    oracle.set_threads(min(16, oracle.threads()))


def softmax_input(code, R, C, seed):
    name = "softmax_bf16" if code == fr.BF16 else "softmax_f32"
    return workloads.make(name, rows=R, cols=C, seed=seed)["x"]


def workspace(R, C):
    return Guarded((max(fr.fr_split_workspace_bytes(R, C) // 4, 4),), torch.float32)


def run_softmax_split(x_np, out_code, offs=(0, 0), inplace=False):
    R, C = x_np.shape
    x = upload(x_np, offs[0])
    ws = workspace(R, C)
    if inplace:
        fr.fr_softmax_fwd_split(x, x, ws.t)
        torch.cuda.synchronize()
        assert ws.canaries_intact()
        return host(x)
    y = Guarded((R, C), TDT[out_code], offs[1])
    fr.fr_softmax_fwd_split(x, y.t, ws.t)
    torch.cuda.synchronize()
    assert y.canaries_intact() and ws.canaries_intact(), "split softmax wrote out of bounds"
    return host(y.t)


def expect_softmax(x_np, out_code, got, what):
    p = oracle.softmax(x_np)
    if out_code == fr.BF16:
        return check_bf16(got, oracle.round_bf16(p), what)
    return check_f32(got, p, what=what)


WIDTHS = [1, 5, 1000, 8191, 8192, 8193, 32768, 50257, 65536, 65537, 100000, 262144]


@pytest.mark.parametrize("C", WIDTHS)
@pytest.mark.parametrize("xin,yout", [(0, 0), (1, 1), (0, 1), (1, 0)])
def test_softmax_split_widths(C, xin, yout):
    for R in (1, 3):
        x = softmax_input(xin, R, C, seed=C + R)
        expect_softmax(x, yout, run_softmax_split(x, yout), f"split softmax {xin}->{yout} {R}x{C}")


def test_softmax_split_one_million_columns():
    x = softmax_input(0, 2, 1 << 20, seed=77)
    expect_softmax(x, 0, run_softmax_split(x, 0), "split softmax 2x1048576")
    x = softmax_input(1, 2, 1 << 20, seed=78)
    expect_softmax(x, 1, run_softmax_split(x, 1), "split softmax bf16 2x1048576")


SEG_SHAPES = [(1024, 8), (512, 8), (256, 8), (1024, 4), (512, 4), (256, 4), (256, 32)]


@pytest.mark.parametrize("t,v", SEG_SHAPES)
def test_every_segment_shape(t, v):
    ran = 0
    for code in (fr.F32, fr.BF16):
        for vp, offs in ((True, (0, 0)), (False, (1, 2))):
            try:
                with fr.forced_variant(fr.OP_SOFTMAX_SPLIT, t, v):
                    tt, vv, e = fr.fr_debug_select_variant(fr.OP_SOFTMAX_SPLIT, 1, code,
                                                           vector_path=vp)
            except fr.FusedRowError:
                continue
            seg = tt * vv * e
            for C in (seg - 3, seg, 2 * seg + 37, 5 * seg):
                x = softmax_input(code, 2, C, seed=C)
                with fr.forced_variant(fr.OP_SOFTMAX_SPLIT, t, v):
                    got = run_softmax_split(x, code, offs)
                expect_softmax(x, code, got, f"split[{t},{v},{vp}] {code} 2x{C}")
                xl, lab = xent_inputs(3, C, code, seed=C, ignore_every=3)
                opts = dict(ignore_index=-100, label_smoothing=0.1, reduction="mean")
                with fr.forced_variant(fr.OP_XENT_SPLIT, t, v):
                    gx = run_xent_split(xl, lab, code, opts, offs=offs)
                expect_xent(xl, lab, code, opts, gx, f"split xent[{t},{v},{vp}] {code} 3x{C}")
                ran += 1
    if not ran:
        pytest.skip(f"no split shape ({t}, {v})")


def test_softmax_split_misaligned_and_in_place():
    for offs in ((1, 1), (3, 3), (1, 0)):
        x = softmax_input(0, 3, 70001, seed=5)
        expect_softmax(x, 0, run_softmax_split(x, 0, offs), f"split softmax offs {offs}")
    x = softmax_input(1, 4, 131072, seed=6)
    expect_softmax(x, 1, run_softmax_split(x, 1, inplace=True), "split softmax in place")


def test_special_rows():
    C = 100000
    rng = np.random.default_rng(9)
    x = rng.normal(0, 3, size=(4, C)).astype(np.float32)
    x[0, ::3] = -np.inf                       # masked entries
    x[1, :] = -np.inf                         # fully masked row: NaN
    x[2, :] = 1.5                             # constant row: 1/C
    x[3, 77777] = 200.0                       # one-hot in a late segment
    got = run_softmax_split(x, 0)
    assert np.all(np.isnan(got[1]))
    keep = [0, 2, 3]
    expect_softmax(x[keep], 0, got[keep], "split softmax special")


# ------------------------------------------------------------- cross-entropy

def run_xent_split(logits, labels, code, opts, argmax=True, offs=(0, 0), inplace=False):
    R, C = logits.shape
    x = upload(logits, offs[0])
    lab = upload(labels)
    loss = Guarded((R,), torch.float32)
    am = Guarded((R,), torch.int32) if argmax else None
    tot = Guarded((1,), torch.float32)
    ws = workspace(R, C)
    if inplace:
        g_t, g = x, None
    else:
        g = Guarded((R, C), TDT[code], offs[1])
        g_t = g.t
    fr.fr_softmax_xent_split(x, lab, loss.t, g_t, ws.t, am.t if am else None, tot.t, **opts)
    torch.cuda.synchronize()
    assert loss.canaries_intact() and tot.canaries_intact() and ws.canaries_intact()
    assert (g is None or g.canaries_intact()) and (am is None or am.canaries_intact())
    return (loss.t.cpu().numpy(), host(g_t), am.t.cpu().numpy() if am else None,
            float(tot.t.cpu()[0]))


XOPTS = [dict(), dict(ignore_index=-100, label_smoothing=0.1, reduction="mean", grad_scale=0.5),
         dict(reduction="sum")]


@pytest.mark.parametrize("C", [1, 7, 50257, 65537, 131072, 262144])
@pytest.mark.parametrize("code", [fr.F32, fr.BF16])
def test_xent_split_widths(C, code):
    for k, opts in enumerate(XOPTS):
        x, lab = xent_inputs(4, C, code, seed=C + k, ignore_every=3 if opts else 0)
        expect_xent(x, lab, code, opts, run_xent_split(x, lab, code, opts, argmax=k != 1),
                    f"split xent {code} 4x{C} {opts}")


def test_xent_split_vocabulary_256k():
    # a 256K-vocabulary batch: 128 rows (33.5M logits), fp32 and bf16
    for code in (fr.F32, fr.BF16):
        x, lab = xent_inputs(128, 262144, code, seed=1234, ignore_every=7)
        opts = dict(ignore_index=-100, label_smoothing=0.1, reduction="mean")
        expect_xent(x, lab, code, opts, run_xent_split(x, lab, code, opts), f"split xent 128x256K {code}")


def test_xent_split_in_place_and_invalid_labels():
    C = 100003
    x, lab = xent_inputs(5, C, fr.F32, seed=12)
    lab[:] = [-100, C, 0, C - 1, 50000]
    opts = dict(ignore_index=-100, label_smoothing=0.05)
    expect_xent(x, lab, fr.F32, opts, run_xent_split(x, lab, fr.F32, opts), "split xent labels")
    expect_xent(x, lab, fr.F32, opts, run_xent_split(x, lab, fr.F32, opts, inplace=True),
                "split xent in place")


def test_split_bitwise_determinism():
    x, lab = xent_inputs(64, 200000, fr.BF16, seed=13, ignore_every=5)
    outs = []
    for _ in range(3):
        r = run_xent_split(x, lab, fr.BF16, dict(ignore_index=-100, reduction="mean"))
        outs.append((r[0].tobytes(), r[1].tobytes(), r[2].tobytes(), np.float32(r[3]).tobytes()))
    assert outs[0] == outs[1] == outs[2]


def test_convenience_routes_wide_rows():
    x = softmax_input(0, 2, 100000, seed=14)
    y = fr.softmax(upload(x))
    expect_softmax(x, 0, y.cpu().numpy(), "softmax() of a wide row")
    xl, lab = xent_inputs(2, 100000, fr.F32, seed=15)
    loss, grad = fr.softmax_xent(upload(xl), upload(lab))
    lo, go, _, _ = oracle.softmax_xent_ex(xl, lab)
    check_f32(loss.cpu().numpy(), lo, scale=np.maximum(np.abs(lo), 1.0), what="softmax_xent() wide")
