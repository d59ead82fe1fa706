"""GPU parity: every fused row kernel against the double-precision oracle,
through the C ABI, on seeded inputs.

Outputs are pre-filled with NaN (an element the kernel fails to write fails
the comparison) and surrounded by guard bands holding a fixed bit pattern
(an out-of-bounds write changes them) — the poisoned-output and memory checks
of "ML Compiler Lab" (Failures the checks caught).

Covered: the five standard workloads at full size (all rows), edge widths
from 1 to the maximum, every compiled kernel variant, misaligned rows (head /
body / tail split and the scalar path), in-place calls, special values,
labels out of range, bitwise determinism and a non-default stream.
"""
import math

import numpy as np
import pytest
import torch

import memory_bound_row_pass_amd as fr
import oracle
import workloads
from gpu_buffers import DEV, TDT, Guarded, host, upload
from parity import FLT_MIN, bf16_bits, check_bf16, check_f32, to_dev

pytestmark = pytest.mark.gpu


def setup_module(module):
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    oracle.set_threads(min(16, oracle.threads()))


def ref_bf16(v):
    return oracle.round_bf16(v)


# ------------------------------------------------------------- runners

def run_softmax(x_np, out_code, x_off=0, y_off=0):
    x = upload(x_np, x_off)
    R, C = x_np.shape
    y = Guarded((R, C), TDT[out_code], y_off)
    fr.fr_softmax_fwd(x, y.t)
    torch.cuda.synchronize()
    assert y.canaries_intact(), "softmax wrote outside its output"
    return host(y.t)


def expect_softmax(x_np, out_code, got, what):
    p = oracle.softmax(x_np)
    if out_code == fr.BF16:
        return check_bf16(got, ref_bf16(p), what)
    return check_f32(got, p, what=what)


def run_layernorm(w_x, w_g, w_b, eps, off=0):
    x, g, b = upload(w_x, off), upload(w_g), upload(w_b)
    R, C = w_x.shape
    y = Guarded((R, C), x.dtype, off)
    mean, rstd = Guarded((R,), torch.float32), Guarded((R,), torch.float32)
    fr.fr_layernorm_fwd(x, g, b, y.t, mean.t, rstd.t, eps)
    torch.cuda.synchronize()
    assert y.canaries_intact() and mean.canaries_intact() and rstd.canaries_intact()
    return host(y.t), mean.t.cpu().numpy(), rstd.t.cpu().numpy()


def expect_layernorm(w_x, w_g, w_b, eps, got, what):
    y, mean, rstd = got
    yo, mo, ro = oracle.layernorm(w_x, w_g, w_b, eps)
    xd = oracle.decode(w_x)
    sd = np.sqrt(np.maximum(xd.var(axis=1), 0))
    if w_x.dtype == np.uint16:
        # y crosses zero through beta: where |y| << 1 the result is a
        # cancellation and carries the fp32 absolute error of the O(1) terms
        hy = check_bf16(y, ref_bf16(yo), what + " y", abs_floor=1e-5)
    else:
        hy = check_f32(y, yo, scale=np.maximum(np.abs(yo), 1.0), what=what + " y")
    check_f32(mean, mo, scale=np.maximum(np.abs(mo), sd), what=what + " mean")
    check_f32(rstd, ro, what=what + " rstd")
    return hy


def run_rmsnorm(w_x, w_r, w_w, eps, off=0, with_res_out=True):
    x, r, wt = upload(w_x, off), upload(w_r, off), upload(w_w)
    R, C = w_x.shape
    y = Guarded((R, C), x.dtype, off)
    ro = Guarded((R, C), x.dtype, off) if with_res_out else None
    fr.fr_add_rmsnorm_fwd(x, r, wt, y.t, ro.t if ro else None, eps)
    torch.cuda.synchronize()
    assert y.canaries_intact() and (ro is None or ro.canaries_intact())
    return host(y.t), (host(ro.t) if ro else None)


def expect_rmsnorm(w_x, w_r, w_w, eps, got, what):
    y, ro = got
    yo, ho, _ = oracle.add_rmsnorm(w_x, w_r, w_w, eps)
    if w_x.dtype == np.uint16:
        hy = check_bf16(y, ref_bf16(yo), what + " y")
        hr = check_bf16(ro, ref_bf16(ho), what + " residual_out") if ro is not None else None
    else:
        hy = check_f32(y, yo, what=what + " y")
        hr = check_f32(ro, ho, what=what + " residual_out") if ro is not None else None
    return hy, hr


def run_xent(logits, labels, x_off=0, g_off=0, with_argmax=True):
    x = upload(logits, x_off)
    lab = upload(labels)
    R, C = logits.shape
    grad = Guarded((R, C), torch.float32, g_off)
    loss = Guarded((R,), torch.float32)
    am = Guarded((R,), torch.int32) if with_argmax else None
    fr.fr_softmax_xent_fwd_bwd(x, lab, loss.t, grad.t, am.t if am else None)
    torch.cuda.synchronize()
    assert grad.canaries_intact() and loss.canaries_intact() and (am is None or am.canaries_intact())
    return loss.t.cpu().numpy(), grad.t.cpu().numpy(), (am.t.cpu().numpy() if am else None)


def expect_xent(logits, labels, got, what):
    loss, grad, am = got
    lo, go, ao = oracle.softmax_xent(logits, labels)
    R, C = logits.shape
    valid = (labels >= 0) & (labels < C)
    p_at = np.abs(go).copy()
    rows = np.nonzero(valid)[0]
    p_at[rows, labels[rows]] = go[rows, labels[rows]] + 1.0
    check_f32(grad, go, scale=np.maximum(np.abs(go), p_at), what=what + " grad")
    assert np.all(np.isnan(loss[~valid])), what + ": out-of-range label must give NaN loss"
    check_f32(loss[valid], lo[valid], scale=np.maximum(np.abs(lo[valid]), 1.0), what=what + " loss")
    if am is not None:
        assert np.array_equal(am, ao), what + " argmax"
    # label sign test: exactly one negative gradient per valid row, at the
    # label (unless p_label rounds to 1 and its gradient is exactly 0)
    for r in rows[:64]:
        neg = np.nonzero(grad[r] < 0)[0]
        want = [labels[r]] if go[r, labels[r]] < -FLT_MIN else []
        assert list(neg) == want, (what, r, neg[:5])


# ------------------------------------------------- full-size workloads

def test_workload_softmax_f32():
    w = workloads.make("softmax_f32")
    got = run_softmax(w["x"], fr.F32)
    st = expect_softmax(w["x"], fr.F32, got, "softmax_f32 64x1000")
    assert np.abs(got.astype(np.float64).sum(1) - 1).max() < 1e-5
    print("softmax_f32", st)


def test_workload_layernorm_f32():
    w = workloads.make("layernorm_f32")
    got = run_layernorm(w["x"], w["gamma"], w["beta"], w.eps)
    expect_layernorm(w["x"], w["gamma"], w["beta"], w.eps, got, "layernorm_f32 4096x1024")


def test_workload_softmax_bf16():
    w = workloads.make("softmax_bf16")
    got = run_softmax(w["x"], fr.BF16)
    p = oracle.softmax(w["x"])
    hist = check_bf16(got, ref_bf16(p), "softmax_bf16 16384x4096")
    sub = int(((p > 0) & (p < 2.0 ** -126)).sum())
    print("softmax_bf16 ulp histogram", hist, "oracle values below 2^-126:", sub)
    assert sub > 0   # the near-one-hot rows do exercise bf16 subnormals


def test_workload_add_rmsnorm_bf16():
    w = workloads.make("add_rmsnorm_bf16")
    hy, hr = expect_rmsnorm(w["x"], w["residual"], w["weight"], w.eps,
                            run_rmsnorm(w["x"], w["residual"], w["weight"], w.eps),
                            "add_rmsnorm_bf16 8192x8192")
    print("add_rmsnorm y ulp", hy, "residual_out ulp", hr)
    # the updated residual is exact except where fp32 could not hold x + r
    assert hr[">1"] == 0 and hr["1"] <= 1e-4 * (hr["0"] + hr["1"])


def test_workload_xent_f32():
    w = workloads.make("xent_f32")
    got = run_xent(w["logits"], w["labels"])
    expect_xent(w["logits"], w["labels"], got, "xent_f32 4096x50257")


# ------------------------------------------------------- edge shapes

EDGE_COLS = [1, 2, 3, 4, 5, 7, 8, 9, 63, 64, 65, 127, 255, 257, 1000, 1023, 1024, 1025,
             2047, 4095, 4096, 4097, 8191, 8192, 12345, 16384, 32769, 50257, 65536]


def _softmax_input(code, R, C, seed):
    if code == fr.BF16:
        return workloads.make("softmax_bf16", rows=R, cols=C, seed=seed)["x"]
    return workloads.make("softmax_f32", rows=R, cols=C, seed=seed)["x"]


@pytest.mark.parametrize("C", EDGE_COLS)
@pytest.mark.parametrize("xin,yout", [(0, 0), (1, 1), (0, 1), (1, 0)])
def test_softmax_edge_cols(C, xin, yout):
    for R in (1, 3):
        x = _softmax_input(xin, R, C, seed=C * 7 + R)
        expect_softmax(x, yout, run_softmax(x, yout), f"softmax {xin}->{yout} {R}x{C}")


@pytest.mark.parametrize("C", EDGE_COLS)
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_layernorm_edge_cols(C, dt):
    w = workloads.make("layernorm_f32", rows=3, cols=C, seed=C, dtype=dt)
    got = run_layernorm(w["x"], w["gamma"], w["beta"], w.eps)
    expect_layernorm(w["x"], w["gamma"], w["beta"], w.eps, got, f"layernorm {dt} 3x{C}")


@pytest.mark.parametrize("C", EDGE_COLS)
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_rmsnorm_edge_cols(C, dt):
    w = workloads.make("add_rmsnorm_bf16", rows=3, cols=C, seed=C, dtype=dt)
    got = run_rmsnorm(w["x"], w["residual"], w["weight"], w.eps)
    expect_rmsnorm(w["x"], w["residual"], w["weight"], w.eps, got, f"add_rmsnorm {dt} 3x{C}")


@pytest.mark.parametrize("C", EDGE_COLS)
def test_xent_edge_cols(C):
    w = workloads.make("xent_f32", rows=4, cols=C, seed=C)
    lab = w["labels"].copy()
    lab[0], lab[-1] = 0, C - 1          # first and last column
    expect_xent(w["logits"], lab, run_xent(w["logits"], lab), f"xent 4x{C}")


def test_many_rows_odd_count():
    # more rows than one grid wave, odd count (partial last workgroup)
    x = _softmax_input(0, 4099, 300, seed=5)
    expect_softmax(x, 0, run_softmax(x, 0), "softmax 4099x300")
    w = workloads.make("xent_f32", rows=1031, cols=777, seed=6)
    expect_xent(w["logits"], w["labels"], run_xent(w["logits"], w["labels"]), "xent 1031x777")


# ----------------------------------------------------- every variant

VARIANT_GRID = [(t, v) for t in (64, 256, 512, 1024) for v in (1, 2, 4, 8, 13, 16, 64)]


def _variant_cols(op, t, v, code, vector_path):
    try:
        with fr.forced_variant(op, t, v):
            tt, vv, e = fr.fr_debug_select_variant(op, 1, code, vector_path=vector_path)
    except fr.FusedRowError:
        return None
    cap = tt * vv * e
    if op in (fr.OP_LAYERNORM, fr.OP_RMSNORM) and e > 1:
        # the norms' 128-bit path needs rows that are whole 16-byte chunks
        return [cap, cap - 5 * e, e * (cap // (2 * e) + 1)]
    return [cap, max(1, cap - 5 * e - 3), max(1, cap // 2 + 1)]


def _grid(uses):
    """The (threads, vecs) pairs of VARIANT_GRID for which the library holds a
    kernel for at least one (op, dtype, vector path) in `uses`; the selection
    call runs on the host, so collection needs no GPU."""
    return [(t, v) for t, v in VARIANT_GRID
            if any(_variant_cols(op, t, v, code, vp) for op, code, vp in uses)]


_BOTH = [(c, vp) for c in (fr.F32, fr.BF16) for vp in (True, False)]
SOFTMAX_GRID = _grid([(fr.OP_SOFTMAX, c, vp) for c, vp in _BOTH])
NORM_XENT_GRID = _grid([(op, c, vp) for op in (fr.OP_LAYERNORM, fr.OP_RMSNORM) for c, vp in _BOTH]
                       + [(fr.OP_XENT, fr.F32, vp) for vp in (True, False)])


@pytest.mark.parametrize("t,v", SOFTMAX_GRID)
def test_every_softmax_variant(t, v):
    ran = 0
    for code in (fr.F32, fr.BF16):
        cols = _variant_cols(fr.OP_SOFTMAX, t, v, code, True)
        if not cols:
            continue
        with fr.forced_variant(fr.OP_SOFTMAX, t, v):
            for C in cols:
                x = _softmax_input(code, 3, C, seed=C)
                expect_softmax(x, code, run_softmax(x, code), f"softmax[{t},{v}] {code} 3x{C}")
                ran += 1
    for code in (fr.F32, fr.BF16):
        cols = _variant_cols(fr.OP_SOFTMAX, t, v, code, False)
        if not cols:
            continue
        with fr.forced_variant(fr.OP_SOFTMAX, t, v):
            for C in cols:
                x = _softmax_input(code, 2, C, seed=C + 1)
                expect_softmax(x, code, run_softmax(x, code, x_off=1, y_off=2),
                               f"softmax scalar[{t},{v}] {code} 2x{C}")
                ran += 1
    if not ran:
        pytest.skip(f"no softmax variant ({t}, {v})")


@pytest.mark.parametrize("t,v", NORM_XENT_GRID)
def test_every_norm_and_xent_variant(t, v):
    ran = 0
    for dt, code in (("f32", fr.F32), ("bf16", fr.BF16)):
        for vp, off in ((True, 0), (False, 1)):
            cols = _variant_cols(fr.OP_LAYERNORM, t, v, code, vp)
            if cols:
                with fr.forced_variant(fr.OP_LAYERNORM, t, v):
                    for C in cols:
                        w = workloads.make("layernorm_f32", rows=2, cols=C, seed=C, dtype=dt)
                        expect_layernorm(w["x"], w["gamma"], w["beta"], w.eps,
                                         run_layernorm(w["x"], w["gamma"], w["beta"], w.eps, off),
                                         f"layernorm[{t},{v},{vp}] {dt} 2x{C}")
                        ran += 1
            cols = _variant_cols(fr.OP_RMSNORM, t, v, code, vp)
            if cols:
                with fr.forced_variant(fr.OP_RMSNORM, t, v):
                    for C in cols:
                        w = workloads.make("add_rmsnorm_bf16", rows=2, cols=C, seed=C, dtype=dt)
                        expect_rmsnorm(w["x"], w["residual"], w["weight"], w.eps,
                                       run_rmsnorm(w["x"], w["residual"], w["weight"], w.eps, off),
                                       f"rmsnorm[{t},{v},{vp}] {dt} 2x{C}")
                        ran += 1
    for vp, off in ((True, 0), (False, 1)):
        cols = _variant_cols(fr.OP_XENT, t, v, fr.F32, vp)
        if cols:
            with fr.forced_variant(fr.OP_XENT, t, v):
                for C in cols:
                    w = workloads.make("xent_f32", rows=3, cols=C, seed=C)
                    for am in (True, False):
                        expect_xent(w["logits"], w["labels"],
                                    run_xent(w["logits"], w["labels"], off, 2 * off, with_argmax=am),
                                    f"xent[{t},{v},{vp}] 3x{C}")
                    ran += 1
    if not ran:
        pytest.skip(f"no variant ({t}, {v})")


# --------------------------------------------------- alignment / aliasing

@pytest.mark.parametrize("xoff,yoff", [(1, 1), (2, 2), (3, 3), (1, 0), (0, 3)])
def test_misaligned_rows(xoff, yoff):
    # equal phases take the head/body/tail vector path, unequal the scalar path
    for C in (5, 1000, 50257):
        x = _softmax_input(0, 5, C, seed=C)
        expect_softmax(x, 0, run_softmax(x, 0, xoff, yoff), f"softmax off {xoff},{yoff} 5x{C}")
        w = workloads.make("xent_f32", rows=5, cols=C, seed=C)
        lab = w["labels"].copy()
        lab[:] = [0, C - 1, min(2, C - 1), C // 2, max(C - 3, 0)]
        expect_xent(w["logits"], lab, run_xent(w["logits"], lab, xoff, yoff), f"xent off 5x{C}")
    for off in (1, 3):
        w = workloads.make("layernorm_f32", rows=4, cols=1000, seed=off)
        expect_layernorm(w["x"], w["gamma"], w["beta"], w.eps,
                         run_layernorm(w["x"], w["gamma"], w["beta"], w.eps, off), "layernorm off")
        w = workloads.make("add_rmsnorm_bf16", rows=4, cols=1000, seed=off)
        expect_rmsnorm(w["x"], w["residual"], w["weight"], w.eps,
                       run_rmsnorm(w["x"], w["residual"], w["weight"], w.eps, off), "rmsnorm off")


def test_in_place():
    x = _softmax_input(1, 64, 4096, seed=3)
    t = to_dev(x)
    fr.fr_softmax_fwd(t, t)
    expect_softmax(x, 1, bf16_bits(t), "softmax in place")

    w = workloads.make("layernorm_f32", rows=64, cols=1024, seed=4)
    t = to_dev(w["x"])
    mean = torch.empty(64, device=DEV)
    rstd = torch.empty(64, device=DEV)
    fr.fr_layernorm_fwd(t, to_dev(w["gamma"]), to_dev(w["beta"]), t, mean, rstd, w.eps)
    expect_layernorm(w["x"], w["gamma"], w["beta"], w.eps,
                     (t.cpu().numpy(), mean.cpu().numpy(), rstd.cpu().numpy()), "layernorm in place")

    w = workloads.make("add_rmsnorm_bf16", rows=64, cols=8192, seed=5)
    for mode in ("res_out=res", "res_out=x", "y=x"):
        xt, rt, wt = to_dev(w["x"]), to_dev(w["residual"]), to_dev(w["weight"])
        if mode == "res_out=res":
            y = torch.empty_like(xt); ro = rt
        elif mode == "res_out=x":
            y = torch.empty_like(xt); ro = xt
        else:
            y = xt; ro = torch.empty_like(xt)
        fr.fr_add_rmsnorm_fwd(xt, rt, wt, y, ro, w.eps)
        expect_rmsnorm(w["x"], w["residual"], w["weight"], w.eps, (bf16_bits(y), bf16_bits(ro)),
                       f"rmsnorm in place {mode}")

    w = workloads.make("xent_f32", rows=64, cols=50257, seed=6)
    t = to_dev(w["logits"])
    loss = torch.empty(64, device=DEV)
    fr.fr_softmax_xent_fwd_bwd(t, to_dev(w["labels"]), loss, t)
    expect_xent(w["logits"], w["labels"], (loss.cpu().numpy(), t.cpu().numpy(), None), "xent in place")


# --------------------------------------------------------- special values

def test_special_values_softmax():
    rng = np.random.default_rng(99)
    C = 1000
    x = rng.normal(0, 3, size=(6, C)).astype(np.float32)
    x[0, ::3] = -np.inf                      # masked entries
    x[1, :] = -np.inf                        # fully masked row -> NaN
    x[2, :] = 7.25                           # constant row -> 1/C
    x[3] += 1000.0                           # shift
    x[4, 5] = 100.0                          # one-hot
    x[5, :] = np.float32(-3.0e38)            # huge negative, finite
    for code in (fr.F32, fr.BF16):
        got = run_softmax(x, code)
        gotf = got.astype(np.float64) if code == fr.F32 else \
            (got.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        assert np.all(np.isnan(gotf[1])), "all -inf row must be NaN"
        keep = [0, 2, 3, 4, 5]
        expect_softmax(x[keep], code, got[keep], f"softmax special {code}")
        assert np.all(gotf[0, ::3] == 0.0)


FAR_DELTAS = [20.0, 31.0, 33.0, 40.0, 50.0, 60.0, 70.0, 75.0, 80.0, 86.0, 88.0, 90.0, 92.0]


def far_rows(R, C, code, seed):
    """Rows N(0, 2^2) with a maximum of 10 and single elements 10 - d for each d
    of FAR_DELTAS (integers, exact in bf16): probabilities from e^-20 down
    into the subnormal range, spread over head, body and tail columns."""
    rng = np.random.default_rng(seed)
    x = np.clip(rng.normal(0, 2, size=(R, C)), -9, 9)
    for r in range(R):
        x[r, (r * 7919) % C] = 10.0
        cols = rng.choice(C, size=min(C - 1, len(FAR_DELTAS)), replace=False)
        cols = cols[cols != (r * 7919) % C]
        for c, d in zip(cols, FAR_DELTAS):
            x[r, c] = 10.0 - d
    x = x.astype(np.float32)
    if code == fr.BF16:
        return oracle.round_bf16(x)
    return x


@pytest.mark.parametrize("C", [1000, 4096, 50257])
def test_softmax_far_below_max(C):
    # elements far below the row maximum: fp32 outputs keep 1e-5 relative
    # (the compensated exponential where a lane's range needs it), bf16
    # outputs reach the subnormal range exactly
    for xin in (fr.F32, fr.BF16):
        x = far_rows(16, C, xin, seed=C + xin)
        for yout in (fr.F32, fr.BF16):
            expect_softmax(x, yout, run_softmax(x, yout), f"softmax far {xin}->{yout} 16x{C}")


def test_special_values_norms():
    # constant rows: LayerNorm gives beta exactly, rstd = 1/sqrt(eps)
    C = 1024
    x = np.full((2, C), 3.5, np.float32)
    g = np.ones(C, np.float32)
    b = np.linspace(-1, 1, C).astype(np.float32)
    got = run_layernorm(x, g, b, 1e-5)
    expect_layernorm(x, g, b, 1e-5, got, "layernorm constant")
    assert np.array_equal(got[0], np.broadcast_to(b, (2, C)))
    # zero input to RMSNorm: y = 0 with eps > 0
    z = np.zeros((2, C), np.float32)
    y, ro = run_rmsnorm(z, z, np.ones(C, np.float32), 1e-6)
    assert np.all(y == 0) and np.all(ro == 0)


def test_labels_out_of_range():
    w = workloads.make("xent_f32", rows=6, cols=3000, seed=8)
    lab = np.array([-1, 3000, 2**31 - 1, -(2**31), 0, 2999], np.int32)
    got = run_xent(w["logits"], lab)
    expect_xent(w["logits"], lab, got, "xent bad labels")
    p = oracle.softmax(w["logits"])
    check_f32(got[1][:4], p[:4], what="grad of rows with bad labels = softmax")


# ------------------------------------------------- determinism / streams

def test_bitwise_determinism():
    w = workloads.make("xent_f32", rows=256, cols=50257, seed=10)
    x, lab = to_dev(w["logits"]), to_dev(w["labels"])
    outs = []
    for _ in range(3):
        loss, grad, am = fr.softmax_xent(x, lab, return_argmax=True)
        outs.append((loss.cpu().numpy().tobytes(), grad.cpu().numpy().tobytes(),
                     am.cpu().numpy().tobytes()))
    assert outs[0] == outs[1] == outs[2]
    w = workloads.make("softmax_bf16", rows=512, seed=11)
    x = to_dev(w["x"])
    r = [bf16_bits(fr.softmax(x)).tobytes() for _ in range(3)]
    assert r[0] == r[1] == r[2]
    w = workloads.make("layernorm_f32", rows=512, seed=12)
    args = [to_dev(w[k]) for k in ("x", "gamma", "beta")]
    r = [tuple(t.cpu().numpy().tobytes() for t in fr.layernorm(*args, w.eps)) for _ in range(3)]
    assert r[0] == r[1] == r[2]


def test_non_default_stream():
    w = workloads.make("add_rmsnorm_bf16", rows=128, seed=13)
    s = torch.cuda.Stream()
    x, r, wt = to_dev(w["x"]), to_dev(w["residual"]), to_dev(w["weight"])
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        y, ro = fr.add_rmsnorm(x, r, wt, w.eps)
    s.synchronize()
    expect_rmsnorm(w["x"], w["residual"], w["weight"], w.eps, (bf16_bits(y), bf16_bits(ro)),
                   "rmsnorm on a side stream")


def test_stream_copy():
    src = torch.randint(0, 2**31 - 1, (1 << 20,), dtype=torch.int32, device=DEV)
    dst = torch.zeros_like(src)
    fr.fr_stream_copy(src, dst)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)
    dst2 = torch.zeros(1000, dtype=torch.uint8, device=DEV)
    src2 = torch.arange(1001, dtype=torch.uint8, device=DEV)[1:]
    fr.fr_stream_copy(src2, dst2)
    torch.cuda.synchronize()
    assert torch.equal(src2, dst2)


def test_rows_zero_is_noop():
    x = torch.empty(0, 100, device=DEV)
    fr.fr_softmax_fwd(x, torch.empty(0, 100, device=DEV))
    loss, grad = fr.softmax_xent(torch.empty(0, 7, device=DEV),
                                 torch.empty(0, dtype=torch.int32, device=DEV))
    assert loss.numel() == 0 and grad.numel() == 0


# ---------------------------------------------------------- graph capture

def test_graph_capture_replays_match_eager():
    # every entry point allocates nothing and never synchronises, so a step of
    # all four ops can be captured; each replay (with eager work and
    # synchronisations in between) must reproduce the eager result exactly
    ws = workloads.make("softmax_bf16", rows=256)
    wl = workloads.make("layernorm_f32", rows=256)
    wr = workloads.make("add_rmsnorm_bf16", rows=64)
    wx = workloads.make("xent_f32", rows=32)
    xs = to_dev(ws["x"]); ys = torch.empty_like(xs)
    xl, gl, bl = to_dev(wl["x"]), to_dev(wl["gamma"]), to_dev(wl["beta"])
    yl = torch.empty_like(xl); ml = torch.empty(256, device=DEV); rl = torch.empty(256, device=DEV)
    xr, rr, wt = to_dev(wr["x"]), to_dev(wr["residual"]), to_dev(wr["weight"])
    yr, ror = torch.empty_like(xr), torch.empty_like(xr)
    xx, lab = to_dev(wx["logits"]), to_dev(wx["labels"])
    loss, grad = torch.empty(32, device=DEV), torch.empty_like(xx)

    def step():
        fr.fr_softmax_fwd(xs, ys)
        fr.fr_layernorm_fwd(xl, gl, bl, yl, ml, rl, wl.eps)
        fr.fr_add_rmsnorm_fwd(xr, rr, wt, yr, ror, wr.eps)
        fr.fr_softmax_xent_fwd_bwd(xx, lab, loss, grad)

    outs = (ys, yl, ml, rl, yr, ror, loss, grad)
    step()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        for o in outs:
            o.fill_(float("nan"))           # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert torch.equal(o.view(torch.int16) if o.dtype == torch.bfloat16 else o.view(torch.int32),
                               e.view(torch.int16) if e.dtype == torch.bfloat16 else e.view(torch.int32)), rep
    # and the eager result itself is right
    check_bf16(bf16_bits(ys), ref_bf16(oracle.softmax(ws["x"])), "graph softmax")


def test_xent_few_rows_shape():
    """Rows that fill the compute units once but not twice (one GPU's share
    of a row-sharded batch) take the 256-lane cross-entropy shape, two rows
    per compute unit: parity with the oracle and the same bits as that shape
    forced; one row per CU, or more than two, keeps the 1024-lane shape."""
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    C = 50257
    assert fr.fr_debug_select_variant_for(fr.OP_XENT, ncu, C, fr.F32) == (1024, 13, 4)
    assert fr.fr_debug_select_variant_for(fr.OP_XENT, 2 * ncu + 1, C, fr.F32) == (1024, 13, 4)
    for R, C in ((2 * ncu, 50257), (ncu + 37, 40001)):
        assert fr.fr_debug_select_variant_for(fr.OP_XENT, R, C, fr.F32) == (256, 50, 4)
        w = workloads.make("xent_f32", rows=R, cols=C, seed=R)
        print(f"xent few rows {R}x{C}", flush=True)
        for am in (True, False):
            got = run_xent(w["logits"], w["labels"], with_argmax=am)
            expect_xent(w["logits"], w["labels"], got, f"xent {R}x{C} argmax={am}")
            with fr.forced_variant(fr.OP_XENT, 256, 50):
                forced = run_xent(w["logits"], w["labels"], with_argmax=am)
            assert all(np.array_equal(a, b) for a, b in zip(got, forced) if a is not None), \
                f"xent {R}x{C}: not the 256-lane shape"
