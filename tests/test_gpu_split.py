"""GPU parity of the split-row kernels (fr_softmax_fwd_split,
fr_softmax_xent_split) against the double-precision oracle, through the C
ABI: widths from 1 to 2^20 (beyond the single-workgroup limit of 65,536),
few-row shapes, every segment shape on the vector and scalar paths, mixed
dtypes, in place, and bitwise reproducibility — the softmax,
cross-entropy, LayerNorm, RMSNorm, softmax backward and norm backward
cases in both the one-pass and the two-pass form.
The tolerances are the forward ones (softmax: 1e-5 relative / one bf16 ulp;
cross-entropy: the rules of test_gpu_xent_ex)."""
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


@pytest.fixture(params=[2, 0], ids=["one-pass", "two-pass"])
def form(request):
    """Runs the test with the one-pass form wherever it applies (any row
    count), then with the two passes only."""
    with fr.split_one_pass(request.param):
        yield request.param


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
def test_softmax_split_widths(C, xin, yout, form):
    for R in (1, 3):
        x = softmax_input(xin, R, C, seed=C + R)
        expect_softmax(x, yout, run_softmax_split(x, yout), f"split softmax {xin}->{yout} {R}x{C}")


def test_softmax_split_one_million_columns(form):
    x = softmax_input(0, 2, 1 << 20, seed=77)
    expect_softmax(x, 0, run_softmax_split(x, 0), "split softmax 2x1048576")
    x = softmax_input(1, 2, 1 << 20, seed=78)
    expect_softmax(x, 1, run_softmax_split(x, 1), "split softmax bf16 2x1048576")


SEG_SHAPES = [(1024, 8), (512, 8), (256, 8), (1024, 4), (512, 4), (256, 4), (512, 16), (256, 32)]
# the softmax / cross-entropy table: 512 x 16 (fp32) and 512 x 8 (fp32 and bf16)
# hold 64 bytes per lane; no 256 x 4
SPLIT_SHAPES = [(1024, 8), (512, 8), (256, 8), (1024, 4), (512, 4), (512, 16), (256, 32)]


@pytest.mark.parametrize("t,v", SPLIT_SHAPES)
def test_every_segment_shape(t, v, form):
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


def test_softmax_split_misaligned_and_in_place(form):
    for offs in ((1, 1), (3, 3), (1, 0)):
        x = softmax_input(0, 3, 70001, seed=5)
        expect_softmax(x, 0, run_softmax_split(x, 0, offs), f"split softmax offs {offs}")
    x = softmax_input(1, 4, 131072, seed=6)
    expect_softmax(x, 1, run_softmax_split(x, 1, inplace=True), "split softmax in place")


def test_special_rows(form):
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
def test_xent_split_widths(C, code, form):
    for k, opts in enumerate(XOPTS):
        x, lab = xent_inputs(4, C, code, seed=C + k, ignore_every=3 if opts else 0)
        expect_xent(x, lab, code, opts, run_xent_split(x, lab, code, opts, argmax=k != 1),
                    f"split xent {code} 4x{C} {opts}")


def test_xent_split_vocabulary_256k(form):
    # a 256K-vocabulary batch: 128 rows (33.5M logits), fp32 and bf16
    for code in (fr.F32, fr.BF16):
        x, lab = xent_inputs(128, 262144, code, seed=1234, ignore_every=7)
        opts = dict(ignore_index=-100, label_smoothing=0.1, reduction="mean")
        expect_xent(x, lab, code, opts, run_xent_split(x, lab, code, opts), f"split xent 128x256K {code}")


def test_xent_split_in_place_and_invalid_labels(form):
    C = 100003
    x, lab = xent_inputs(5, C, fr.F32, seed=12)
    lab[:] = [-100, C, 0, C - 1, 50000]
    opts = dict(ignore_index=-100, label_smoothing=0.05)
    expect_xent(x, lab, fr.F32, opts, run_xent_split(x, lab, fr.F32, opts), "split xent labels")
    expect_xent(x, lab, fr.F32, opts, run_xent_split(x, lab, fr.F32, opts, inplace=True),
                "split xent in place")


def test_split_bitwise_determinism(form):
    x, lab = xent_inputs(64, 200000, fr.BF16, seed=13, ignore_every=5)
    outs = []
    for _ in range(3):
        r = run_xent_split(x, lab, fr.BF16, dict(ignore_index=-100, reduction="mean"))
        outs.append((r[0].tobytes(), r[1].tobytes(), r[2].tobytes(), np.float32(r[3]).tobytes()))
    assert outs[0] == outs[1] == outs[2]


def _softmax_split_ws(x_np, ws):
    R, C = x_np.shape
    y = Guarded((R, C), torch.float32)
    fr.fr_softmax_fwd_split(upload(x_np), y.t, ws.t)
    torch.cuda.synchronize()
    assert y.canaries_intact() and ws.canaries_intact()
    return host(y.t)


def test_one_pass_form_runs():
    """White-box: the one-pass form of [64, 131072] fp32 (segments of 32768:
    64 rows x 4 work items) leaves its ticket counter at 256 (every
    workgroup took one), the abort word at 0, and in the slot of (row r,
    segment j) the word {m, s} of that segment — m its maximum, s >= 1. The
    two passes (segments of 8192) leave row 0's first segment state (max,
    sum, ...) at the start of the workspace instead."""
    R, C = 64, 131072
    x = softmax_input(fr.F32, R, C, seed=41)
    seg_max = lambda r, j, n: x[r, j * n:(j + 1) * n].max().view(np.uint32)
    for mode in (2, 0):
        with fr.split_one_pass(mode):
            ws = workspace(R, C)
            got = _softmax_split_ws(x, ws)
        expect_softmax(x, fr.F32, got, f"split softmax {R}x{C} mode {mode}")
        words = ws.t.cpu().numpy().view(np.uint32)
        if mode:
            assert (words[0], words[1]) == (R * 4, 0), words[:4]
            for r, j in ((0, 0), (5, 3), (63, 2)):
                k = 4 + 4 * (r * 4 + j)
                assert words[k] == seg_max(r, j, 32768), (r, j, words[k:k + 4])
                assert words[k + 1] >= np.float32(1.0).view(np.uint32)
        else:
            assert words[0] == seg_max(0, 0, 8192), words[:4]
            assert words[1] >= np.float32(1.0).view(np.uint32)       # the exponential sum


def test_one_pass_wait_bound():
    """The bounded wait, forced to give up: with the poll bound at 0 a member
    gives up whenever its first poll does not find every state of its row
    (and every later wait gives up once one has). The launch still ends, and
    each row is either the oracle's or holds NaN (a member that gave up);
    the next call, with the default bound, is right throughout (its slots
    and abort word are cleared again)."""
    R, C = 96, 131072
    x = softmax_input(fr.F32, R, C, seed=42)
    with fr.split_one_pass(2):
        with fr.coop_spin_limit(0):
            got = _softmax_split_ws(x, workspace(R, C))
        nan_rows = np.isnan(got).any(axis=1)
        print(f"rows with NaN after forced give-ups: {int(nan_rows.sum())} of {R}", flush=True)
        keep = np.flatnonzero(~nan_rows)
        if keep.size:
            expect_softmax(x[keep], fr.F32, got[keep], "split softmax, rows not given up")
        expect_softmax(x, fr.F32, _softmax_split_ws(x, workspace(R, C)), "split softmax after")


def test_convenience_routes_wide_rows():
    x = softmax_input(0, 2, 100000, seed=14)
    y = fr.softmax(upload(x))
    expect_softmax(x, 0, y.cpu().numpy(), "softmax() of a wide row")
    xl, lab = xent_inputs(2, 100000, fr.F32, seed=15)
    loss, grad = fr.softmax_xent(upload(xl), upload(lab))
    lo, go, _, _ = oracle.softmax_xent_ex(xl, lab)
    check_f32(loss.cpu().numpy(), lo, scale=np.maximum(np.abs(lo), 1.0), what="softmax_xent() wide")


# ------------------------------------------------------ LayerNorm / RMSNorm

from test_gpu_parity import expect_layernorm, expect_rmsnorm  # noqa: E402


def run_ln_split(w_x, w_g, w_b, eps, offs=(0, 0), inplace=False):
    x, g, b = upload(w_x, offs[0]), upload(w_g, offs[1]), upload(w_b, offs[1])
    R, C = w_x.shape
    ws = workspace(R, C)
    mean, rstd = Guarded((R,), torch.float32), Guarded((R,), torch.float32)
    y = None if inplace else Guarded((R, C), x.dtype, offs[0])
    yt = x if inplace else y.t
    fr.fr_layernorm_fwd_split(x, g, b, yt, ws.t, mean.t, rstd.t, eps)
    torch.cuda.synchronize()
    assert ws.canaries_intact() and mean.canaries_intact() and rstd.canaries_intact()
    assert y is None or y.canaries_intact(), "split LayerNorm wrote out of bounds"
    return host(yt), mean.t.cpu().numpy(), rstd.t.cpu().numpy()


def run_rms_split(w_x, w_r, w_w, eps, offs=(0, 0), inplace=False, with_res_out=True):
    x, r, wt = upload(w_x, offs[0]), upload(w_r, offs[0]), upload(w_w, offs[1])
    R, C = w_x.shape
    ws = workspace(R, C)
    if inplace:  # y over x, residual_out over the residual
        fr.fr_add_rmsnorm_fwd_split(x, r, wt, x, ws.t, r, eps)
        torch.cuda.synchronize()
        assert ws.canaries_intact()
        return host(x), host(r)
    y = Guarded((R, C), x.dtype, offs[0])
    ro = Guarded((R, C), x.dtype, offs[0]) if with_res_out else None
    fr.fr_add_rmsnorm_fwd_split(x, r, wt, y.t, ws.t, ro.t if ro else None, eps)
    torch.cuda.synchronize()
    assert ws.canaries_intact() and y.canaries_intact() and (ro is None or ro.canaries_intact())
    return host(y.t), (host(ro.t) if ro else None)


NORM_WIDTHS = [1, 5, 1000, 8191, 8192, 8193, 65536, 65537, 100000, 262144]


@pytest.mark.parametrize("C", NORM_WIDTHS)
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_layernorm_split_widths(C, dt, form):
    for R in (1, 3):
        w = workloads.make("layernorm_f32", rows=R, cols=C, seed=C + R, dtype=dt)
        got = run_ln_split(w["x"], w["gamma"], w["beta"], w.eps)
        expect_layernorm(w["x"], w["gamma"], w["beta"], w.eps, got, f"split layernorm {dt} {R}x{C}")


@pytest.mark.parametrize("C", NORM_WIDTHS)
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_rmsnorm_split_widths(C, dt, form):
    for R in (1, 3):
        w = workloads.make("add_rmsnorm_bf16", rows=R, cols=C, seed=C + R, dtype=dt)
        got = run_rms_split(w["x"], w["residual"], w["weight"], w.eps, with_res_out=R == 3)
        expect_rmsnorm(w["x"], w["residual"], w["weight"], w.eps, got,
                       f"split add_rmsnorm {dt} {R}x{C}")


@pytest.mark.parametrize("t,v", SEG_SHAPES)
def test_norm_split_every_segment_shape(t, v, form):
    ran = 0
    for dt, code in (("f32", fr.F32), ("bf16", fr.BF16)):
        for vp, offs in ((True, (0, 0)), (False, (1, 3))):
            for op in (fr.OP_LAYERNORM_SPLIT, fr.OP_RMSNORM_SPLIT):
                try:
                    with fr.forced_variant(op, t, v):
                        tt, vv, e = fr.fr_debug_select_variant(op, 1, code, vector_path=vp)
                except fr.FusedRowError:
                    continue
                seg = tt * vv * e
                # the vector path needs every row on the 16-byte grid (the
                # parameter vectors share the rows' phase): widths of 8k
                widths = (seg - 8, seg, 2 * seg + 40, 5 * seg) if vp else (seg - 3, 2 * seg + 37)
                for C in widths:
                    with fr.forced_variant(op, t, v):
                        if op == fr.OP_LAYERNORM_SPLIT:
                            w = workloads.make("layernorm_f32", rows=2, cols=C, seed=C, dtype=dt)
                            got = run_ln_split(w["x"], w["gamma"], w["beta"], w.eps, offs)
                        else:
                            w = workloads.make("add_rmsnorm_bf16", rows=2, cols=C, seed=C, dtype=dt)
                            got = run_rms_split(w["x"], w["residual"], w["weight"], w.eps, offs)
                    what = f"split norm op {op} [{t},{v},{vp}] {dt} 2x{C}"
                    if op == fr.OP_LAYERNORM_SPLIT:
                        expect_layernorm(w["x"], w["gamma"], w["beta"], w.eps, got, what)
                    else:
                        expect_rmsnorm(w["x"], w["residual"], w["weight"], w.eps, got, what)
                    ran += 1
    if not ran:
        pytest.skip(f"no split norm shape ({t}, {v})")


def test_norm_split_in_place_and_misaligned(form):
    for dt in ("f32", "bf16"):
        w = workloads.make("layernorm_f32", rows=4, cols=70001, seed=21, dtype=dt)
        expect_layernorm(w["x"], w["gamma"], w["beta"], w.eps,
                         run_ln_split(w["x"], w["gamma"], w["beta"], w.eps, inplace=True),
                         f"split layernorm in place {dt}")
        for offs in ((1, 1), (3, 0), (0, 5)):
            expect_layernorm(w["x"], w["gamma"], w["beta"], w.eps,
                             run_ln_split(w["x"], w["gamma"], w["beta"], w.eps, offs),
                             f"split layernorm offs {offs} {dt}")
        w = workloads.make("add_rmsnorm_bf16", rows=4, cols=131072, seed=22, dtype=dt)
        expect_rmsnorm(w["x"], w["residual"], w["weight"], w.eps,
                       run_rms_split(w["x"], w["residual"], w["weight"], w.eps, inplace=True),
                       f"split add_rmsnorm in place {dt}")
        expect_rmsnorm(w["x"], w["residual"], w["weight"], w.eps,
                       run_rms_split(w["x"], w["residual"], w["weight"], w.eps, (1, 2)),
                       f"split add_rmsnorm misaligned {dt}")


def test_norm_split_special_rows(form):
    C = 100000
    w = workloads.make("layernorm_f32", rows=3, cols=C, seed=23)
    x = w["x"].copy()
    x[0, :] = 2.5                                   # constant row: y = beta, rstd = 1/sqrt(eps)
    x[1, :C // 2] = -7.0                            # two-valued row across the segments
    x[1, C // 2:] = 9.0
    got = run_ln_split(x, w["gamma"], w["beta"], w.eps)
    expect_layernorm(x, w["gamma"], w["beta"], w.eps, got, "split layernorm special rows")
    assert np.array_equal(got[0][0], w["beta"])
    w = workloads.make("add_rmsnorm_bf16", rows=2, cols=C, seed=24, dtype="f32")
    xr = w["x"].copy()
    rr = w["residual"].copy()
    rr[0] = -xr[0]                                  # h = 0: y = 0
    got = run_rms_split(xr, rr, w["weight"], w.eps)
    expect_rmsnorm(xr, rr, w["weight"], w.eps, got, "split add_rmsnorm zero row")
    assert np.all(got[0][0] == 0)


def test_norm_split_determinism_and_convenience(form):
    w = workloads.make("layernorm_f32", rows=8, cols=200000, seed=25, dtype="bf16")
    a = run_ln_split(w["x"], w["gamma"], w["beta"], w.eps)
    b = run_ln_split(w["x"], w["gamma"], w["beta"], w.eps)
    assert all(np.array_equal(p, q) for p, q in zip(a, b))
    y, m, r = fr.layernorm(upload(w["x"]), upload(w["gamma"]), upload(w["beta"]), w.eps)
    assert np.array_equal(host(y), a[0]) and np.array_equal(m.cpu().numpy(), a[1])
    w = workloads.make("add_rmsnorm_bf16", rows=2, cols=100000, seed=26)
    y, ro = fr.add_rmsnorm(upload(w["x"]), upload(w["residual"]), upload(w["weight"]), w.eps)
    expect_rmsnorm(w["x"], w["residual"], w["weight"], w.eps, (host(y), host(ro)),
                   "add_rmsnorm() of a wide row")


# ---------------------------------------------------------- softmax backward

from test_gpu_backward import expect_softmax_bwd, softmax_bwd_inputs  # noqa: E402


def run_softmax_bwd_split(p, dy, offs=(0, 0, 0), inplace=None):
    R, C = p.shape
    pt, dyt = upload(p, offs[0]), upload(dy, offs[1])
    ws = workspace(R, C)
    if inplace:
        tgt = pt if inplace == "p" else dyt
        fr.fr_softmax_bwd_split(pt, dyt, tgt, ws.t)
        torch.cuda.synchronize()
        assert ws.canaries_intact()
        return host(tgt)
    dx = Guarded((R, C), pt.dtype, offs[2])
    fr.fr_softmax_bwd_split(pt, dyt, dx.t, ws.t)
    torch.cuda.synchronize()
    assert dx.canaries_intact() and ws.canaries_intact(), "split softmax_bwd wrote out of bounds"
    return host(dx.t)


@pytest.mark.parametrize("C", [1, 7, 8192, 8193, 16385, 65537, 262144])
@pytest.mark.parametrize("code", [fr.F32, fr.BF16])
def test_softmax_bwd_split_widths(C, code, form):
    for R in (1, 3):
        p, dy = softmax_bwd_inputs(R, C, code, seed=C + R)
        expect_softmax_bwd(p, dy, code, run_softmax_bwd_split(p, dy), f"split softmax_bwd {code} {R}x{C}")


def test_softmax_bwd_split_shapes_in_place_misaligned(form):
    for t, v in SEG_SHAPES:
        for code in (fr.F32, fr.BF16):
            for vp, offs in ((True, (0, 0, 0)), (False, (1, 2, 0))):
                try:
                    with fr.forced_variant(fr.OP_SOFTMAX_BWD_SPLIT, t, v):
                        tt, vv, e = fr.fr_debug_select_variant(fr.OP_SOFTMAX_BWD_SPLIT, 1, code,
                                                               vector_path=vp)
                except fr.FusedRowError:
                    continue
                C = 2 * tt * vv * e + 37
                p, dy = softmax_bwd_inputs(2, C, code, seed=C + t)
                with fr.forced_variant(fr.OP_SOFTMAX_BWD_SPLIT, t, v):
                    got = run_softmax_bwd_split(p, dy, offs)
                expect_softmax_bwd(p, dy, code, got, f"split softmax_bwd [{t},{v},{vp}] {code} 2x{C}")
    for code in (fr.F32, fr.BF16):
        p, dy = softmax_bwd_inputs(3, 100003, code, seed=31)
        for ip in ("p", "dy"):
            expect_softmax_bwd(p, dy, code, run_softmax_bwd_split(p, dy, inplace=ip),
                               f"split softmax_bwd in place ({ip}) {code}")
    p, dy = softmax_bwd_inputs(2, 70000, fr.F32, seed=32)
    dx = fr.softmax_bwd(upload(p), upload(dy))
    expect_softmax_bwd(p, dy, fr.F32, dx.cpu().numpy(), "softmax_bwd() of a wide row")


# ------------------------------------------------------- norm backward, split

from test_gpu_backward import (expect_ln_bwd, expect_rms_bwd, ln_bwd_inputs,  # noqa: E402
                               rms_bwd_inputs)
from parity import to_dev  # noqa: E402


def bwd_workspace(op, R, C):
    return Guarded((max(fr.fr_norm_bwd_split_workspace_bytes(op, R, C) // 4, 4),), torch.float32)


def run_rms_bwd_split(w, code, with_dres=True, off=0, inplace=None):
    R, C = w["h"].shape
    h, dy, wt = upload(w["h"], off), upload(w["dy"], off), upload(w["weight"], off)
    dres = upload(w["dres"], off) if with_dres else None
    dw = Guarded((C,), torch.float32)
    ws = bwd_workspace(fr.OP_RMSNORM_BWD, R, C)
    if inplace:
        dh, dh_t = None, {"dy": dy, "h": h, "dres": dres}[inplace]
    else:
        dh = Guarded((R, C), TDT[code], off)
        dh_t = dh.t
    fr.fr_add_rmsnorm_bwd_split(h, dy, wt, dh_t, dw.t, ws.t, dres=dres, eps=w.eps)
    torch.cuda.synchronize()
    assert dw.canaries_intact() and ws.canaries_intact() and (dh is None or dh.canaries_intact())
    return host(dh_t), dw.t.cpu().numpy()


def run_ln_bwd_split(w, mean, rstd, code, off=0, inplace=None):
    R, C = w["x"].shape
    x, dy, g = upload(w["x"], off), upload(w["dy"], off), upload(w["gamma"], off)
    m, r = to_dev(mean), to_dev(rstd)
    dg, db = Guarded((C,), torch.float32), Guarded((C,), torch.float32)
    ws = bwd_workspace(fr.OP_LAYERNORM_BWD, R, C)
    if inplace:
        dx, dx_t = None, {"x": x, "dy": dy}[inplace]
    else:
        dx = Guarded((R, C), TDT[code], off)
        dx_t = dx.t
    fr.fr_layernorm_bwd_split(x, dy, g, m, r, dx_t, dg.t, db.t, ws.t)
    torch.cuda.synchronize()
    assert dg.canaries_intact() and db.canaries_intact() and ws.canaries_intact()
    assert dx is None or dx.canaries_intact()
    return host(dx_t), dg.t.cpu().numpy(), db.t.cpu().numpy()


BWD_WIDTHS = [16385, 24576, 65537, 100000]


@pytest.mark.parametrize("C", BWD_WIDTHS)
@pytest.mark.parametrize("code", [fr.F32, fr.BF16])
def test_rms_bwd_split_widths(C, code, form):
    for R, dres in ((1, True), (5, False)):
        w = rms_bwd_inputs(R, C, code, seed=C + R)
        expect_rms_bwd(w, code, run_rms_bwd_split(w, code, with_dres=dres),
                       f"split rms_bwd {code} {R}x{C} dres={dres}", with_dres=dres)


@pytest.mark.parametrize("C", BWD_WIDTHS)
@pytest.mark.parametrize("code", [fr.F32, fr.BF16])
def test_ln_bwd_split_widths(C, code, form):
    for R in (1, 5):
        w, mean, rstd = ln_bwd_inputs(R, C, code, seed=C + R)
        expect_ln_bwd(w, mean, rstd, code, run_ln_bwd_split(w, mean, rstd, code),
                      f"split ln_bwd {code} {R}x{C}")


def test_norm_bwd_split_many_rows_in_place_misaligned(form):
    # more rows than row groups (each workgroup takes several rows), the
    # scalar path (misaligned), and outputs over their inputs
    for code in (fr.F32, fr.BF16):
        w = rms_bwd_inputs(700, 32768, code, seed=41)
        expect_rms_bwd(w, code, run_rms_bwd_split(w, code), f"split rms_bwd {code} 700x32768")
        w = rms_bwd_inputs(3, 40000, code, seed=42)
        expect_rms_bwd(w, code, run_rms_bwd_split(w, code, off=1), f"split rms_bwd {code} misaligned")
        for ip in ("h", "dy", "dres"):
            expect_rms_bwd(w, code, run_rms_bwd_split(w, code, inplace=ip),
                           f"split rms_bwd {code} in place ({ip})")
        w, mean, rstd = ln_bwd_inputs(600, 32768, code, seed=43)
        expect_ln_bwd(w, mean, rstd, code, run_ln_bwd_split(w, mean, rstd, code),
                      f"split ln_bwd {code} 600x32768")
        w, mean, rstd = ln_bwd_inputs(3, 40001, code, seed=44)
        expect_ln_bwd(w, mean, rstd, code, run_ln_bwd_split(w, mean, rstd, code, off=1),
                      f"split ln_bwd {code} misaligned")
        for ip in ("x", "dy"):
            expect_ln_bwd(w, mean, rstd, code, run_ln_bwd_split(w, mean, rstd, code, inplace=ip),
                          f"split ln_bwd {code} in place ({ip})")


def test_norm_bwd_split_determinism_rows_zero_and_convenience(form):
    w = rms_bwd_inputs(64, 50000, fr.BF16, seed=45)
    a = run_rms_bwd_split(w, fr.BF16)
    b = run_rms_bwd_split(w, fr.BF16)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    dw = torch.full((30000,), 5.0, device=DEV)
    e = torch.empty(0, 30000, device=DEV)
    ws = torch.empty(16, dtype=torch.uint8, device=DEV)
    fr.fr_add_rmsnorm_bwd_split(e, e, torch.ones(30000, device=DEV), e, dw, ws)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dw).item() == 0
    dh, dwc = fr.add_rmsnorm_bwd(upload(w["h"]), upload(w["dy"]), upload(w["weight"]), w.eps,
                                 dres=upload(w["dres"]))
    assert np.array_equal(host(dh), a[0]) and np.array_equal(dwc.cpu().numpy(), a[1])
    w, mean, rstd = ln_bwd_inputs(4, 30000, fr.F32, seed=46)
    dx, dg, db = fr.layernorm_bwd(upload(w["x"]), upload(w["dy"]), upload(w["gamma"]),
                                  to_dev(mean), to_dev(rstd))
    expect_ln_bwd(w, mean, rstd, fr.F32, (host(dx), dg.cpu().numpy(), db.cpu().numpy()),
                  "layernorm_bwd() of a wide row")


# ------------------------------------------- bounded waits, every one-pass kernel

def _as_f64(a):
    a = np.asarray(a)
    if a.dtype == np.uint16:  # bf16 bit patterns
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def _wait_bound_cases():
    """(name, run) pairs: run() returns the call's row outputs (arrays of rows)
    and its per-column outputs."""
    cases = []
    x = softmax_input(fr.F32, 96, 131072, seed=51)
    cases.append(("softmax fp32", lambda: ((run_softmax_split(x, fr.F32),), ())))
    xl, lab = xent_inputs(64, 262144, fr.BF16, seed=52, ignore_every=5)
    opts = dict(ignore_index=-100, label_smoothing=0.1)
    cases.append(("cross-entropy bf16", lambda: (lambda r: ((r[1], r[0][:, None], r[2][:, None]), ()))(
        run_xent_split(xl, lab, fr.BF16, opts))))
    wr = workloads.make("add_rmsnorm_bf16", rows=48, cols=262144, seed=53)
    cases.append(("add_rmsnorm bf16", lambda: (run_rms_split(wr["x"], wr["residual"], wr["weight"],
                                                             wr.eps), ())))
    wl = workloads.make("layernorm_f32", rows=64, cols=131072, seed=54)
    cases.append(("layernorm fp32", lambda: (lambda r: ((r[0], r[1][:, None], r[2][:, None]), ()))(
        run_ln_split(wl["x"], wl["gamma"], wl["beta"], wl.eps))))
    p, dy = softmax_bwd_inputs(96, 131072, fr.BF16, seed=55)
    cases.append(("softmax_bwd bf16", lambda: ((run_softmax_bwd_split(p, dy),), ())))
    wb = rms_bwd_inputs(64, 65536, fr.F32, seed=56)
    cases.append(("add_rmsnorm_bwd fp32", lambda: (lambda r: ((r[0],), (r[1],)))(
        run_rms_bwd_split(wb, fr.F32))))
    wn, mean, rstd = ln_bwd_inputs(64, 65536, fr.F32, seed=57)
    cases.append(("layernorm_bwd fp32", lambda: (lambda r: ((r[0],), (r[1], r[2])))(
        run_ln_bwd_split(wn, mean, rstd, fr.F32))))
    return cases


def test_one_pass_wait_bound_every_kernel():
    """Every one-pass kernel with its waits forced to give up (poll bound 0:
    a workgroup gives up whenever its first poll does not find all of its
    row's states): the launch ends, and every row of every row output is
    either bitwise the one of a call with the default bound or holds NaN (a
    workgroup that gave up; an ignored row of the cross-entropy, whose loss
    and gradient are 0 regardless, shows it as argmax -1); the per-column
    outputs (parameter gradients)
    are bitwise the same when no row gave up. The next call, with the
    default bound, is bitwise the same throughout."""
    with fr.split_one_pass(2):
        for name, run in _wait_bound_cases():
            print(f"bounded waits: {name}", flush=True)
            ref_rows, ref_cols = run()
            with fr.coop_spin_limit(0):
                got_rows, got_cols = run()
            # a row given up: NaN in one of its float outputs, or an argmax of
            # -1 (an ignored row's loss and gradient are 0 all the same)
            nan_any = np.zeros(len(ref_rows[0]), dtype=bool)
            for g in got_rows:
                g = np.asarray(g)
                if g.dtype == np.int32:
                    nan_any |= (g.reshape(len(g), -1) == -1).any(axis=1)
                else:
                    nan_any |= np.isnan(_as_f64(g)).reshape(len(g), -1).any(axis=1)
            for g, r in zip(got_rows, ref_rows):
                g2 = np.ascontiguousarray(np.asarray(g).reshape(len(g), -1))
                r2 = np.ascontiguousarray(np.asarray(r).reshape(len(r), -1))
                same = (g2.view(np.uint8) == r2.view(np.uint8)).all(axis=1)
                ok = same | nan_any
                assert ok.all(), f"{name}: rows {np.flatnonzero(~ok)[:8]} neither right nor NaN"
            if not nan_any.any():
                for g, r in zip(got_cols, ref_cols):
                    assert np.array_equal(g, r), f"{name}: per-column outputs differ"
            print(f"  rows given up: {int(nan_any.sum())} of {len(nan_any)}", flush=True)
            after_rows, after_cols = run()
            for g, r in zip(after_rows + after_cols, ref_rows + ref_cols):
                g2, r2 = np.ascontiguousarray(g), np.ascontiguousarray(r)
                assert np.array_equal(g2.view(np.uint8), r2.view(np.uint8)), \
                    f"{name}: the call after differs"


def test_one_pass_repeated_calls_bitwise():
    """Each one-pass kernel called 20 times on the same inputs (a different
    interleaving of its workgroups' posts and waits each time): every call
    bitwise the same, and no row given up."""
    with fr.split_one_pass(2):
        for name, run in _wait_bound_cases():
            print(f"repeated calls: {name}", flush=True)
            first = run()
            flat0 = [np.ascontiguousarray(a).view(np.uint8) for a in first[0] + first[1]]
            for a in first[0]:
                a = np.asarray(a)
                if a.dtype == np.int32:
                    assert not (a == -1).any(), f"{name}: a row given up"
                else:
                    assert not np.isnan(_as_f64(a)).any(), f"{name}: a row given up"
            for k in range(19):
                got = run()
                flat = [np.ascontiguousarray(a).view(np.uint8) for a in got[0] + got[1]]
                assert all(np.array_equal(x, y) for x, y in zip(flat0, flat)), \
                    f"{name}: call {k + 2} differs from the first"


def test_bench_split_shapes_sampled():
    """The benchmark's split workloads at their full sizes, in the form the
    default selection takes there (one pass for each), checked against the
    oracle on sampled rows (the first two, two in the middle, the last two):
    cross-entropy bf16 [1024, 262144] (every 7th row ignored, smoothing 0.1,
    argmax), LayerNorm fp32 [512, 131072], residual-add + RMSNorm bf16
    [256, 262144], softmax backward bf16 [1024, 131072]."""
    def pick(R):
        return np.array(sorted({0, 1, R // 2 - 1, R // 2, R - 2, R - 1}))
    for op, R, C, dt in ((fr.OP_XENT_SPLIT, 1024, 262144, fr.BF16),
                         (fr.OP_LAYERNORM_SPLIT, 512, 131072, fr.F32),
                         (fr.OP_RMSNORM_SPLIT, 256, 262144, fr.BF16),
                         (fr.OP_SOFTMAX_BWD_SPLIT, 1024, 131072, fr.BF16)):
        t, v, e = fr.fr_debug_select_variant_for(op, R, C, dt)
        assert (t, v * e) == (512, 32 if op == fr.OP_LAYERNORM_SPLIT else 64), (op, t, v, e)
    rows = pick(1024)
    xl, lab = xent_inputs(1024, 262144, fr.BF16, seed=61, ignore_every=7)
    opts = dict(ignore_index=-100, label_smoothing=0.1)
    loss, grad, am, _ = run_xent_split(xl, lab, fr.BF16, opts)
    expect_xent(xl[rows], lab[rows], fr.BF16, opts, (loss[rows], grad[rows], am[rows], 0.0),
                "split xent bf16 1024x262144 (sampled)")
    del xl, grad
    rows = pick(512)
    wl = workloads.make("layernorm_f32", rows=512, cols=131072, seed=62)
    y, m, r = run_ln_split(wl["x"], wl["gamma"], wl["beta"], wl.eps)
    expect_layernorm(wl["x"][rows], wl["gamma"], wl["beta"], wl.eps, (y[rows], m[rows], r[rows]),
                     "split layernorm fp32 512x131072 (sampled)")
    del wl, y
    rows = pick(256)
    wr = workloads.make("add_rmsnorm_bf16", rows=256, cols=262144, seed=63)
    y, ro = run_rms_split(wr["x"], wr["residual"], wr["weight"], wr.eps)
    expect_rmsnorm(wr["x"][rows], wr["residual"][rows], wr["weight"], wr.eps, (y[rows], ro[rows]),
                   "split add_rmsnorm bf16 256x262144 (sampled)")
    del wr, y, ro
    rows = pick(1024)
    p, dy = softmax_bwd_inputs(1024, 131072, fr.BF16, seed=64)
    dx = run_softmax_bwd_split(p, dy)
    expect_softmax_bwd(p[rows], dy[rows], fr.BF16, dx[rows], "split softmax_bwd bf16 1024x131072 (sampled)")


# ------------------------------------------------------------ row batches

def _bits(*arrays):
    return tuple(None if a is None else np.ascontiguousarray(a).tobytes() for a in arrays)


@pytest.mark.parametrize("batch_rows", [1, 3, 64])
def test_split_row_batches(batch_rows):
    """The two-pass launches (the one-pass form switched off) run both passes
    over one batch of rows at a time (bounded by input bytes): batches of 1 and 3 rows (a ragged last batch of
    7 rows) and one batch of all of them, for every split entry point. Each
    result matches the oracle and has the same bits as the unbatched call."""
    R = 7
    cases = []
    x = softmax_input(fr.F32, R, 20000, seed=31)
    cases.append(("softmax f32", 20000 * 4, lambda: (run_softmax_split(x, fr.F32),),
                  lambda got: expect_softmax(x, fr.F32, got[0], "split softmax batches")))
    xb = softmax_input(fr.BF16, R, 70001, seed=32)
    cases.append(("softmax bf16", 70001 * 2, lambda: (run_softmax_split(xb, fr.BF16, offs=(1, 1)),),
                  lambda got: expect_softmax(xb, fr.BF16, got[0], "split softmax bf16 batches")))
    opts = dict(ignore_index=-100, label_smoothing=0.1, reduction="mean")
    for code, es in ((fr.F32, 4), (fr.BF16, 2)):
        xl, lab = xent_inputs(R, 70000, code, seed=33 + code, ignore_every=3)
        cases.append((f"xent {code}", 70000 * es,
                      lambda xl=xl, lab=lab, code=code: run_xent_split(xl, lab, code, opts),
                      lambda got, xl=xl, lab=lab, code=code: expect_xent(
                          xl, lab, code, opts, got, f"split xent {code} batches")))
    wl = workloads.make("layernorm_f32", rows=R, cols=20000, seed=35)
    cases.append(("layernorm f32", 20000 * 4,
                  lambda: run_ln_split(wl["x"], wl["gamma"], wl["beta"], wl.eps),
                  lambda got: expect_layernorm(wl["x"], wl["gamma"], wl["beta"], wl.eps, got,
                                               "split layernorm batches")))
    wr = workloads.make("add_rmsnorm_bf16", rows=R, cols=20000, seed=36)
    cases.append(("rmsnorm bf16", 20000 * 2 * 2,
                  lambda: run_rms_split(wr["x"], wr["residual"], wr["weight"], wr.eps),
                  lambda got: expect_rmsnorm(wr["x"], wr["residual"], wr["weight"], wr.eps, got,
                                             "split rmsnorm batches")))
    p, dy = softmax_bwd_inputs(R, 20000, fr.BF16, seed=37)
    cases.append(("softmax bwd bf16", 20000 * 2 * 2, lambda: (run_softmax_bwd_split(p, dy),),
                  lambda got: expect_softmax_bwd(p, dy, fr.BF16, got[0], "split softmax_bwd batches")))
    for name, row_bytes, run, expect in cases:
        print(f"row batches of {batch_rows}: {name}", flush=True)
        with fr.split_one_pass(0), fr.split_batch_bytes(batch_rows * row_bytes):
            got = run()
        with fr.split_one_pass(0), fr.split_batch_bytes(0):
            whole = run()
        expect(got)
        assert _bits(*got) == _bits(*whole), f"{name}: batched and unbatched results differ"
