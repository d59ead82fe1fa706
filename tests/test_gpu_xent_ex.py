"""GPU parity of the cross-entropy variants (fr_softmax_xent_ex: bf16 or fp32
logits, ignore_index, label smoothing, sum / mean reduction, gradient scale)
against the double-precision oracle, through the C ABI.

Tolerances: the fp32 rule of parity.py (|g - o| <= 1e-5 * scale + 2^-126) at
scales that bound each output's rounding error:
  grad_j      |g| (p_j + q_j)    (g p_j - g q_j is a cancellation near p_j = q_j)
  loss_r      max(|loss_r|, |lse| + (1 - eps)|x_label| + eps mean_j |x_j|)
  total       sum_r of the loss scales (/ n_valid for the mean)
Ignored rows must be exactly zero (loss and gradient). bf16 gradients pass
within one ulp of the rounded oracle or by the rule above plus their final
rounding.
"""
import numpy as np
import pytest
import torch

import memory_bound_row_pass_amd as fr
import oracle
import workloads
from gpu_buffers import DEV, TDT, Guarded, host, upload
from parity import check_bf16, check_f32

pytestmark = pytest.mark.gpu


def setup_module(module):
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    oracle.set_threads(min(16, oracle.threads()))


def inputs(R, C, code, seed, ignore_every=0):
    w = workloads.make("xent_f32", rows=R, cols=C, seed=seed,
                       dtype="bf16" if code == fr.BF16 else "f32")
    lab = w["labels"].copy()
    if ignore_every:
        lab[::ignore_every] = -100
    return w["logits"], lab


def run(logits, labels, code, opts, argmax=True, offs=(0, 0), inplace=False, stream=None):
    R, C = logits.shape
    x = upload(logits, offs[0])
    lab = upload(labels)
    loss = Guarded((R,), torch.float32)
    am = Guarded((R,), torch.int32) if argmax else None
    tot = Guarded((1,), torch.float32)
    if inplace:
        g_t, g = x, None
    else:
        g = Guarded((R, C), TDT[code], offs[1])
        g_t = g.t
    fr.fr_softmax_xent_ex(x, lab, loss.t, g_t, am.t if am else None, tot.t, stream=stream, **opts)
    torch.cuda.synchronize()
    assert loss.canaries_intact() and tot.canaries_intact()
    assert (g is None or g.canaries_intact()) and (am is None or am.canaries_intact())
    return (loss.t.cpu().numpy(), host(g_t), am.t.cpu().numpy() if am else None,
            float(tot.t.cpu()[0]))


def expect(logits, labels, code, opts, got, what):
    loss, grad, am, tot = got
    eps = float(np.float32(opts.get("label_smoothing", 0.0)))
    scale = float(np.float32(opts.get("grad_scale", 1.0)))
    red = opts.get("reduction", "none")
    ign = opts.get("ignore_index")
    lo, go, ao, to = oracle.softmax_xent_ex(logits, labels, ignore_index=ign, label_smoothing=eps,
                                            reduction=red, grad_scale=scale)
    R, C = logits.shape
    xd = oracle.decode(logits)
    p = oracle.softmax(logits)
    ignored = (labels == ign) if ign is not None else np.zeros(R, bool)
    valid = (labels >= 0) & (labels < C) & ~ignored
    nv = int((~ignored).sum())
    g = scale / nv if red == "mean" else scale
    q = np.full((R, C), eps / C)
    q[ignored] = 0.0
    rows = np.nonzero(valid)[0]
    q[rows, labels[rows]] += 1 - eps
    s_grad = abs(g) * (p + q)
    if code == fr.BF16:
        hist = check_bf16(grad, oracle.round_bf16(go), what + " grad",
                          cond=(go, np.maximum(s_grad, np.abs(go))))
    else:
        hist = check_f32(grad, go, scale=np.maximum(s_grad, np.abs(go)), what=what + " grad")
    gfl = grad.astype(np.float64) if code == fr.F32 else \
        (grad.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.all(gfl[ignored] == 0), what + ": ignored rows must have a zero gradient"
    assert np.all(loss[ignored] == 0), what + ": ignored rows must have loss 0"
    bad = ~valid & ~ignored
    assert np.all(np.isnan(loss[bad])), what + ": an invalid label must give a NaN loss"
    lse = np.log(np.exp(xd - xd.max(1, keepdims=True)).sum(1)) + xd.max(1)
    xl = np.where(valid, xd[np.arange(R), np.clip(labels, 0, C - 1)], 0.0)
    smooth = eps * np.abs(xd).mean(1) if eps else 0.0
    s_loss = np.maximum(np.abs(lo), np.abs(lse) + (1 - eps) * np.abs(xl) + smooth)
    check_f32(loss[valid], lo[valid], scale=s_loss[valid], what=what + " loss")
    if am is not None:
        assert np.array_equal(am, ao), what + " argmax"
    if red != "none":
        if np.isnan(to):
            assert np.isnan(tot), what + " total"
        else:
            st = s_loss[valid].sum() / (nv if red == "mean" else 1)
            check_f32(np.array([tot]), np.array([to]), scale=np.array([max(st, abs(to))]),
                      what=what + " total")
    return hist


OPTS = [
    dict(),
    dict(ignore_index=-100),
    dict(label_smoothing=0.1),
    dict(ignore_index=-100, label_smoothing=0.1, reduction="mean", grad_scale=0.5),
    dict(reduction="sum", grad_scale=2.0),
    dict(ignore_index=7, label_smoothing=1.0, reduction="mean"),
]


# ------------------------------------------------- full-size workloads

@pytest.mark.parametrize("code", [fr.F32, fr.BF16])
def test_workload_xent_with_options(code):
    x, lab = inputs(4096, 50257, code, seed=1005, ignore_every=9)
    opts = dict(ignore_index=-100, label_smoothing=0.1, reduction="mean", grad_scale=1.0)
    h = expect(x, lab, code, opts, run(x, lab, code, opts), f"xent_ex {code} 4096x50257")
    print("xent_ex grad ulp / stats", h)


# ------------------------------------------------------- edge shapes

EDGE_COLS = [1, 2, 3, 7, 8, 9, 63, 64, 65, 1000, 1025, 4096, 8191, 12345, 32768, 50257, 65536]


@pytest.mark.parametrize("C", EDGE_COLS)
@pytest.mark.parametrize("code", [fr.F32, fr.BF16])
def test_edge_cols(C, code):
    for k, opts in enumerate(OPTS):
        x, lab = inputs(5, C, code, seed=C + k, ignore_every=3 if "ignore_index" in opts else 0)
        if opts.get("ignore_index") == 7:
            lab[1] = 7 % C if C > 7 else lab[1]
        expect(x, lab, code, opts, run(x, lab, code, opts, argmax=k % 2 == 0),
               f"xent_ex {code} 5x{C} {opts}")


# ----------------------------------------------------- every variant

VARIANT_GRID = [(t, v) for t in (64, 256, 512, 1024) for v in (1, 2, 4, 7, 8, 13, 16, 25, 50, 64)]


def _caps(t, v, code, vector_path):
    try:
        with fr.forced_variant(fr.OP_XENT, t, v):
            tt, vv, e = fr.fr_debug_select_variant(fr.OP_XENT, 1, code, vector_path=vector_path)
    except fr.FusedRowError:
        return None
    cap = tt * vv * e
    return [cap, max(1, cap - 5 * e - 3), max(1, cap // 2 + 1)]


# only the pairs with a kernel for some (dtype, vector path); the selection
# call runs on the host, so collection needs no GPU
XENT_GRID = [(t, v) for t, v in VARIANT_GRID
             if any(_caps(t, v, c, vp) for c in (fr.F32, fr.BF16) for vp in (True, False))]


@pytest.mark.parametrize("t,v", XENT_GRID)
def test_every_variant(t, v):
    ran = 0
    opts = dict(ignore_index=-100, label_smoothing=0.2, reduction="mean", grad_scale=0.25)
    for code in (fr.F32, fr.BF16):
        for vp, offs in ((True, (0, 0)), (False, (1, 2))):
            for C in _caps(t, v, code, vp) or []:
                x, lab = inputs(4, C, code, seed=C, ignore_every=3)
                with fr.forced_variant(fr.OP_XENT, t, v):
                    got = run(x, lab, code, opts, argmax=True, offs=offs)
                    got2 = run(x, lab, code, dict(label_smoothing=0.05), argmax=False, offs=offs)
                expect(x, lab, code, opts, got, f"xent_ex[{t},{v},{vp}] {code} 4x{C}")
                expect(x, lab, code, dict(label_smoothing=0.05), got2,
                       f"xent_ex[{t},{v},{vp}] {code} 4x{C} no argmax")
                ran += 1
    if not ran:
        pytest.skip(f"no cross-entropy variant ({t}, {v})")


# --------------------------------------------------- alignment / aliasing

@pytest.mark.parametrize("offs", [(1, 1), (3, 3), (1, 0), (0, 2)])
def test_misaligned(offs):
    for code in (fr.F32, fr.BF16):
        for C in (5, 1000, 50257):
            x, lab = inputs(4, C, code, seed=C, ignore_every=2)
            opts = dict(ignore_index=-100, label_smoothing=0.1)
            expect(x, lab, code, opts, run(x, lab, code, opts, offs=offs), f"xent_ex offs {offs}")


def test_in_place():
    for code in (fr.F32, fr.BF16):
        x, lab = inputs(64, 50257, code, seed=6, ignore_every=5)
        opts = dict(ignore_index=-100, label_smoothing=0.1, reduction="sum")
        expect(x, lab, code, opts, run(x, lab, code, opts, inplace=True), f"xent_ex in place {code}")


# ------------------------------------------------------------ special cases

def test_labels_invalid_masked_logits_and_all_ignored():
    C = 3000
    x, _ = inputs(6, C, fr.F32, seed=8)
    x[2, ::5] = -np.inf                           # masked classes
    lab = np.array([-1, C, 17, 2**31 - 1, -100, 0], np.int32)
    for opts in (dict(ignore_index=-100), dict(ignore_index=-100, label_smoothing=0.1,
                                                reduction="sum")):
        expect(x, lab, fr.F32, opts, run(x, lab, fr.F32, opts), f"xent_ex special {opts}")
    lab = np.full(6, -100, np.int32)
    opts = dict(ignore_index=-100, reduction="mean")
    got = run(x, lab, fr.F32, opts)
    assert np.isnan(got[3]) and np.all(got[0] == 0) and np.all(got[1] == 0)


@pytest.mark.parametrize("C", [1000, 4096, 50257])
def test_far_below_max(C):
    # logits far below the row maximum: fp32 gradients keep 1e-5 relative,
    # bf16 gradients reach the bf16 subnormal range (p down to ~1e-40)
    from test_gpu_parity import far_rows
    for code in (fr.F32, fr.BF16):
        x = far_rows(12, C, code, seed=C + 5 * code)
        lab = np.random.default_rng(C).integers(0, C, size=12).astype(np.int32)
        for opts in (dict(), dict(ignore_index=-100, reduction="sum"),
                     dict(label_smoothing=0.1, reduction="mean")):
            for am in (True, False):
                expect(x, lab, code, opts, run(x, lab, code, opts, argmax=am),
                       f"xent_ex far {code} 12x{C} {opts} argmax={am}")


def test_rows_zero():
    e = torch.empty(0, 10, device=DEV)
    lab = torch.empty(0, dtype=torch.int32, device=DEV)
    loss = torch.empty(0, device=DEV)
    for red, want in (("sum", 0.0), ("mean", float("nan"))):
        tot = torch.full((1,), 7.0, device=DEV)
        fr.fr_softmax_xent_ex(e, lab, loss, e, None, tot, reduction=red)
        torch.cuda.synchronize()
        v = float(tot.cpu()[0])
        assert (np.isnan(v) and np.isnan(want)) or v == want


def test_convenience_routes():
    x, lab = inputs(32, 50257, fr.F32, seed=9)
    xt, lt = upload(x), upload(lab)
    l0, g0 = fr.softmax_xent(xt, lt)                                  # plain kernel
    l1, g1 = fr.softmax_xent(xt, lt, ignore_index=-100)               # options kernel, none ignored
    assert torch.equal(l0, l1) and torch.equal(g0, g1)
    tot, g2 = fr.softmax_xent(xt, lt, reduction="mean")
    lo, _, _, to = oracle.softmax_xent_ex(x, lab, reduction="mean")
    assert abs(float(tot.cpu()[0]) - to) <= 1e-5 * abs(to)


def test_bitwise_determinism_and_graph_replay():
    x, lab = inputs(512, 50257, fr.BF16, seed=10, ignore_every=4)
    xt, lt = upload(x), upload(lab)
    loss = torch.empty(512, device=DEV)
    grad = torch.empty_like(xt)
    tot = torch.empty(1, device=DEV)
    kw = dict(ignore_index=-100, label_smoothing=0.1, reduction="mean")

    def step():
        fr.fr_softmax_xent_ex(xt, lt, loss, grad, None, tot, **kw)

    step()
    torch.cuda.synchronize()
    ref = (loss.clone(), grad.clone(), tot.clone())
    for _ in range(2):
        step()
        torch.cuda.synchronize()
        assert torch.equal(loss, ref[0]) and torch.equal(grad.view(torch.int16), ref[1].view(torch.int16))
        assert torch.equal(tot, ref[2])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        step()
    for rep in range(3):
        loss.fill_(float("nan"))
        tot.fill_(float("nan"))
        grad.fill_(float("nan"))
        torch.cuda.synchronize()
        gr.replay()
        torch.cuda.synchronize()
        assert torch.equal(loss, ref[0]) and torch.equal(tot, ref[2]), rep
        assert torch.equal(grad.view(torch.int16), ref[1].view(torch.int16)), rep
    expect(x, lab, fr.BF16, kw, (ref[0].cpu().numpy(), host(ref[1]), None, float(ref[2].cpu()[0])),
           "xent_ex graph")


def test_non_default_stream():
    x, lab = inputs(64, 4096, fr.F32, seed=11, ignore_every=3)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    opts = dict(ignore_index=-100, label_smoothing=0.1, reduction="mean")
    expect(x, lab, fr.F32, opts, run(x, lab, fr.F32, opts, stream=s.cuda_stream), "xent_ex side stream")


# ------------------------------------------- several rows per workgroup

@pytest.mark.parametrize("C", [50257, 40001])
def test_many_rows_per_workgroup(C):
    """More rows than compute units, so each workgroup of the 1024-lane
    kernels loops over several rows; the bf16 kernel stages the next row in
    LDS while it reduces and writes the current one. Ignored rows are
    interleaved (the first row among them), with and without argmax,
    misaligned and in place."""
    R = 700
    assert fr.fr_debug_select_variant(fr.OP_XENT, C, fr.BF16) == (1024, 7, 8)
    opts = dict(ignore_index=-100, label_smoothing=0.1, reduction="mean")
    for code in (fr.BF16, fr.F32):
        x, lab = inputs(R, C, code, seed=C + code, ignore_every=3)
        print(f"many rows: {code} {R}x{C}", flush=True)
        for am in (True, False):
            expect(x, lab, code, opts, run(x, lab, code, opts, argmax=am),
                   f"xent_ex {code} {R}x{C} argmax={am}")
        expect(x, lab, code, opts, run(x, lab, code, opts, argmax=False, offs=(1, 1)),
               f"xent_ex {code} {R}x{C} misaligned")
        expect(x, lab, code, dict(), run(x, lab, code, dict(), argmax=False, inplace=True),
               f"xent_ex {code} {R}x{C} in place")


def test_few_rows_shape_with_options():
    # two rows per compute unit (256-lane shape) with options, fp32 logits
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    R, C = 2 * ncu - 3, 50257
    assert fr.fr_debug_select_variant_for(fr.OP_XENT, R, C, fr.F32) == (256, 50, 4)
    x, lab = inputs(R, C, fr.F32, seed=77, ignore_every=5)
    opts = dict(ignore_index=-100, label_smoothing=0.1, reduction="mean")
    got = run(x, lab, fr.F32, opts, argmax=False)
    expect(x, lab, fr.F32, opts, got, f"xent_ex f32 {R}x{C} few rows")
    with fr.forced_variant(fr.OP_XENT, 256, 50):
        forced = run(x, lab, fr.F32, opts, argmax=False)
    assert np.array_equal(got[0], forced[0]) and np.array_equal(got[1], forced[1])


@pytest.mark.parametrize("R,C", [(300, 32769), (513, 40000), (1000, 57344), (257, 50257),
                                 (1537, 33000)])
def test_staged_row_widths_and_counts(R, C):
    """bf16 logits on the staged 1024-lane shape: widths whose whole slots
    number fewer than NV - 1 (a full wait before a staged row) and NV - 1 or
    NV (the counted wait), row counts from one to several rows per compute
    unit; options, argmax, misaligned rows."""
    assert fr.fr_debug_select_variant(fr.OP_XENT, C, fr.BF16) == (1024, 7, 8)
    rng = np.random.default_rng(R * 7 + C)
    x, lab = inputs(R, C, fr.BF16, seed=R + C, ignore_every=int(rng.integers(2, 6)))
    opts = dict(ignore_index=-100, label_smoothing=float(rng.choice([0.0, 0.05])),
                reduction=str(rng.choice(["none", "mean"])))
    print(f"staged bf16 {R}x{C} {opts}", flush=True)
    for am, offs in ((False, (0, 0)), (True, (1, 1))):
        expect(x, lab, fr.BF16, opts, run(x, lab, fr.BF16, opts, argmax=am, offs=offs),
               f"xent_ex bf16 {R}x{C} argmax={am} offs={offs}")


def test_staged_bf16_plain_and_ignored_runs():
    """The staged bf16 1024-lane kernel looping over many rows per workgroup:
    without options (out of place, misaligned), and with runs of consecutive
    ignored rows — the first and last rows among them — so that a row staged
    after an ignored row's zero stores, a staged row followed by an ignored
    one, and ignored rows with nothing to stage all occur."""
    R, C = 1500, 50257  # a workgroup takes rows w, w + ncu, ...: ~6 rows each
    assert fr.fr_debug_select_variant(fr.OP_XENT, C, fr.BF16) == (1024, 7, 8)
    x, lab = inputs(R, C, fr.BF16, seed=4242)
    print(f"staged bf16 plain {R}x{C}", flush=True)
    for am, offs in ((False, (0, 0)), (False, (3, 1)), (True, (0, 0))):
        expect(x, lab, fr.BF16, dict(), run(x, lab, fr.BF16, dict(), argmax=am, offs=offs),
               f"xent_ex bf16 plain {R}x{C} argmax={am} offs={offs}")
    rng = np.random.default_rng(4243)
    runs = lab.copy()
    r = 0
    while r < R:  # alternate runs of 1-400 kept rows and 1-400 ignored rows
        n_keep, n_ign = int(rng.integers(1, 400)), int(rng.integers(1, 400))
        runs[r + n_keep:r + n_keep + n_ign] = -100
        r += n_keep + n_ign
    runs[0] = runs[-1] = -100
    opts = dict(ignore_index=-100, label_smoothing=0.1, reduction="mean")
    print(f"staged bf16 ignored runs: {int((runs == -100).sum())} of {R} rows ignored", flush=True)
    for am in (False, True):
        expect(x, runs, fr.BF16, opts, run(x, runs, fr.BF16, opts, argmax=am),
               f"xent_ex bf16 ignored runs argmax={am}")


# --------------------------------------------- totals in the row kernel

@pytest.mark.parametrize("code", [fr.F32, fr.BF16])
def test_mean_over_many_rows_counted_first(code):
    """Past 8192 rows the rows not ignored are counted by a kernel of their
    own before the row pass (below, every workgroup counts them itself); the
    sum / mean is added up by the row kernel's last workgroup either way."""
    for R in (8192, 8193, 20000):
        x, lab = inputs(R, 300, code, seed=R, ignore_every=5)
        for opts in (dict(ignore_index=-100, reduction="mean", label_smoothing=0.05),
                     dict(ignore_index=-100, reduction="sum")):
            print(f"many-row total {code} {R}x300 {opts['reduction']}", flush=True)
            expect(x, lab, code, opts, run(x, lab, code, opts, argmax=False),
                   f"xent_ex {code} {R}x300 {opts['reduction']}")


def test_completion_counters_reused():
    """More calls than the pool has completion counters (256), alternating
    sum and mean and two row counts: every call's total matches its first
    call's bitwise (each counter is back at zero when its call ends)."""
    shapes = [(300, 1000, 21), (4100, 64, 22)]
    data = []
    for R, C, seed in shapes:
        x, lab = inputs(R, C, fr.F32, seed=seed, ignore_every=4)
        xt, lt = upload(x), upload(lab)
        data.append((xt, lt, torch.empty(R, device=DEV), torch.empty_like(xt)))
    tot = torch.empty(1, device=DEV)
    first = {}
    for i in range(300):
        xt, lt, loss, grad = data[i % 2]
        red = "mean" if (i // 2) % 2 else "sum"
        fr.fr_softmax_xent_ex(xt, lt, loss, grad, None, tot, ignore_index=-100, reduction=red)
        torch.cuda.synchronize()
        key = (i % 2, red)
        v = float(tot.cpu()[0])
        if key not in first:
            first[key] = v
            x = data[i % 2][0].cpu().numpy()
            lab = data[i % 2][1].cpu().numpy()
            to = oracle.softmax_xent_ex(x, lab, ignore_index=-100, reduction=red)[3]
            assert abs(v - to) <= 1e-5 * abs(to) + 1e-30, (key, v, to)
        else:
            assert v == first[key], (i, key, v, first[key])
