"""GPU parity of the backward kernels against the double-precision oracle,
through the C ABI, on seeded inputs.

The per-row forward statistics the backward consumes come from the oracle:
p = softmax(x) rounded to the storage dtype, and LayerNorm's mean / rstd
rounded to fp32 (the GPU and the oracle are given the same stored values).
Outputs and the workspace are NaN-poisoned inside canary guard bands.

Tolerances. Each output is compared with the fp32 rule of parity.py
(|g - o| <= 1e-5 * scale + 2^-126) at a scale that bounds the magnitude its
fp32 rounding error grows with, because these outputs are formed by
cancellation and a relative bound on |o| alone is ill-posed:
  softmax   dx_j: p_j (|dy_j| + sum_k |p_k dy_k|)
  RMSNorm   dh_j: r |w_j dy_j| + |h_j| r^3 sum_k |dy_k w_k h_k| / C + |dres_j|
            dw_j: sum_rows |dy_j h_j| r
  LayerNorm dx_j: rstd (|g_j| + sum_k |g_k| / C + |n_j| sum_k |g_k n_k| / C)
            dgamma_j: sum_rows |dy_j n_j|,  dbeta_j: sum_rows |dy_j|
(r and n recomputed in double from the inputs, g = dy gamma). The fp32 sums
behind them run over at most ~100 sequential terms per lane, tree levels and
fixed-order merges, a worst-case relative error below 100 * 2^-24 = 6e-6 of
the scale. bf16 outputs pass within one ulp of the rounded oracle or by the
same rule plus their one final rounding (parity.check_bf16, cond=).
"""
import numpy as np
import pytest
import torch

import memory_bound_row_pass_amd as fr
import oracle
import workloads
from gpu_buffers import DEV, TDT, Guarded, host, upload
from parity import bf16_bits, check_bf16, check_f32, to_dev

pytestmark = pytest.mark.gpu


def setup_module(module):
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    oracle.set_threads(min(16, oracle.threads()))


def dec(a):
    return oracle.decode(a)


def store(v, code):
    """Double values -> the storage dtype (fp32 array or bf16 bit patterns)."""
    return oracle.round_bf16(v) if code == fr.BF16 else np.asarray(v, np.float32)


def compare(got, ref, scale, code, what):
    if code == fr.BF16:
        return check_bf16(got, oracle.round_bf16(ref), what, cond=(ref, np.maximum(scale, np.abs(ref))))
    return check_f32(got, ref, scale=np.maximum(scale, np.abs(ref)), what=what)


def workspace(op, R, C):
    n = fr.fr_norm_bwd_workspace_bytes(op, R, C)
    return Guarded((max(n // 4, 4),), torch.float32)


# ------------------------------------------------------------ softmax bwd

def softmax_bwd_inputs(R, C, code, seed):
    w = workloads.make("softmax_bwd_bf16", rows=R, cols=C, seed=seed,
                       dtype="bf16" if code == fr.BF16 else "f32")
    p = store(oracle.softmax(w["x"]), code)
    return p, w["dy"]


def run_softmax_bwd(p, dy, code, offs=(0, 0, 0), inplace=None):
    R, C = p.shape
    pt, dyt = upload(p, offs[0]), upload(dy, offs[1])
    if inplace == "dy":
        fr.fr_softmax_bwd(pt, dyt, dyt)
        torch.cuda.synchronize()
        return host(dyt)
    if inplace == "p":
        fr.fr_softmax_bwd(pt, dyt, pt)
        torch.cuda.synchronize()
        return host(pt)
    dx = Guarded((R, C), TDT[code], offs[2])
    fr.fr_softmax_bwd(pt, dyt, dx.t)
    torch.cuda.synchronize()
    assert dx.canaries_intact(), "softmax_bwd wrote outside dx"
    return host(dx.t)


def expect_softmax_bwd(p, dy, code, got, what):
    ref = oracle.softmax_bwd(p, dy)
    pd, dyd = dec(p), dec(dy)
    scale = pd * (np.abs(dyd) + np.abs(pd * dyd).sum(1, keepdims=True))
    return compare(got, ref, scale, code, what)


# ------------------------------------------------------------ RMSNorm bwd

def rms_bwd_inputs(R, C, code, seed):
    return workloads.make("add_rmsnorm_bwd_bf16", rows=R, cols=C, seed=seed,
                          dtype="bf16" if code == fr.BF16 else "f32")


def run_rms_bwd(w, code, with_dres=True, off=0, inplace=None, stream=None):
    R, C = w["h"].shape
    h, dy, wt = upload(w["h"], off), upload(w["dy"], off), upload(w["weight"], off)
    dres = upload(w["dres"], off) if with_dres else None
    dw = Guarded((C,), torch.float32)
    ws = workspace(fr.OP_RMSNORM_BWD, R, C)
    if inplace:
        dh_t = {"dy": dy, "h": h, "dres": dres}[inplace]
        dh = None
    else:
        dh = Guarded((R, C), TDT[code], off)
        dh_t = dh.t
    fr.fr_add_rmsnorm_bwd(h, dy, wt, dh_t, dw.t, ws.t, dres=dres, eps=w.eps, stream=stream)
    torch.cuda.synchronize()
    assert dw.canaries_intact() and ws.canaries_intact() and (dh is None or dh.canaries_intact())
    return host(dh_t), dw.t.cpu().numpy()


def expect_rms_bwd(w, code, got, what, with_dres=True):
    dh, dw = got
    eps = float(np.float32(w.eps))
    dres = w["dres"] if with_dres else None
    dh_o, dw_o = oracle.rmsnorm_bwd(w["h"], w["dy"], w["weight"], np.float32(w.eps), dres=dres)
    hd, dyd, wd = dec(w["h"]), dec(w["dy"]), dec(w["weight"])
    C = hd.shape[1]
    r = 1.0 / np.sqrt((hd * hd).mean(1, keepdims=True) + eps)
    t = np.abs(dyd * wd * hd).sum(1, keepdims=True) / C
    s_dh = r * np.abs(wd * dyd) + np.abs(hd) * r ** 3 * t
    if with_dres:
        s_dh = s_dh + np.abs(dec(dres))
    hdh = compare(dh, dh_o, s_dh, code, what + " dh")
    check_f32(dw, dw_o, scale=np.maximum(np.abs(dw_o), (np.abs(dyd * hd) * r).sum(0)),
              what=what + " dweight")
    return hdh


# ----------------------------------------------------------- LayerNorm bwd

def ln_bwd_inputs(R, C, code, seed):
    w = workloads.make("layernorm_bwd_f32", rows=R, cols=C, seed=seed,
                       dtype="bf16" if code == fr.BF16 else "f32")
    _, mean, rstd = oracle.layernorm(w["x"], w["gamma"], w["gamma"], np.float32(w.eps))
    return w, mean.astype(np.float32), rstd.astype(np.float32)


def run_ln_bwd(w, mean, rstd, code, off=0, inplace=None):
    R, C = w["x"].shape
    x, dy, g = upload(w["x"], off), upload(w["dy"], off), upload(w["gamma"], off)
    m, r = to_dev(mean), to_dev(rstd)
    dg, db = Guarded((C,), torch.float32), Guarded((C,), torch.float32)
    ws = workspace(fr.OP_LAYERNORM_BWD, R, C)
    if inplace:
        dx_t, dx = {"x": x, "dy": dy}[inplace], None
    else:
        dx = Guarded((R, C), TDT[code], off)
        dx_t = dx.t
    fr.fr_layernorm_bwd(x, dy, g, m, r, dx_t, dg.t, db.t, ws.t)
    torch.cuda.synchronize()
    assert dg.canaries_intact() and db.canaries_intact() and ws.canaries_intact()
    assert dx is None or dx.canaries_intact()
    return host(dx_t), dg.t.cpu().numpy(), db.t.cpu().numpy()


def expect_ln_bwd(w, mean, rstd, code, got, what):
    dx, dg, db = got
    m64, r64 = mean.astype(np.float64), rstd.astype(np.float64)
    dx_o, dg_o, db_o = oracle.layernorm_bwd(w["x"], w["dy"], w["gamma"], m64, r64)
    xd, dyd, gd = dec(w["x"]), dec(w["dy"]), dec(w["gamma"])
    C = xd.shape[1]
    n = (xd - m64[:, None]) * r64[:, None]
    g = dyd * gd
    s_dx = r64[:, None] * (np.abs(g) + np.abs(g).sum(1, keepdims=True) / C
                           + np.abs(n) * np.abs(g * n).sum(1, keepdims=True) / C)
    hdx = compare(dx, dx_o, s_dx, code, what + " dx")
    check_f32(dg, dg_o, scale=np.maximum(np.abs(dg_o), np.abs(dyd * n).sum(0)), what=what + " dgamma")
    check_f32(db, db_o, scale=np.maximum(np.abs(db_o), np.abs(dyd).sum(0)), what=what + " dbeta")
    return hdx


# ------------------------------------------------- full-size workloads

def test_workload_softmax_bwd_bf16():
    w = workloads.make("softmax_bwd_bf16")
    p = store(oracle.softmax(w["x"]), fr.BF16)
    h = expect_softmax_bwd(p, w["dy"], fr.BF16, run_softmax_bwd(p, w["dy"], fr.BF16),
                           "softmax_bwd_bf16 16384x4096")
    print("softmax_bwd dx ulp", h)


def test_workload_layernorm_bwd_f32():
    w, m, r = ln_bwd_inputs(None, None, fr.F32, None)
    expect_ln_bwd(w, m, r, fr.F32, run_ln_bwd(w, m, r, fr.F32), "layernorm_bwd_f32 4096x1024")


def test_workload_add_rmsnorm_bwd_bf16():
    w = workloads.make("add_rmsnorm_bwd_bf16")
    h = expect_rms_bwd(w, fr.BF16, run_rms_bwd(w, fr.BF16), "add_rmsnorm_bwd_bf16 8192x8192")
    print("rmsnorm_bwd dh ulp", h)


# ------------------------------------------------------- edge shapes

EDGE_COLS = [1, 2, 3, 4, 7, 8, 9, 16, 63, 64, 65, 255, 256, 1000, 1024, 1025, 2048, 4095,
             4096, 8192, 12345, 16384]


def _norm_vec_ok(C, code):
    return (C * (2 if code == fr.BF16 else 4)) % 16 == 0


@pytest.mark.parametrize("C", EDGE_COLS)
@pytest.mark.parametrize("code", [fr.F32, fr.BF16])
def test_softmax_bwd_edge_cols(C, code):
    for R in (1, 5):
        p, dy = softmax_bwd_inputs(R, C, code, seed=C * 3 + R)
        expect_softmax_bwd(p, dy, code, run_softmax_bwd(p, dy, code), f"softmax_bwd {code} {R}x{C}")


@pytest.mark.parametrize("C", EDGE_COLS)
@pytest.mark.parametrize("code", [fr.F32, fr.BF16])
def test_rms_bwd_edge_cols(C, code):
    # 16-byte rows take the vector path, others (odd widths) the scalar path
    for R, dres in ((1, True), (37, False)):
        w = rms_bwd_inputs(R, C, code, seed=C + R)
        expect_rms_bwd(w, code, run_rms_bwd(w, code, with_dres=dres), f"rms_bwd {code} {R}x{C}",
                       with_dres=dres)


@pytest.mark.parametrize("C", EDGE_COLS)
@pytest.mark.parametrize("code", [fr.F32, fr.BF16])
def test_ln_bwd_edge_cols(C, code):
    for R in (1, 37):
        w, m, r = ln_bwd_inputs(R, C, code, seed=C + 2 * R)
        expect_ln_bwd(w, m, r, code, run_ln_bwd(w, m, r, code), f"ln_bwd {code} {R}x{C}")


@pytest.mark.parametrize("R", [2, 15, 16, 17, 255, 4095, 4096, 4097, 8229])
def test_norm_bwd_row_counts(R):
    # row groups per workgroup (16 at 64 lanes per row) and the grid of at
    # most 256 workgroups: partial last groups, one and several sweeps
    C = 256
    w = rms_bwd_inputs(R, C, fr.F32, seed=R)
    expect_rms_bwd(w, fr.F32, run_rms_bwd(w, fr.F32), f"rms_bwd f32 {R}x{C}")
    w, m, r = ln_bwd_inputs(R, C, fr.F32, seed=R + 1)
    expect_ln_bwd(w, m, r, fr.F32, run_ln_bwd(w, m, r, fr.F32), f"ln_bwd f32 {R}x{C}")
    p, dy = softmax_bwd_inputs(R, C, fr.F32, seed=R + 2)
    expect_softmax_bwd(p, dy, fr.F32, run_softmax_bwd(p, dy, fr.F32), f"softmax_bwd f32 {R}x{C}")


# ----------------------------------------------------- every variant

VARIANT_GRID = [(t, v) for t in (64, 256, 512, 1024) for v in (1, 2, 4, 8, 16)]


def _caps(op, t, v, code, vector_path):
    try:
        with fr.forced_variant(op, t, v):
            tt, vv, e = fr.fr_debug_select_variant(op, 1, code, vector_path=vector_path)
    except fr.FusedRowError:
        return None
    cap = tt * vv * e
    if e > 1 and op != fr.OP_SOFTMAX_BWD:
        return [cap, max(e, cap - 5 * e), e * (cap // (2 * e) + 1)]
    return [cap, max(1, cap - 5 * e - 3), max(1, cap // 2 + 1)]


def _rows_for(C):
    return max(3, min(700, (1 << 20) // C))


# only the pairs with a kernel for some (op, dtype, vector path); the
# selection call runs on the host, so collection needs no GPU
BWD_GRID = [(t, v) for t, v in VARIANT_GRID
            if any(_caps(op, t, v, c, vp)
                   for op in (fr.OP_SOFTMAX_BWD, fr.OP_RMSNORM_BWD, fr.OP_LAYERNORM_BWD)
                   for c in (fr.F32, fr.BF16) for vp in (True, False))]


@pytest.mark.parametrize("t,v", BWD_GRID)
def test_every_backward_variant(t, v):
    ran = 0
    for code in (fr.F32, fr.BF16):
        for vp, off in ((True, 0), (False, 1)):
            for C in _caps(fr.OP_SOFTMAX_BWD, t, v, code, vp) or []:
                p, dy = softmax_bwd_inputs(3, C, code, seed=C)
                offs = (0, 0, 0) if vp else (1, 2, 1)
                with fr.forced_variant(fr.OP_SOFTMAX_BWD, t, v):
                    got = run_softmax_bwd(p, dy, code, offs)
                expect_softmax_bwd(p, dy, code, got, f"softmax_bwd[{t},{v},{vp}] {code} 3x{C}")
                ran += 1
            for C in _caps(fr.OP_RMSNORM_BWD, t, v, code, vp) or []:
                w = rms_bwd_inputs(_rows_for(C), C, code, seed=C + 1)
                with fr.forced_variant(fr.OP_RMSNORM_BWD, t, v):
                    got = run_rms_bwd(w, code, off=off)
                expect_rms_bwd(w, code, got, f"rms_bwd[{t},{v},{vp}] {code} {w.rows}x{C}")
                ran += 1
            for C in _caps(fr.OP_LAYERNORM_BWD, t, v, code, vp) or []:
                w, m, r = ln_bwd_inputs(_rows_for(C), C, code, seed=C + 2)
                with fr.forced_variant(fr.OP_LAYERNORM_BWD, t, v):
                    got = run_ln_bwd(w, m, r, code, off=off)
                expect_ln_bwd(w, m, r, code, got, f"ln_bwd[{t},{v},{vp}] {code} {w.rows}x{C}")
                ran += 1
    if not ran:
        pytest.skip(f"no backward variant ({t}, {v})")


# --------------------------------------------------- alignment / aliasing

@pytest.mark.parametrize("offs", [(1, 1, 1), (3, 3, 3), (1, 0, 0), (0, 2, 1)])
def test_softmax_bwd_misaligned(offs):
    # equal phases: head/body/tail vector path; unequal: scalar path
    for C in (5, 1000, 4099):
        p, dy = softmax_bwd_inputs(4, C, fr.F32, seed=C)
        expect_softmax_bwd(p, dy, fr.F32, run_softmax_bwd(p, dy, fr.F32, offs),
                           f"softmax_bwd offs {offs} 4x{C}")


def test_in_place():
    p, dy = softmax_bwd_inputs(64, 4096, fr.BF16, seed=3)
    for mode in ("dy", "p"):
        expect_softmax_bwd(p, dy, fr.BF16, run_softmax_bwd(p, dy, fr.BF16, inplace=mode),
                           f"softmax_bwd dx={mode}")
    w = rms_bwd_inputs(64, 8192, fr.BF16, seed=4)
    for mode in ("dy", "h", "dres"):
        expect_rms_bwd(w, fr.BF16, run_rms_bwd(w, fr.BF16, inplace=mode), f"rms_bwd dh={mode}")
    w, m, r = ln_bwd_inputs(64, 1024, fr.F32, seed=5)
    for mode in ("x", "dy"):
        expect_ln_bwd(w, m, r, fr.F32, run_ln_bwd(w, m, r, fr.F32, inplace=mode), f"ln_bwd dx={mode}")


# ------------------------------------------------------------ special cases

def test_rows_zero_zeroes_parameter_gradients():
    C = 1000
    dw = torch.full((C,), float("nan"), device=DEV)
    e = torch.empty(0, C, device=DEV)
    fr.fr_add_rmsnorm_bwd(e, e, torch.ones(C, device=DEV), e, dw, None)
    dg = torch.full((C,), float("nan"), device=DEV)
    db = torch.full((C,), float("nan"), device=DEV)
    z = torch.empty(0, device=DEV)
    fr.fr_layernorm_bwd(e, e, torch.ones(C, device=DEV), z, z, e, dg, db, None)
    fr.fr_softmax_bwd(e, e, e)
    torch.cuda.synchronize()
    assert bool((dw == 0).all()) and bool((dg == 0).all()) and bool((db == 0).all())


def test_softmax_bwd_one_hot_and_uniform():
    # p one-hot: dx = 0 exactly; p uniform: dx = (dy - mean dy) / C
    C = 1024
    p = np.zeros((2, C), np.float32)
    p[0, 17] = 1.0
    p[1, :] = 1.0 / C
    dy = np.random.default_rng(1).normal(size=(2, C)).astype(np.float32)
    got = run_softmax_bwd(p, dy, fr.F32)
    assert np.all(got[0] == 0.0)
    expect_softmax_bwd(p, dy, fr.F32, got, "softmax_bwd one-hot / uniform")


def test_norm_bwd_constant_dy_zero():
    # dy = 0: every gradient is exactly zero (RMS: dh = dres)
    w = rms_bwd_inputs(40, 512, fr.F32, seed=9)
    w.arrays["dy"] = np.zeros_like(w["dy"])
    dh, dw = run_rms_bwd(w, fr.F32)
    assert np.array_equal(dh, w["dres"]) and np.all(dw == 0)
    w, m, r = ln_bwd_inputs(40, 512, fr.F32, seed=10)
    w.arrays["dy"] = np.zeros_like(w["dy"])
    dx, dg, db = run_ln_bwd(w, m, r, fr.F32)
    assert np.all(dx == 0) and np.all(dg == 0) and np.all(db == 0)


# ------------------------------------------------- determinism / streams

def test_bitwise_determinism():
    w = rms_bwd_inputs(3000, 4096, fr.BF16, seed=11)
    args = [to_dev(w[k]) for k in ("h", "dy", "weight")]
    dres = to_dev(w["dres"])
    r = []
    for _ in range(3):
        dh, dw = fr.add_rmsnorm_bwd(*args, eps=w.eps, dres=dres)
        r.append((bf16_bits(dh).tobytes(), dw.cpu().numpy().tobytes()))
    assert r[0] == r[1] == r[2]
    w, m, rs = ln_bwd_inputs(3000, 1024, fr.F32, seed=12)
    args = [to_dev(a) for a in (w["x"], w["dy"], w["gamma"], m, rs)]
    r = [tuple(t.cpu().numpy().tobytes() for t in fr.layernorm_bwd(*args)) for _ in range(3)]
    assert r[0] == r[1] == r[2]


def test_non_default_stream():
    w = rms_bwd_inputs(256, 2048, fr.BF16, seed=13)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    got = run_rms_bwd(w, fr.BF16, stream=s.cuda_stream)
    expect_rms_bwd(w, fr.BF16, got, "rms_bwd on a side stream")


def test_graph_capture_replays_match_eager():
    # the norm backward is two launches (row pass, column sums) and no
    # memset, so a backward step can be captured; every replay must match
    p, dyp = softmax_bwd_inputs(128, 4096, fr.BF16, seed=14)
    wr = rms_bwd_inputs(256, 8192, fr.BF16, seed=15)
    wl, m, r = ln_bwd_inputs(512, 1024, fr.F32, seed=16)
    pt, dypt = to_dev(p), to_dev(dyp)
    dx = torch.empty_like(pt)
    h, dy, wt, dres = (to_dev(wr[k]) for k in ("h", "dy", "weight", "dres"))
    dh, dw = torch.empty_like(h), torch.empty(8192, device=DEV)
    wsr = torch.empty(fr.fr_norm_bwd_workspace_bytes(fr.OP_RMSNORM_BWD, 256, 8192), dtype=torch.uint8,
                      device=DEV)
    x, dyl, g, mt, rt = (to_dev(a) for a in (wl["x"], wl["dy"], wl["gamma"], m, r))
    dxl, dg, db = torch.empty_like(x), torch.empty(1024, device=DEV), torch.empty(1024, device=DEV)
    wsl = torch.empty(fr.fr_norm_bwd_workspace_bytes(fr.OP_LAYERNORM_BWD, 512, 1024),
                      dtype=torch.uint8, device=DEV)

    def step():
        fr.fr_softmax_bwd(pt, dypt, dx)
        fr.fr_add_rmsnorm_bwd(h, dy, wt, dh, dw, wsr, dres=dres, eps=wr.eps)
        fr.fr_layernorm_bwd(x, dyl, g, mt, rt, dxl, dg, db, wsl)

    outs = (dx, dh, dw, dxl, dg, db)
    step()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        step()
    for rep in range(4):
        for o in outs:
            o.fill_(float("nan"))
        wsr.fill_(255)
        wsl.fill_(255)
        torch.cuda.synchronize()
        gr.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            iv = torch.int16 if o.dtype == torch.bfloat16 else torch.int32
            assert torch.equal(o.view(iv), e.view(iv)), rep
    expect_rms_bwd(wr, fr.BF16, (bf16_bits(eager[1]), eager[2].cpu().numpy()), "graph rms_bwd")


@pytest.mark.parametrize("C", [8192, 5000])
def test_rms_bwd_several_sweeps(C):
    """More rows than one sweep of the persistent grid (256 workgroups x 2 row
    groups): every workgroup walks several rows; without dres the bf16
    8192-column shape stages its next rows in LDS. Rows past the last sweep's
    end (a partial sweep) take part with no data."""
    code = fr.BF16
    assert fr.fr_debug_select_variant(fr.OP_RMSNORM_BWD, C, code) == (512, 2, 8)
    R = 1100
    w = rms_bwd_inputs(R, C, code, seed=C + 3)
    print(f"rms_bwd sweeps bf16 {R}x{C}", flush=True)
    for with_dres in (False, True):
        expect_rms_bwd(w, code, run_rms_bwd(w, code, with_dres=with_dres),
                       f"rms_bwd bf16 {R}x{C} dres={with_dres}", with_dres=with_dres)
    expect_rms_bwd(w, code, run_rms_bwd(w, code, with_dres=False, inplace="dy"),
                   f"rms_bwd bf16 {R}x{C} in place", with_dres=False)


@pytest.mark.parametrize("code,C", [(fr.F32, 4096), (fr.BF16, 4096), (fr.F32, 1024), (fr.BF16, 1000)])
def test_ln_bwd_several_sweeps(code, C):
    """More rows than one sweep of the persistent grid: every workgroup walks
    several rows, staging the next rows' x and dy (and their mean and rstd)
    while it reduces and writes the current ones, with gamma in registers;
    the last sweep is partial (row groups with no row take part with no
    data). Also misaligned (scalar path) and in place."""
    t, v, e = fr.fr_debug_select_variant(fr.OP_LAYERNORM_BWD, C, code)
    R = 256 * (1024 // t) * 2 + 77
    w, m, r = ln_bwd_inputs(R, C, code, seed=C + R)
    print(f"ln_bwd sweeps {code} {R}x{C} variant {(t, v, e)}", flush=True)
    expect_ln_bwd(w, m, r, code, run_ln_bwd(w, m, r, code), f"ln_bwd {code} {R}x{C}")
    expect_ln_bwd(w, m, r, code, run_ln_bwd(w, m, r, code, off=1), f"ln_bwd {code} {R}x{C} misaligned")
    expect_ln_bwd(w, m, r, code, run_ln_bwd(w, m, r, code, inplace="x"), f"ln_bwd {code} {R}x{C} in place")


@pytest.mark.parametrize("R,C,code", [(600, 4104, fr.BF16), (1100, 6000, fr.BF16),
                                      (1025, 8192, fr.BF16), (520, 7000, fr.F32)])
def test_staged_norm_bwd_shapes(R, C, code):
    """The staged norm backward shapes at widths with and without a partial
    slot (a full wait instead of the counted one) and row counts that end in
    a partial sweep: RMSNorm with and without dres, LayerNorm."""
    w = rms_bwd_inputs(R, C, code, seed=R + C)
    print(f"staged norm bwd {code} {R}x{C}", flush=True)
    for with_dres in (True, False):
        expect_rms_bwd(w, code, run_rms_bwd(w, code, with_dres=with_dres),
                       f"rms_bwd {code} {R}x{C} dres={with_dres}", with_dres=with_dres)
    wl, m, r = ln_bwd_inputs(R, C, code, seed=R + C + 1)
    expect_ln_bwd(wl, m, r, code, run_ln_bwd(wl, m, r, code), f"ln_bwd {code} {R}x{C}")
