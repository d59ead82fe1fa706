"""Pins of the double-precision CPU oracle against facts fixed outside it.

Nothing here re-types the oracle's formula and compares it with itself. Each
pin is an invariant, a closed form, an independent library routine (torch CPU
float64), brute-force finite differences, or the IEEE definition of rounding,
chosen so that a plausible slip in the oracle (a dropped term, a wrong sign or
index, a swapped operand, variance divided by C-1, eps outside the root,
rounding through fp32) fails at least one of them.

Sources: "Engineering a CUDA Machine Learning Framework from Scratch" §3.1
(online softmax: rows sum to one, max subtraction, the online recurrence) and
§3.2 (Welford moments); "NexusGrad", "Verified VJP Operators" (central
finite differences) and "Mathematical Correctness & Verification" (parity with
a reference implementation).
"""
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import workloads

RNG = np.random.default_rng(20240601)


def rel_err(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.max(np.abs(a - b) / np.maximum(np.abs(b), 1e-300)))


# ------------------------------------------------------------------ I1, I2

@pytest.mark.parametrize("shape,scale", [((50, 777), 4.0), ((7, 4096), 60.0), ((3, 1), 1.0),
                                         ((5, 50257), 2.0)])
def test_softmax_rows_sum_to_one(shape, scale):
    x = (RNG.normal(0, scale, size=shape)).astype(np.float32)
    p = oracle.softmax(x)
    assert np.all(p >= 0)
    assert np.abs(p.sum(1) - 1.0).max() <= 1e-13


def test_softmax_rows_sum_to_one_bf16_near_one_hot():
    w = workloads.make("softmax_bf16", rows=16, cols=4096)
    p = oracle.softmax(w["x"])
    assert np.abs(p.sum(1) - 1.0).max() <= 1e-13
    # the largest per-row scales make near-one-hot rows
    assert p.max() > 0.5


@pytest.mark.parametrize("c", [1000.0, -1000.0, 1024.0, -1024.0])
def test_softmax_shift_invariance(c):
    # values on a 2^-8 grid so that x + c is exact in fp32
    k = RNG.integers(-2048, 2048, size=(9, 333))
    x = (k / 256.0).astype(np.float32)
    xs = (k / 256.0 + c).astype(np.float32)
    assert np.array_equal(xs.astype(np.float64) - c, x.astype(np.float64))
    p0, p1 = oracle.softmax(x), oracle.softmax(xs)
    assert np.all(np.isfinite(p1))
    assert rel_err(p1, p0) <= 1e-12


# ------------------------------------------------------------------ I3

def _three_pass_stats(x):
    m = float(np.max(x))
    s = math.fsum(math.exp(v - m) for v in x)
    return m, s


@pytest.mark.parametrize("n,scale", [(1, 1.0), (2, 3.0), (1000, 4.0), (4096, 60.0), (50257, 2.0)])
def test_online_recurrence_equals_three_pass(n, scale):
    x = RNG.normal(0, scale, size=n)
    m_on, d_on = oracle.online_softmax_stats(x)
    m3, s3 = _three_pass_stats(x)
    assert m_on == m3
    assert abs(d_on - s3) <= 1e-13 * s3


def test_online_recurrence_chunked_merge_any_order():
    x = RNG.normal(0, 8.0, size=3000)
    m3, s3 = _three_pass_stats(x)
    for trial in range(20):
        cuts = np.sort(RNG.choice(np.arange(0, 3001), size=RNG.integers(1, 40), replace=True))
        pieces = np.split(x, cuts)          # may contain empty chunks
        states = [oracle.online_softmax_stats(p) for p in pieces]
        order = RNG.permutation(len(states))
        states = [states[i] for i in order]
        while len(states) > 1:             # random pairwise tree
            i = int(RNG.integers(0, len(states) - 1))
            a, b = states[i], states[i + 1]
            if RNG.random() < 0.5:
                a, b = b, a
            states[i:i + 2] = [oracle.softmax_stats_merge(a, b)]
        m, d = states[0]
        assert m == m3
        assert abs(d - s3) <= 1e-13 * s3


def test_online_merge_identity_and_neg_inf_entries():
    empty = oracle.online_softmax_stats(np.array([], dtype=np.float64))
    assert empty == (-math.inf, 0.0)
    a = oracle.online_softmax_stats(np.array([1.0, 2.0]))
    assert oracle.softmax_stats_merge(empty, a) == a
    assert oracle.softmax_stats_merge(a, empty) == a
    x = np.array([-math.inf, 0.5, -math.inf, 2.0])
    m, d = oracle.online_softmax_stats(x)
    assert m == 2.0 and abs(d - (1 + math.exp(-1.5))) <= 1e-15


def test_softmax_consistent_with_online_stats():
    # p_j * d == exp(x_j - m): ties the definition to the recurrence
    x = RNG.normal(0, 4, size=(4, 1000)).astype(np.float32)
    p = oracle.softmax(x)
    for r in range(4):
        xr = x[r].astype(np.float64)
        m, d = oracle.online_softmax_stats(xr)
        assert rel_err(p[r] * d, np.exp(xr - m)) <= 1e-13


# ------------------------------------------------------------------ I4

def _two_pass_moments(x):
    n = len(x)
    mu = math.fsum(x) / n
    m2 = math.fsum((v - mu) ** 2 for v in x)
    return float(n), mu, m2


@pytest.mark.parametrize("mu,sigma,n", [(0.0, 1.0, 1000), (3.0, 2.0, 1024), (-5.0, 0.1, 77)])
def test_welford_equals_two_pass(mu, sigma, n):
    x = RNG.normal(mu, sigma, size=n)
    cw, mw, qw = oracle.welford(x)
    c2, m2_, q2 = _two_pass_moments(x)
    assert cw == c2
    assert abs(mw - m2_) <= 1e-14 * max(abs(m2_), sigma)
    assert abs(qw - q2) <= 1e-12 * q2


def test_chan_merge_random_chunkings():
    x = RNG.normal(3.0, 2.0, size=2048)
    ref = _two_pass_moments(x)
    for trial in range(20):
        cuts = np.sort(RNG.choice(np.arange(0, 2049), size=RNG.integers(1, 64), replace=True))
        states = [oracle.welford(p) for p in np.split(x, cuts)]
        while len(states) > 1:
            i = int(RNG.integers(0, len(states) - 1))
            states[i:i + 2] = [oracle.chan_merge(states[i], states[i + 1])]
        n, mu, m2 = states[0]
        assert n == ref[0]
        assert abs(mu - ref[1]) <= 1e-14 * abs(ref[1])
        assert abs(m2 - ref[2]) <= 1e-12 * ref[2]


def test_chan_merge_identity():
    a = oracle.welford(np.array([1.0, 4.0, 7.0]))
    assert oracle.chan_merge((0.0, 0.0, 0.0), a) == a
    assert oracle.chan_merge(a, (0.0, 0.0, 0.0)) == a
    assert oracle.chan_merge((0.0, 0.0, 0.0), (0.0, 0.0, 0.0)) == (0.0, 0.0, 0.0)


def test_welford_stress_large_mean():
    # mean 1e8, sd 1: the naive E[x^2] - E[x]^2 loses everything, Welford does not
    x = 1e8 + RNG.normal(0, 1.0, size=4096)
    _, mu, m2 = oracle.welford(x)
    _, mu2, m2ref = _two_pass_moments(x)
    assert abs(m2 - m2ref) <= 1e-8 * m2ref
    naive = float(np.sum(x * x) - len(x) * np.mean(x) ** 2)
    assert abs(naive - m2ref) > 1e-3 * m2ref


def test_layernorm_moments_match_welford():
    w = workloads.make("layernorm_f32", rows=8, cols=1024)
    y, mean, rstd = oracle.layernorm(w["x"], w["gamma"], w["beta"], w.eps)
    for r in range(8):
        n, mu, m2 = oracle.welford(w["x"][r].astype(np.float64))
        assert abs(mean[r] - mu) <= 1e-14 * abs(mu)
        ref = 1.0 / math.sqrt(m2 / n + float(np.float32(w.eps)))
        assert abs(rstd[r] - ref) <= 1e-13 * ref


# ------------------------------------------------------------------ I5, I6

def test_layernorm_normalized_moments():
    x = RNG.normal(3.0, 2.0, size=(6, 1024)).astype(np.float32)
    ones, zeros = np.ones(1024, np.float32), np.zeros(1024, np.float32)
    eps = np.float32(1e-5)
    y, mean, rstd = oracle.layernorm(x, ones, zeros, eps)
    for r in range(6):
        xr = x[r].astype(np.float64)
        var = _two_pass_moments(xr)[2] / 1024
        assert abs(math.fsum(y[r]) / 1024) <= 1e-13
        vn = math.fsum(v * v for v in y[r]) / 1024
        assert abs(vn - var / (var + float(eps))) <= 1e-13
    # gamma/beta enter as y = n * gamma + beta
    g = RNG.uniform(0.5, 1.5, size=1024).astype(np.float32)
    b = RNG.normal(0, 0.3, size=1024).astype(np.float32)
    y2, _, _ = oracle.layernorm(x, g, b, eps)
    assert np.max(np.abs((y2 - b.astype(np.float64)) / g.astype(np.float64) - y)) <= 1e-13


def test_add_rmsnorm_normalized_moment_and_exact_h():
    w = workloads.make("add_rmsnorm_bf16", rows=5, cols=2048)
    y, h, rstd = oracle.add_rmsnorm(w["x"], w["residual"], w["weight"], w.eps)
    hx = oracle.decode(w["x"]) + oracle.decode(w["residual"])
    assert np.array_equal(h, hx)
    wt = oracle.decode(w["weight"])
    for r in range(5):
        n = y[r] / wt
        ms = math.fsum(v * v for v in h[r]) / 2048
        mn = math.fsum(v * v for v in n) / 2048
        assert abs(mn - ms / (ms + float(np.float32(w.eps)))) <= 1e-13
        assert abs(rstd[r] - 1 / math.sqrt(ms + float(np.float32(w.eps)))) <= 1e-13 * rstd[r]


# ------------------------------------------------------------------ I7

@pytest.mark.parametrize("C", [2, 3, 4, 5, 6, 7, 8])
def test_xent_gradient_by_central_differences(C):
    x = RNG.normal(0, 2.0, size=(3, C))
    labels = RNG.integers(0, C, size=3).astype(np.int32)
    loss, grad, _ = oracle.softmax_xent(x, labels)
    eps = 1e-6
    for r in range(3):
        for j in range(C):
            xp, xm = x.copy(), x.copy()
            xp[r, j] += eps
            xm[r, j] -= eps
            lp = oracle.softmax_xent(xp, labels)[0][r]
            lm = oracle.softmax_xent(xm, labels)[0][r]
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - grad[r, j]) <= 1e-8, (r, j, fd, grad[r, j])
    assert np.max(np.abs(grad.sum(1))) <= 1e-15 * C * 4
    p = oracle.softmax(x)
    for r in range(3):
        assert abs(loss[r] - (-math.log(p[r, labels[r]]))) <= 1e-13 * max(loss[r], 1e-3)
    assert np.all(loss >= 0)


def test_xent_label_sign_and_out_of_range_label():
    x = RNG.normal(0, 2.0, size=(4, 9)).astype(np.float32)
    labels = np.array([0, 8, -1, 9], dtype=np.int32)
    loss, grad, _ = oracle.softmax_xent(x, labels)
    p = oracle.softmax(x)
    for r in (0, 1):
        neg = np.nonzero(grad[r] < 0)[0]
        assert list(neg) == [labels[r]]
        assert np.isfinite(loss[r])
    for r in (2, 3):
        assert math.isnan(loss[r])
        assert np.array_equal(grad[r], p[r])


def test_xent_argmax_lowest_index_on_ties():
    x = np.array([[1, 3, 3, 2], [5, 5, 5, 5], [0, 0, 0, 7], [-1, -2, -1, -3]], dtype=np.float32)
    _, _, am = oracle.softmax_xent(x, np.zeros(4, np.int32))
    assert list(am) == [1, 0, 3, 0]


# ------------------------------------------------------------------ I8

def test_closed_forms_softmax_and_xent():
    # one column
    x1 = RNG.normal(0, 5, size=(4, 1)).astype(np.float32)
    assert np.all(oracle.softmax(x1) == 1.0)
    loss, grad, am = oracle.softmax_xent(x1, np.zeros(4, np.int32))
    assert np.all(loss == 0.0) and np.all(grad == 0.0) and np.all(am == 0)
    # constant rows
    for C in (2, 7, 1000, 50257):
        xc = np.full((2, C), 3.25, dtype=np.float32)
        p = oracle.softmax(xc)
        assert np.max(np.abs(p * C - 1.0)) <= 1e-13
        lab = np.array([0, C - 1], np.int32)
        loss, grad, _ = oracle.softmax_xent(xc, lab)
        assert np.max(np.abs(loss - math.log(C))) <= 1e-13 * math.log(C)
        assert abs(grad[1, C - 1] - (1.0 / C - 1.0)) <= 1e-13
    # two columns: the logistic function
    x2 = RNG.normal(0, 3, size=(50, 2)).astype(np.float32).astype(np.float64)
    p2 = oracle.softmax(x2.astype(np.float32))
    for r in range(50):
        sig = 1.0 / (1.0 + math.exp(x2[r, 1] - x2[r, 0]))
        assert abs(p2[r, 0] - sig) <= 1e-14 * max(sig, 1e-300) + 1e-300


def test_closed_forms_layernorm():
    ones, zeros = np.ones(2, np.float32), np.zeros(2, np.float32)
    for a, b in [(1.0, 2.0), (-3.5, 7.25), (100.0, 100.5)]:
        for eps in (0.0, 1e-5, 0.5):
            e = float(np.float32(eps))
            x = np.array([[a, b]], dtype=np.float32)
            y, mean, rstd = oracle.layernorm(x, ones, zeros, eps)
            var = ((a - b) / 2) ** 2
            n = math.sqrt(var / (var + e))
            assert abs(y[0, 0] - (-n if a < b else n)) <= 1e-14
            assert abs(y[0, 1] - (n if a < b else -n)) <= 1e-14
            assert abs(mean[0] - (a + b) / 2) <= 1e-15 * abs((a + b) / 2)
            assert abs(rstd[0] - 1 / math.sqrt(var + e)) <= 1e-14 / math.sqrt(var + e)
    # [1, 2, 3, 4], eps = 0: mean 2.5, var 1.25
    x = np.array([[1, 2, 3, 4]], dtype=np.float32)
    y, mean, rstd = oracle.layernorm(x, np.ones(4, np.float32), np.zeros(4, np.float32), 0.0)
    ref = [(v - 2.5) / math.sqrt(1.25) for v in (1, 2, 3, 4)]
    assert np.max(np.abs(y[0] - ref)) <= 1e-15
    # constant row: normalised part is zero, y = beta, rstd = 1/sqrt(eps)
    xc = np.full((1, 16), 7.0, np.float32)
    beta = RNG.normal(0, 1, size=16).astype(np.float32)
    y, mean, rstd = oracle.layernorm(xc, np.ones(16, np.float32), beta, 1e-5)
    assert np.array_equal(y[0], beta.astype(np.float64))
    assert abs(rstd[0] - 1 / math.sqrt(float(np.float32(1e-5)))) <= 1e-12 * rstd[0]


def test_closed_forms_rmsnorm():
    for c in (0.5, -3.0, 1e-3):
        for eps in (0.0, 1e-6, 0.25):
            C = 8
            x = np.full((1, C), c, np.float32)
            r = np.zeros((1, C), np.float32)
            w = RNG.uniform(0.8, 1.2, size=C).astype(np.float32)
            y, h, rstd = oracle.add_rmsnorm(x, r, w, eps)
            e = float(np.float32(eps))
            cs = float(np.float32(c))       # the stored input value
            ref = cs * w.astype(np.float64) / math.sqrt(cs * cs + e)
            assert np.max(np.abs(y[0] - ref) / np.abs(ref)) <= 1e-14
    x = np.array([[3.0, 1.0]], np.float32)
    r = np.array([[0.0, 3.0]], np.float32)
    y, h, _ = oracle.add_rmsnorm(x, r, np.ones(2, np.float32), 0.0)
    assert list(h[0]) == [3.0, 4.0]
    assert np.max(np.abs(y[0] - np.array([3.0, 4.0]) / math.sqrt(12.5))) <= 1e-15


# ------------------------------------------------------------------ I9

def test_torch_float64_cross_check():
    x = RNG.normal(0, 4, size=(16, 1000)).astype(np.float32)
    p = oracle.softmax(x)
    pt = torch.softmax(torch.from_numpy(x.astype(np.float64)), dim=1).numpy()
    assert rel_err(p, pt) <= 1e-12

    w = workloads.make("softmax_bf16", rows=8, cols=4096)
    p = oracle.softmax(w["x"])
    pt = torch.softmax(torch.from_numpy(oracle.decode(w["x"])), dim=1).numpy()
    big = pt > 1e-290
    assert rel_err(p[big], pt[big]) <= 1e-12

    w = workloads.make("layernorm_f32", rows=32, cols=1024)
    y, mean, rstd = oracle.layernorm(w["x"], w["gamma"], w["beta"], w.eps)
    yt = F.layer_norm(torch.from_numpy(w["x"].astype(np.float64)), (1024,),
                      torch.from_numpy(w["gamma"].astype(np.float64)),
                      torch.from_numpy(w["beta"].astype(np.float64)),
                      eps=float(np.float32(w.eps))).numpy()
    assert np.max(np.abs(y - yt)) <= 1e-12

    w = workloads.make("add_rmsnorm_bf16", rows=8, cols=8192)
    y, h, _ = oracle.add_rmsnorm(w["x"], w["residual"], w["weight"], w.eps)
    ht = torch.from_numpy(oracle.decode(w["x"]) + oracle.decode(w["residual"]))
    yt = F.rms_norm(ht, (8192,), torch.from_numpy(oracle.decode(w["weight"])),
                    eps=float(np.float32(w.eps))).numpy()
    assert rel_err(y, yt) <= 1e-12

    w = workloads.make("xent_f32", rows=6, cols=50257)
    loss, grad, am = oracle.softmax_xent(w["logits"], w["labels"])
    lt = torch.from_numpy(w["logits"].astype(np.float64)).requires_grad_(True)
    lab = torch.from_numpy(w["labels"].astype(np.int64))
    l = F.cross_entropy(lt, lab, reduction="none")
    l.sum().backward()
    assert rel_err(loss, l.detach().numpy()) <= 1e-12
    assert np.max(np.abs(grad - lt.grad.numpy())) <= 1e-15
    assert np.array_equal(am, torch.argmax(lt.detach(), dim=1).numpy().astype(np.int32))


# ------------------------------------------------------------------ I10

def _bits(v):
    return oracle.round_bf16_scalar(v)


def test_round_bf16_hand_cases():
    one = 1.0
    assert _bits(one) == 0x3F80
    assert _bits(1 + 2**-8) == 0x3F80                 # tie -> even (down)
    assert _bits(1 + 3 * 2**-8) == 0x3F82             # tie -> even (up)
    assert _bits(1 + 2**-8 + 2**-30) == 0x3F81        # just above a tie
    assert _bits(1 + 2**-8 - 2**-30) == 0x3F80        # just below a tie
    # direct from double: through fp32 this would hit the tie and go to even
    assert _bits(1 + 2**-8 + 2**-40) == 0x3F81
    assert _bits(-(1 + 2**-8 + 2**-40)) == 0xBF81
    maxf = (2 - 2**-7) * 2.0**127
    assert _bits(maxf) == 0x7F7F
    assert _bits((2 - 2**-8) * 2.0**127) == 0x7F80    # overflow tie -> inf
    assert _bits((2 - 2**-8) * 2.0**127 * (1 - 2**-40)) == 0x7F7F
    assert _bits(2.0**-126) == 0x0080
    assert _bits(2.0**-133) == 0x0001                  # smallest subnormal
    assert _bits(2.0**-134) == 0x0000                  # half of it: tie -> even (zero)
    assert _bits(2.0**-134 * (1 + 2**-20)) == 0x0001
    assert _bits(3 * 2.0**-134) == 0x0002              # tie between 1 and 2 -> 2
    assert _bits(127.5 * 2.0**-133) == 0x0080          # rounds up into the normal range
    assert _bits(0.0) == 0x0000 and _bits(-0.0) == 0x8000
    assert _bits(math.inf) == 0x7F80 and _bits(-math.inf) == 0xFF80
    assert (_bits(math.nan) & 0x7FFF) > 0x7F80
    assert _bits(1e300) == 0x7F80 and _bits(-1e-300) == 0x8000


def _check_f32_range(u32):
    f = u32.view(np.float32)
    with np.errstate(invalid="ignore"):
        f64 = f.astype(np.float64)
    got = oracle.round_bf16(f64)
    ref = workloads.f32_to_bf16_bits(f)        # independent bit-pattern routine
    nan = np.isnan(f)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.all((got[nan] & 0x7FFF) > 0x7F80)


def test_round_bf16_all_exponents_and_tie_patterns():
    hi = np.arange(0, 1 << 16, dtype=np.uint32) << 16
    lows = np.array([0x0000, 0x0001, 0x3FFF, 0x7FFE, 0x7FFF, 0x8000, 0x8001, 0xBFFF,
                     0xC000, 0xFFFE, 0xFFFF], dtype=np.uint32)
    u = (hi[:, None] | lows[None, :]).reshape(-1)
    _check_f32_range(u)
    _check_f32_range(RNG.integers(0, 1 << 32, size=1 << 22, dtype=np.uint64).astype(np.uint32))


@pytest.mark.skipif(os.environ.get("FR_EXHAUSTIVE_BF16", "1") == "0",
                    reason="all 2^32 fp32 inputs (about two minutes): FR_EXHAUSTIVE_BF16=0 set")
def test_round_bf16_exhaustive_fp32():
    step = 1 << 24
    for start in range(0, 1 << 32, step):
        _check_f32_range(np.arange(start, start + step, dtype=np.uint64).astype(np.uint32))


# ------------------------------------------------------------------ misc

def test_decode_is_exact():
    bits = np.array([0x3F80, 0x0001, 0x8000, 0x7F7F, 0xC2F7], dtype=np.uint16)
    ref = [1.0, 2.0**-133, -0.0, (2 - 2**-7) * 2.0**127, -123.5]
    assert list(oracle.decode(bits)) == ref
