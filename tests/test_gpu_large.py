"""GPU parity on buffers larger than 4 GiB: rows whose element offsets pass
2^31 and whose byte offsets pass 2^32 (the kernels address a row from a 64-bit
row base; the split path also walks row batches), through the C ABI.

Inputs are drawn on the device from torch's seeded generator (standard normal
or uniform, scaled like the standard workloads); the rows around each
boundary are copied to the host and given to the double-precision oracle,
by the same comparison rules as the other parity tests. Where an output
depends on every row (the parameter gradients), dy is zero outside the
sampled rows, so the oracle on the sampled rows gives the exact expected
value, and every other row has a known exact result, checked on the device
over the whole buffer.
"""
import numpy as np
import pytest
import torch

import memory_bound_row_pass_amd as fr
from gpu_buffers import DEV
from parity import bf16_bits
from test_gpu_backward import expect_rms_bwd, expect_softmax_bwd
from test_gpu_parity import expect_layernorm, expect_rmsnorm, expect_softmax, expect_xent

pytestmark = pytest.mark.gpu

GIB = 1 << 30


@pytest.fixture(autouse=True)
def _free_device_memory():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def gen(seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    return g


def rows_of(t, rows):
    """The given rows of a device tensor as host arrays (bf16 as bit patterns)."""
    sub = t[torch.tensor(rows, device=DEV)]
    return bf16_bits(sub) if sub.dtype == torch.bfloat16 else sub.cpu().numpy()


def samples(R, *bounds):
    """Rows 0 and R-1 and the two rows on each side of every boundary row."""
    s = {0, R - 1}
    for b in bounds:
        s.update(r for r in (b - 1, b) if 0 <= r < R)
    return sorted(s)


def test_softmax_f32_beyond_4gib():
    R, C = (4 * GIB) // (1024 * 4) + 4, 1024            # byte offsets pass 2^31 and 2^32
    x = torch.randn(R, C, device=DEV, generator=gen(31)) * 4.0
    y = torch.full_like(x, float("nan"))
    assert x.numel() * 4 > 4 * GIB
    fr.fr_softmax_fwd(x, y)
    torch.cuda.synchronize()
    rows = samples(R, (2 * GIB) // (C * 4), (4 * GIB) // (C * 4), R // 2)
    expect_softmax(rows_of(x, rows), fr.F32, rows_of(y, rows), f"softmax f32 [{R}, {C}] rows {rows}")


def test_softmax_bf16_beyond_2e31_elements():
    R, C = (1 << 31) // 4096 + 4, 4096                  # element offsets pass 2^31
    x = (torch.randn(R, C, device=DEV, generator=gen(32)) * 8.0).bfloat16()
    y = torch.empty_like(x)
    assert x.numel() > 1 << 31
    fr.fr_softmax_fwd(x, y)
    torch.cuda.synchronize()
    rows = samples(R, (1 << 30) // C, (1 << 31) // C)
    expect_softmax(rows_of(x, rows), fr.BF16, rows_of(y, rows), f"softmax bf16 [{R}, {C}]")


def test_layernorm_f32_beyond_4gib():
    R, C = (4 * GIB) // (1024 * 4) + 3, 1024
    g = gen(33)
    x = torch.randn(R, C, device=DEV, generator=g) * 2.0 + 3.0
    gamma = torch.rand(C, device=DEV, generator=g) + 0.5
    beta = torch.randn(C, device=DEV, generator=g) * 0.1
    y = torch.full_like(x, float("nan"))
    mean = torch.full((R,), float("nan"), device=DEV)
    rstd = torch.full((R,), float("nan"), device=DEV)
    fr.fr_layernorm_fwd(x, gamma, beta, y, mean, rstd, 1e-5)
    torch.cuda.synchronize()
    rows = samples(R, (2 * GIB) // (C * 4), (4 * GIB) // (C * 4))
    got = (rows_of(y, rows), mean[rows].cpu().numpy(), rstd[rows].cpu().numpy())
    expect_layernorm(rows_of(x, rows), gamma.cpu().numpy(), beta.cpu().numpy(), 1e-5, got,
                     f"layernorm f32 [{R}, {C}]")


def test_add_rmsnorm_bf16_beyond_2e31_elements():
    R, C = (1 << 31) // 8192 + 4, 8192
    g = gen(34)
    x = torch.randn(R, C, device=DEV, generator=g).bfloat16()
    r = torch.randn(R, C, device=DEV, generator=g).bfloat16()
    w = (torch.rand(C, device=DEV, generator=g) * 0.4 + 0.8).bfloat16()
    y, ro = torch.empty_like(x), torch.empty_like(x)
    fr.fr_add_rmsnorm_fwd(x, r, w, y, ro, 1e-6)
    torch.cuda.synchronize()
    rows = samples(R, (1 << 30) // C, (1 << 31) // C)
    expect_rmsnorm(rows_of(x, rows), rows_of(r, rows), bf16_bits(w), 1e-6,
                   (rows_of(y, rows), rows_of(ro, rows)), f"add_rmsnorm bf16 [{R}, {C}]")


def test_xent_f32_beyond_4gib():
    C = 50257
    R = (4 * GIB) // (C * 4) + 5                        # rows straddle 2^31 and 2^32 bytes
    g = gen(35)
    logits = torch.randn(R, C, device=DEV, generator=g) * 2.0
    labels = torch.randint(0, C, (R,), device=DEV, generator=g, dtype=torch.int32)
    loss = torch.full((R,), float("nan"), device=DEV)
    grad = torch.full_like(logits, float("nan"))
    am = torch.full((R,), -7, device=DEV, dtype=torch.int32)
    fr.fr_softmax_xent_fwd_bwd(logits, labels, loss, grad, am)
    torch.cuda.synchronize()
    rows = samples(R, (2 * GIB) // (C * 4), (2 * GIB) // (C * 4) + 1,
                   (4 * GIB) // (C * 4), (4 * GIB) // (C * 4) + 1)
    got = (loss[rows].cpu().numpy(), rows_of(grad, rows), am[rows].cpu().numpy())
    expect_xent(rows_of(logits, rows), labels[rows].cpu().numpy(), got, f"xent f32 [{R}, {C}]")


def test_xent_split_f32_beyond_2e31_elements():
    C = 131072
    R = (1 << 31) // C + 4                              # element offsets pass 2^31
    g = gen(36)
    logits = torch.randn(R, C, device=DEV, generator=g) * 2.0
    labels = torch.randint(0, C, (R,), device=DEV, generator=g, dtype=torch.int32)
    loss = torch.full((R,), float("nan"), device=DEV)
    grad = torch.full_like(logits, float("nan"))
    am = torch.full((R,), -7, device=DEV, dtype=torch.int32)
    ws = torch.empty(max(fr.fr_split_workspace_bytes(R, C), 16), dtype=torch.uint8, device=DEV)
    fr.fr_softmax_xent_split(logits, labels, loss, grad, ws, argmax=am)
    torch.cuda.synchronize()
    rows = samples(R, (1 << 30) // C, (1 << 31) // C)
    got = (loss[rows].cpu().numpy(), rows_of(grad, rows), am[rows].cpu().numpy())
    expect_xent(rows_of(logits, rows), labels[rows].cpu().numpy(), got, f"xent split f32 [{R}, {C}]")


def test_softmax_bwd_bf16_beyond_2e31_elements():
    R, C = (1 << 31) // 4096 + 4, 4096
    g = gen(37)
    p = (torch.rand(R, C, device=DEV, generator=g) * (2.0 / C)).bfloat16()
    dy = torch.randn(R, C, device=DEV, generator=g).bfloat16()
    dx = torch.empty_like(p)
    fr.fr_softmax_bwd(p, dy, dx)
    torch.cuda.synchronize()
    rows = samples(R, (1 << 30) // C, (1 << 31) // C)
    expect_softmax_bwd(rows_of(p, rows), rows_of(dy, rows), fr.BF16, rows_of(dx, rows),
                       f"softmax bwd bf16 [{R}, {C}]")


class _Rows:
    """Host copies of the sampled rows, in the form the backward checks take."""

    def __init__(self, arrays, eps):
        self.arrays, self.eps = arrays, eps

    def __getitem__(self, k):
        return self.arrays[k]


def test_rmsnorm_bwd_bf16_beyond_2e31_elements():
    R, C = (1 << 31) // 8192 + 4, 8192
    g = gen(38)
    h = (torch.randn(R, C, device=DEV, generator=g) * 1.4).bfloat16()
    dres = torch.randn(R, C, device=DEV, generator=g).bfloat16()
    w = (torch.rand(C, device=DEV, generator=g) * 0.4 + 0.8).bfloat16()
    rows = samples(R, (1 << 30) // C, (1 << 31) // C)
    ridx = torch.tensor(rows, device=DEV)
    # dy is zero outside the sampled rows: there dh = dres exactly and the
    # weight gradient is the sampled rows' sum alone
    dy = torch.zeros(R, C, device=DEV, dtype=torch.bfloat16)
    dy[ridx] = torch.randn(len(rows), C, device=DEV, generator=g).bfloat16()
    dh = torch.empty_like(h)
    dw = torch.full((C,), float("nan"), device=DEV)
    ws = torch.empty(fr.fr_norm_bwd_workspace_bytes(fr.OP_RMSNORM_BWD, R, C), dtype=torch.uint8,
                     device=DEV)
    fr.fr_add_rmsnorm_bwd(h, dy, w, dh, dw, ws, dres=dres, eps=1e-6)
    torch.cuda.synchronize()
    sub = _Rows({"h": rows_of(h, rows), "dy": rows_of(dy, rows), "dres": rows_of(dres, rows),
                 "weight": bf16_bits(w)}, 1e-6)
    expect_rms_bwd(sub, fr.BF16, (rows_of(dh, rows), dw.cpu().numpy()),
                   f"rmsnorm bwd bf16 [{R}, {C}]", with_dres=True)
    differ = dh.view(torch.int16) != dres.view(torch.int16)
    differ[ridx] = False
    assert not bool(differ.any()), "rows with dy = 0 must give dh = dres exactly"
