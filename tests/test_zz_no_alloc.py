"""GPU: the allocation-free RMSNorm backward (fr_add_rmsnorm_bwd_noalloc,
the library's own device array in place of a workspace) gives bitwise the
results of fr_add_rmsnorm_bwd with a caller workspace, through the C ABI, on
consecutive calls that reuse the array: a large call, then a smaller one
(its fewer partial rows must not mix with the larger call's leftovers), in
both dtypes, with and without the residual's gradient."""
import numpy as np
import pytest
import torch

import memory_bound_row_pass_amd as fr

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def setup_module(module):
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"


def inputs(R, C, dt, seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    h = (torch.randn(R, C, device=DEV, generator=g) * 1.4).to(dt)
    dy = torch.randn(R, C, device=DEV, generator=g).to(dt)
    dres = torch.randn(R, C, device=DEV, generator=g).to(dt)
    w = (torch.rand(C, device=DEV, generator=g) * 0.4 + 0.8).to(dt)
    return h, dy, dres, w


def bits(t):
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32)


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("with_dres", [True, False])
def test_noalloc_matches_workspace_call(dt, with_dres):
    # 8192 x 8192 bf16 fills the array (256 partial rows x 8192 columns);
    # then fewer rows and columns, and rows that are not a multiple of the
    # workgroup's row groups, and a single row
    for (R, C) in [(8192, 8192), (1000, 1536), (37, 8192), (1, 64)]:
        h, dy, dres, w = inputs(R, C, dt, R + C)
        dr = dres if with_dres else None
        dh_ref = torch.empty_like(h)
        dw_ref = torch.empty(C, device=DEV)
        ws = torch.empty(max(fr.fr_norm_bwd_workspace_bytes(fr.OP_RMSNORM_BWD, R, C), 16),
                         dtype=torch.uint8, device=DEV)
        fr.fr_add_rmsnorm_bwd(h, dy, w, dh_ref, dw_ref, ws, dres=dr, eps=1e-6)
        dh = torch.full_like(h, float("nan"))
        dw = torch.full((C,), float("nan"), device=DEV)
        fr.fr_add_rmsnorm_bwd_noalloc(h, dy, w, dh, dw, dres=dr, eps=1e-6)
        torch.cuda.synchronize()
        print(f"noalloc {dt} dres={with_dres} [{R}, {C}]", flush=True)
        assert torch.equal(bits(dh), bits(dh_ref)), (R, C)
        assert torch.equal(bits(dw), bits(dw_ref)), (R, C)


def test_noalloc_twice_in_a_row_second_smaller():
    """Two calls back to back on one stream, the second smaller, each checked
    against the workspace entry point's results."""
    runs = []
    for (R, C, seed) in [(4096, 4096, 1), (513, 2048, 2)]:
        h, dy, dres, w = inputs(R, C, torch.bfloat16, seed)
        dh, dw = torch.empty_like(h), torch.empty(C, device=DEV)
        fr.fr_add_rmsnorm_bwd_noalloc(h, dy, w, dh, dw, dres=dres, eps=1e-6)
        runs.append((h, dy, dres, w, dh, dw))
    torch.cuda.synchronize()
    for h, dy, dres, w, dh, dw in runs:
        R, C = h.shape
        dh_ref, dw_ref = torch.empty_like(h), torch.empty(C, device=DEV)
        ws = torch.empty(fr.fr_norm_bwd_workspace_bytes(fr.OP_RMSNORM_BWD, R, C),
                         dtype=torch.uint8, device=DEV)
        fr.fr_add_rmsnorm_bwd(h, dy, w, dh_ref, dw_ref, ws, dres=dres, eps=1e-6)
        torch.cuda.synchronize()
        assert torch.equal(bits(dh), bits(dh_ref))
        assert torch.equal(bits(dw), bits(dw_ref))


def test_noalloc_rejects_partials_beyond_the_array():
    # 16384 bf16 columns over 256 partial rows need 16 MiB: refused before
    # any launch, and the outputs are untouched
    R, C = 4096, 16384
    h, dy, dres, w = inputs(R, C, torch.bfloat16, 5)
    dh = torch.zeros_like(h)
    dw = torch.zeros(C, device=DEV)
    with pytest.raises(fr.FusedRowError) as e:
        fr.fr_add_rmsnorm_bwd_noalloc(h, dy, w, dh, dw, eps=1e-6)
    assert e.value.status == 2
    # rows == 0 writes zeros and needs no array
    dw0 = torch.full((C,), 7.0, device=DEV)
    fr.fr_add_rmsnorm_bwd_noalloc(h[:0], dy[:0], w, dh[:0], dw0, eps=1e-6)
    torch.cuda.synchronize()
    assert bool(torch.all(dw0 == 0)) and bool(torch.all(dh == 0))
