"""The C ABI without a GPU: the library loads, exports every entry point the
header declares, and rejects bad arguments with the documented status codes
before making any HIP call (so no call here launches anything)."""
import ctypes
import os
import re

import pytest

import memory_bound_row_pass_amd as fr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fusedrow.h")

OK, E_NULL, E_SHAPE, E_DTYPE, E_ALIAS, E_LAUNCH, E_ALIGN, E_VALUE, E_VARIANT = range(9)

# fake, never dereferenced: every call below fails validation first
A = 0x7F0000000000          # 16-byte aligned
B = 0x7F0100000000
P = ctypes.c_void_p


def test_exports_every_declared_symbol():
    names = re.findall(r"^FR_API [^;(]*?\b(fr_\w+)\s*\(", open(HEADER).read(), re.M)
    assert len(names) >= 9
    for n in names:
        assert hasattr(fr.lib, n), n
    out = os.popen(f"nm -D --defined-only {fr.LIB_PATH}").read()
    exported = set(re.findall(r" T (\w+)$", out, re.M))
    assert set(names) == exported, (set(names) ^ exported)


def test_status_strings_and_version():
    for s in range(9):
        assert fr.status_str(s).startswith("FR_")
    assert "unknown" in fr.status_str(99)
    assert "gfx950" in fr.version()


def sm(x, y, rows, cols, xd=0, yd=0):
    return fr.lib.fr_softmax_fwd(P(x), P(y), rows, cols, xd, yd, None)


def test_softmax_validation():
    assert sm(A, B, 0, 10) == OK                 # no-op, nothing launched
    assert sm(0, 0, 0, 10) == OK                 # NULL allowed when rows == 0
    assert sm(A, B, -1, 10) == E_SHAPE
    assert sm(A, B, 4, 0) == E_SHAPE
    assert sm(A, B, 4, fr.FR_MAX_COLS + 1) == E_SHAPE
    assert sm(A, B, 2**62, 2**10) == E_SHAPE     # size overflow
    assert sm(A, B, 4, 10, 2, 0) == E_DTYPE
    assert sm(A, B, 4, 10, 0, 7) == E_DTYPE
    assert sm(0, B, 4, 10) == E_NULL
    assert sm(A, 0, 4, 10) == E_NULL
    assert sm(A + 2, B, 4, 10) == E_ALIGN        # fp32 needs 4-byte alignment
    assert sm(A, B + 1, 4, 10, 0, 1) == E_ALIGN  # bf16 needs 2-byte alignment
    # partial overlap is rejected, exact in-place is not an alias error
    assert sm(A, A + 4, 4, 10) == E_ALIAS
    assert sm(A, A + 40 * 4 - 4, 4, 10) == E_ALIAS
    # same base, different element size: rows would overlap
    assert sm(A, A, 4, 10, 0, 1) == E_ALIAS


def test_layernorm_validation():
    f = fr.lib.fr_layernorm_fwd
    G, Bt, M, R = A + 0x100000, A + 0x200000, A + 0x300000, A + 0x400000
    assert f(P(A), P(G), P(Bt), P(B), P(M), P(R), 0, 8, 1e-5, 0, None) == OK
    assert f(P(A), P(G), P(Bt), P(B), P(M), P(R), 4, 8, -1.0, 0, None) == E_VALUE
    assert f(P(A), P(G), P(Bt), P(B), P(M), P(R), 4, 8, float("nan"), 0, None) == E_VALUE
    assert f(P(A), P(G), P(Bt), P(B), P(M), P(R), 4, 8, float("inf"), 0, None) == E_VALUE
    assert f(P(A), None, P(Bt), P(B), P(M), P(R), 4, 8, 1e-5, 0, None) == E_NULL
    assert f(P(A), P(G), P(Bt), P(B), P(M), P(R), 4, 8, 1e-5, 3, None) == E_DTYPE
    assert f(P(A), P(G), P(Bt), P(B), P(M + 2), P(R), 4, 8, 1e-5, 0, None) == E_ALIGN
    # an output over a per-column parameter, or two outputs overlapping
    assert f(P(A), P(G), P(Bt), P(G), P(M), P(R), 1, 8, 1e-5, 0, None) == E_ALIAS
    assert f(P(A), P(G), P(Bt), P(B), P(M), P(M + 4), 4, 8, 1e-5, 0, None) == E_ALIAS
    assert f(P(A), P(G), P(Bt), P(B), P(A), P(R), 4, 8, 1e-5, 0, None) == E_ALIAS


def test_add_rmsnorm_validation():
    f = fr.lib.fr_add_rmsnorm_fwd
    Rz, W, Y, RO = A + 0x100000, A + 0x200000, A + 0x300000, A + 0x400000
    assert f(P(A), P(Rz), P(W), P(Y), P(RO), 0, 8, 1e-6, 1, None) == OK
    assert f(P(A), None, P(W), P(Y), P(RO), 4, 8, 1e-6, 1, None) == E_NULL
    assert f(P(A), P(Rz), P(W), P(Y), P(RO), 4, 8, -1e-6, 1, None) == E_VALUE
    assert f(P(A), P(Rz), P(W), P(Y), P(Y), 4, 8, 1e-6, 1, None) == E_ALIAS      # two outputs
    assert f(P(A), P(Rz), P(W), P(Y), P(Rz + 2), 4, 8, 1e-6, 1, None) == E_ALIAS  # partial
    assert f(P(A), P(Rz), P(W), P(Y), P(A + 1), 4, 8, 1e-6, 1, None) == E_ALIGN


# The interface of the four row operations and the status string, as the
# contract fixes it (whitespace aside): a caller compiled against these
# prototypes must find exactly them in the header.
CONTRACT = [
    "fr_status_t fr_softmax_fwd(const void* x, void* y, int64_t rows, int64_t cols, "
    "fr_dtype_t x_dtype, fr_dtype_t y_dtype, void* stream);",
    "fr_status_t fr_layernorm_fwd(const void* x, const void* gamma, const void* beta, "
    "void* y, float* mean, float* rstd, int64_t rows, int64_t cols, float eps, "
    "fr_dtype_t dtype, void* stream);",
    "fr_status_t fr_add_rmsnorm_fwd(const void* x, const void* residual, const void* weight, "
    "void* y, void* residual_out, int64_t rows, int64_t cols, float eps, fr_dtype_t dtype, "
    "void* stream);",
    "fr_status_t fr_softmax_xent_fwd_bwd(const float* logits, const int32_t* labels, "
    "float* loss, float* grad, int32_t* argmax, int64_t rows, int64_t cols, void* stream);",
    "const char* fr_status_str(fr_status_t s);",
]


def _declarations():
    """Every FR_API declaration of the header, comments removed, FR_API
    dropped and whitespace collapsed (one space, none inside parentheses)."""
    text = re.sub(r"/\*.*?\*/", " ", open(HEADER).read(), flags=re.S)
    out = {}
    for m in re.finditer(r"^FR_API\s+([^;]*;)", text, re.M):
        d = re.sub(r"\s+", " ", m.group(1)).replace("( ", "(").replace(" )", ")")
        out[re.search(r"\b(fr_\w+)\s*\(", d).group(1)] = d
    return out


def test_contract_prototypes():
    decl = _declarations()
    for proto in CONTRACT:
        name = re.search(r"\b(fr_\w+)\(", proto).group(1)
        assert name in decl, name
        assert decl[name] == proto, f"{name}:\n header   {decl[name]}\n contract {proto}"
    # the enums' values are part of the binary interface
    text = open(HEADER).read()
    for name, value in [("FR_F32", 0), ("FR_BF16", 1), ("FR_OK", 0), ("FR_E_NULL", 1),
                        ("FR_E_SHAPE", 2), ("FR_E_DTYPE", 3), ("FR_E_ALIAS", 4),
                        ("FR_E_LAUNCH", 5)]:
        assert re.search(rf"\b{name}\s*=\s*{value}\b", text), name


def test_xent_validation():
    # the contract's argument list: logits, labels, loss, grad, argmax, rows,
    # cols, stream (fp32 logits and gradient; no dtype argument)
    f = fr.lib.fr_softmax_xent_fwd_bwd
    L, LS, G, AM = A + 0x100000, A + 0x200000, A + 0x300000, A + 0x400000
    assert f(P(A), P(L), P(LS), P(G), P(AM), 0, 8, None) == OK
    assert f(None, None, None, None, None, 0, 8, None) == OK    # rows == 0: nothing read
    assert f(P(A), P(L), P(LS), P(G), P(AM), -1, 8, None) == E_SHAPE
    assert f(P(A), P(L), P(LS), P(G), P(AM), 4, 0, None) == E_SHAPE
    assert f(P(A), P(L), P(LS), P(G), P(AM), 4, fr.FR_MAX_COLS + 1, None) == E_SHAPE
    assert f(P(A), None, P(LS), P(G), None, 4, 8, None) == E_NULL
    assert f(P(A), P(L), P(LS), None, None, 4, 8, None) == E_NULL
    assert f(P(A + 2), P(L), P(LS), P(G), None, 4, 8, None) == E_ALIGN   # fp32 logits
    assert f(P(A), P(L), P(LS), P(G + 2), None, 4, 8, None) == E_ALIGN
    assert f(P(A), P(L), P(LS), P(G), P(LS), 4, 8, None) == E_ALIAS   # argmax over loss
    assert f(P(A), P(L), P(L), P(G), None, 4, 8, None) == E_ALIAS     # loss over labels
    assert f(P(A), P(L), P(LS), P(A + 4), None, 4, 8, None) == E_ALIAS
    # a non-NULL stream is the last argument, not a dtype: still validated first
    assert f(P(A), P(L), P(LS), P(A + 4), None, 4, 8, P(0x1234)) == E_ALIAS


def test_softmax_bwd_validation():
    f = fr.lib.fr_softmax_bwd
    D, X = A + 0x100000, A + 0x200000
    assert f(P(A), P(D), P(X), 0, 8, 0, None) == OK
    assert f(None, None, None, 0, 8, 1, None) == OK
    assert f(P(A), P(D), P(X), 4, fr.FR_BWD_MAX_COLS + 1, 0, None) == E_SHAPE
    assert f(P(A), None, P(X), 4, 8, 0, None) == E_NULL
    assert f(P(A), P(D), P(X), 4, 8, 2, None) == E_DTYPE
    assert f(P(A), P(D), P(D + 4), 4, 8, 0, None) == E_ALIAS   # partial overlap with dy
    assert f(P(A), P(A), P(A + 4), 4, 8, 0, None) == E_ALIAS
    assert f(P(A), P(D), P(X + 2), 4, 8, 0, None) == E_ALIGN


def test_rmsnorm_bwd_noalloc_validation():
    f = fr.lib.fr_add_rmsnorm_bwd_noalloc
    D, W, DH, DW = A + 0x10000000, A + 0x20000000, A + 0x30000000, A + 0x40000000
    assert f(P(A), P(D), None, P(W), P(DH), None, 4, 8, 1e-6, 1, None) == E_NULL  # dweight
    assert f(P(A), P(D), None, P(W), P(DH), P(DW), 4, fr.FR_BWD_MAX_COLS + 1, 1e-6, 1,
             None) == E_SHAPE
    assert f(P(A), P(D), None, P(W), P(DH), P(DW), 4, 8, -1.0, 1, None) == E_VALUE
    assert f(P(A), P(D), None, P(W), P(DH), P(DW), 4, 8, 1e-6, 5, None) == E_DTYPE
    assert f(P(A), P(D), None, P(W), P(A + 2), P(DW), 4, 8, 1e-6, 1, None) == E_ALIAS
    # partial rows beyond the library's array: 256 rows x 16384 columns x 4 B
    assert f(P(A), P(D), None, P(W), P(DH), P(DW), 4096, 16384, 1e-6, 1, None) == E_SHAPE
    assert fr.FR_NOALLOC_SCRATCH_BYTES == 8 << 20
    assert re.search(r"#define FR_NOALLOC_SCRATCH_BYTES \(8 << 20\)", open(HEADER).read())


def test_norm_bwd_workspace_bytes():
    f = fr.fr_norm_bwd_workspace_bytes
    assert f(fr.OP_RMSNORM_BWD, 8192, 8192) == fr.FR_BWD_PARTIALS * 8192 * 4
    assert f(fr.OP_LAYERNORM_BWD, 4096, 1024) == fr.FR_BWD_PARTIALS * 1024 * 4 * 2
    assert f(fr.OP_RMSNORM_BWD, 3, 100) == 3 * 100 * 4
    assert f(fr.OP_LAYERNORM_BWD, 0, 100) == 0
    for op, r, c in ((fr.OP_SOFTMAX, 4, 8), (fr.OP_RMSNORM_BWD, -1, 8),
                     (fr.OP_RMSNORM_BWD, 4, fr.FR_BWD_MAX_COLS + 1), (fr.OP_LAYERNORM_BWD, 4, 0)):
        with pytest.raises(ValueError):
            f(op, r, c)


def test_rmsnorm_bwd_validation():
    f = fr.lib.fr_add_rmsnorm_bwd
    DY, DR, W, DH, DW, WS = (A + k * 0x100000 for k in range(1, 7))
    need = 4 * 8 * 4

    def call(h=A, dy=DY, dres=DR, w=W, dh=DH, dw=DW, ws=WS, wsb=need, rows=4, cols=8, eps=1e-6,
             dt=0):
        return f(P(h), P(dy), P(dres), P(w), P(dh), P(dw), P(ws), wsb, rows, cols, eps, dt, None)

    assert call(dw=0, rows=0) == E_NULL                # dweight is written even for rows == 0
    assert call(dw=DW + 2, rows=0) == E_ALIGN
    assert call(wsb=need - 1) == E_SHAPE
    assert call(cols=fr.FR_BWD_MAX_COLS + 1) == E_SHAPE
    assert call(eps=-1.0) == E_VALUE
    assert call(dt=5) == E_DTYPE
    assert call(ws=0) == E_NULL
    assert call(dy=0) == E_NULL
    assert call(ws=WS + 4) == E_ALIGN                  # workspace: 16-byte aligned
    assert call(dres=DR + 2) == E_ALIGN
    assert call(ws=DH + 64) == E_ALIAS                 # workspace inside dh
    assert call(dw=W) == E_ALIAS                       # dweight over weight
    assert call(dh=DY + 4) == E_ALIAS                  # partial overlap with dy


def test_layernorm_bwd_validation():
    f = fr.lib.fr_layernorm_bwd
    DY, G, M, R, DX, DG, DB, WS = (A + k * 0x100000 for k in range(1, 9))
    need = 4 * 8 * 4 * 2

    def call(x=A, dy=DY, g=G, m=M, r=R, dx=DX, dg=DG, db=DB, ws=WS, wsb=need, rows=4, cols=8, dt=1):
        return f(P(x), P(dy), P(g), P(m), P(r), P(dx), P(dg), P(db), P(ws), wsb, rows, cols, dt,
                 None)

    assert call(db=0, rows=0) == E_NULL
    assert call(dg=DB, rows=0) == E_ALIAS              # the two gradients may not coincide
    assert call(wsb=need - 4) == E_SHAPE
    assert call(m=0) == E_NULL
    assert call(r=R + 2) == E_ALIGN
    assert call(x=A + 1) == E_ALIGN                    # bf16 needs 2-byte alignment
    assert call(ws=DX) == E_ALIAS
    assert call(dg=M) == E_ALIAS                       # an output over an input
    assert call(dx=DY + 2) == E_ALIAS


def test_xent_ex_validation():
    f = fr.lib.fr_softmax_xent_ex
    L, LS, G, AM, T = (A + k * 0x100000 for k in range(1, 6))

    def call(lg=A, lab=L, ls=LS, g=G, am=AM, tot=T, rows=4, cols=8, dt=1, **o):
        opts = fr.XentOptions(o.get("use", 1), o.get("ign", -100), o.get("eps", 0.1),
                              o.get("scale", 1.0), o.get("red", fr.REDUCE_MEAN))
        return f(P(lg), P(lab), P(ls), P(g), P(am), P(tot), rows, cols, dt, ctypes.byref(opts), None)

    assert call(rows=0, red=fr.REDUCE_NONE) == OK          # nothing to do, nothing launched
    assert call(rows=0, tot=0) == E_NULL                    # a total needs somewhere to go
    assert call(eps=-0.1) == E_VALUE
    assert call(eps=1.5) == E_VALUE
    assert call(eps=float("nan")) == E_VALUE
    assert call(scale=float("inf")) == E_VALUE
    assert call(red=7) == E_VALUE
    assert call(dt=4) == E_DTYPE
    assert call(tot=0) == E_NULL
    assert call(tot=T + 2) == E_ALIGN
    assert call(lg=A + 1) == E_ALIGN                        # bf16 needs 2-byte alignment
    assert call(tot=LS + 4) == E_ALIAS                      # total inside the per-row losses
    assert call(tot=L) == E_ALIAS                           # total over the labels
    assert call(g=A + 2) == E_ALIAS


def test_split_validation():
    f = fr.lib.fr_softmax_fwd_split
    Y, WS = A + 0x100000, A + 0x200000
    need = fr.fr_split_workspace_bytes(4, 100000)
    assert need == 4 * 13 * 16 + 16                   # ceil(100000 / 8192) = 13 segments per row
    assert f(P(A), P(Y), 0, 100000, 0, 0, None, 0, None) == OK
    assert f(P(A), P(Y), 4, 100000, 0, 0, P(WS), need - 1, None) == E_SHAPE
    assert f(P(A), P(Y), 4, fr.FR_SPLIT_MAX_COLS + 1, 0, 0, P(WS), 1 << 40, None) == E_SHAPE
    assert f(P(A), P(Y), 4, 100000, 0, 0, None, need, None) == E_NULL
    assert f(P(A), P(Y), 4, 100000, 0, 0, P(WS + 8), need, None) == E_ALIGN
    assert f(P(A), P(Y), 4, 100000, 3, 0, P(WS), need, None) == E_DTYPE
    assert f(P(A), P(A + 4), 4, 100000, 0, 0, P(WS), need, None) == E_ALIAS
    assert f(P(A), P(Y), 4, 100000, 0, 0, P(Y + 16), need, None) == E_ALIAS   # workspace in y
    g = fr.lib.fr_softmax_xent_split
    L, LS, G = A + 0x300000, A + 0x400000, A + 0x500000
    opts = fr.XentOptions(0, 0, 2.0, 1.0, 0)
    assert g(P(A), P(L), P(LS), P(G), None, None, 4, 100000, 0, ctypes.byref(opts), P(WS), need,
             None) == E_VALUE
    opts = fr.XentOptions(0, 0, 0.0, 1.0, fr.REDUCE_SUM)
    assert g(P(A), P(L), P(LS), P(G), None, None, 4, 100000, 0, ctypes.byref(opts), P(WS), need,
             None) == E_NULL
    with pytest.raises(ValueError):
        fr.fr_split_workspace_bytes(4, 0)


def test_split_norm_validation():
    f = fr.lib.fr_layernorm_fwd_split
    Gm, Bt, Y, M, RS, WS = (A + k * 0x100000 for k in range(1, 7))
    need = fr.fr_split_workspace_bytes(4, 100000)

    def ln(x=A, g=Gm, b=Bt, y=Y, m=M, r=RS, rows=4, cols=100000, eps=1e-5, dt=0, ws=WS, wn=need):
        return f(P(x), P(g), P(b), P(y), P(m), P(r), rows, cols, eps, dt, P(ws), wn, None)

    assert ln(rows=0, ws=0, wn=0) == OK
    assert ln(wn=need - 1) == E_SHAPE
    assert ln(cols=fr.FR_SPLIT_MAX_COLS + 1, wn=1 << 40) == E_SHAPE
    assert ln(ws=0) == E_NULL
    assert ln(g=0) == E_NULL
    assert ln(ws=WS + 8) == E_ALIGN
    assert ln(dt=3) == E_DTYPE
    assert ln(eps=-1.0) == E_VALUE
    assert ln(eps=float("nan")) == E_VALUE
    assert ln(m=M + 2) == E_ALIGN
    assert ln(y=A + 4) == E_ALIAS                       # partial overlap with x
    assert ln(ws=Y + 16) == E_ALIAS                     # workspace inside y
    assert ln(r=M) == E_ALIAS                           # mean and rstd the same buffer
    g = fr.lib.fr_add_rmsnorm_fwd_split
    R_, W_, RO = A + 0x700000, A + 0x800000, A + 0x900000

    def rn(x=A, r=R_, w=W_, y=Y, ro=RO, rows=4, cols=100000, eps=1e-6, dt=1, ws=WS, wn=need):
        return g(P(x), P(r), P(w), P(y), P(ro), rows, cols, eps, dt, P(ws), wn, None)

    assert rn(rows=0, ws=0, wn=0) == OK
    assert rn(wn=need - 1) == E_SHAPE
    assert rn(w=0) == E_NULL
    assert rn(dt=2) == E_DTYPE
    assert rn(eps=float("inf")) == E_VALUE
    assert rn(x=A + 1) == E_ALIGN                      # bf16 needs 2-byte alignment
    assert rn(ro=R_ + 2) == E_ALIAS                    # residual_out overlapping the residual
    assert rn(ws=RO) == E_ALIAS                        # workspace over residual_out


def test_softmax_bwd_split_validation():
    f = fr.lib.fr_softmax_bwd_split
    DY, DX, WS = A + 0x100000, A + 0x200000, A + 0x300000
    need = fr.fr_split_workspace_bytes(4, 100000)

    def call(p=A, dy=DY, dx=DX, rows=4, cols=100000, dt=0, ws=WS, wn=need):
        return f(P(p), P(dy), P(dx), rows, cols, dt, P(ws), wn, None)

    assert call(rows=0, ws=0, wn=0) == OK
    assert call(wn=need - 1) == E_SHAPE
    assert call(cols=0) == E_SHAPE
    assert call(dy=0) == E_NULL
    assert call(ws=0) == E_NULL
    assert call(dt=5) == E_DTYPE
    assert call(dx=DX + 2) == E_ALIGN
    assert call(dx=A + 4) == E_ALIAS
    assert call(ws=DX + 64) == E_ALIAS


def test_norm_bwd_split_validation():
    n = fr.fr_norm_bwd_split_workspace_bytes
    assert n(fr.OP_RMSNORM_BWD, 4, 100000) == 1024 + 4 * 100000 * 4  # 13 segments, 4 row groups
    assert n(fr.OP_LAYERNORM_BWD, 1000, 32768) == 64256 + 256 * 32768 * 4 * 2   # 64000 + 16, padded
    with pytest.raises(ValueError):
        n(fr.OP_SOFTMAX, 4, 100000)
    with pytest.raises(ValueError):
        n(fr.OP_RMSNORM_BWD, 4, fr.FR_SPLIT_MAX_COLS + 1)
    f = fr.lib.fr_add_rmsnorm_bwd_split
    DY, DR, W, DH, DW, WS = (A + k * 0x1000000 for k in range(1, 7))
    need = n(fr.OP_RMSNORM_BWD, 4, 100000)

    def rn(h=A, dy=DY, dres=DR, w=W, dh=DH, dw=DW, ws=WS, wn=need, rows=4, cols=100000, eps=1e-6,
           dt=1):
        return f(P(h), P(dy), P(dres), P(w), P(dh), P(dw), P(ws), wn, rows, cols, eps, dt, None)

    assert rn(wn=need - 1) == E_SHAPE
    assert rn(cols=0) == E_SHAPE
    assert rn(dw=0) == E_NULL
    assert rn(ws=0) == E_NULL
    assert rn(dt=3) == E_DTYPE
    assert rn(eps=-1.0) == E_VALUE
    assert rn(ws=WS + 8) == E_ALIGN
    assert rn(dh=A + 2) == E_ALIAS
    assert rn(ws=DW) == E_ALIAS
    g = fr.lib.fr_layernorm_bwd_split
    M, RS, DG, DB = A + 0x8000000, A + 0x9000000, A + 0xA000000, A + 0xB000000
    need = n(fr.OP_LAYERNORM_BWD, 4, 100000)

    def ln(x=A, dy=DY, gm=W, m=M, r=RS, dx=DH, dg=DG, db=DB, ws=WS, wn=need, rows=4, cols=100000,
           dt=0):
        return g(P(x), P(dy), P(gm), P(m), P(r), P(dx), P(dg), P(db), P(ws), wn, rows, cols, dt,
                 None)

    assert ln(wn=need - 1) == E_SHAPE
    assert ln(m=0) == E_NULL
    assert ln(db=0) == E_NULL
    assert ln(dt=9) == E_DTYPE
    assert ln(r=RS + 2) == E_ALIGN
    assert ln(db=DG) == E_ALIAS
    assert ln(dx=DY + 4) == E_ALIAS


def test_attention_validation():
    f = fr.lib.fr_attention_fwd
    K, V, O, LSE = A + 0x100000, A + 0x200000, A + 0x300000, A + 0x400000

    def call(q=A, k=K, v=V, o=O, lse=LSE, b=1, h=2, sq=16, sk=16, d=64, causal=0, scale=0.125, dt=1):
        return f(P(q), P(k), P(v), P(o), P(lse), b, h, sq, sk, d, causal, scale, dt, None)

    assert call(sq=0) == OK
    assert call(d=96) == E_SHAPE
    assert call(b=70000) == E_SHAPE                      # batch * heads > 65535
    assert call(b=2**62, h=2**40) == E_SHAPE             # batch * heads overflows int64
    assert call(dt=0) == E_DTYPE                         # bf16 only
    assert call(scale=float("nan")) == E_VALUE
    assert call(k=0) == E_NULL
    assert call(o=O + 8) == E_ALIGN                      # 16-byte alignment
    assert call(o=K) == E_ALIAS                          # output over the keys
    assert call(lse=A + 64) == E_ALIAS                   # lse inside q


def test_stream_copy_validation():
    f = fr.lib.fr_stream_copy
    assert f(P(A), P(B), 0, None) == OK
    assert f(P(A), P(B), -1, None) == E_SHAPE
    assert f(None, P(B), 16, None) == E_NULL
    assert f(P(A), P(A + 8), 16, None) == E_ALIAS


def test_stream_probe_validation():
    f = fr.lib.fr_stream_probe
    S = A + 0x100000
    READ, WRITE, COPY = fr.PROBE_READ, fr.PROBE_WRITE, fr.PROBE_COPY
    assert f(READ, P(A), None, 0, 0, 0, P(S), 256, 8, 1, None) == OK        # nothing to do
    assert f(3, P(A), P(B), 16, 0, 0, None, 256, 8, 1, None) == E_VALUE     # unknown probe
    assert f(COPY, P(A), P(B), 16, 0, 0, None, 256, 7, 1, None) == E_VARIANT  # no such shape
    assert f(COPY, P(A), P(B), 16, 0, 0, None, 256, 8, 4, None) == E_VALUE    # unknown policy bit
    assert f(COPY, P(A), P(B), 24, 0, 0, None, 256, 8, 1, None) == E_SHAPE  # not whole chunks
    assert f(COPY, P(A), P(B), -16, 0, 0, None, 256, 8, 1, None) == E_SHAPE
    assert f(COPY, P(A), P(B), 32, 24, 0, None, 256, 8, 1, None) == E_SHAPE  # row not chunks
    assert f(COPY, P(A), P(B), 32, 256 * 8 * 16 + 16, 0, None, 256, 8, 1, None) == E_SHAPE
    assert f(READ, P(A), None, 16, 0, 0, None, 256, 8, 1, None) == E_NULL   # read needs a sink
    assert f(WRITE, None, None, 16, 0, 7, None, 256, 8, 1, None) == E_NULL
    assert f(COPY, P(A + 4), P(B), 16, 0, 0, None, 256, 8, 1, None) == E_ALIGN
    assert f(READ, P(A), None, 16, 0, 0, P(S + 2), 256, 8, 1, None) == E_ALIGN
    assert f(COPY, P(A), P(A + 16), 32, 0, 0, None, 256, 8, 1, None) == E_ALIAS
    assert f(READ, P(A), None, 64, 0, 0, P(A + 32), 64, 4, 1, None) == E_ALIAS  # sink in src
    assert fr.lib.fr_stream_read(P(A), 24, P(S), None) == E_SHAPE
    assert fr.lib.fr_stream_write(P(A + 8), 16, 1, None) == E_ALIGN
    # rows of a length: one sink word per row, partial last row included
    assert fr.fr_stream_probe_rows(1 << 20) == 32
    assert fr.fr_stream_probe_rows((1 << 20) + 16, 201040) == (1 << 20) // 201040 + 1
    assert fr.lib.fr_stream_probe_rows(16, 24) == -1


def test_mfma_probe_validation():
    f = fr.lib.fr_mfma_probe
    assert f(0, 1, 0, P(A), None) == E_SHAPE
    assert f((1 << 20) + 1, 1, 0, P(A), None) == E_SHAPE
    assert f(1, 0, 1, P(A), None) == E_SHAPE
    assert f(1, (1 << 19) + 1, 1, P(A), None) == E_SHAPE
    assert f(1, 1, 2, P(A), None) == E_VALUE
    assert f(1, 1, -1, P(A), None) == E_VALUE
    assert f(1, 1, 0, None, None) == E_NULL
    assert f(1, 1, 1, P(A + 2), None) == E_ALIGN


def test_variant_selection():
    # one wavefront per row for short rows, a workgroup per row for long ones
    assert fr.fr_debug_select_variant(fr.OP_SOFTMAX, 1000, fr.F32) == (64, 4, 4)
    assert fr.fr_debug_select_variant(fr.OP_SOFTMAX, 2048, fr.BF16) == (64, 4, 8)
    assert fr.fr_debug_select_variant(fr.OP_SOFTMAX, 4096, fr.BF16) == (128, 4, 8)
    assert fr.fr_debug_select_variant(fr.OP_SOFTMAX, 4096, fr.F32) == (64, 16, 4)
    t, v, e = fr.fr_debug_select_variant(fr.OP_XENT, 50257, fr.F32)
    assert t * v * e >= 50257 and t >= 256
    t, v, e = fr.fr_debug_select_variant(fr.OP_SOFTMAX, 50257, fr.F32, vector_path=False)
    assert e == 1 and t * v >= 50257
    for op in (fr.OP_SOFTMAX, fr.OP_LAYERNORM, fr.OP_RMSNORM, fr.OP_XENT):
        for c in (1, 2, 3, 64, 1000, 4096, 8192, 50257, fr.FR_MAX_COLS):
            for vp in (True, False):
                t, v, e = fr.fr_debug_select_variant(op, c, fr.F32, vector_path=vp)
                assert t * v * e >= c
    for op in (fr.OP_SOFTMAX_BWD, fr.OP_RMSNORM_BWD, fr.OP_LAYERNORM_BWD):
        for dt in (fr.F32, fr.BF16):
            for c in (1, 3, 8, 64, 1000, 1024, 4096, 8192, fr.FR_BWD_MAX_COLS):
                for vp in (True, False):
                    t, v, e = fr.fr_debug_select_variant(op, c, dt, vector_path=vp)
                    assert t * v * e >= c
            with pytest.raises(fr.FusedRowError) as ei:
                fr.fr_debug_select_variant(op, fr.FR_BWD_MAX_COLS + 1, dt)
            assert ei.value.status == E_SHAPE
    for op in (fr.OP_SOFTMAX_SPLIT, fr.OP_XENT_SPLIT, fr.OP_LAYERNORM_SPLIT, fr.OP_RMSNORM_SPLIT,
               fr.OP_SOFTMAX_BWD_SPLIT):
        for dt in (fr.F32, fr.BF16):
            for vp in (True, False):
                t, v, e = fr.fr_debug_select_variant(op, 262144, dt, vector_path=vp)
                assert t * v * e >= 8192
    with fr.forced_variant(fr.OP_SOFTMAX, 1024, 16):
        assert fr.fr_debug_select_variant(fr.OP_SOFTMAX, 1000, fr.F32) == (1024, 16, 4)
    assert fr.fr_debug_select_variant(fr.OP_SOFTMAX, 1000, fr.F32) == (64, 4, 4)
    with fr.forced_variant(fr.OP_SOFTMAX, 64, 1):
        with pytest.raises(fr.FusedRowError) as ei:
            fr.fr_debug_select_variant(fr.OP_SOFTMAX, 1000, fr.F32)
        assert ei.value.status == E_VARIANT
    with pytest.raises(fr.FusedRowError):
        fr.fr_debug_force_variant(12, 64, 1)


def test_binding_rejects_host_tensors():
    torch = pytest.importorskip("torch")
    x = torch.zeros(2, 3)
    with pytest.raises(ValueError):
        fr.fr_softmax_fwd(x, torch.zeros(2, 3))


def test_split_batch_setting():
    # host-side setting only: returns the previous value; < 0 restores the
    # built-in 256 MiB bound; 0 means one batch of all rows
    L = fr.lib
    default = 256 << 20
    prev = L.fr_debug_set_split_batch_bytes(12345)
    try:
        assert prev == default
        assert L.fr_debug_set_split_batch_bytes(0) == 12345
        assert L.fr_debug_set_split_batch_bytes(-7) == 0
        assert L.fr_debug_set_split_batch_bytes(-1) == default
        with fr.split_batch_bytes(1):
            assert L.fr_debug_set_split_batch_bytes(1) == 1
        assert L.fr_debug_set_split_batch_bytes(-1) == default
    finally:
        L.fr_debug_set_split_batch_bytes(-1)


def test_split_one_pass_settings():
    # host-side settings only: each returns the previous value
    L = fr.lib
    assert L.fr_debug_set_split_one_pass(0) == 1          # 1 by default
    try:
        assert L.fr_debug_set_split_one_pass(2) == 0
        assert L.fr_debug_set_split_one_pass(7) == 2      # out of range: 1
        assert L.fr_debug_set_split_one_pass(-1) == 1
        assert L.fr_debug_set_split_one_pass(1) == 1
        with fr.split_one_pass(0):
            assert L.fr_debug_set_split_one_pass(0) == 0
        assert L.fr_debug_set_split_one_pass(1) == 1
    finally:
        L.fr_debug_set_split_one_pass(1)
    default = 1 << 18
    assert L.fr_debug_set_coop_spin_limit(5) == default
    try:
        assert L.fr_debug_set_coop_spin_limit(0) == 5
        assert L.fr_debug_set_coop_spin_limit(-3) == 0
        assert L.fr_debug_set_coop_spin_limit(-1) == default
        with fr.coop_spin_limit(0):
            assert L.fr_debug_set_coop_spin_limit(0) == 0
        assert L.fr_debug_set_coop_spin_limit(-1) == default
    finally:
        L.fr_debug_set_coop_spin_limit(-1)


def test_split_form_selection():
    # host-side selection only (no GPU: 256 compute units assumed): the
    # one-pass shape (512 lanes x 64 elements; the fp32 LayerNorm 512 x 32)
    # when the rows give at least 4 work items per compute unit, else the
    # two passes' first shape; mode 0 never, mode 2 always (where the row
    # has at most 64 one-pass segments)
    import torch
    if torch.cuda.is_available():
        pytest.skip("compute-unit count of the host without a GPU")
    sel = fr.fr_debug_select_variant_for
    X, SM, LN, RN, SB = (fr.OP_XENT_SPLIT, fr.OP_SOFTMAX_SPLIT, fr.OP_LAYERNORM_SPLIT,
                         fr.OP_RMSNORM_SPLIT, fr.OP_SOFTMAX_BWD_SPLIT)
    cases = [  # (op, rows, cols, dtype, mode 1 shape)
        (X, 2048, 131072, fr.F32, (512, 16, 4)),    # 2048 x 4 work items
        (X, 96, 131072, fr.F32, (256, 8, 4)),       # 384 < 1024: two passes
        (X, 1024, 262144, fr.BF16, (512, 8, 8)),
        (X, 64, 262144, fr.BF16, (256, 8, 8)),
        (X, 512, 50257, fr.F32, (512, 16, 4)),      # 512 x 2 = 1024
        (X, 511, 50257, fr.F32, (256, 8, 4)),
        (SM, 2048, 131072, fr.F32, (512, 16, 4)),
        (LN, 512, 131072, fr.F32, (512, 8, 4)),     # fp32 LayerNorm: 512 x 32
        (LN, 512, 131072, fr.BF16, (256, 4, 8)),    # bf16 LayerNorm: two passes
        (RN, 256, 262144, fr.BF16, (512, 8, 8)),
        (SB, 1024, 131072, fr.BF16, (512, 8, 8)),
        (X, 4, 1 << 22, fr.F32, (256, 8, 4)),       # 128 one-pass segments > 64
    ]
    for op, R, C, dt, want in cases:
        assert sel(op, R, C, dt) == want, (op, R, C, dt)
    first = {fr.F32: (256, 8, 4), fr.BF16: (256, 8, 8)}
    with fr.split_one_pass(0):
        for op, R, C, dt, _ in cases:
            want = (256, 4, 8) if (op in (LN, RN, SB) and dt == fr.BF16) else first[dt]
            assert sel(op, R, C, dt) == want, (op, R, C, dt, "mode 0")
    with fr.split_one_pass(2):
        assert sel(X, 1, 131072, fr.F32) == (512, 16, 4)
        assert sel(LN, 1, 131072, fr.BF16) == (256, 4, 8)   # no one-pass shape: the first
        assert sel(X, 4, 1 << 22, fr.F32) == (256, 8, 4)


def test_row_aware_selection():
    # the cross-entropy takes the 256-lane shape (two rows per compute unit)
    # when the rows fill the compute units once but not twice; without a GPU
    # the compute-unit count falls back to 256
    import torch
    if torch.cuda.is_available():
        pytest.skip("compute-unit count of the host without a GPU")
    sel = fr.fr_debug_select_variant_for
    for R, want in ((100, (1024, 13, 4)), (256, (1024, 13, 4)), (257, (256, 50, 4)),
                    (512, (256, 50, 4)), (513, (1024, 13, 4)), (4096, (1024, 13, 4))):
        assert sel(fr.OP_XENT, R, 50257, fr.F32) == want, R
    assert sel(fr.OP_XENT, 300, 50257, fr.BF16) == (1024, 7, 8)   # no 256-lane bf16 shape holds it
    assert sel(fr.OP_SOFTMAX, 300, 50257, fr.F32) == fr.fr_debug_select_variant(fr.OP_SOFTMAX, 50257)
    with fr.forced_variant(fr.OP_XENT, 1024, 13):                    # a forced shape is kept
        assert sel(fr.OP_XENT, 300, 50257, fr.F32) == (1024, 13, 4)
    with pytest.raises(fr.FusedRowError):
        sel(fr.OP_XENT, -1, 50257, fr.F32)
