"""C-ABI checks that need no GPU: librownorm.so loads, exports every function
include/rownorm.h and include/rownorm_bench.h declare (with the argument
count the binding declares), and rejects bad arguments before anything is
enqueued (all of these return before the library's first HIP call, so no
compute call is made here).  Pointers below are fake, suitably aligned
addresses that are never dereferenced."""
import ctypes
import os
import re

import pytest

import rmsnorm_row_welford_amd as rn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("rownorm.h", "rownorm_bench.h")]

OK, EINVAL, EDTYPE, EOVERLAP, EWORKSPACE, EHIP, EUNSUP = 0, -1, -2, -3, -4, -5, -6
F32, BF16, F16, BF16_F32W, F16_F32W = 0, 1, 2, 3, 4


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(rn.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return rn.lib()


def declarations():
    """name -> parameter count of every function the headers declare."""
    out = {}
    for h in HEADERS:
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^\s*(?:const\s+)?(?:int|int64_t|size_t|char|void)\s*\*?\s*"
                             r"(\w+)\s*\(([^)]*)\)\s*;", text, flags=re.M):
            params = [p for p in m.group(2).split(",") if p.strip() and p.strip() != "void"]
            out[m.group(1)] = len(params)
    return out


def declared_functions():
    return sorted(declarations())


def test_header_declares_the_boundary():
    names = declared_functions()
    for must in ("ln_fwd", "rms_fwd", "fused_add_rms_fwd", "ln_bwd", "rms_bwd",
                 "rn_bwd_workspace_bytes", "rn_status_str"):
        assert must in names


def test_library_exports_every_declared_symbol(L):
    decl = declarations()
    assert sorted(decl) == sorted(rn.SIGNATURES), "binding and headers disagree"
    for n, nargs in decl.items():
        assert hasattr(L, n), f"{n} not exported"
        assert len(rn.SIGNATURES[n][0]) == nargs, f"{n}: binding has the wrong arity"


def test_bench_helpers_live_in_their_own_header():
    main = open(HEADERS[0]).read()
    for n in ("rn_copy", "rn_add"):
        assert n + "(" not in re.sub(r"/\*.*?\*/", "", main, flags=re.S)


def test_status_strings(L):
    for code in (OK, EINVAL, EDTYPE, EOVERLAP, EWORKSPACE, EHIP, EUNSUP):
        s = L.rn_status_str(code).decode()
        assert s and s != "unknown status"
    assert L.rn_status_str(12345).decode() == "unknown status"


MAXH = 1 << 22


def test_max_hidden(L):
    for dt in (F32, BF16, F16, BF16_F32W, F16_F32W):
        assert L.rn_max_hidden(dt, 1) == MAXH
        assert L.rn_max_hidden(dt, 0) == MAXH
    assert L.rn_max_hidden(9, 1) == 0
    assert L.rn_max_hidden(5, 1) == 0


A = 1 << 30          # fake device addresses, far apart, 256-byte aligned
X, Y, G, B, M, R, H_, DY, DX, DG, DB, W, RES = (A * k for k in range(1, 14))
S = None             # stream: never reached


def ln_fwd(L, x=X, ldx=1024, g=G, b=B, y=Y, ldy=1024, m=M, r=R, N=8,
           H=1024, dt=BF16, eps=1e-5):
    return L.ln_fwd(x, ldx, g, b, y, ldy, m, r, N, H, dt, eps, S)


@pytest.mark.parametrize("kw,want", [
    (dict(eps=0.0), EINVAL), (dict(eps=-1e-5), EINVAL),
    (dict(eps=float("nan")), EINVAL), (dict(eps=float("inf")), EINVAL),
    (dict(eps=1e-40), EINVAL),               # subnormal in binary32
    (dict(dt=7), EDTYPE), (dict(H=0), EINVAL), (dict(N=-1), EINVAL),
    (dict(H=MAXH + 1, ldx=MAXH + 1, ldy=MAXH + 1), EUNSUP),
    (dict(H=MAXH + 8, ldx=MAXH + 8, ldy=MAXH + 8), EUNSUP),
    (dict(ldx=1000), EINVAL), (dict(ldy=1023), EINVAL),
    (dict(x=None), EINVAL), (dict(g=None), EINVAL), (dict(y=None), EINVAL),
    (dict(x=X + 1), EINVAL),                 # bf16 pointer not 2-aligned
    (dict(m=M + 2), EINVAL),                 # float pointer not 4-aligned
    (dict(y=X + 512), EOVERLAP),             # y inside x
    (dict(y=G - 8), EOVERLAP),               # y runs into gamma
    (dict(m=R), EOVERLAP),                   # mean == rstd
    (dict(r=Y + 100), EOVERLAP),             # rstd inside y
    (dict(N=0), OK),                         # no rows: nothing to do
    (dict(N=0, b=None, m=None, r=None), OK),
    (dict(N=0, x=None, y=None), OK),         # torch gives NULL for 0 rows
    (dict(N=0, g=None), EINVAL),             # gamma is always required
    (dict(N=0, H=MAXH, ldx=MAXH, ldy=MAXH), OK),        # the longest row
    (dict(N=0, H=8193, ldx=8193, ldy=8193), OK),        # long odd rows too
])
def test_ln_fwd_argument_errors(L, kw, want):
    assert ln_fwd(L, **kw) == want


def test_rms_fwd_argument_errors(L):
    assert L.rms_fwd(X, 64, G, Y, 64, R, 4, 64, BF16, 0.0, S) == EINVAL
    assert L.rms_fwd(X, 64, G, X, 64, R, 4, 64, BF16, 1e-6, S) == EOVERLAP
    assert L.rms_fwd(X, 64, G, Y, 64, None, 0, 64, F32, 1e-6, S) == OK
    assert L.rms_fwd(X, 64, G, Y, 64, None, 4, 64, 5, 1e-6, S) == EDTYPE
    assert L.rms_fwd(X, 64, G, Y, 64, None, 4, 64, -1, 1e-6, S) == EDTYPE


def fused(L, x=X, ldx=4096, res=RES, ldr=4096, g=G, y=Y, ldy=4096, h=H_,
          ldh=4096, r=R, N=0, H=4096, dt=BF16, eps=1e-6):
    return L.fused_add_rms_fwd(x, ldx, res, ldr, g, y, ldy, h, ldh, r, N, H,
                               dt, eps, S)


@pytest.mark.parametrize("kw,want", [
    (dict(), OK),
    (dict(h=X), OK),                 # in place over x
    (dict(h=RES), OK),               # in place over the residual
    (dict(h=X, ldh=4104), EOVERLAP),  # same base, different stride
    (dict(h=X + 64), EOVERLAP),      # partial overlap
    (dict(res=X, h=X), EOVERLAP),    # x == residual == h
    (dict(y=X), EOVERLAP),
    (dict(y=H_), EOVERLAP),          # y == h
    (dict(res=None), EINVAL), (dict(h=None), EINVAL),
    (dict(ldr=4000), EINVAL), (dict(ldh=100), EINVAL),
])
def test_fused_argument_errors(L, kw, want):
    kw.setdefault("N", 16)
    if want == OK:
        kw["N"] = 0     # valid: N = 0 returns before touching the device
    assert fused(L, **kw) == want


def ln_bwd(L, dy=DY, lddy=1024, x=X, ldx=1024, g=G, m=M, r=R, dx=DX,
           lddx=1024, dg=DG, db=DB, w=W, wb=1 << 24, N=8, H=1024, dt=BF16,
           eps=1e-5):
    return L.ln_bwd(dy, lddy, x, ldx, g, m, r, dx, lddx, dg, db, w, wb, N, H,
                    dt, eps, S)


@pytest.mark.parametrize("kw,want", [
    (dict(m=None), EINVAL), (dict(r=None), EINVAL), (dict(db=None), EINVAL),
    (dict(dg=None), EINVAL), (dict(dx=None), EINVAL),
    (dict(w=W + 16), EINVAL),              # workspace not 256-aligned
    (dict(dx=DY), EOVERLAP), (dict(dx=X + 2048), EOVERLAP),
    (dict(dg=DB), EOVERLAP), (dict(w=X), EOVERLAP),
    (dict(dg=G), EOVERLAP),
    (dict(eps=0.0), EINVAL), (dict(dt=5), EDTYPE),
    (dict(H=MAXH + 1, lddy=MAXH + 1, ldx=MAXH + 1, lddx=MAXH + 1), EUNSUP),
    (dict(lddx=1000), EINVAL),
])
def test_ln_bwd_argument_errors(L, kw, want):
    assert ln_bwd(L, **kw) == want


def test_rms_bwd_argument_errors(L):
    a = (DY, 256, X, 256, G, R, DX, 256, DG, W, 1 << 20)
    assert L.rms_bwd(*a, 4, 256, BF16, -1.0, S) == EINVAL
    b = (DY, 256, X, 256, G, None, DX, 256, DG, W, 1 << 20)
    assert L.rms_bwd(*b, 4, 256, BF16, 1e-5, S) == EINVAL
    c = (DY, 256, X, 256, G, R, X, 256, DG, W, 1 << 20)
    assert L.rms_bwd(*c, 4, 256, BF16, 1e-5, S) == EOVERLAP


def test_workspace_query_without_device(L):
    # (N, H, dtype, is_layernorm, device, &bytes); device -1 = current
    out = ctypes.c_size_t(123)
    assert L.rn_bwd_workspace_bytes(0, 1024, BF16, 1, -1, ctypes.byref(out)) == OK
    assert out.value == 0
    out.value = 7
    assert L.rn_bwd_workspace_bytes(0, 1024, BF16, 0, 3, ctypes.byref(out)) == OK
    assert out.value == 0                    # N = 0 touches no device
    assert L.rn_bwd_workspace_bytes(10, 1024, 9, 1, -1, ctypes.byref(out)) == EDTYPE
    assert L.rn_bwd_workspace_bytes(10, 0, BF16, 1, -1, ctypes.byref(out)) == EINVAL
    assert L.rn_bwd_workspace_bytes(10, 1024, BF16, 1, -1, None) == EINVAL
    assert L.rn_bwd_workspace_bytes(10, 1024, BF16, 1, -2, ctypes.byref(out)) == EINVAL


def test_partial_rows_query_without_device(L):
    # (N, H, dtype, is_layernorm, vectorizable, &rows)
    out = ctypes.c_int(123)
    assert L.rn_bwd_partial_rows(0, 1024, BF16, 1, 1, ctypes.byref(out)) == OK
    assert out.value == 0                    # N = 0 touches no device
    assert L.rn_bwd_partial_rows(10, 1024, 9, 1, 1, ctypes.byref(out)) == EDTYPE
    assert L.rn_bwd_partial_rows(10, 0, BF16, 1, 1, ctypes.byref(out)) == EINVAL
    assert L.rn_bwd_partial_rows(10, MAXH + 1, BF16, 1, 1, ctypes.byref(out)) == EUNSUP
    assert L.rn_bwd_partial_rows(10, 1024, BF16, 1, 1, None) == EINVAL


def test_copy_argument_errors(L):
    assert L.rn_copy(X, Y, 0, S) == OK
    assert L.rn_copy(None, Y, 16, S) == EINVAL
    assert L.rn_copy(X, X + 8, 64, S) == EOVERLAP


DH = A * 14


def fused_bwd(L, dy=DY, lddy=1024, h=H_, ldh=1024, g=G, r=R, dh=DH, lddh=1024,
              dx=DX, lddx=1024, dres=RES, lddres=1024, dg=DG, w=W, wb=1 << 24,
              N=8, H=1024, dt=BF16, eps=1e-6):
    return L.fused_add_rms_bwd(dy, lddy, h, ldh, g, r, dh, lddh, dx, lddx, dres,
                               lddres, dg, w, wb, N, H, dt, eps, S)


@pytest.mark.parametrize("kw,want", [
    # dx == dh_in with equal strides is accepted (the GPU tests cover it);
    # even N = 0 launches the dgamma fill, so no OK case runs here
    (dict(dx=DH, lddx=1032), EOVERLAP),       # same base, other stride
    (dict(dx=DH + 64), EOVERLAP),             # partial overlap with dh_in
    (dict(dres=DH), EOVERLAP),                # dres may not alias dh_in
    (dict(dres=DX), EOVERLAP),                # dres == dx
    (dict(dres=H_), EOVERLAP), (dict(dx=DY), EOVERLAP),
    (dict(dg=DH + 8), EOVERLAP), (dict(w=DH), EOVERLAP),
    (dict(r=None), EINVAL), (dict(h=None), EINVAL), (dict(dg=None), EINVAL),
    (dict(dh=DH + 1), EINVAL), (dict(dres=RES + 1), EINVAL),
    (dict(lddh=1000), EINVAL), (dict(lddres=512), EINVAL),
    (dict(eps=0.0), EINVAL), (dict(dt=5), EDTYPE),
    (dict(H=MAXH + 1, lddy=MAXH + 1, ldh=MAXH + 1, lddx=MAXH + 1, lddh=MAXH + 1,
          lddres=MAXH + 1), EUNSUP),
])
def test_fused_bwd_argument_errors(L, kw, want):
    assert fused_bwd(L, **kw) == want


@pytest.mark.parametrize("kw,want", [
    # float32 parameters beside 16-bit activations: gamma/beta 4-byte
    # aligned, and their extent is 4*H bytes
    (dict(dt=BF16_F32W, g=G + 2), EINVAL),
    (dict(dt=F16_F32W, b=B + 2), EINVAL),
    (dict(dt=BF16_F32W, x=X + 2), OK),        # 2-byte activations: fine
    (dict(dt=BF16_F32W, y=G + 2048), EOVERLAP),   # inside gamma's 4 KiB
    (dict(dt=F16, g=G + 1), EINVAL),
    (dict(dt=F16, m=R), EOVERLAP),
])
def test_mixed_param_argument_checks(L, kw, want):
    if want == OK:
        kw["N"] = 0     # valid: N = 0 returns before touching the device
    assert ln_fwd(L, **kw) == want


def test_mixed_param_backward_checks(L):
    # dgamma float32 with bf16 activations: 4-aligned, 4*H bytes long
    assert ln_bwd(L, dt=BF16_F32W, dg=DG + 2) == EINVAL
    assert ln_bwd(L, dt=BF16_F32W, db=DG + 2048) == EOVERLAP
    assert fused_bwd(L, dt=F16_F32W, dg=DG + 2) == EINVAL
    assert fused_bwd(L, dt=F16_F32W, dx=G + 2048) == EOVERLAP


def test_add_argument_errors(L):
    assert L.rn_add(X, Y, H_, 0, BF16, S) == OK
    assert L.rn_add(X, Y, H_, -1, BF16, S) == EINVAL
    assert L.rn_add(None, Y, H_, 8, BF16, S) == EINVAL
    assert L.rn_add(X, Y, H_, 8, 9, S) == EDTYPE
    assert L.rn_add(X + 1, Y, H_, 8, BF16, S) == EINVAL
    assert L.rn_add(X, Y, X + 4, 8, BF16, S) == EOVERLAP
    assert L.rn_add(X, Y, Y + 4, 8, F32, S) == EOVERLAP


def test_headers_serve_a_plain_c_caller(L, tmp_path):
    """Both headers compile as C99 with gcc (not hipcc), and a C program that
    takes the address of every declared function links against
    librownorm.so and runs the device-free workspace query."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    rocm_inc = "/opt/rocm/include"
    if gcc is None or not os.path.isdir(rocm_inc):
        pytest.skip("needs gcc and the ROCm headers")
    names = sorted(declarations())
    src = tmp_path / "use.c"
    src.write_text(
        '#include "rownorm.h"\n#include "rownorm_bench.h"\n#include <stdio.h>\n'
        "int main(void) {\n"
        "    void *fns[] = {" + ", ".join(f"(void *)&{n}" for n in names) + "};\n"
        "    size_t bytes = 123;\n"
        "    int st = rn_bwd_workspace_bytes(0, 1024, RN_BF16, 1, -1, &bytes);\n"
        '    printf("%d %zu %d %s\\n", st, bytes, (int)(sizeof fns / sizeof fns[0]),\n'
        "           rn_status_str(RN_EOVERLAP));\n"
        "    return 0;\n}\n")
    exe = tmp_path / "use"
    libdir = os.path.dirname(rn.LIB_PATH)
    r = subprocess.run([gcc, "-std=c99", "-Wall", "-Werror=implicit-function-declaration",
                        "-D__HIP_PLATFORM_AMD__", "-I" + os.path.join(ROOT, "include"),
                        "-I" + rocm_inc, str(src), "-L" + libdir, "-lrownorm",
                        "-Wl,-rpath," + libdir, "-o", str(exe)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert out.returncode == 0, out.stderr
    st, nbytes, nfn, msg = out.stdout.split(" ", 3)
    assert (int(st), int(nbytes), int(nfn)) == (OK, 0, len(names))
    assert msg.strip() == L.rn_status_str(EOVERLAP).decode()
