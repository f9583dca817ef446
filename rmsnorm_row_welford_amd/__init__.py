"""Row-wise LayerNorm / RMSNorm / fused residual-add + RMSNorm, forward and
backward, on AMD Instinct MI355X (gfx950).

This package is a thin binding over librownorm.so (C ABI, include/rownorm.h):
it turns torch tensors into device pointers, sizes and the current HIP stream,
allocates outputs the caller did not pass, and raises on a non-zero status.
All arithmetic runs in the library's HIP kernels; there is no CPU fallback —
if the library is missing every call raises.

Tensors are 2-D [N, H] with contiguous rows (stride(1) == 1, any row stride
>= H), on one GPU, dtype torch.float32, torch.bfloat16 or torch.float16.
gamma/beta are [H] tensors of the activation dtype or float32 (with 16-bit
activations); the parameter gradients take gamma's dtype.  mean/rstd are
float32 [N] tensors.
"""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librownorm.so")

RN_F32, RN_BF16, RN_F16, RN_BF16_F32W, RN_F16_F32W = 0, 1, 2, 3, 4
RN_OK = 0
STATUS_NAMES = {0: "RN_OK", -1: "RN_EINVAL", -2: "RN_EDTYPE",
                -3: "RN_EOVERLAP", -4: "RN_EWORKSPACE", -5: "RN_EHIP",
                -6: "RN_EUNSUPPORTED"}

# name -> (argtypes, restype); mirrors include/rownorm.h and (the benchmark
# helpers rn_copy, rn_add, rn_bwd_partial_rows) include/rownorm_bench.h
_P, _I64, _I, _F, _SZ = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                         ctypes.c_float, ctypes.c_size_t)
SIGNATURES = {
    "ln_fwd": ([_P, _I64, _P, _P, _P, _I64, _P, _P, _I64, _I64, _I, _F, _P], _I),
    "rms_fwd": ([_P, _I64, _P, _P, _I64, _P, _I64, _I64, _I, _F, _P], _I),
    "fused_add_rms_fwd": ([_P, _I64, _P, _I64, _P, _P, _I64, _P, _I64, _P,
                           _I64, _I64, _I, _F, _P], _I),
    "ln_bwd": ([_P, _I64, _P, _I64, _P, _P, _P, _P, _I64, _P, _P, _P, _SZ,
                _I64, _I64, _I, _F, _P], _I),
    "ln_bwd_noalloc": ([_P, _I64, _P, _I64, _P, _P, _P, _P, _I64, _P, _P,
                        _I64, _I64, _I, _F, _P], _I),
    "rms_bwd": ([_P, _I64, _P, _I64, _P, _P, _P, _I64, _P, _P, _SZ, _I64,
                 _I64, _I, _F, _P], _I),
    "fused_add_rms_bwd": ([_P, _I64, _P, _I64, _P, _P, _P, _I64, _P, _I64, _P,
                           _I64, _P, _P, _SZ, _I64, _I64, _I, _F, _P], _I),
    "rn_bwd_workspace_bytes": ([_I64, _I64, _I, _I, _I, ctypes.POINTER(_SZ)], _I),
    "rn_max_hidden": ([_I, _I], _I64),
    "rn_status_str": ([_I], ctypes.c_char_p),
    "rn_copy": ([_P, _P, _SZ, _P], _I),
    "rn_add": ([_P, _P, _P, _I64, _I, _P], _I),
    "rn_bwd_partial_rows": ([_I64, _I64, _I, _I, _I, ctypes.POINTER(_I)], _I),
}

_lib = None


class RowNormError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        msg = lib().rn_status_str(status).decode()
        super().__init__(f"{fn}: {STATUS_NAMES.get(status, status)} ({msg})")


def lib() -> ctypes.CDLL:
    """The loaded librownorm.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -c 'import __graft_entry__ as g; g.build()'` "
                "(or python rmsnorm_row_welford_amd/build.py)")
        h = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in SIGNATURES.items():
            f = getattr(h, name)
            f.argtypes = args
            f.restype = res
        _lib = h
    return _lib


def _check(fn, status):
    if status != RN_OK:
        raise RowNormError(fn, status)


# ------------------------------------------------------------ marshalling --
def _code_of(act, param):
    """rn_dtype code for (activation dtype, parameter dtype)."""
    import torch
    table = {(torch.float32, torch.float32): RN_F32,
             (torch.bfloat16, torch.bfloat16): RN_BF16,
             (torch.float16, torch.float16): RN_F16,
             (torch.bfloat16, torch.float32): RN_BF16_F32W,
             (torch.float16, torch.float32): RN_F16_F32W}
    if (act, param) not in table:
        raise TypeError(f"unsupported dtypes: activations {act}, parameters {param}")
    return table[(act, param)]


def _dtype_code(t, gamma):
    return _code_of(t.dtype, gamma.dtype)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _rows(t, name):
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D [N, H], got {tuple(t.shape)}")
    if t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError(f"{name} rows must be contiguous")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    return t.stride(0) if t.shape[0] > 1 else max(t.shape[1], t.stride(0))


def _vec(t, H, name):
    if t is None:
        return None
    if t.dim() != 1 or t.shape[0] != H or (H > 1 and t.stride(0) != 1):
        raise ValueError(f"{name} must be a contiguous [{H}] vector")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    return t


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _stats(t, N, name):
    import torch
    if t is None:
        return None
    if t.dtype != torch.float32 or t.dim() != 1 or t.shape[0] != N or \
            (N > 1 and t.stride(0) != 1):
        raise ValueError(f"{name} must be a contiguous float32 [{N}] tensor")
    return t


# ---------------------------------------------------------------- forward --
def ln_fwd(x, gamma, beta=None, eps=1e-5, *, y=None, mean=None, rstd=None,
           save_stats=True, stream=None):
    """LayerNorm forward.  Returns (y, mean, rstd); mean/rstd are None when
    save_stats is False and none were passed."""
    import torch
    N, H = x.shape
    ldx = _rows(x, "x")
    _vec(gamma, H, "gamma")
    _vec(beta, H, "beta")
    if y is None:
        y = torch.empty((N, H), dtype=x.dtype, device=x.device)
    if save_stats and mean is None:
        mean = torch.empty(N, dtype=torch.float32, device=x.device)
    if save_stats and rstd is None:
        rstd = torch.empty(N, dtype=torch.float32, device=x.device)
    _stats(mean, N, "mean")
    _stats(rstd, N, "rstd")
    _check("ln_fwd", lib().ln_fwd(
        _ptr(x), ldx, _ptr(gamma), _ptr(beta), _ptr(y), _rows(y, "y"),
        _ptr(mean), _ptr(rstd), N, H, _dtype_code(x, gamma), float(eps),
        _stream(stream)))
    return y, mean, rstd


def rms_fwd(x, gamma, eps=1e-5, *, y=None, rstd=None, save_stats=True,
            stream=None):
    """RMSNorm forward.  Returns (y, rstd)."""
    import torch
    N, H = x.shape
    ldx = _rows(x, "x")
    _vec(gamma, H, "gamma")
    if y is None:
        y = torch.empty((N, H), dtype=x.dtype, device=x.device)
    if save_stats and rstd is None:
        rstd = torch.empty(N, dtype=torch.float32, device=x.device)
    _stats(rstd, N, "rstd")
    _check("rms_fwd", lib().rms_fwd(
        _ptr(x), ldx, _ptr(gamma), _ptr(y), _rows(y, "y"), _ptr(rstd), N, H,
        _dtype_code(x, gamma), float(eps), _stream(stream)))
    return y, rstd


def fused_add_rms_fwd(x, residual, gamma, eps=1e-6, *, y=None, h=None,
                      rstd=None, save_stats=True, stream=None):
    """Fused residual add + RMSNorm forward.  Returns (y, h, rstd) with
    h = x + residual.  Pass h=x or h=residual for the in-place update."""
    import torch
    N, H = x.shape
    ldx = _rows(x, "x")
    ldr = _rows(residual, "residual")
    _vec(gamma, H, "gamma")
    if y is None:
        y = torch.empty((N, H), dtype=x.dtype, device=x.device)
    if h is None:
        h = torch.empty((N, H), dtype=x.dtype, device=x.device)
    if save_stats and rstd is None:
        rstd = torch.empty(N, dtype=torch.float32, device=x.device)
    _stats(rstd, N, "rstd")
    _check("fused_add_rms_fwd", lib().fused_add_rms_fwd(
        _ptr(x), ldx, _ptr(residual), ldr, _ptr(gamma), _ptr(y),
        _rows(y, "y"), _ptr(h), _rows(h, "h"), _ptr(rstd), N, H,
        _dtype_code(x, gamma), float(eps), _stream(stream)))
    return y, h, rstd


# --------------------------------------------------------------- backward --
def workspace_bytes(N, H, dtype, layernorm: bool, param_dtype=None,
                    device=None) -> int:
    """Backward workspace size (rn_bwd_workspace_bytes) for activations of
    `dtype` and parameters of `param_dtype` (default: the same) on GPU
    `device` (an index or torch.device; default: the current device)."""
    code = _code_of(dtype, dtype if param_dtype is None else param_dtype)
    if device is None:
        dev = -1
    else:
        dev = device if isinstance(device, int) else device.index
        dev = -1 if dev is None else dev
    out = ctypes.c_size_t(0)
    _check("rn_bwd_workspace_bytes", lib().rn_bwd_workspace_bytes(
        N, H, code, 1 if layernorm else 0, dev, ctypes.byref(out)))
    return int(out.value)


def _workspace(workspace, N, H, x, gamma, layernorm):
    import torch
    need = workspace_bytes(N, H, x.dtype, layernorm, gamma.dtype, x.device)
    if workspace is None:
        # 256-byte aligned by torch's caching allocator
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    return workspace, workspace.numel() * workspace.element_size()


def ln_bwd(dy, x, gamma, mean, rstd, eps=1e-5, *, dx=None, dgamma=None,
           dbeta=None, workspace=None, stream=None):
    """LayerNorm backward.  Returns (dx, dgamma, dbeta)."""
    import torch
    N, H = x.shape
    ldx = _rows(x, "x")
    lddy = _rows(dy, "dy")
    _vec(gamma, H, "gamma")
    _stats(mean, N, "mean")
    _stats(rstd, N, "rstd")
    if dx is None:
        dx = torch.empty((N, H), dtype=x.dtype, device=x.device)
    if dgamma is None:
        dgamma = torch.empty(H, dtype=gamma.dtype, device=x.device)
    if dbeta is None:
        dbeta = torch.empty(H, dtype=gamma.dtype, device=x.device)
    ws, wsb = _workspace(workspace, N, H, x, gamma, True)
    _check("ln_bwd", lib().ln_bwd(
        _ptr(dy), lddy, _ptr(x), ldx, _ptr(gamma), _ptr(mean), _ptr(rstd),
        _ptr(dx), _rows(dx, "dx"), _ptr(dgamma), _ptr(dbeta), _ptr(ws), wsb,
        N, H, _dtype_code(x, gamma), float(eps), _stream(stream)))
    return dx, dgamma, dbeta


def ln_bwd_noalloc(dy, x, gamma, mean, rstd, eps=1e-5, *, dx=None, dgamma=None,
                   dbeta=None, stream=None):
    """LayerNorm backward with the library's static per-GPU partial-row
    array instead of a workspace (the entry point allocates nothing; pass
    dx, dgamma and dbeta to allocate nothing here either).  Returns
    (dx, dgamma, dbeta)."""
    import torch
    N, H = x.shape
    ldx = _rows(x, "x")
    lddy = _rows(dy, "dy")
    _vec(gamma, H, "gamma")
    _stats(mean, N, "mean")
    _stats(rstd, N, "rstd")
    if dx is None:
        dx = torch.empty((N, H), dtype=x.dtype, device=x.device)
    if dgamma is None:
        dgamma = torch.empty(H, dtype=gamma.dtype, device=x.device)
    if dbeta is None:
        dbeta = torch.empty(H, dtype=gamma.dtype, device=x.device)
    _check("ln_bwd_noalloc", lib().ln_bwd_noalloc(
        _ptr(dy), lddy, _ptr(x), ldx, _ptr(gamma), _ptr(mean), _ptr(rstd),
        _ptr(dx), _rows(dx, "dx"), _ptr(dgamma), _ptr(dbeta), N, H,
        _dtype_code(x, gamma), float(eps), _stream(stream)))
    return dx, dgamma, dbeta


def rms_bwd(dy, x, gamma, rstd, eps=1e-5, *, dx=None, dgamma=None,
            workspace=None, stream=None):
    """RMSNorm backward.  Returns (dx, dgamma)."""
    import torch
    N, H = x.shape
    ldx = _rows(x, "x")
    lddy = _rows(dy, "dy")
    _vec(gamma, H, "gamma")
    _stats(rstd, N, "rstd")
    if dx is None:
        dx = torch.empty((N, H), dtype=x.dtype, device=x.device)
    if dgamma is None:
        dgamma = torch.empty(H, dtype=gamma.dtype, device=x.device)
    ws, wsb = _workspace(workspace, N, H, x, gamma, False)
    _check("rms_bwd", lib().rms_bwd(
        _ptr(dy), lddy, _ptr(x), ldx, _ptr(gamma), _ptr(rstd), _ptr(dx),
        _rows(dx, "dx"), _ptr(dgamma), _ptr(ws), wsb, N, H,
        _dtype_code(x, gamma), float(eps), _stream(stream)))
    return dx, dgamma


def fused_add_rms_bwd(dy, h, gamma, rstd, eps=1e-6, *, dh_in=None, dx=None,
                      dres=None, write_dres=False, dgamma=None, workspace=None,
                      stream=None):
    """Fused add+RMSNorm backward on the stored h.  Returns (dx, dres,
    dgamma); dres is None unless passed or write_dres is set (dx holds the
    gradient of both inputs).  Pass dx=dh_in to accumulate in place."""
    import torch
    N, H = h.shape
    ldh = _rows(h, "h")
    lddy = _rows(dy, "dy")
    _vec(gamma, H, "gamma")
    _stats(rstd, N, "rstd")
    if dx is None:
        dx = torch.empty((N, H), dtype=h.dtype, device=h.device)
    if dres is None and write_dres:
        dres = torch.empty((N, H), dtype=h.dtype, device=h.device)
    if dgamma is None:
        dgamma = torch.empty(H, dtype=gamma.dtype, device=h.device)
    ws, wsb = _workspace(workspace, N, H, h, gamma, False)
    _check("fused_add_rms_bwd", lib().fused_add_rms_bwd(
        _ptr(dy), lddy, _ptr(h), ldh, _ptr(gamma), _ptr(rstd), _ptr(dh_in),
        _rows(dh_in, "dh_in") if dh_in is not None else H, _ptr(dx),
        _rows(dx, "dx"), _ptr(dres), _rows(dres, "dres") if dres is not None else H,
        _ptr(dgamma), _ptr(ws), wsb, N, H, _dtype_code(h, gamma), float(eps),
        _stream(stream)))
    return dx, dres, dgamma


# ------------------------------------------------------------------ misc --
def max_hidden(dtype_code: int, vectorizable: bool = True) -> int:
    return int(lib().rn_max_hidden(dtype_code, 1 if vectorizable else 0))


def bwd_partial_rows(N, H, dtype, layernorm: bool, param_dtype=None,
                     vectorizable: bool = True) -> int:
    """The float32 partial rows per parameter the backward's kernel 1
    writes at (N, H) on the current device (0: none, the column sums or one
    workgroup); see rn_bwd_partial_rows."""
    code = _code_of(dtype, dtype if param_dtype is None else param_dtype)
    out = ctypes.c_int(0)
    _check("rn_bwd_partial_rows", lib().rn_bwd_partial_rows(
        N, H, code, 1 if layernorm else 0, 1 if vectorizable else 0, ctypes.byref(out)))
    return int(out.value)


def copy(src, dst, nbytes=None, stream=None):
    """Device-to-device byte copy with the library's streaming copy kernel."""
    n = src.numel() * src.element_size() if nbytes is None else nbytes
    _check("rn_copy", lib().rn_copy(_ptr(src), _ptr(dst), n, _stream(stream)))


def add(a, b, out=None, stream=None):
    """out = a + b (element-wise, float32 add rounded to the storage type)
    with the library's streaming add kernel; a benchmark helper."""
    import torch
    if a.shape != b.shape or a.dtype != b.dtype:
        raise ValueError("a and b must match in shape and dtype")
    if not (a.is_contiguous() and b.is_contiguous()):
        raise ValueError("a and b must be contiguous")
    if out is None:
        out = torch.empty_like(a)
    code = _code_of(a.dtype, a.dtype)
    _check("rn_add", lib().rn_add(_ptr(a), _ptr(b), _ptr(out), a.numel(), code,
                                  _stream(stream)))
    return out
