"""HIP path vs the binary64 oracle, element by element, on the same seeded
inputs (rmsnorm_row_welford_amd.synth), through the C ABI.

Every output element of every workload is compared, the full-size ones
included: they run on the GPU exactly as the benchmark launches them, and
the oracle computes every row.  Bars: tests/tolerance.py.  Each check is
labelled with its workload; the session prints, per label, the largest ulp
distance and how many elements passed only through the cancellation floor.
On the workloads the pages name, RMSNorm and fused y must hold 1 ulp
everywhere (no floor), and the floor may carry at most FLOOR_FRAC of the
LayerNorm y and dx elements.
"""
import numpy as np
import pytest
import torch

import oracle
import tolerance as tol
import rmsnorm_row_welford_amd as rn
from rmsnorm_row_welford_amd import synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


TORCH_DT = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}


def to_dev(a, dt="bf16"):
    """Storage array -> GPU tensor; uint16 patterns are bf16 or fp16 (dt),
    float32 arrays stay float32 whatever dt says."""
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(TORCH_DT[dt]).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    t = t.detach().cpu()
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def pdt(arr, dtype):
    """Storage type of the parameters: float32 or the activation type."""
    return "f32" if arr["gamma"].dtype == np.float32 else dtype


# Share of LayerNorm y and dx elements that may pass only through the
# cancellation floor on the named workloads: only |v| below about 2^-14 of
# the row scale can need it, about 5e-5 of a normal sample (measured on
# MI355X: at most 5.4e-6 on any of them).
FLOOR_FRAC = 5e-5


def dec(orc, arr, k, dtype):
    return orc.decode(arr[k], pdt(arr, dtype) if k in ("gamma", "beta") else dtype)


# ----------------------------------------------------------------- helpers --
def _lab(tag, what):
    return f"{tag}: {what}" if tag else f"edge: {what}"


def check_ln_fwd(orc, arr, dtype, eps, use_beta=True, tag=None):
    """tag: the workload's name for the statistics; a named workload also
    bounds the share of floored y elements."""
    x = to_dev(arr["x"], dtype)
    g = to_dev(arr["gamma"], dtype)
    b = to_dev(arr["beta"], dtype) if (use_beta and "beta" in arr) else None
    y, mean, rstd = rn.ln_fwd(x, g, b, eps)
    torch.cuda.synchronize()
    xd = orc.decode(arr["x"], dtype)
    e = oracle.eps_at_boundary(eps)
    bd = dec(orc, arr, "beta", dtype) if b is not None else None
    y_o, m_o, r_o = orc.ln_fwd(xd, dec(orc, arr, "gamma", dtype), bd, e)
    del xd
    var_o = 1.0 / (r_o * r_o) - e
    stats = tol.check_out(host(y), y_o, dtype, orc, _lab(tag, f"LN y {dtype}"),
                          max_floored_frac=FLOOR_FRAC if tag else None)
    tol.check_mean(host(mean), m_o, var_o, e, _lab(tag, "LN mean"))
    tol.check_rstd(host(rstd), r_o, _lab(tag, "LN rstd"))
    return y, mean, rstd, stats


def check_rms_fwd(orc, arr, dtype, eps, tag=None):
    """RMSNorm y is a product (no cancellation): 1 ulp everywhere."""
    x = to_dev(arr["x"], dtype)
    g = to_dev(arr["gamma"], dtype)
    y, rstd = rn.rms_fwd(x, g, eps)
    torch.cuda.synchronize()
    xd = orc.decode(arr["x"], dtype)
    y_o, r_o = orc.rms_fwd(xd, dec(orc, arr, "gamma", dtype),
                           oracle.eps_at_boundary(eps))
    del xd
    stats = tol.check_out(host(y), y_o, dtype, orc, _lab(tag, f"RMS y {dtype}"),
                          strict=True)
    tol.check_rstd(host(rstd), r_o, _lab(tag, "RMS rstd"))
    return y, rstd, stats


def check_bwd(orc, arr, dtype, eps, layernorm, tag=None):
    """GPU forward (for the saved stats), GPU backward, oracle backward."""
    x = to_dev(arr["x"], dtype)
    dy = to_dev(arr["dy"], dtype)
    g = to_dev(arr["gamma"], dtype)
    e = oracle.eps_at_boundary(eps)
    xd = orc.decode(arr["x"], dtype)
    dyd = orc.decode(arr["dy"], dtype)
    gd = dec(orc, arr, "gamma", dtype)
    if layernorm:
        _, mean, rstd = rn.ln_fwd(x, g, None, eps)
        dx, dg, db = rn.ln_bwd(dy, x, g, mean, rstd, eps)
        torch.cuda.synchronize()
        dx_o, dg_o, db_o, _, rstd_o = orc.ln_bwd(dyd, xd, gd, e)
    else:
        _, rstd = rn.rms_fwd(x, g, eps)
        dx, dg = rn.rms_bwd(dy, x, g, rstd, eps)
        torch.cuda.synchronize()
        dx_o, dg_o, rstd_o = orc.rms_bwd(dyd, xd, gd, e)
    assert dg.dtype == TORCH_DT[pdt(arr, dtype)] and dx.dtype == TORCH_DT[dtype]
    ts = tol.dx_term_scale(dyd, gd, rstd_o)
    del xd, dyd
    nm = "LN" if layernorm else "RMS"
    stats = tol.check_out(host(dx), dx_o, dtype, orc, _lab(tag, f"{nm} dx {dtype}"),
                          term_scale=ts, max_floored_frac=FLOOR_FRAC if tag else None)
    rr = tol.check_param(orc.decode(host(dg), pdt(arr, dtype)), dg_o,
                         _lab(tag, f"{nm} dgamma"))
    if layernorm:
        tol.check_param(orc.decode(host(db), pdt(arr, dtype)), db_o, _lab(tag, "LN dbeta"))
    return stats, rr


def fused_bwd_oracle(orc, arr, dtype, eps, with_dh=True):
    """Oracle side of the fused backward: its own forward gives the stored h
    (RNE of the exact sum) and the saved rstd (of the exact sum)."""
    e = oracle.eps_at_boundary(eps)
    xd, rd = orc.decode(arr["x"], dtype), orc.decode(arr["residual"], dtype)
    gd, dyd = dec(orc, arr, "gamma", dtype), orc.decode(arr["dy"], dtype)
    _, h_o, rs_o = orc.fused_add_rms_fwd(xd, rd, gd, e)
    h_stored = orc.decode(orc.encode(h_o, dtype), dtype)
    dhd = orc.decode(arr["dh"], dtype) if with_dh else None
    dx_o, dg_o = orc.fused_add_rms_bwd(dyd, h_stored, gd, rs_o, dhd)
    return dx_o, dg_o, tol.dx_term_scale(dyd, gd, rs_o), h_o


def check_fused_bwd(orc, arr, dtype, eps, with_dh=True, write_dres=True,
                    in_place=False, tag=None):
    """GPU fused forward (h, rstd), GPU fused backward, oracle backward."""
    x, r, g, dy = (to_dev(arr[k], dtype) for k in ("x", "residual", "gamma", "dy"))
    _, h, rstd = rn.fused_add_rms_fwd(x, r, g, eps)
    dh = to_dev(arr["dh"], dtype) if with_dh else None
    dx, dres, dg = rn.fused_add_rms_bwd(
        dy, h, g, rstd, eps, dh_in=dh, dx=dh if in_place else None,
        write_dres=write_dres)
    torch.cuda.synchronize()
    if in_place:
        assert dx.data_ptr() == dh.data_ptr()
    dx_o, dg_o, ts, h_o = fused_bwd_oracle(orc, arr, dtype, eps, with_dh)
    assert np.array_equal(host(h), orc.encode(h_o, dtype)), "h not RNE(x + r)"
    del h_o
    stats = tol.check_out(host(dx), dx_o, dtype, orc, _lab(tag, f"fused dx {dtype}"),
                          term_scale=ts, max_floored_frac=FLOOR_FRAC if tag else None)
    if write_dres:
        assert torch.equal(dres, dx), "dres differs from dx"
    else:
        assert dres is None
    rr = tol.check_param(orc.decode(host(dg), pdt(arr, dtype)), dg_o,
                         _lab(tag, "fused dgamma"))
    return stats, rr


# ------------------------------------------------------- the workloads --
def test_ln_f32_64x1000_fwd_bwd(orc):
    w = synth.WORKLOADS["ln_f32_64x1000"]
    arr = synth.generate(w)
    check_ln_fwd(orc, arr, "f32", w.eps, tag=w.name)
    check_bwd(orc, arr, "f32", w.eps, layernorm=True, tag=w.name)


@pytest.mark.parametrize("op", ["ln", "rms"])
def test_fwd_bf16_8192x1024(orc, op):
    w = synth.WORKLOADS["fwd_bf16_8192x1024"]
    arr = synth.generate(w)
    if op == "ln":
        y, mean, rstd, _ = check_ln_fwd(orc, arr, "bf16", w.eps, use_beta=False,
                                        tag=w.name)
        # rows [N/2, N) are exactly 50.0 after rounding: zero variance,
        # y = beta = 0, mean = 50, rstd = 1/sqrt(eps) (in float32)
        lo = w.N // 2
        assert np.all(host(y)[lo:] == 0)
        assert np.all(host(mean)[lo:] == 50.0)
        want = np.float32(1.0) / np.sqrt(np.float32(w.eps))
        assert np.allclose(host(rstd)[lo:], want, rtol=1e-6)
    else:
        check_rms_fwd(orc, arr, "bf16", w.eps, tag=w.name)


def test_fused_bf16_32768x4096(orc):
    w = synth.WORKLOADS["fused_bf16_32768x4096"]
    arr = synth.generate(w)
    x = to_dev(arr["x"])
    r = to_dev(arr["residual"])
    g = to_dev(arr["gamma"])
    y, h, rstd = rn.fused_add_rms_fwd(x, r, g, w.eps)
    torch.cuda.synchronize()
    # h: every element, bit-exact
    h_exact = orc.decode(arr["x"], "bf16") + orc.decode(arr["residual"], "bf16")
    assert np.array_equal(host(h), orc.bf16_encode(h_exact)), "h not RNE(x + r)"
    del h_exact
    y_o, h_o, r_o = orc.fused_add_rms_fwd(
        orc.decode(arr["x"], "bf16"), orc.decode(arr["residual"], "bf16"),
        orc.decode(arr["gamma"], "bf16"), oracle.eps_at_boundary(w.eps))
    del h_o
    tol.check_bf16(host(y), y_o, orc, _lab(w.name, "fused y bf16"), strict=True)
    tol.check_rstd(host(rstd), r_o, _lab(w.name, "fused rstd"))


def test_fused_bwd_bf16_32768x4096(orc):
    w = synth.WORKLOADS["fused_bwd_bf16_32768x4096"]
    arr = synth.generate(w)
    check_fused_bwd(orc, arr, "bf16", w.eps, tag=w.name)


@pytest.mark.parametrize("name", ["mixed_bf16_f32w_32768x1024", "f16_32768x1024"])
def test_storage_workloads(orc, name):
    """Full-size runs of the float32-parameter and fp16 paths: every op,
    every row."""
    w = synth.WORKLOADS[name]
    arr = synth.generate(w)
    y, _, _, _ = check_ln_fwd(orc, arr, w.dtype, w.eps, tag=name)
    assert y.dtype == TORCH_DT[w.dtype]
    check_rms_fwd(orc, arr, w.dtype, w.eps, tag=name)
    check_bwd(orc, arr, w.dtype, w.eps, layernorm=True, tag=name)
    check_bwd(orc, arr, w.dtype, w.eps, layernorm=False, tag=name)
    check_fused_bwd(orc, arr, w.dtype, w.eps, tag=name)


def test_step_workload(orc):
    """The benchmark step's own inputs (32768 x 1024 bf16, with a residual):
    the five ops in the step's order, every row."""
    w = synth.WORKLOADS["step_bf16_32768x1024"]
    arr = synth.generate(w)
    check_ln_fwd(orc, arr, "bf16", w.eps, tag=w.name)
    check_rms_fwd(orc, arr, "bf16", w.eps, tag=w.name)
    x, r, g = (to_dev(arr[k]) for k in ("x", "residual", "gamma"))
    y, h, rstd = rn.fused_add_rms_fwd(x, r, g, 1e-6)
    torch.cuda.synchronize()
    y_o, h_o, r_o = orc.fused_add_rms_fwd(
        orc.decode(arr["x"], "bf16"), orc.decode(arr["residual"], "bf16"),
        orc.decode(arr["gamma"], "bf16"), oracle.eps_at_boundary(1e-6))
    assert np.array_equal(host(h), orc.bf16_encode(h_o)), "h not RNE(x + r)"
    del h_o
    tol.check_bf16(host(y), y_o, orc, _lab(w.name, "fused y bf16"), strict=True)
    tol.check_rstd(host(rstd), r_o, _lab(w.name, "fused rstd"))
    check_bwd(orc, arr, "bf16", w.eps, layernorm=True, tag=w.name)
    check_bwd(orc, arr, "bf16", w.eps, layernorm=False, tag=w.name)


# the named backward workloads, then the other shapes of the backward
# page's timing table (timed by the benchmark beside them)
BWD = ["bwd_bf16_32768x1024", "bwd_bf16_16384x2048", "bwd_bf16_512x16384",
       "bwd_bf16_2048x16384", "bwdtab_bf16_8192x1024", "bwdtab_bf16_16384x1024",
       "bwdtab_bf16_2048x4096", "bwdtab_bf16_4096x4096", "bwdtab_bf16_8192x4096",
       "bwdtab_bf16_1024x8192"]


@pytest.mark.parametrize("name", BWD)
@pytest.mark.parametrize("op", ["ln", "rms"])
def test_bwd_workloads(orc, name, op):
    w = synth.WORKLOADS[name]
    arr = synth.generate(w)
    if op == "ln":
        check_ln_fwd(orc, arr, "bf16", w.eps, tag=name)
    else:
        check_rms_fwd(orc, arr, "bf16", w.eps, tag=name)
    check_bwd(orc, arr, "bf16", w.eps, layernorm=(op == "ln"), tag=name)


# The benchmark's long-row shapes (rows past the register-resident plans):
# every element of the forward outputs and of dx, in the launch
# configuration the benchmark times.
LONG_W = [("long_bf16_2048x32768", "ln"), ("long_bf16_2048x32768", "rms"),
          ("long_bf16_2048x32768", "fused"), ("long_bf16_256x131072", "ln"),
          ("long_bf16_256x131072", "rms")]


@pytest.mark.parametrize("name,op", LONG_W)
def test_long_workloads(orc, name, op):
    w = synth.WORKLOADS[name]
    arr = synth.generate(w)
    if op == "fused":
        x, r, g = (to_dev(arr[k]) for k in ("x", "residual", "gamma"))
        y, h, rstd = rn.fused_add_rms_fwd(x, r, g, w.eps)
        torch.cuda.synchronize()
        y_o, h_o, r_o = orc.fused_add_rms_fwd(
            orc.decode(arr["x"], "bf16"), orc.decode(arr["residual"], "bf16"),
            orc.decode(arr["gamma"], "bf16"), oracle.eps_at_boundary(w.eps))
        assert np.array_equal(host(h), orc.bf16_encode(h_o)), "h not RNE(x + r)"
        del h_o
        tol.check_bf16(host(y), y_o, orc, _lab(name, "fused y bf16"), strict=True)
        tol.check_rstd(host(rstd), r_o, _lab(name, "fused rstd"))
        return
    if op == "ln":
        check_ln_fwd(orc, arr, "bf16", w.eps, tag=name)
    else:
        check_rms_fwd(orc, arr, "bf16", w.eps, tag=name)
    check_bwd(orc, arr, "bf16", w.eps, layernorm=(op == "ln"), tag=name)


# ------------------------------------------------------------ edge cases --
# The LayerNorm page's validation list (64 ... 2049) plus tiny rows, ragged
# tails, element-wise-path shapes and the largest rows.
# Row lengths that fill a plan's span exactly (64 ... 16384: no masking) and
# ragged ones (masked tails, element-wise plans; 4097 and 6002 take the
# row-major partial rows with a length that is not a multiple of 4).
SHAPES = [64, 128, 256, 512, 768, 1024, 2048, 2049, 1, 2, 3, 1000, 3000, 4095,
          4096, 4097, 6002, 8192, 12288, 16384]


# storage pairs: activations[/parameters]
STORAGE = ["bf16", "f32", "f16", "bf16/f32", "f16/f32"]


def check_all_ops(orc, arr, dtype):
    """Every op on one input set: LN and RMS forward and backward, the fused
    forward (h bit-exact) and the fused backward."""
    check_ln_fwd(orc, arr, dtype, 1e-5)
    check_rms_fwd(orc, arr, dtype, 1e-5)
    check_bwd(orc, arr, dtype, 1e-5, layernorm=True)
    check_bwd(orc, arr, dtype, 1e-5, layernorm=False)
    x, r, g = (to_dev(arr[k], dtype) for k in ("x", "residual", "gamma"))
    y, h, rstd = rn.fused_add_rms_fwd(x, r, g, 1e-6)
    torch.cuda.synchronize()
    xd, rd = orc.decode(arr["x"], dtype), orc.decode(arr["residual"], dtype)
    y_o, h_o, r_o = orc.fused_add_rms_fwd(xd, rd, dec(orc, arr, "gamma", dtype),
                                          oracle.eps_at_boundary(1e-6))
    assert np.array_equal(host(h), orc.encode(h_o, dtype))
    tol.check_out(host(y), y_o, dtype, orc, f"edge: fused y {dtype}", strict=True)
    tol.check_rstd(host(rstd), r_o, "edge: fused rstd")
    check_fused_bwd(orc, arr, dtype, 1e-6)


@pytest.mark.parametrize("storage", STORAGE)
@pytest.mark.parametrize("H", SHAPES)
def test_shapes_all_ops(orc, storage, H):
    N = 67 if H <= 4096 else 19
    dtype, _, wdt = storage.partition("/")
    arr = synth.custom(100 + H, N, H, dtype, wdtype=wdt or None)
    check_all_ops(orc, arr, dtype)


def _sweep_cases(n=120, seed=20261202):
    """(N, H, storage) drawn log-uniformly: H in [1, 140000] (every plan, the
    segment and long-row kernels, masked tails and the element-wise path),
    N in [1, 4000] with N*H at most about 3 M elements (the persistent
    grids' rounds, the few-row plans and the one-workgroup backward)."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        H = max(1, int(np.exp(rng.uniform(0.0, np.log(140000.0)))))
        N = max(1, int(np.exp(rng.uniform(0.0, np.log(4000.0)))))
        N = min(N, max(1, (3 << 20) // H))
        out.append((N, H, STORAGE[int(rng.integers(len(STORAGE)))]))
    return out


# A seeded sweep of shapes and storage pairs that no list above was written
# for, every op against the oracle.
@pytest.mark.parametrize("case", list(enumerate(_sweep_cases())),
                         ids=lambda c: f"{c[0]}-{c[1][0]}x{c[1][1]}-{c[1][2]}")
def test_shape_sweep(orc, case):
    i, (N, H, storage) = case
    dtype, _, wdt = storage.partition("/")
    arr = synth.custom(5000 + i, N, H, dtype, wdtype=wdt or None)
    check_all_ops(orc, arr, dtype)


# Short rows, several per wave: every segment width (8, 16, 32 lanes) on the
# 16-byte path and the element-wise path, ragged in N against the rows a
# workgroup holds.
SHORT = [8, 16, 24, 32, 40, 56, 96, 136, 200, 256, 5, 7, 17, 31, 33, 63]


@pytest.mark.parametrize("storage", ["bf16", "f32", "f16/f32"])
@pytest.mark.parametrize("H", SHORT)
def test_short_rows(orc, storage, H):
    dtype, _, wdt = storage.partition("/")
    arr = synth.custom(300 + H, 333, H, dtype, wdtype=wdt or None)
    check_ln_fwd(orc, arr, dtype, 1e-5)
    check_rms_fwd(orc, arr, dtype, 1e-5)
    check_bwd(orc, arr, dtype, 1e-5, layernorm=True)
    check_bwd(orc, arr, dtype, 1e-5, layernorm=False)
    check_fused_bwd(orc, arr, dtype, 1e-6)


# Short rows in numbers that make every wave of the persistent backward grid
# take several row groups, ending on a ragged group: the row group after a
# wave's last one is requested too, and must read nothing and change nothing.
@pytest.mark.parametrize("storage,H", [("bf16", 24), ("bf16", 128), ("bf16", 200),
                                       ("f32", 40), ("f16/f32", 7)])
def test_short_rows_persistent_tail(orc, storage, H):
    dtype, _, wdt = storage.partition("/")
    arr = synth.custom(700 + H, 150001, H, dtype, wdtype=wdt or None)
    check_bwd(orc, arr, dtype, 1e-5, layernorm=True)
    check_bwd(orc, arr, dtype, 1e-5, layernorm=False)
    check_fused_bwd(orc, arr, dtype, 1e-6)


def test_qk_norm_bf16_1048576x128(orc):
    """Head-dimension rows (a million rows of 128), every row."""
    w = synth.WORKLOADS["rows_bf16_1048576x128"]
    arr = synth.generate(w)
    check_ln_fwd(orc, arr, "bf16", w.eps, tag=w.name)
    check_rms_fwd(orc, arr, "bf16", w.eps, tag=w.name)
    check_bwd(orc, arr, "bf16", w.eps, layernorm=True, tag=w.name)
    check_bwd(orc, arr, "bf16", w.eps, layernorm=False, tag=w.name)


# Rows whose mean dwarfs their spread, on single-wave rows (1024) and on
# rows split over 4 and 16 waves (4096, 16384), where each wave shifts by its
# own first element and the waves' means meet relative to wave 0's.
@pytest.mark.parametrize("H", [1024, 4096, 16384])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_small_variance_rows(orc, dtype, H):
    # rows with |mean|/sigma = 50, and constant rows
    N = 40
    arr = synth.custom(5, N, H, dtype, x=(0.0, 1.0), half_shifted=(2.0, 0.04))
    check_ln_fwd(orc, arr, dtype, 1e-5)
    check_bwd(orc, arr, dtype, 1e-5, layernorm=True)
    c = arr["x"].copy()
    c[:] = c[0, 0]      # every row constant
    arr2 = dict(arr, x=c)
    y, mean, rstd, _ = check_ln_fwd(orc, arr2, dtype, 1e-5)
    assert np.all(orc.decode(host(y), dtype) == orc.decode(arr["beta"], dtype)[None, :])
    if dtype == "f32":
        # |mean|/sigma = 2e4: x - mean formed against a float32 mean of 1000
        # would be off by ~1e-3 relative; the pivot shift keeps it exact
        arr3 = synth.custom(6, N, H, dtype, x=(1000.0, 0.05))
        check_ln_fwd(orc, arr3, dtype, 1e-5)


# (H, pad): every plan family; the element-wise path (pad 3) ends at 8192
STRIDED = [(H, pad) for H in (1024, 128, 40, 24, 4096) for pad in (24, 3)] + \
          [(8192, 24), (16384, 24), (16384, 40)]


def check_strided(orc, dtype, pad, H, N=33, seed=11):
    """Rows at stride H + pad: LN and RMS forward and backward and the fused
    forward leave the padding between rows and a guard row after the last
    row untouched, and match the oracle."""
    arr = synth.custom(seed, N, H, dtype)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    SENT = -7.0

    def buf(a=None):
        t = torch.full((N + 1, H + pad), SENT, dtype=tdt, device=DEV)
        if a is not None:
            t[:N, :H] = to_dev(a)
        return t

    def view(t):
        return t.as_strided((N, H), (H + pad, 1))

    X, DY, R = buf(arr["x"]), buf(arr["dy"]), buf(arr["residual"])
    Y, DX, HH, Y2, Y3, DX3 = buf(), buf(), buf(), buf(), buf(), buf()
    g, b = to_dev(arr["gamma"]), to_dev(arr["beta"])
    _, mean, rstd = rn.ln_fwd(view(X), g, b, 1e-5, y=view(Y))
    rn.ln_bwd(view(DY), view(X), g, mean, rstd, 1e-5, dx=view(DX))
    rn.fused_add_rms_fwd(view(X), view(R), g, 1e-6, y=view(Y2), h=view(HH))
    _, rstd3 = rn.rms_fwd(view(X), g, 1e-5, y=view(Y3))
    _, dg3 = rn.rms_bwd(view(DY), view(X), g, rstd3, 1e-5, dx=view(DX3))
    torch.cuda.synchronize()
    for t, name in ((Y, "y"), (DX, "dx"), (HH, "h"), (Y2, "fused y"), (Y3, "RMS y"),
                    (DX3, "RMS dx")):
        hb = t.float().cpu().numpy()
        assert np.all(hb[:N, H:] == SENT), f"{name}: row padding written"
        assert np.all(hb[N, :] == SENT), f"{name}: guard row written"
    e = oracle.eps_at_boundary(1e-5)
    xd = orc.decode(arr["x"], dtype)
    gd, bd = orc.decode(arr["gamma"], dtype), orc.decode(arr["beta"], dtype)
    y_o, _, _ = orc.ln_fwd(xd, gd, bd, e)
    tol.check_out(host(Y[:N, :H].contiguous()), y_o, dtype, orc, f"edge: strided LN y {dtype}")
    dyd = orc.decode(arr["dy"], dtype)
    dx_o, _, _, _, r_o = orc.ln_bwd(dyd, xd, gd, e)
    tol.check_out(host(DX[:N, :H].contiguous()), dx_o, dtype, orc, f"edge: strided dx {dtype}",
                  term_scale=tol.dx_term_scale(dyd, gd, r_o))
    h_o = xd + orc.decode(arr["residual"], dtype)
    assert np.array_equal(host(HH[:N, :H].contiguous()), orc.encode(h_o, dtype))
    y3_o, _ = orc.rms_fwd(xd, gd, e)
    tol.check_out(host(Y3[:N, :H].contiguous()), y3_o, dtype, orc,
                  f"edge: strided RMS y {dtype}", strict=True)
    dx3_o, dg3_o, r3_o = orc.rms_bwd(dyd, xd, gd, e)
    tol.check_out(host(DX3[:N, :H].contiguous()), dx3_o, dtype, orc,
                  f"edge: strided RMS dx {dtype}", term_scale=tol.dx_term_scale(dyd, gd, r3_o))
    tol.check_param(orc.decode(host(dg3), dtype), dg3_o, "edge: strided RMS dgamma")


@pytest.mark.parametrize("H,pad", STRIDED)
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_strided_rows_and_canaries(orc, dtype, pad, H):
    """Row strides > H (pad 24 or 40 keeps 16-byte rows, pad 3 forces the
    element-wise path).  Short rows run several rows per wave, addressed
    through one range per row group; 16384 runs the persistent plan, whose
    ring reads rows past N from empty ranges."""
    check_strided(orc, dtype, pad, H)


def _strided_cases(n=40, seed=7702):
    """(N, H, pad, dtype): H log-uniform in [1, 70000], pads that keep or
    break 16-byte rows, N up to 600 (about 2 M elements at most)."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        H = max(1, int(np.exp(rng.uniform(0.0, np.log(70000.0)))))
        N = max(1, int(np.exp(rng.uniform(0.0, np.log(600.0)))))
        N = min(N, max(1, (2 << 20) // H))
        pad = int(rng.choice([1, 3, 8, 24, 40, 129]))
        out.append((N, H, pad, ["bf16", "f32"][int(rng.integers(2))]))
    return out


@pytest.mark.parametrize("case", list(enumerate(_strided_cases())),
                         ids=lambda c: f"{c[0]}-{c[1][0]}x{c[1][1]}+{c[1][2]}-{c[1][3]}")
def test_strided_sweep(orc, case):
    i, (N, H, pad, dtype) = case
    check_strided(orc, dtype, pad, H, N=N, seed=6000 + i)


@pytest.mark.parametrize("alias", ["x", "residual"])
def test_fused_in_place(orc, alias):
    N, H = 129, 4096
    arr = synth.custom(12, N, H, "bf16")
    x, r, g = (to_dev(arr[k]) for k in ("x", "residual", "gamma"))
    target = x if alias == "x" else r
    y, h, _ = rn.fused_add_rms_fwd(x, r, g, 1e-6, h=target)
    torch.cuda.synchronize()
    assert h.data_ptr() == target.data_ptr()
    xd, rd = orc.decode(arr["x"], "bf16"), orc.decode(arr["residual"], "bf16")
    y_o, h_o, _ = orc.fused_add_rms_fwd(xd, rd, orc.decode(arr["gamma"], "bf16"),
                                        oracle.eps_at_boundary(1e-6))
    assert np.array_equal(host(target), orc.bf16_encode(h_o))
    tol.check_bf16(host(y), y_o, orc, "edge: in-place fused y bf16", strict=True)


@pytest.mark.parametrize("with_dh,write_dres,in_place", [
    (True, True, False), (True, False, False), (False, True, False),
    (False, False, False), (True, True, True), (True, False, True)])
@pytest.mark.parametrize("N,H", [(129, 4096), (300, 16384), (2051, 1000)])
def test_fused_bwd_variants(orc, N, H, with_dh, write_dres, in_place):
    """With and without the residual-stream gradient, one or two outputs,
    dx accumulated in place over dh_in; a short-wide shape (column sums),
    and H = 1000 (element-wise path)."""
    arr = synth.custom(16 + H, N, H, "bf16")
    check_fused_bwd(orc, arr, "bf16", 1e-6, with_dh=with_dh,
                    write_dres=write_dres, in_place=in_place)


@pytest.mark.parametrize("pad", [24, 3])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_fused_bwd_strided(orc, dtype, pad):
    """Fused backward with every row tensor at stride H + pad: padding and a
    guard row after the last row stay untouched."""
    N, H = 33, 2048
    arr = synth.custom(17, N, H, dtype)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    SENT = -7.0

    def buf(a=None):
        t = torch.full((N + 1, H + pad), SENT, dtype=tdt, device=DEV)
        if a is not None:
            t[:N, :H] = to_dev(a)
        return t

    def view(t):
        return t.as_strided((N, H), (H + pad, 1))

    X, R, DY, DH = (buf(arr[k]) for k in ("x", "residual", "dy", "dh"))
    HH, Y, DX, DR = buf(), buf(), buf(), buf()
    g = to_dev(arr["gamma"])
    _, _, rstd = rn.fused_add_rms_fwd(view(X), view(R), g, 1e-6, y=view(Y),
                                      h=view(HH))
    rn.fused_add_rms_bwd(view(DY), view(HH), g, rstd, 1e-6, dh_in=view(DH),
                         dx=view(DX), dres=view(DR))
    torch.cuda.synchronize()
    for t, name in ((DX, "dx"), (DR, "dres")):
        hb = t.float().cpu().numpy()
        assert np.all(hb[:N, H:] == SENT), f"{name}: row padding written"
        assert np.all(hb[N, :] == SENT), f"{name}: guard row written"
    dx_o, _, ts, _ = fused_bwd_oracle(orc, arr, dtype, 1e-6)
    tol.check_out(host(DX[:N, :H].contiguous()), dx_o, dtype, orc,
                  f"edge: strided fused dx {dtype}", term_scale=ts)
    assert torch.equal(DX, DR)


# (4099, 16384) reduces through partial rows, (300, 16384) through column
# sums of the rows (too few rows for partial rows to pay off).
@pytest.mark.parametrize("N,H", [(4099, 1024), (4099, 16384), (300, 16384)])
def test_bitwise_deterministic(N, H):
    arr = synth.custom(13, N, H, "bf16")
    x, dy, g, b = (to_dev(arr[k]) for k in ("x", "dy", "gamma", "beta"))
    outs = []
    for _ in range(2):
        y, mean, rstd = rn.ln_fwd(x, g, b, 1e-5)
        dx, dg, db = rn.ln_bwd(dy, x, g, mean, rstd, 1e-5)
        _, rs2 = rn.rms_fwd(x, g, 1e-5)
        dx2, dg2 = rn.rms_bwd(dy, x, g, rs2, 1e-5)
        dx3, _, dg3 = rn.fused_add_rms_bwd(dy, x, g, rs2, 1e-5, dh_in=dy)
        torch.cuda.synchronize()
        outs.append([t.clone() for t in (y, mean, rstd, dx, dg, db, dx2, dg2,
                                         dx3, dg3)])
    for a, b_ in zip(*outs):
        assert torch.equal(a, b_)


# Tall shapes on the one-workgroup-per-CU team plans (H 1024/2048/4096:
# 8/4/2 rows per team step; N ragged), and wide rows.
@pytest.mark.parametrize("N,H", [(32771, 1024), (12293, 2048), (6151, 4096),
                                 (1000, 16384)])
def test_workspace_contents_on_entry(orc, N, H):
    """Whatever the workspace holds on entry (zeros, all-ones bytes, 0xFE
    bytes, random bytes, what this call or a call of another shape left),
    the backward gives the same bits, and they match the oracle."""
    arr = synth.custom(31 + H, N, H, "bf16")
    x, dy, g, dh = (to_dev(arr[k]) for k in ("x", "dy", "gamma", "dh"))
    bf = torch.bfloat16
    ws = torch.empty(max(rn.workspace_bytes(N, H, bf, True),
                         rn.workspace_bytes(N, H, bf, False)), dtype=torch.uint8, device=DEV)
    _, mean, rstd = rn.ln_fwd(x, g, None, 1e-5)
    _, rs2 = rn.rms_fwd(x, g, 1e-5)

    def run():
        dx, dg, db = rn.ln_bwd(dy, x, g, mean, rstd, 1e-5, workspace=ws)
        dx2, dg2 = rn.rms_bwd(dy, x, g, rs2, 1e-5, workspace=ws)
        dx3, _, dg3 = rn.fused_add_rms_bwd(dy, x, g, rs2, 1e-5, dh_in=dh, workspace=ws)
        torch.cuda.synchronize()
        return [t.clone() for t in (dx, dg, db, dx2, dg2, dx3, dg3)]

    gen = torch.Generator(device="cpu").manual_seed(5)
    rand = torch.randint(0, 256, (ws.numel(),), dtype=torch.uint8, generator=gen)
    ws.zero_()
    want = run()
    # the first result against the oracle (LayerNorm: dx rows, dgamma, dbeta)
    e = oracle.eps_at_boundary(1e-5)
    xd, dyd, gd = (orc.decode(arr[k], "bf16") for k in ("x", "dy", "gamma"))
    dx_o, dg_o, db_o, _, rstd_o = orc.ln_bwd(dyd, xd, gd, e)
    tol.check_out(host(want[0]), dx_o, "bf16", orc, "edge: workspace states LN dx",
                  term_scale=tol.dx_term_scale(dyd, gd, rstd_o))
    tol.check_param(orc.decode(host(want[1]), "bf16"), dg_o, "edge: workspace states dgamma")
    tol.check_param(orc.decode(host(want[2]), "bf16"), db_o, "edge: workspace states dbeta")
    _, dg_r, _ = orc.rms_bwd(dyd, xd, gd, e)
    tol.check_param(orc.decode(host(want[4]), "bf16"), dg_r, "edge: workspace states RMS dgamma")

    states = {"reused": None, "ones": 0xFF, "fe": 0xFE, "random": rand}
    for name, fill in states.items():
        if isinstance(fill, int):
            ws.fill_(fill)
        elif fill is not None:
            ws.copy_(fill.to(DEV))
        got = run()
        for a, b in zip(want, got):
            assert torch.equal(a, b), f"workspace state {name!r} changed the result"
    # a call of another shape on the same workspace, then this one again
    n2 = N // 2 + 3
    rn.rms_bwd(dy[:n2], x[:n2], g, rs2[:n2], 1e-5, workspace=ws)
    for a, b in zip(want, run()):
        assert torch.equal(a, b), "a call of another shape changed the result"


# Wide rows at ragged row counts: row lengths that leave the last 2048-column
# blocks empty (9000, 12288), fp16, and fp32 parameters.
WIDE = [(1001, 16384, "bf16"), (37, 9000, "bf16"), (300, 12288, "f16"),
        (513, 16384, "bf16/f32"), (600, 16384, "f32")]


@pytest.mark.parametrize("N,H,storage", WIDE)
def test_wide_rows(orc, N, H, storage):
    """LN, RMS and fused forward and backward against the oracle, and bit for
    bit the same run to run.  On the persistent 16384 plan, 1001, 600 and
    513 rows give each workgroup 2-4 rows: whole turns of its prefetch ring
    (four buffers for 2-byte rows, two for float32) and every remainder."""
    dtype, _, wdt = storage.partition("/")
    arr = synth.custom(60 + N, N, H, dtype, wdtype=wdt or None)
    check_ln_fwd(orc, arr, dtype, 1e-5)
    check_rms_fwd(orc, arr, dtype, 1e-5)
    xf, rf, gf = (to_dev(arr[k], dtype) for k in ("x", "residual", "gamma"))
    yf, hf, rsf = rn.fused_add_rms_fwd(xf, rf, gf, 1e-5)
    torch.cuda.synchronize()
    y_o, h_o, r_o = orc.fused_add_rms_fwd(
        orc.decode(arr["x"], dtype), orc.decode(arr["residual"], dtype),
        dec(orc, arr, "gamma", dtype), oracle.eps_at_boundary(1e-5))
    assert np.array_equal(host(hf), orc.encode(h_o, dtype)), "h not RNE(x + r)"
    tol.check_out(host(yf), y_o, dtype, orc, f"edge: fused y {dtype}", strict=True)
    tol.check_rstd(host(rsf), r_o, "edge: fused rstd")
    check_bwd(orc, arr, dtype, 1e-5, layernorm=True)
    check_bwd(orc, arr, dtype, 1e-5, layernorm=False)
    check_fused_bwd(orc, arr, dtype, 1e-5)
    x, dy, g, dh = (to_dev(arr[k], dtype) for k in ("x", "dy", "gamma", "dh"))

    def run():
        _, mean, rstd = rn.ln_fwd(x, g, None, 1e-5)
        _, rs2 = rn.rms_fwd(x, g, 1e-5)
        dx, dg, db = rn.ln_bwd(dy, x, g, mean, rstd, 1e-5)
        dx2, dg2 = rn.rms_bwd(dy, x, g, rs2, 1e-5)
        dx3, dr3, dg3 = rn.fused_add_rms_bwd(dy, x, g, rs2, 1e-5, dh_in=dh,
                                             write_dres=True)
        torch.cuda.synchronize()
        return [t.clone() for t in (dx, dg, db, dx2, dg2, dx3, dr3, dg3)]

    for a_, b_ in zip(run(), run()):
        assert torch.equal(a_, b_), "not reproducible run to run"


def test_tensors_past_4gib(orc):
    """Row tensors of more than 4 GiB: 2^21 + 5 rows of 1024 bf16, so the
    byte offset of every row from 2^21 on is at or past 2^32.  Every op runs
    once at that size (inputs drawn on the GPU, seeded: synth.device_normal).
    y, h, mean, rstd and dx of rows on both sides of the 2^32-byte mark and
    of the last rows are compared with the oracle (each row's outputs depend
    on that row alone).  dbeta and dgamma, which sum every row, are checked
    against their definitions evaluated in float64 over all rows: dbeta =
    the column sums of dy, dgamma = the column sums of dy * (x - mean) * rstd
    with the saved statistics (float32 parameters, so the sums come back
    unrounded)."""
    N, H = (1 << 21) + 5, 1024
    assert (1 << 21) * H * 2 == 1 << 32
    bf = torch.bfloat16
    x = synth.device_normal(7001, (N, H), 0.0, 1.0, "bf16", DEV)
    r = synth.device_normal(7002, (N, H), 0.0, 1.0, "bf16", DEV)
    dy = synth.device_normal(7003, (N, H), 0.0, 1.0, "bf16", DEV)
    g = synth.device_normal(7004, (H,), 1.0, 0.1, "f32", DEV)
    b = synth.device_normal(7005, (H,), 0.0, 0.1, "f32", DEV)
    rows = [0, 1, 1 << 20, (1 << 21) - 1, 1 << 21, (1 << 21) + 1, N - 2, N - 1]
    e = oracle.eps_at_boundary(1e-5)
    gd = host(g).astype(np.float64)
    bd = host(b).astype(np.float64)

    def rows_of(t):
        return host(t[rows].contiguous())

    xd = orc.decode(rows_of(x), "bf16")
    rd = orc.decode(rows_of(r), "bf16")
    dyd = orc.decode(rows_of(dy), "bf16")

    y, mean, rstd = rn.ln_fwd(x, g, b, 1e-5)
    torch.cuda.synchronize()
    y_o, m_o, r_o = orc.ln_fwd(xd, gd, bd, e)
    tol.check_out(rows_of(y), y_o, "bf16", orc, "edge: past 4 GiB LN y")
    tol.check_mean(host(mean[rows]), m_o, 1.0 / (r_o * r_o) - e, e, "edge: past 4 GiB LN mean")
    tol.check_rstd(host(rstd[rows]), r_o, "edge: past 4 GiB LN rstd")
    dx, dg, db = rn.ln_bwd(dy, x, g, mean, rstd, 1e-5)
    torch.cuda.synchronize()
    dx_o, _, _, _, rs_o = orc.ln_bwd(dyd, xd, gd, e)
    tol.check_out(rows_of(dx), dx_o, "bf16", orc, "edge: past 4 GiB LN dx",
                  term_scale=tol.dx_term_scale(dyd, gd, rs_o))
    # dgamma / dbeta against their definitions over all rows, in float64
    want_dg = torch.zeros(H, dtype=torch.float64, device=DEV)
    want_db = torch.zeros(H, dtype=torch.float64, device=DEV)
    for r0 in range(0, N, 1 << 18):
        sl = slice(r0, min(r0 + (1 << 18), N))
        d64 = dy[sl].double()
        xh = (x[sl].double() - mean[sl].double()[:, None]) * rstd[sl].double()[:, None]
        want_dg += (d64 * xh).sum(0)
        want_db += d64.sum(0)
        del d64, xh
    tol.check_param(host(dg).astype(np.float64), host(want_dg), "edge: past 4 GiB dgamma")
    tol.check_param(host(db).astype(np.float64), host(want_db), "edge: past 4 GiB dbeta")
    del dx, y

    y2, rs2 = rn.rms_fwd(x, g, 1e-5)
    torch.cuda.synchronize()
    y_o, r_o = orc.rms_fwd(xd, gd, e)
    tol.check_out(rows_of(y2), y_o, "bf16", orc, "edge: past 4 GiB RMS y", strict=True)
    tol.check_rstd(host(rs2[rows]), r_o, "edge: past 4 GiB RMS rstd")
    dx2, dg2 = rn.rms_bwd(dy, x, g, rs2, 1e-5)
    torch.cuda.synchronize()
    dx_o, _, rs_o = orc.rms_bwd(dyd, xd, gd, e)
    tol.check_out(rows_of(dx2), dx_o, "bf16", orc, "edge: past 4 GiB RMS dx",
                  term_scale=tol.dx_term_scale(dyd, gd, rs_o))
    want_dg.zero_()
    for r0 in range(0, N, 1 << 18):
        sl = slice(r0, min(r0 + (1 << 18), N))
        want_dg += (dy[sl].double() * (x[sl].double() * rs2[sl].double()[:, None])).sum(0)
    tol.check_param(host(dg2).astype(np.float64), host(want_dg), "edge: past 4 GiB RMS dgamma")
    del dx2, y2

    y3, h3, rs3 = rn.fused_add_rms_fwd(x, r, g, 1e-5)
    torch.cuda.synchronize()
    y_o, h_o, r_o = orc.fused_add_rms_fwd(xd, rd, gd, e)
    assert np.array_equal(rows_of(h3), orc.encode(h_o, "bf16")), "h not RNE(x + r)"
    tol.check_out(rows_of(y3), y_o, "bf16", orc, "edge: past 4 GiB fused y", strict=True)
    tol.check_rstd(host(rs3[rows]), r_o, "edge: past 4 GiB fused rstd")


def test_partial_rows_query():
    """rn_bwd_partial_rows agrees with the workspace the backward asks for:
    P partial rows per parameter fit in it (P rounded up to 8 slots), none
    when the workspace is empty; the tall shapes use a bounded P that does
    not grow with N, the 512 x 16384 LayerNorm the column sums."""
    bf = torch.bfloat16
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for N, H in [(32768, 1024), (16384, 2048), (2048, 16384), (512, 16384),
                 (1048576, 128), (65536, 1024), (4, 4096), (600, 20480)]:
        for ln in (True, False):
            p = rn.bwd_partial_rows(N, H, bf, ln)
            ws = rn.workspace_bytes(N, H, bf, ln)
            need = ((p + 7) // 8 * 8) * H * 4 * (2 if ln else 1)
            assert need <= ws, (N, H, ln, p, ws)
            assert (p == 0) == (ws == 0) or p == 0, (N, H, ln, p, ws)
            assert p <= 16 * cus, (N, H, ln, p)
    assert rn.bwd_partial_rows(32768, 1024, bf, True) == rn.bwd_partial_rows(65536, 1024, bf, True)
    assert rn.bwd_partial_rows(512, 16384, bf, True) == 0


@pytest.mark.parametrize("N", [0, 1, 2, 7, 255, 513])
def test_row_counts(orc, N):
    """N = 0 (no rows: dgamma = dbeta = 0), N below the partial-row count,
    and N just above it."""
    H = 1024
    if N == 0:
        x = torch.empty((0, H), dtype=torch.bfloat16, device=DEV)
        g = torch.ones(H, dtype=torch.bfloat16, device=DEV)
        y, mean, rstd = rn.ln_fwd(x, g, None, 1e-5)
        dg = torch.full((H,), 3.0, dtype=torch.bfloat16, device=DEV)
        db = torch.full((H,), 3.0, dtype=torch.bfloat16, device=DEV)
        rn.ln_bwd(x, x, g, mean, rstd, 1e-5, dgamma=dg, dbeta=db)
        _, _, dg2 = rn.fused_add_rms_bwd(x, x, g, rstd, 1e-5, dh_in=x)
        torch.cuda.synchronize()
        assert torch.all(dg == 0) and torch.all(db == 0)
        assert torch.all(dg2 == 0)
        return
    arr = synth.custom(14 + N, N, H, "bf16")
    check_ln_fwd(orc, arr, "bf16", 1e-5)
    check_bwd(orc, arr, "bf16", 1e-5, layernorm=True)
    check_bwd(orc, arr, "bf16", 1e-5, layernorm=False)
    check_fused_bwd(orc, arr, "bf16", 1e-5)


@pytest.mark.parametrize("N", [1, 8, 9, 16, 64])
def test_decode_sizes(orc, N):
    """Few rows at H = 4096: N <= 8 runs the backward as one workgroup that
    writes dgamma/dbeta itself (one launch), N = 9 just past it, 16 and 64
    two launches; LN, RMS and fused backward against the oracle."""
    arr = synth.custom(500 + N, N, 4096, "bf16")
    check_ln_fwd(orc, arr, "bf16", 1e-5)
    check_bwd(orc, arr, "bf16", 1e-5, layernorm=True)
    check_bwd(orc, arr, "bf16", 1e-5, layernorm=False)
    check_fused_bwd(orc, arr, "bf16", 1e-6)
    if N <= 4:
        # one workgroup on the 16-byte and the element-wise plans alike (the
        # query sizes for both): no workspace at all
        assert rn.workspace_bytes(N, 4096, torch.bfloat16, True) == 0
    if N <= 8:
        # one workgroup on the 16-byte plan: the call needs no workspace
        x, dy, g = (to_dev(arr[k]) for k in ("x", "dy", "gamma"))
        _, mean, rstd = rn.ln_fwd(x, g, None, 1e-5)
        empty = torch.empty(0, dtype=torch.uint8, device=DEV)
        dx, dg, db = rn.ln_bwd(dy, x, g, mean, rstd, 1e-5, workspace=empty)
        dx2, dg2, db2 = rn.ln_bwd(dy, x, g, mean, rstd, 1e-5)
        torch.cuda.synchronize()
        assert torch.equal(dx, dx2) and torch.equal(dg, dg2) and torch.equal(db, db2)


def test_many_short_rows(orc):
    """Persistent loops with many iterations per workgroup."""
    N, H = 200003, 64
    arr = synth.custom(15, N, H, "bf16")
    check_ln_fwd(orc, arr, "bf16", 1e-5)
    check_rms_fwd(orc, arr, "bf16", 1e-5)
    check_bwd(orc, arr, "bf16", 1e-5, layernorm=True)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("n,off", [(1000003, 0), (4096, 0), (777, 1)])
def test_add_helper(orc, dtype, n, off):
    """The unfused baseline's add: RNE(a + b) bit-exact, on the 16-byte path
    with a tail and element by element (offset views)."""
    arr = synth.custom(18, 1, n + off, dtype)
    a = to_dev(arr["x"], dtype)[0, off:]
    b = to_dev(arr["residual"], dtype)[0, off:]
    out = rn.add(a, b)
    torch.cuda.synchronize()
    want = orc.encode(orc.decode(arr["x"][0, off:], dtype) +
                      orc.decode(arr["residual"][0, off:], dtype), dtype)
    assert np.array_equal(host(out), want)
    rn.add(a, b, out=a)      # in place over a
    torch.cuda.synchronize()
    assert np.array_equal(host(a), want)


@pytest.mark.parametrize("N,H", [(64, 4096), (1, 8192), (333, 128), (16389, 1024),
                                 (300, 16384)])
def test_graph_capture_replays(N, H):
    """The entry points enqueue only kernels on the caller's stream, so a HIP
    graph can capture them: fused forward + fused backward + LayerNorm
    forward/backward captured once and replayed four times, with eager work
    and synchronizations between replays; every replay must reproduce the
    eager results bit for bit; (16389, 1024) is a tall ragged shape on a
    persistent team plan, (300, 16384) a wide one."""
    arr = synth.custom(19, N, H, "bf16")
    x, r, g, b, dy, dh = (to_dev(arr[k]) for k in ("x", "residual", "gamma", "beta",
                                                   "dy", "dh"))
    bf = torch.bfloat16
    y, hh, dx, dx2, y2 = (torch.empty((N, H), dtype=bf, device=DEV) for _ in range(5))
    rstd, mean, rstd2 = (torch.empty(N, dtype=torch.float32, device=DEV) for _ in range(3))
    dg, dg2, db2 = (torch.empty(H, dtype=bf, device=DEV) for _ in range(3))
    # one workspace for both backward ops (LayerNorm may need none where
    # RMSNorm needs partial rows)
    ws = torch.empty(max(1, rn.workspace_bytes(N, H, bf, True),
                         rn.workspace_bytes(N, H, bf, False)), dtype=torch.uint8, device=DEV)

    def step():
        rn.fused_add_rms_fwd(x, r, g, 1e-6, y=y, h=hh, rstd=rstd)
        rn.fused_add_rms_bwd(dy, hh, g, rstd, 1e-6, dh_in=dh, dx=dx, dgamma=dg,
                             workspace=ws)
        rn.ln_fwd(x, g, b, 1e-5, y=y2, mean=mean, rstd=rstd2)
        rn.ln_bwd(dy, x, g, mean, rstd2, 1e-5, dx=dx2, dgamma=dg2, dbeta=db2,
                  workspace=ws)

    outs = (y, hh, rstd, dx, dg, y2, mean, rstd2, dx2, dg2, db2)
    step()
    torch.cuda.synchronize()
    want = [t.clone() for t in outs]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        for t in outs:
            t.fill_(7.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for t, w_ in zip(outs, want):
            assert torch.equal(t, w_), f"replay {rep} differs from eager"


def test_two_streams_at_once(orc):
    """Backward calls on two streams at once, each with its own workspace
    (the library keeps no per-call state): both results equal the same calls
    made one after the other, and the first matches the oracle."""
    shapes = [(32771, 1024), (4099, 4096)]
    arrs = [synth.custom(600 + i, N, H, "bf16") for i, (N, H) in enumerate(shapes)]
    ins = []
    for a in arrs:
        x, dy, g = (to_dev(a[k]) for k in ("x", "dy", "gamma"))
        _, mean, rstd = rn.ln_fwd(x, g, None, 1e-5)
        ins.append((x, dy, g, mean, rstd))
    torch.cuda.synchronize()
    want = [rn.ln_bwd(dy, x, g, m, r, 1e-5) for (x, dy, g, m, r) in ins]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    got = [None, None]
    for rep in range(3):
        for i, st in enumerate(streams):
            st.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(st):
                x, dy, g, m, r = ins[i]
                got[i] = rn.ln_bwd(dy, x, g, m, r, 1e-5, stream=st)
        torch.cuda.synchronize()
        for i in range(2):
            for a_, b_ in zip(want[i], got[i]):
                assert torch.equal(a_, b_), f"stream {i}, repetition {rep}"
    a = arrs[0]
    e = oracle.eps_at_boundary(1e-5)
    xd, dyd, gd = (orc.decode(a[k], "bf16") for k in ("x", "dy", "gamma"))
    dx_o, dg_o, db_o, _, r_o = orc.ln_bwd(dyd, xd, gd, e)
    tol.check_out(host(got[0][0]), dx_o, "bf16", orc, "edge: two streams LN dx",
                  term_scale=tol.dx_term_scale(dyd, gd, r_o))
    tol.check_param(orc.decode(host(got[0][1]), "bf16"), dg_o, "edge: two streams dgamma")


@pytest.mark.parametrize("N,H", [(600, 20480), (37, 40960), (5, 4096), (3, 16384)])
def test_graph_capture_long_and_one_workgroup(N, H):
    """HIP graph capture of the long-row kernels (partial rows at 600 x 20480,
    column sums at 37 x 40960) and of the one-launch backward of a few rows
    (5 x 4096, 3 x 16384): replayed four times with eager work and
    synchronizations between replays, every replay reproduces the eager
    results bit for bit."""
    arr = synth.custom(23, N, H, "bf16")
    x, r, g, b, dy, dh = (to_dev(arr[k]) for k in ("x", "residual", "gamma", "beta",
                                                   "dy", "dh"))
    bf = torch.bfloat16
    y, hh, dx, dx2, y2 = (torch.empty((N, H), dtype=bf, device=DEV) for _ in range(5))
    rstd, mean, rstd2 = (torch.empty(N, dtype=torch.float32, device=DEV) for _ in range(3))
    dg, dg2, db2 = (torch.empty(H, dtype=bf, device=DEV) for _ in range(3))
    ws = torch.empty(max(1, rn.workspace_bytes(N, H, bf, True),
                         rn.workspace_bytes(N, H, bf, False)), dtype=torch.uint8, device=DEV)

    def step():
        rn.fused_add_rms_fwd(x, r, g, 1e-6, y=y, h=hh, rstd=rstd)
        rn.fused_add_rms_bwd(dy, hh, g, rstd, 1e-6, dh_in=dh, dx=dx, dgamma=dg,
                             workspace=ws)
        rn.ln_fwd(x, g, b, 1e-5, y=y2, mean=mean, rstd=rstd2)
        rn.ln_bwd(dy, x, g, mean, rstd2, 1e-5, dx=dx2, dgamma=dg2, dbeta=db2,
                  workspace=ws)

    outs = (y, hh, rstd, dx, dg, y2, mean, rstd2, dx2, dg2, db2)
    step()
    torch.cuda.synchronize()
    want = [t.clone() for t in outs]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        for t in outs:
            t.fill_(7.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for t, w_ in zip(outs, want):
            assert torch.equal(t, w_), f"replay {rep} differs from eager"


def test_unsupported_sizes():
    H = (1 << 22) + 8          # past the longest supported row
    g = torch.ones(H, dtype=torch.bfloat16, device=DEV)
    x = torch.ones((2, H), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(rn.RowNormError) as ei:
        rn.rms_fwd(x, g, 1e-5)
    assert ei.value.status == -6
    with pytest.raises(rn.RowNormError) as ei:
        rn.workspace_bytes(2, H, torch.bfloat16, True)
    assert ei.value.status == -6


# Rows past the register plans (forward: 2-byte rows with 2-byte parameters
# above 32768 elements, other 16-byte rows above 16384, the element-wise
# path above 8192; backward: 16-byte rows above 16384, element-wise above
# 8192).  The forward holds such a row on chip where it fits (its first
# segments in registers, the next ones in LDS) and reads it twice
# otherwise; the backward walks it in segments, caching x and dy in LDS
# where they fit, and writes partial rows for rows of up to 32768 elements
# when N makes them pay, else column sums.  Cases (forward; backward):
#   (600, 20480, bf16)     32768-element register plan, masked tail; LDS
#                          cache, RMS partial rows, LN column sums
#   (37, 32768, bf16)      register plan, full; x and dy on chip, column
#                          sums (few rows)
#   (300, 32768, bf16/f32) float32 parameters: on chip in registers (two
#                          workgroups per CU); column sums
#   (3, 49152, bf16)       registers (6 segments; fused: 4 + 2 in LDS);
#                          column sums (rows past 32768 always take them)
#   (5, 98304, bf16)       registers + 4 LDS segments (fused: read twice);
#                          x and dy partly on chip, the rest read twice
#   (30, 98304, bf16/f32)  the same with float32 parameters
#   (600, 24576, f32)      float32 rows in registers; read twice, partial
#                          rows (LN and RMS)
#   (50, 40000, f32)       registers + LDS for LN/RMS (fused: read twice)
#   (300, 8193, bf16)      element-wise path (odd H), registers, two
#                          workgroups per CU; column sums
#   (600, 12002, f16)      element-wise (rows not 16-byte multiples); RMS
#                          partial rows with 12 segments of accumulators
#   (20, 24577, f16)       element-wise, the 32-segment register kernel
#   (40, 40001, bf16)      element-wise, registers + LDS
#   (1, 16392, bf16), (2, 8201, f32)  one or two rows just past the
#                          register plans (16-byte and element-wise paths)
#   (2, 2^22, bf16), (1, 2^22, f32), (2, 2^22 - 1, f16/f32)  the longest rows
#                          the library takes, on both paths (read twice): 4096
#                          values per lane in each fp32 sum, column sums over
#                          2^22 columns
# Below 1024 rows the column sums past 32768 elements use tiles 32 lanes
# wide (every case above); from 1024 rows on, 8 lanes wide:
#   (1024, 33024, bf16)    16-byte path: x and dy in registers, column sums
#                          over 8-lane tiles of 128 row slots
#   (1030, 32777, f16)     element-wise path: x and dy in registers and LDS,
#                          the same tiles
MAXH = 1 << 22
LONG = [(600, 20480, "bf16"), (37, 32768, "bf16"), (300, 32768, "bf16/f32"),
        (3, 49152, "bf16"), (5, 98304, "bf16"), (30, 98304, "bf16/f32"),
        (600, 24576, "f32"), (50, 40000, "f32"), (300, 8193, "bf16"),
        (600, 12002, "f16"), (20, 24577, "f16"), (40, 40001, "bf16"),
        (1, 16392, "bf16"), (2, 8201, "f32"),
        (2, MAXH, "bf16"), (1, MAXH, "f32"), (2, MAXH - 1, "f16/f32"),
        (1024, 33024, "bf16"), (1030, 32777, "f16")]


@pytest.mark.parametrize("N,H,storage", LONG)
def test_long_rows(orc, N, H, storage):
    """LN, RMS and fused forward and backward against the oracle on every
    element, and bit for bit the same run to run."""
    dtype, _, wdt = storage.partition("/")
    arr = synth.custom(80 + H % 97, N, H, dtype, wdtype=wdt or None)
    print(f"long rows N={N} H={H} {storage}", flush=True)
    check_ln_fwd(orc, arr, dtype, 1e-5)
    check_rms_fwd(orc, arr, dtype, 1e-5)
    xf, rf, gf = (to_dev(arr[k], dtype) for k in ("x", "residual", "gamma"))
    yf, hf, rsf = rn.fused_add_rms_fwd(xf, rf, gf, 1e-5)
    torch.cuda.synchronize()
    y_o, h_o, r_o = orc.fused_add_rms_fwd(
        orc.decode(arr["x"], dtype), orc.decode(arr["residual"], dtype),
        dec(orc, arr, "gamma", dtype), oracle.eps_at_boundary(1e-5))
    assert np.array_equal(host(hf), orc.encode(h_o, dtype)), "h not RNE(x + r)"
    tol.check_out(host(yf), y_o, dtype, orc, f"edge: long fused y {dtype}", strict=True)
    tol.check_rstd(host(rsf), r_o, "edge: long fused rstd")
    check_bwd(orc, arr, dtype, 1e-5, layernorm=True)
    check_bwd(orc, arr, dtype, 1e-5, layernorm=False)
    check_fused_bwd(orc, arr, dtype, 1e-5)
    x, dy, g, dh = (to_dev(arr[k], dtype) for k in ("x", "dy", "gamma", "dh"))

    def run():
        _, mean, rstd = rn.ln_fwd(x, g, None, 1e-5)
        _, rs2 = rn.rms_fwd(x, g, 1e-5)
        dx, dg, db = rn.ln_bwd(dy, x, g, mean, rstd, 1e-5)
        dx2, dg2 = rn.rms_bwd(dy, x, g, rs2, 1e-5)
        dx3, dr3, dg3 = rn.fused_add_rms_bwd(dy, x, g, rs2, 1e-5, dh_in=dh,
                                             write_dres=True)
        torch.cuda.synchronize()
        return [t.clone() for t in (mean, rstd, rs2, dx, dg, db, dx2, dg2, dx3, dr3, dg3)]

    for a_, b_ in zip(run(), run()):
        assert torch.equal(a_, b_), "not reproducible run to run"


@pytest.mark.parametrize("H,pad", [(20480, 24), (20480, 3), (40960, 8), (98304, 8)])
def test_long_rows_strided_in_place(orc, H, pad):
    """Long rows at a row stride of H + pad (pad 3: the element-wise path):
    the padding and a guard row stay untouched; the fused forward writes h
    over x.  Forward paths: 20480 the 32768-element register plan (pad 3:
    the element-wise on-chip kernel); 40960 on chip (LN: registers; fused:
    registers and LDS); 98304 LN on chip with LDS, the fused op read twice
    (h may only be written in the second pass, from values the same lane
    read there).  The backward at 98304 holds part of x and dy on chip and
    reads the rest twice."""
    N = 7
    arr = synth.custom(21, N, H, "bf16")
    SENT = -7.0

    def buf(a=None):
        t = torch.full((N + 1, H + pad), SENT, dtype=torch.bfloat16, device=DEV)
        if a is not None:
            t[:N, :H] = to_dev(a)
        return t

    def view(t):
        return t.as_strided((N, H), (H + pad, 1))

    X, DY, R = buf(arr["x"]), buf(arr["dy"]), buf(arr["residual"])
    Y, DX, Y2 = buf(), buf(), buf()
    g, b = to_dev(arr["gamma"]), to_dev(arr["beta"])
    _, mean, rstd = rn.ln_fwd(view(X), g, b, 1e-5, y=view(Y))
    rn.ln_bwd(view(DY), view(X), g, mean, rstd, 1e-5, dx=view(DX))
    torch.cuda.synchronize()
    e = oracle.eps_at_boundary(1e-5)
    xd = orc.decode(arr["x"], "bf16")
    gd, bd = orc.decode(arr["gamma"], "bf16"), orc.decode(arr["beta"], "bf16")
    y_o, _, _ = orc.ln_fwd(xd, gd, bd, e)
    tol.check_out(host(Y[:N, :H].contiguous()), y_o, "bf16", orc, "edge: long strided LN y")
    dyd = orc.decode(arr["dy"], "bf16")
    dx_o, _, _, _, r_o = orc.ln_bwd(dyd, xd, gd, e)
    tol.check_out(host(DX[:N, :H].contiguous()), dx_o, "bf16", orc, "edge: long strided dx",
                  term_scale=tol.dx_term_scale(dyd, gd, r_o))
    # fused, h over x
    rn.fused_add_rms_fwd(view(X), view(R), g, 1e-6, y=view(Y2), h=view(X))
    torch.cuda.synchronize()
    y3_o, h_o, _ = orc.fused_add_rms_fwd(xd, orc.decode(arr["residual"], "bf16"), gd,
                                         oracle.eps_at_boundary(1e-6))
    assert np.array_equal(host(X[:N, :H].contiguous()), orc.bf16_encode(h_o))
    tol.check_out(host(Y2[:N, :H].contiguous()), y3_o, "bf16", orc,
                  "edge: long in-place fused y", strict=True)
    for t, name in ((X, "h"), (Y, "y"), (DX, "dx"), (Y2, "fused y")):
        hb = t.float().cpu().numpy()
        assert np.all(hb[:N, H:] == SENT), f"{name}: row padding written"
        assert np.all(hb[N, :] == SENT), f"{name}: guard row written"


def test_workspace_errors():
    H = 1024
    x = torch.ones((64, H), dtype=torch.bfloat16, device=DEV)
    g = torch.ones(H, dtype=torch.bfloat16, device=DEV)
    _, rstd = rn.rms_fwd(x, g, 1e-5)
    need = rn.workspace_bytes(64, H, torch.bfloat16, False)
    assert need >= H * 4          # at least one float32 partial row
    # the same size when the device is named explicitly
    assert rn.workspace_bytes(64, H, torch.bfloat16, False, device=0) == need
    small = torch.empty(H * 4 - 4, dtype=torch.uint8, device=DEV)
    with pytest.raises(rn.RowNormError) as ei:
        rn.rms_bwd(x, x, g, rstd, 1e-5, workspace=small)
    assert ei.value.status == -4
    # the workspace does not grow with N past the partial-row cap
    assert rn.workspace_bytes(10 ** 6, H, torch.bfloat16, True) == \
        rn.workspace_bytes(10 ** 7, H, torch.bfloat16, True)


# Forward with some or all saved statistics omitted (null mean / rstd): y
# and h do not depend on which statistics are stored, and a statistic that
# is stored is the same either way.  The shapes cover every forward plan
# family: several rows per wave, a row per wave, 4- and 8-wave teams, and
# the persistent 16-wave plan with partial ring turns (N below, between and
# above multiples of the grid).
STATLESS = [(1000, 128), (257, 1024), (129, 2048), (70, 4096), (33, 8192),
            (7, 16384), (300, 16384), (1029, 16384)]


@pytest.mark.parametrize("N,H", STATLESS)
def test_forward_without_stats(N, H):
    arr = synth.custom(90 + N, N, H, "bf16")
    x, g, b, r = (to_dev(arr[k]) for k in ("x", "gamma", "beta", "residual"))
    y1, m1, s1 = rn.ln_fwd(x, g, b, 1e-5)
    y0, m0, s0 = rn.ln_fwd(x, g, b, 1e-5, save_stats=False)
    assert m0 is None and s0 is None
    assert torch.equal(y0, y1)
    ym, mm, sm = rn.ln_fwd(x, g, b, 1e-5, mean=torch.empty_like(m1), save_stats=False)
    assert sm is None and torch.equal(ym, y1) and torch.equal(mm, m1)
    ys, ms, ss = rn.ln_fwd(x, g, b, 1e-5, rstd=torch.empty_like(s1), save_stats=False)
    assert ms is None and torch.equal(ys, y1) and torch.equal(ss, s1)

    y1, s1 = rn.rms_fwd(x, g, 1e-5)
    y0, s0 = rn.rms_fwd(x, g, 1e-5, save_stats=False)
    assert s0 is None and torch.equal(y0, y1)

    y1, h1, s1 = rn.fused_add_rms_fwd(x, r, g, 1e-5)
    y0, h0, s0 = rn.fused_add_rms_fwd(x, r, g, 1e-5, save_stats=False)
    assert s0 is None and torch.equal(y0, y1) and torch.equal(h0, h1)


@pytest.mark.parametrize("H", [64, 128, 200])
def test_short_rows_huge_stride(orc, H):
    """Short rows run several rows per wave through one buffer range per row
    group, which needs (rows per wave) * stride * e < 2^31; a stride just past
    that bound makes the host take the one-row-per-wave plan instead (the
    backward keeps the segment plan's partial-row count).  Forward,
    backward and fused forward/backward against the oracle, with the bytes
    after each row and after the last row untouched."""
    N, e = 3, 2
    rpw = 8 if H <= 64 else 4 if H <= 128 else 2
    ld = (1 << 31) // (rpw * e) + 8          # 16-byte rows, bound just crossed
    assert rpw * ld * e >= 1 << 31
    arr = synth.custom(70 + H, N, H, "bf16")
    SENT = -7.0
    n_el = (N - 1) * ld + H + 64

    def buf(a=None):
        t = torch.full((n_el,), SENT, dtype=torch.bfloat16, device=DEV)
        if a is not None:
            view(t).copy_(to_dev(a))
        return t

    def view(t):
        return t.as_strided((N, H), (ld, 1))

    X, DY, R, DH = (buf(arr[k]) for k in ("x", "dy", "residual", "dh"))
    Y, DX, HH, Y2, DX2 = buf(), buf(), buf(), buf(), buf()
    g, b = to_dev(arr["gamma"]), to_dev(arr["beta"])
    _, mean, rstd = rn.ln_fwd(view(X), g, b, 1e-5, y=view(Y))
    _, _, db = rn.ln_bwd(view(DY), view(X), g, mean, rstd, 1e-5, dx=view(DX))
    _, _, rs3 = rn.fused_add_rms_fwd(view(X), view(R), g, 1e-6, y=view(Y2), h=view(HH))
    rn.fused_add_rms_bwd(view(DY), view(HH), g, rs3, 1e-6, dh_in=view(DH), dx=view(DX2))
    torch.cuda.synchronize()
    for t, name in ((Y, "y"), (DX, "dx"), (HH, "h"), (Y2, "fused y"), (DX2, "fused dx")):
        for r in range(N):
            tail = t[r * ld + H: r * ld + H + 64].float().cpu().numpy()
            assert np.all(tail == SENT), f"{name}: bytes after row {r} written"
    e64 = oracle.eps_at_boundary(1e-5)
    xd, dyd = orc.decode(arr["x"], "bf16"), orc.decode(arr["dy"], "bf16")
    gd, bd = orc.decode(arr["gamma"], "bf16"), orc.decode(arr["beta"], "bf16")
    y_o, _, _ = orc.ln_fwd(xd, gd, bd, e64)
    tol.check_out(host(view(Y).contiguous()), y_o, "bf16", orc, "edge: huge-stride LN y")
    dx_o, _, db_o, _, r_o = orc.ln_bwd(dyd, xd, gd, e64)
    tol.check_out(host(view(DX).contiguous()), dx_o, "bf16", orc, "edge: huge-stride LN dx",
                  term_scale=tol.dx_term_scale(dyd, gd, r_o))
    tol.check_param(orc.decode(host(db), "bf16"), db_o, "edge: huge-stride LN dbeta")
    y3_o, h_o, _ = orc.fused_add_rms_fwd(xd, orc.decode(arr["residual"], "bf16"), gd,
                                         oracle.eps_at_boundary(1e-6))
    assert np.array_equal(host(view(HH).contiguous()), orc.bf16_encode(h_o))
    tol.check_out(host(view(Y2).contiguous()), y3_o, "bf16", orc,
                  "edge: huge-stride fused y", strict=True)
    arr2 = dict(arr, x=arr["x"])
    dx2_o, _, ts2, _ = fused_bwd_oracle(orc, arr2, "bf16", 1e-6)
    tol.check_out(host(view(DX2).contiguous()), dx2_o, "bf16", orc,
                  "edge: huge-stride fused dx", term_scale=ts2)
