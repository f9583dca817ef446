"""Pins for the CPU oracle: checks that tie it to something other than itself.

Each ``check_*`` function takes an ``oracle.Oracle`` and raises
AssertionError when the oracle disagrees with a fact the pages or the
mathematics fix.  test_oracle_pins.py runs them on the real oracle;
test_oracle_mutants.py runs them on copies of the oracle with a mistake
planted in the C source and requires that some check catches each one.

What each check leans on (never the oracle's own formula retyped):
  closed-form moments of the normalized row, scale laws, RMSNorm ==
  LayerNorm on exactly zero-mean rows, hand-derived tiny cases
  (tests/golden/closed_forms.txt), central finite differences of
  L = sum(dy * y), exact backward invariants, torch's binary64 CPU
  layer_norm / rms_norm and autograd (an independent library routine),
  and for the codecs: exact rational rounding against the enumerated set of
  all bfloat16 / binary16 values (binary32: against the three binary32
  neighbours of each input), plus torch's and numpy's own casts.
"""
import math
import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    scale = max(1.0, float(np.max(np.abs(b))) if b.size else 1.0)
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol * scale, f"{what}: max err {err:.3e} > {tol:.1e}*{scale:.3g}"


# ----------------------------------------------------------------- forward --
def check_ln_moments(orc):
    """Normalized rows (gamma=1, beta=0) have mean 0 and mean square
    v/(v+eps), v the population variance (numpy's np.var, ddof=0)."""
    rng = _rng(11)
    for eps in (1e-5, 0.3):
        for mu, sd, H in ((0.0, 1.0, 37), (1000.0, 2.0, 64), (-3.0, 0.5, 5)):
            x = mu + sd * rng.standard_normal((6, H))
            y, mean, rstd = orc.ln_fwd(x, np.ones(H), None, eps)
            v = np.var(x, axis=1)
            _close(y.mean(axis=1), 0.0, 1e-12, "LN row mean")
            _close((y * y).mean(axis=1), v / (v + eps), 1e-12, "LN row mean square")
            _close(mean, x.mean(axis=1), 1e-13, "LN saved mean")
            _close(rstd * np.sqrt(v + eps), 1.0, 1e-13, "LN saved rstd")


def check_ln_scale_law(orc):
    """LN with eps of (a*x + b) equals LN with eps/a^2 of x, a > 0."""
    rng = _rng(12)
    H = 33
    x = rng.standard_normal((5, H))
    g = 1 + 0.1 * rng.standard_normal(H)
    b = 0.1 * rng.standard_normal(H)
    a, off, eps = 3.0, -7.0, 0.2
    y1, _, _ = orc.ln_fwd(a * x + off, g, b, eps)
    y2, _, _ = orc.ln_fwd(x, g, b, eps / (a * a))
    _close(y1, y2, 1e-12, "LN scale law")


def check_ln_affine(orc):
    """y is x_hat * gamma + beta: subtracting beta and dividing by gamma
    recovers the gamma=1, beta=0 output (per column)."""
    rng = _rng(13)
    H = 19
    x = rng.standard_normal((4, H))
    g = 1 + 0.3 * rng.standard_normal(H)
    b = rng.standard_normal(H)
    y, _, _ = orc.ln_fwd(x, g, b, 1e-5)
    y0, _, _ = orc.ln_fwd(x, np.ones(H), None, 1e-5)
    _close((y - b) / g, y0, 1e-12, "LN affine")
    yb, _, _ = orc.ln_fwd(x, np.ones(H), np.zeros(H), 1e-5)
    _close(yb, y0, 0.0, "LN beta=NULL equals beta=0")


def check_rms_moments(orc):
    """RMSNorm (gamma=1): y/x is the same for every column of a row (no mean
    subtraction), and mean(y^2) = m2/(m2+eps) with m2 = mean(x^2)."""
    rng = _rng(14)
    for eps in (1e-6, 0.25):
        x = 2.0 + rng.standard_normal((5, 29))
        y, rstd = orc.rms_fwd(x, np.ones(29), eps)
        m2 = (x * x).mean(axis=1)
        ratio = y / x
        _close(ratio - ratio[:, :1], 0.0, 1e-14, "RMS proportional")
        _close((y * y).mean(axis=1), m2 / (m2 + eps), 1e-12, "RMS mean square")
        _close(rstd * np.sqrt(m2 + eps), 1.0, 1e-13, "RMS saved rstd")


def check_rms_scale_law(orc):
    rng = _rng(15)
    x = rng.standard_normal((4, 21))
    g = 1 + 0.1 * rng.standard_normal(21)
    a, eps = 0.125, 1e-3
    y1, _ = orc.rms_fwd(a * x, g, eps)
    y2, _ = orc.rms_fwd(x, g, eps / (a * a))
    _close(y1, y2, 1e-12, "RMS scale law")


def _zero_mean_rows(rng, N, H):
    """Rows built from +/- pairs (plus a zero for odd H) of multiples of
    2^-10 below 2^6 in magnitude: every partial sum is exactly representable
    in binary64, so the row sum is exactly 0 in any summation order."""
    half = np.round(rng.standard_normal((N, H // 2)) * 1024.0) / 1024.0
    x = np.concatenate([half, -half[:, ::-1]], axis=1)
    if H % 2:
        x = np.concatenate([x, np.zeros((N, 1))], axis=1)
    return x


def check_rms_equals_ln_zero_mean(orc):
    rng = _rng(16)
    for H in (2, 16, 31):
        x = _zero_mean_rows(rng, 3, H)
        g = 1 + 0.1 * rng.standard_normal(H)
        y_ln, mean, _ = orc.ln_fwd(x, g, None, 1e-5)
        y_rms, _ = orc.rms_fwd(x, g, 1e-5)
        assert np.all(mean == 0.0)
        _close(y_ln, y_rms, 1e-15, "RMS == LN on zero-mean rows")


def check_fused(orc):
    """Fused add+RMSNorm: h is exactly x + r and y is RMSNorm of the
    unrounded h; gamma enters once."""
    rng = _rng(17)
    H = 24
    x = rng.standard_normal((5, H))
    r = rng.standard_normal((5, H))
    g = 1 + 0.05 * rng.standard_normal(H)
    y, h, rstd = orc.fused_add_rms_fwd(x, r, g, 1e-6)
    assert np.array_equal(h, x + r)
    y_ref, rstd_ref = orc.rms_fwd(x + r, g, 1e-6)
    _close(y, y_ref, 1e-15, "fused y")
    _close(rstd, rstd_ref, 1e-15, "fused rstd")
    m2 = ((x + r) ** 2).mean(axis=1)
    _close(rstd * np.sqrt(m2 + 1e-6), 1.0, 1e-13, "fused rstd closed form")


def check_against_torch_fwd(orc):
    """torch's binary64 CPU layer_norm / rms_norm (independent code)."""
    import torch
    import torch.nn.functional as F
    rng = _rng(18)
    N, H = 7, 129
    x = rng.standard_normal((N, H)) * 3 + 1
    g = 1 + 0.1 * rng.standard_normal(H)
    b = 0.1 * rng.standard_normal(H)
    tx, tg, tb = (torch.from_numpy(a) for a in (x, g, b))
    y, _, _ = orc.ln_fwd(x, g, b, 1e-5)
    _close(y, F.layer_norm(tx, (H,), tg, tb, 1e-5).numpy(), 1e-12, "torch LN")
    y, _ = orc.rms_fwd(x, g, 1e-5)
    _close(y, F.rms_norm(tx, (H,), tg, 1e-5).numpy(), 1e-12, "torch RMS")


def _eval_list(s, env):
    return [float(eval(t, {"__builtins__": {}}, env)) for t in s.split()]


def check_golden_closed_forms(orc):
    """Hand-derived tiny cases, tests/golden/closed_forms.txt."""
    path = os.path.join(GOLDEN, "closed_forms.txt")
    n = 0
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            fields = dict(kv.split("=", 1) for kv in
                          (p.strip() for p in line.split("|")))
            eps = float(fields["eps"])
            env = {"sqrt": math.sqrt, "eps": eps}
            op = fields["op"]
            x = np.array([_eval_list(fields["x"], env)])
            g = np.array(_eval_list(fields["gamma"], env))
            H = x.shape[1]
            if op == "ln_fwd":
                b = np.array(_eval_list(fields["beta"], env))
                y, _, _ = orc.ln_fwd(x, g, b, eps)
                _close(y[0], _eval_list(fields["y"], env), 1e-14, line)
            elif op == "rms_fwd":
                y, _ = orc.rms_fwd(x, g, eps)
                _close(y[0], _eval_list(fields["y"], env), 1e-14, line)
            elif op == "fused_fwd":
                r = np.array([_eval_list(fields["r"], env)])
                y, h, _ = orc.fused_add_rms_fwd(x, r, g, eps)
                _close(y[0], _eval_list(fields["y"], env), 1e-14, line)
                _close(h[0], _eval_list(fields["h"], env), 0.0, line)
            elif op == "ln_bwd":
                dy = np.array([_eval_list(fields["dy"], env)])
                dx, dg, db, _, _ = orc.ln_bwd(dy, x, g, eps)
                _close(dx[0], _eval_list(fields["dx"], env), 1e-14, line)
                _close(dg, _eval_list(fields["dgamma"], env), 1e-14, line)
                _close(db, _eval_list(fields["dbeta"], env), 1e-14, line)
            elif op == "rms_bwd":
                dy = np.array([_eval_list(fields["dy"], env)])
                dx, dg, _ = orc.rms_bwd(dy, x, g, eps)
                _close(dx[0], _eval_list(fields["dx"], env), 1e-14, line)
                _close(dg, _eval_list(fields["dgamma"], env), 1e-14, line)
            else:
                raise AssertionError(f"unknown op {op}")
            assert H >= 1
            n += 1
    assert n >= 8, "golden file lost its cases"


# ------------------------------------------------------------- statistics --
def check_welford(orc):
    """Sequential Welford and the parallel merge over random splits
    (including empty parts) equal the two-pass mean and M2."""
    rng = _rng(19)
    for mu, sd, n in ((0.0, 1.0, 1000), (50.0, 0.01, 777), (1e3, 1e-3, 64)):
        x = mu + sd * rng.standard_normal(n)
        m_ref = x.mean()
        q_ref = float(np.sum((x - m_ref) ** 2))
        c, m, q = orc.welford(x)
        assert c == n
        _close(m, m_ref, 1e-14, "welford mean")
        assert abs(q - q_ref) <= 1e-9 * q_ref, (q, q_ref)
        for trial in range(5):
            cuts = np.sort(rng.integers(0, n + 1, size=6))
            parts = np.split(x, cuts)     # some parts may be empty
            acc = (0.0, 0.0, 0.0)
            for p in parts:
                acc = orc.welford_merge(acc, orc.welford(p))
            assert acc[0] == n
            _close(acc[1], m_ref, 1e-14, "merged mean")
            assert abs(acc[2] - q_ref) <= 1e-9 * q_ref, (acc[2], q_ref)
    # count-0 identity on both sides
    s = orc.welford(np.array([1.0, 2.0, 4.0]))
    assert orc.welford_merge((0.0, 0.0, 0.0), s) == s
    assert orc.welford_merge(s, (0.0, 0.0, 0.0)) == s
    assert orc.welford_merge((0.0, 0.0, 0.0), (0.0, 0.0, 0.0)) == (0.0, 0.0, 0.0)


# ---------------------------------------------------------------- backward --
def _loss_ln(orc, x, g, b, dy, eps):
    y, _, _ = orc.ln_fwd(x, g, b, eps)
    return float(np.sum(dy * y))


def _loss_rms(orc, x, g, dy, eps):
    y, _ = orc.rms_fwd(x, g, eps)
    return float(np.sum(dy * y))


def check_bwd_finite_differences(orc):
    """Central differences of L = sum(dy * y) w.r.t. x, gamma, beta."""
    rng = _rng(20)
    for N in (1, 3):
        for H in (1, 2, 3, 5, 8, 17):
            for eps in (1e-5, 0.5):
                x = rng.standard_normal((N, H))
                dy = rng.standard_normal((N, H))
                g = 1 + 0.1 * rng.standard_normal(H)
                b = 0.1 * rng.standard_normal(H)
                dx, dg, db, _, _ = orc.ln_bwd(dy, x, g, eps)
                dxr, dgr, _ = orc.rms_bwd(dy, x, g, eps)
                fx = np.zeros_like(x)
                fxr = np.zeros_like(x)
                for i in range(N):
                    for j in range(H):
                        h = 1e-6 * max(1.0, abs(x[i, j]))
                        xp = x.copy(); xp[i, j] += h
                        xm = x.copy(); xm[i, j] -= h
                        fx[i, j] = (_loss_ln(orc, xp, g, b, dy, eps) -
                                    _loss_ln(orc, xm, g, b, dy, eps)) / (2 * h)
                        fxr[i, j] = (_loss_rms(orc, xp, g, dy, eps) -
                                     _loss_rms(orc, xm, g, dy, eps)) / (2 * h)
                fg = np.zeros(H); fb = np.zeros(H); fgr = np.zeros(H)
                for j in range(H):
                    h = 1e-6 * max(1.0, abs(g[j]))
                    gp = g.copy(); gp[j] += h
                    gm = g.copy(); gm[j] -= h
                    fg[j] = (_loss_ln(orc, x, gp, b, dy, eps) -
                             _loss_ln(orc, x, gm, b, dy, eps)) / (2 * h)
                    fgr[j] = (_loss_rms(orc, x, gp, dy, eps) -
                              _loss_rms(orc, x, gm, dy, eps)) / (2 * h)
                    bp = b.copy(); bp[j] += 1e-6
                    bm = b.copy(); bm[j] -= 1e-6
                    fb[j] = (_loss_ln(orc, x, g, bp, dy, eps) -
                             _loss_ln(orc, x, g, bm, dy, eps)) / 2e-6
                tag = f"N={N} H={H} eps={eps}"
                _close(dx, fx, 1e-7, "LN dx vs FD " + tag)
                _close(dg, fg, 1e-7, "LN dgamma vs FD " + tag)
                _close(db, fb, 1e-7, "LN dbeta vs FD " + tag)
                _close(dxr, fxr, 1e-7, "RMS dx vs FD " + tag)
                _close(dgr, fgr, 1e-7, "RMS dgamma vs FD " + tag)


def check_fused_bwd_finite_differences(orc):
    """Fused add+RMSNorm backward: central differences of
    L(x, r) = sum(dy * y) + sum(dh * h), (y, h) = fused(x, r), with respect
    to x AND to r both equal the oracle's gradient at the forward's h and
    rstd; with dh omitted, the y-path alone."""
    rng = _rng(26)
    for N, H, eps in ((1, 1, 1e-5), (2, 3, 0.2), (3, 8, 1e-6), (2, 17, 1e-3)):
        x = rng.standard_normal((N, H))
        r = rng.standard_normal((N, H))
        dy = rng.standard_normal((N, H))
        dh = rng.standard_normal((N, H))
        g = 1 + 0.05 * rng.standard_normal(H)
        for use_dh in (False, True):
            def L(xx, rr):
                y, h, _ = orc.fused_add_rms_fwd(xx, rr, g, eps)
                v = float(np.sum(dy * y))
                return v + (float(np.sum(dh * h)) if use_dh else 0.0)
            _, h, rs = orc.fused_add_rms_fwd(x, r, g, eps)
            dx, dg = orc.fused_add_rms_bwd(dy, h, g, rs, dh if use_dh else None)
            fx = np.zeros_like(x)
            fr = np.zeros_like(x)
            for i in range(N):
                for j in range(H):
                    st = 1e-6 * max(1.0, abs(x[i, j]))
                    e = np.zeros_like(x)
                    e[i, j] = st
                    fx[i, j] = (L(x + e, r) - L(x - e, r)) / (2 * st)
                    st = 1e-6 * max(1.0, abs(r[i, j]))
                    e = np.zeros_like(x)
                    e[i, j] = st
                    fr[i, j] = (L(x, r + e) - L(x, r - e)) / (2 * st)
            fg = np.zeros(H)
            for j in range(H):
                st = 1e-6 * max(1.0, abs(g[j]))
                gp = g.copy(); gp[j] += st
                gm = g.copy(); gm[j] -= st
                yp, _, _ = orc.fused_add_rms_fwd(x, r, gp, eps)
                ym, _, _ = orc.fused_add_rms_fwd(x, r, gm, eps)
                fg[j] = (float(np.sum(dy * yp)) - float(np.sum(dy * ym))) / (2 * st)
            tag = f"N={N} H={H} dh={use_dh}"
            _close(dx, fx, 1e-7, "fused dx vs FD in x " + tag)
            _close(dx, fr, 1e-7, "fused dres vs FD in r " + tag)
            _close(dg, fg, 1e-7, "fused dgamma vs FD " + tag)


def check_bwd_invariants(orc):
    """LayerNorm: each dx row sums to 0 and sum_j dx*x_hat equals
    rstd*H*c2*eps/(v+eps).  RMSNorm: sum_j dx*x_hat equals
    rstd*H*c2*eps/(m2+eps).  Zero-mean rows: LN dx - RMS dx = -rstd*c1.
    dbeta is the column sum of dy."""
    rng = _rng(21)
    N, H, eps = 6, 40, 0.05
    x = 1.5 * rng.standard_normal((N, H)) + 0.7
    dy = rng.standard_normal((N, H))
    g = 1 + 0.2 * rng.standard_normal(H)
    dx, dg, db, mean, rstd = orc.ln_bwd(dy, x, g, eps)
    v = np.var(x, axis=1)
    s = 1.0 / np.sqrt(v + eps)
    xhat = (x - x.mean(axis=1, keepdims=True)) * s[:, None]
    c2 = (dy * g * xhat).mean(axis=1)
    _close(dx.sum(axis=1), 0.0, 1e-12, "LN sum dx")
    _close((dx * xhat).sum(axis=1), s * H * c2 * eps / (v + eps), 1e-11,
           "LN sum dx*xhat")
    _close(db, dy.sum(axis=0), 1e-13, "dbeta column sums")
    dxr, dgr, rstd_r = orc.rms_bwd(dy, x, g, eps)
    m2 = (x * x).mean(axis=1)
    sr = 1.0 / np.sqrt(m2 + eps)
    xr = x * sr[:, None]
    c2r = (dy * g * xr).mean(axis=1)
    _close((dxr * xr).sum(axis=1), sr * H * c2r * eps / (m2 + eps), 1e-11,
           "RMS sum dx*xhat")
    z = _zero_mean_rows(rng, 4, 18)
    dyz = rng.standard_normal(z.shape)
    gz = 1 + 0.1 * rng.standard_normal(18)
    dxl, _, _, _, rz = orc.ln_bwd(dyz, z, gz, 1e-5)
    dxm, _, _ = orc.rms_bwd(dyz, z, gz, 1e-5)
    c1 = (dyz * gz).mean(axis=1)
    _close(dxl - dxm, -(rz * c1)[:, None] * np.ones((1, 18)), 1e-13,
           "LN - RMS on zero-mean rows")


def check_bwd_against_torch(orc):
    import torch
    import torch.nn.functional as F
    rng = _rng(22)
    N, H, eps = 5, 66, 1e-5
    x = rng.standard_normal((N, H))
    dy = rng.standard_normal((N, H))
    g = 1 + 0.1 * rng.standard_normal(H)
    b = 0.1 * rng.standard_normal(H)
    tx = torch.from_numpy(x.copy()).requires_grad_()
    tg = torch.from_numpy(g.copy()).requires_grad_()
    tb = torch.from_numpy(b.copy()).requires_grad_()
    F.layer_norm(tx, (H,), tg, tb, eps).backward(torch.from_numpy(dy))
    dx, dg, db, _, _ = orc.ln_bwd(dy, x, g, eps)
    _close(dx, tx.grad.numpy(), 1e-12, "torch LN dx")
    _close(dg, tg.grad.numpy(), 1e-12, "torch LN dgamma")
    _close(db, tb.grad.numpy(), 1e-12, "torch LN dbeta")
    tx = torch.from_numpy(x.copy()).requires_grad_()
    tg = torch.from_numpy(g.copy()).requires_grad_()
    F.rms_norm(tx, (H,), tg, eps).backward(torch.from_numpy(dy))
    dx, dg, _ = orc.rms_bwd(dy, x, g, eps)
    _close(dx, tx.grad.numpy(), 1e-12, "torch RMS dx")
    _close(dg, tg.grad.numpy(), 1e-12, "torch RMS dgamma")


def check_special_cases(orc):
    """H = 1 and constant rows."""
    rng = _rng(23)
    x = rng.standard_normal((5, 1))
    g = np.array([1.7])
    b = np.array([-0.3])
    dy = rng.standard_normal((5, 1))
    y, mean, rstd = orc.ln_fwd(x, g, b, 1e-5)
    _close(y, np.full((5, 1), -0.3), 0.0, "LN H=1: y = beta")
    dx, _, _, _, _ = orc.ln_bwd(dy, x, g, 1e-5)
    _close(dx, 0.0, 0.0, "LN H=1: dx = 0")
    y, _ = orc.rms_fwd(x, g, 1e-5)
    _close(y, x * 1.7 / np.sqrt(x * x + 1e-5), 1e-14, "RMS H=1")
    # constant row c: mean c, var 0, rstd 1/sqrt(eps), y = beta,
    # dx = rstd * (g - mean(g))
    H, c, eps = 12, 50.0, 1e-5
    xc = np.full((2, H), c)
    gg = 1 + 0.1 * rng.standard_normal(H)
    bb = 0.1 * rng.standard_normal(H)
    y, mean, rstd = orc.ln_fwd(xc, gg, bb, eps)
    _close(y, np.tile(bb, (2, 1)), 1e-15, "LN constant row: y = beta")
    assert np.all(mean == c)
    _close(rstd, 1.0 / math.sqrt(eps), 1e-15, "LN constant row rstd")
    dyc = rng.standard_normal((2, H))
    dx, _, _, _, _ = orc.ln_bwd(dyc, xc, gg, eps)
    gc = dyc * gg
    _close(dx, (gc - gc.mean(axis=1, keepdims=True)) / math.sqrt(eps), 1e-13,
           "LN constant row dx")


# ------------------------------------------------------------------ codec --
def _all_bf16_values():
    bits = np.arange(0, 1 << 16, dtype=np.uint32)
    with np.errstate(invalid="ignore"):
        f = (bits << 16).view(np.float32).astype(np.float64)
    return bits.astype(np.uint16), f


def _exact_round_bf16(v: float, finite_sorted, finite_bits):
    """Reference RNE to bfloat16 by exact rational comparison against the
    enumerated set of all finite bfloat16 values."""
    if math.isnan(v):
        return None
    if v == 0.0:
        return 0x8000 if math.copysign(1.0, v) < 0 else 0
    maxv = finite_sorted[-1]
    # overflow: at or beyond max + half an ulp (ulp at max is 2^120)
    half = Fraction(2) ** 119
    if Fraction(abs(v)) >= Fraction(maxv) + half:
        return 0xFF80 if v < 0 else 0x7F80
    i = int(np.searchsorted(finite_sorted, v))
    cands = [k for k in (i - 1, i) if 0 <= k < len(finite_sorted)]
    fv = Fraction(v)
    best = None
    for k in cands:
        d = abs(Fraction(finite_sorted[k]) - fv)
        key = (d, int(finite_bits[k]) & 1)
        if best is None or key < best[0]:
            best = (key, k)
    bits = int(finite_bits[best[1]])
    if Fraction(finite_sorted[best[1]]) == 0:
        # rounded to zero: sign follows the input
        bits = 0x8000 if v < 0 else 0
    return bits


def check_bf16_codec(orc):
    bits, vals = _all_bf16_values()
    # decode: every pattern (NaNs compared as NaN)
    dec = orc.bf16_decode(bits)
    nan = np.isnan(vals)
    assert np.array_equal(np.isnan(dec), nan)
    assert np.array_equal(dec[~nan], vals[~nan])
    assert np.array_equal(np.signbit(dec[~nan]), np.signbit(vals[~nan]))
    # encode: exact rational rounding against the enumerated finite set
    fin = np.isfinite(vals)
    order = np.argsort(vals[fin], kind="stable")
    fs = vals[fin][order]
    fb = bits[fin][order]
    # drop -0.0 duplicates so the sorted list is strictly increasing
    keep = np.concatenate([[True], np.diff(fs) > 0])
    fs, fb = fs[keep], fb[keep]
    rng = _rng(24)
    tests = list(rng.standard_normal(2000) * 10.0 ** rng.integers(-40, 38, 2000))
    # exact midpoints (ties) between neighbours, both parities, and near them
    for k in rng.integers(0, len(fs) - 1, 400):
        mid = (fs[k] + fs[k + 1]) / 2.0      # exact in binary64
        tests += [mid, np.nextafter(mid, np.inf), np.nextafter(mid, -np.inf)]
    tiny = 2.0 ** -133
    tests += [0.0, -0.0, tiny, tiny / 2, tiny * 0.75, tiny * 1.5, -tiny * 2.5,
              2.0 ** -126, 2.0 ** -126 * (1 - 2 ** -9), fs[-1],
              fs[-1] + 2.0 ** 119, np.nextafter(fs[-1] + 2.0 ** 119, 0),
              1e39, -1e39, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8]
    tests = np.array(tests, dtype=np.float64)
    got = orc.bf16_encode(tests)
    for v, gb in zip(tests, got):
        want = _exact_round_bf16(float(v), fs, fb)
        assert int(gb) == want, f"bf16({v!r}) = {int(gb):#06x}, want {want:#06x}"
    # specials
    sp = orc.bf16_encode(np.array([np.inf, -np.inf, np.nan]))
    assert int(sp[0]) == 0x7F80 and int(sp[1]) == 0xFF80
    assert (int(sp[2]) & 0x7F80) == 0x7F80 and (int(sp[2]) & 0x7F) != 0


def check_bf16_encode_vs_torch(orc):
    """binary32 inputs: one-step rounding from binary64 equals torch's
    float32 -> bfloat16 cast (round to nearest even)."""
    import torch
    rng = _rng(25)
    u = rng.integers(0, 1 << 32, size=1 << 20, dtype=np.uint64).astype(np.uint32)
    f = u.view(np.float32)
    f = f[np.isfinite(f)]
    want = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16)
    want = want.numpy().view(np.uint16)
    got = orc.bf16_encode(f.astype(np.float64))
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"{bad.size} mismatches, e.g. {f[bad[:3]]}"


def _exact_round_f16(v: float, finite_sorted, finite_bits):
    """Reference RNE to binary16 by exact rational comparison against the
    enumerated set of all finite binary16 values (overflow at or beyond
    65504 + 16, half an ulp past the largest value)."""
    if v == 0.0:
        return 0x8000 if math.copysign(1.0, v) < 0 else 0
    if Fraction(abs(v)) >= Fraction(65504) + 16:
        return 0xFC00 if v < 0 else 0x7C00
    i = int(np.searchsorted(finite_sorted, v))
    fv = Fraction(v)
    best = None
    for k in (i - 1, i):
        if 0 <= k < len(finite_sorted):
            key = (abs(Fraction(finite_sorted[k]) - fv), int(finite_bits[k]) & 1)
            if best is None or key < best[0]:
                best = (key, k)
    bits = int(finite_bits[best[1]])
    if Fraction(finite_sorted[best[1]]) == 0:
        return 0x8000 if v < 0 else 0
    return bits


def check_f16_codec(orc):
    """IEEE binary16: decode of all 2^16 patterns equals numpy's exact
    float16 -> float64 widening; encode equals exact rational rounding to
    the nearest finite value (ties to the even pattern) on random, tie,
    subnormal and overflow inputs, and equals numpy's direct float64 ->
    float16 cast on a million random binary64 values."""
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = bits.view(np.float16).astype(np.float64)
    dec = orc.f16_decode(bits)
    nan = np.isnan(vals)
    assert np.array_equal(np.isnan(dec), nan)
    assert np.array_equal(dec[~nan], vals[~nan])
    assert np.array_equal(np.signbit(dec[~nan]), np.signbit(vals[~nan]))
    fin = np.isfinite(vals)
    order = np.argsort(vals[fin], kind="stable")
    fs, fb = vals[fin][order], bits[fin][order]
    keep = np.concatenate([[True], np.diff(fs) > 0])
    fs, fb = fs[keep], fb[keep]
    rng = _rng(27)
    tests = list(rng.standard_normal(2000) * 10.0 ** rng.integers(-9, 6, 2000))
    for k in rng.integers(0, len(fs) - 1, 400):
        mid = (fs[k] + fs[k + 1]) / 2.0
        tests += [mid, np.nextafter(mid, np.inf), np.nextafter(mid, -np.inf)]
    tiny = 2.0 ** -24
    tests += [0.0, -0.0, tiny, tiny / 2, tiny * 0.75, tiny * 1.5, -tiny * 2.5,
              2.0 ** -14, 2.0 ** -14 * (1 - 2 ** -12), 65504.0, 65519.99,
              65520.0, -65520.0, 1e6, 1.0 + 2 ** -11, 1.0 + 3 * 2 ** -11,
              2047.5, 2048.5, 2049.0]
    tests = np.array(tests, dtype=np.float64)
    got = orc.f16_encode(tests)
    for v, gb in zip(tests, got):
        want = _exact_round_f16(float(v), fs, fb)
        assert int(gb) == want, f"f16({v!r}) = {int(gb):#06x}, want {want:#06x}"
    sp = orc.f16_encode(np.array([np.inf, -np.inf, np.nan]))
    assert int(sp[0]) == 0x7C00 and int(sp[1]) == 0xFC00
    assert (int(sp[2]) & 0x7C00) == 0x7C00 and (int(sp[2]) & 0x3FF) != 0
    w = rng.standard_normal(1 << 20) * 10.0 ** rng.integers(-8, 5, 1 << 20)
    with np.errstate(over="ignore"):
        want = w.astype(np.float16).view(np.uint16)
    bad = np.nonzero(orc.f16_encode(w) != want)[0]
    assert bad.size == 0, f"{bad.size} mismatches vs numpy, e.g. {w[bad[:3]]}"


def check_f16_encode_vs_torch(orc):
    """binary32 inputs: one-step rounding from binary64 equals torch's
    float32 -> float16 cast (round to nearest even)."""
    import torch
    rng = _rng(28)
    u = rng.integers(0, 1 << 32, size=1 << 20, dtype=np.uint64).astype(np.uint32)
    f = u.view(np.float32)
    f = f[np.isfinite(f)]
    want = torch.from_numpy(f.copy()).to(torch.float16).view(torch.int16)
    want = want.numpy().view(np.uint16)
    got = orc.f16_encode(f.astype(np.float64))
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"{bad.size} mismatches, e.g. {f[bad[:3]]}"


def _exact_round_f32(v: float):
    """Reference RNE to binary32 by exact rational comparison: the answer is
    one of the binary32 neighbours of a nearby candidate (three consecutive
    binary32 values around it), chosen by exact distance, ties to the even
    significand; at or beyond FLT_MAX + half an ulp (2^103) it overflows."""
    fmax = float(np.finfo(np.float32).max)
    if v == 0.0:
        return np.float32(v)
    if Fraction(abs(v)) >= Fraction(fmax) + Fraction(2) ** 103:
        return np.float32(np.inf if v > 0 else -np.inf)
    with np.errstate(over="ignore"):
        c = np.float32(min(max(v, -fmax), fmax))
    with np.errstate(over="ignore"):
        cands = {np.nextafter(c, np.float32(-np.inf)), c,
                 np.nextafter(c, np.float32(np.inf))}
    cands = [k for k in cands if np.isfinite(k)]
    fv = Fraction(v)
    best = None
    for k in cands:
        key = (abs(Fraction(float(k)) - fv), int(np.array(k).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, k)
    r = best[1]
    if r == 0:   # rounded to zero: the sign follows the input
        return np.float32(-0.0) if v < 0 else np.float32(0.0)
    return r


def check_f32_encode(orc):
    """binary64 -> binary32 (the expected value of every float32 output and of
    the bit-exact float32 h): exact rational rounding to the nearest binary32
    value, ties to even, on random values over the whole exponent range,
    exact midpoints between neighbours (and one binary64 step either side),
    subnormals and the subnormal/normal boundary, overflow, signed zeros;
    then numpy's float64 -> float32 cast on a million random values."""
    rng = _rng(29)
    tests = list(rng.standard_normal(2000) * 10.0 ** rng.integers(-46, 39, 2000))
    u = rng.integers(1, 0x7F7FFFFF, 600, dtype=np.uint64).astype(np.uint32)
    for f in u.view(np.float32):
        nb = np.nextafter(f, np.float32(np.inf))
        mid = (float(f) + float(nb)) / 2.0        # exact in binary64
        tests += [mid, -mid, np.nextafter(mid, np.inf), np.nextafter(mid, -np.inf)]
    tiny = 2.0 ** -149
    fmax = float(np.finfo(np.float32).max)
    tests += [0.0, -0.0, tiny, tiny / 2, tiny * 0.75, tiny * 1.5, -tiny * 2.5,
              tiny * 3.5, 2.0 ** -126, 2.0 ** -126 * (1 - 2 ** -24),
              2.0 ** -126 - tiny / 2, fmax, -fmax, fmax + 2.0 ** 103,
              np.nextafter(fmax + 2.0 ** 103, 0), 1e39, -1e39, 1.0 + 2 ** -24,
              1.0 + 3 * 2 ** -24, 1.0 - 2 ** -25, 1.0 + 2 ** -52]
    tests = np.array(tests, dtype=np.float64)
    got = orc.f32_encode(tests)
    for v, g in zip(tests, got):
        want = _exact_round_f32(float(v))
        same = (np.array(g).view(np.uint32) == np.array(want).view(np.uint32))
        assert same, f"f32({v!r}) = {g!r}, want {want!r}"
    w = rng.standard_normal(1 << 20) * 10.0 ** rng.integers(-45, 38, 1 << 20)
    with np.errstate(over="ignore"):
        want = w.astype(np.float32)
    bad = np.nonzero(orc.f32_encode(w).view(np.uint32) != want.view(np.uint32))[0]
    assert bad.size == 0, f"{bad.size} mismatches vs numpy, e.g. {w[bad[:3]]}"


ALL_CHECKS = [
    check_ln_moments, check_ln_scale_law, check_ln_affine, check_rms_moments,
    check_rms_scale_law, check_rms_equals_ln_zero_mean, check_fused,
    check_against_torch_fwd, check_golden_closed_forms, check_welford,
    check_bwd_finite_differences, check_fused_bwd_finite_differences,
    check_bwd_invariants,
    check_bwd_against_torch, check_special_cases, check_bf16_codec,
    check_bf16_encode_vs_torch, check_f16_codec, check_f16_encode_vs_torch,
    check_f32_encode,
]
