"""Parity bars between the HIP path and the binary64 oracle.

bf16 and fp16 outputs (same rule, each in its own format):
  the GPU value must be within 1 ulp of the correctly rounded oracle value
  (distance measured on the ordered integer image of the bit patterns,
  +0 == -0), or, for values produced by cancellation, within an absolute
  floor of ulp_bf16(2^-10 * row scale), i.e. between 2^-18 and 2^-17 times
  the row's scale.  Why a floor at all: the float32 pipeline's own error is
  a few float32 ulps of the scale of the terms that cancel (about
  2^-22 * scale), while a bf16 ulp at |v| is 2^-8..2^-7 * |v|; only outputs
  far below the row's scale (|v| below about 2^-14 * scale) can land more
  than one ulp away, and the floor (16-32 float32 ulps of the scale) covers
  exactly those.  The row scale is the RMS of the oracle output, or for dx
  the larger of that and rstd * RMS(dy * gamma): dx = rstd * (g - c1 -
  x_hat * c2) is a difference of terms of size rstd * |g|, and for short rows
  it cancels almost completely (H = 1 RMSNorm: dx = rstd * g * eps / (x^2 +
  eps)), so the RMS of dx itself understates the terms' size.
  Outputs formed without cancellation (RMSNorm and fused y = x * rstd *
  gamma, products only) may not use the floor at all (strict=True): a few
  float32 roundings cannot move a correctly rounded bf16 value by more than
  one ulp.  Every check records the element count, the largest ulp distance
  and how many elements passed only through the floor (STATS), and the
  session prints them.
fp32 outputs: |gpu - oracle| <= 1e-5 * max(|oracle|, row scale).
mean (fp32): |gpu - oracle| <= 1e-5 * max(|mean|, sqrt(var + eps)).
rstd (fp32): relative 1e-5.
dgamma/dbeta: relative RMS error ||gpu - oracle|| / ||oracle|| <= 5e-3.
h of the fused op: bit-exact to RNE(x + residual).
"""
import numpy as np

FLOOR_REL_EXP = -10          # floor = ulp_bf16(2^-10 * row scale)
F32_REL = 1e-5
PARAM_REL_RMS = 5e-3
CHUNK_ELEMS = 1 << 22        # compare in row blocks of about this many elements

# label -> {"n", "max_ulp", "floored", "max_rel"}; filled by every check
STATS = {}


def _record(what, n, max_ulp=None, floored=None, max_rel=None):
    s = STATS.setdefault(what, {"n": 0, "max_ulp": 0, "floored": 0, "max_rel": 0.0})
    s["n"] += int(n)
    if max_ulp is not None:
        s["max_ulp"] = max(s["max_ulp"], int(max_ulp))
    if floored is not None:
        s["floored"] += int(floored)
    if max_rel is not None:
        s["max_rel"] = max(s["max_rel"], float(max_rel))


def ordered(bits_u16: np.ndarray) -> np.ndarray:
    """Map bfloat16 / binary16 bit patterns (sign-magnitude) to integers
    ordered like their values."""
    b = bits_u16.astype(np.int32)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def ulp_bf16(v: np.ndarray) -> np.ndarray:
    """Spacing of bfloat16 values at |v| (normal range): 2^(k-7) for
    |v| in [2^k, 2^(k+1)); 0 at v = 0 (a row whose scale is 0 gets no
    floor)."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    _, e = np.frexp(a)
    return np.where(a > 0, np.ldexp(1.0, e - 8), 0.0)


def row_rms(v: np.ndarray) -> np.ndarray:
    v = np.atleast_2d(v)
    return np.sqrt(np.mean(v * v, axis=1, keepdims=True))


def _scale(oracle_vals, term_scale):
    s = row_rms(oracle_vals)
    if term_scale is not None:
        s = np.maximum(s, np.asarray(term_scale, dtype=np.float64).reshape(-1, 1))
    return s


def _row_blocks(N, H):
    step = max(1, CHUNK_ELEMS // max(H, 1))
    for r0 in range(0, N, step):
        yield r0, min(N, r0 + step)


def check_bf16(gpu_bits, oracle_vals, orc, what, term_scale=None, dtype="bf16",
               strict=False, max_floored_frac=None):
    """gpu_bits: uint16 [N, H] (bf16, or fp16 with dtype="f16");
    oracle_vals: float64 [N, H] (unrounded); term_scale: optional per-row
    scale of the terms that cancel.  strict: no floor (1 ulp everywhere).
    max_floored_frac: bound on the fraction of elements that may pass only
    through the floor."""
    gpu_bits = np.atleast_2d(gpu_bits)
    oracle_vals = np.atleast_2d(oracle_vals)
    N, H = oracle_vals.shape
    ts = None if term_scale is None else np.asarray(term_scale, dtype=np.float64).reshape(-1)
    max_ulp, floored, nbad, first = 0, 0, 0, None
    for r0, r1 in _row_blocks(N, H):
        o = oracle_vals[r0:r1]
        want = orc.encode(o, dtype)
        ulp = np.abs(ordered(gpu_bits[r0:r1]) - ordered(want))
        ok1 = ulp <= 1
        if strict:
            ok = ok1
        else:
            floor = ulp_bf16(np.ldexp(_scale(o, None if ts is None else ts[r0:r1]),
                                      FLOOR_REL_EXP))
            gv = orc.decode(gpu_bits[r0:r1], dtype)
            ok = ok1 | (np.abs(gv - o) <= floor)
        if ulp.size:
            max_ulp = max(max_ulp, int(ulp.max()))
        floored += int(np.sum(ok & ~ok1))
        bad = np.argwhere(~ok)
        nbad += len(bad)
        if len(bad) and first is None:
            i, j = bad[0]
            gv1 = orc.decode(gpu_bits[r0 + i, j:j + 1], dtype)[0]
            first = (r0 + i, j, gv1, o[i, j], int(ulp[i, j]))
    _record(what, oracle_vals.size, max_ulp, floored)
    if nbad:
        i, j, g, o, u = first
        raise AssertionError(
            f"{what}: {nbad} of {oracle_vals.size} elements off"
            f"{' (strict 1 ulp)' if strict else ''}; first at [{i},{j}] "
            f"gpu={g!r} oracle={o!r} ulp={u}")
    if max_floored_frac is not None and oracle_vals.size:
        frac = floored / oracle_vals.size
        assert frac <= max_floored_frac, \
            f"{what}: {floored} elements needed the floor ({frac:.2e} > {max_floored_frac:.0e})"
    return {"max_ulp": max_ulp, "floored": floored}


def check_f32(gpu, oracle_vals, what, rel=F32_REL, term_scale=None):
    gpu = np.atleast_2d(np.asarray(gpu, dtype=np.float64))
    oracle_vals = np.atleast_2d(oracle_vals)
    scale = np.maximum(np.abs(oracle_vals), _scale(oracle_vals, term_scale))
    err = np.abs(gpu - oracle_vals)
    ok = err <= rel * scale
    bad = np.argwhere(~ok)
    mr = float(np.max(err / np.maximum(scale, 1e-300))) if err.size else 0.0
    _record(what, oracle_vals.size, max_rel=mr)
    if bad.size:
        i, j = bad[0]
        raise AssertionError(
            f"{what}: {len(bad)} of {ok.size} off; first at [{i},{j}] "
            f"gpu={gpu[i, j]!r} oracle={oracle_vals[i, j]!r}")
    return mr


def check_out(gpu_host, oracle_vals, dtype, orc, what, term_scale=None,
              strict=False, max_floored_frac=None):
    if dtype in ("bf16", "f16"):
        return check_bf16(gpu_host, oracle_vals, orc, what, term_scale, dtype,
                          strict=strict, max_floored_frac=max_floored_frac)
    return check_f32(gpu_host, oracle_vals, what, term_scale=term_scale)


def dx_term_scale(dy, gamma, rstd):
    """Per-row scale of the terms dx is the difference of: rstd*RMS(dy*gamma)."""
    g = np.atleast_2d(dy) * np.asarray(gamma)[None, :]
    return np.asarray(rstd) * np.sqrt(np.mean(g * g, axis=1))


def check_mean(gpu, mean_o, var_o, eps, what):
    gpu = np.asarray(gpu, dtype=np.float64)
    scale = np.maximum(np.abs(mean_o), np.sqrt(var_o + eps))
    err = np.abs(gpu - mean_o)
    _record(what, gpu.size, max_rel=float(np.max(err / scale)) if err.size else 0.0)
    assert np.all(err <= F32_REL * scale), \
        f"{what}: max scaled err {np.max(err / scale):.3e}"


def check_rstd(gpu, rstd_o, what):
    gpu = np.asarray(gpu, dtype=np.float64)
    rel = np.abs(gpu - rstd_o) / np.abs(rstd_o)
    _record(what, gpu.size, max_rel=float(rel.max()) if rel.size else 0.0)
    assert np.all(rel <= F32_REL), f"{what}: max rel err {rel.max():.3e}"


def check_param(gpu_vals, oracle_vals, what):
    gpu_vals = np.asarray(gpu_vals, dtype=np.float64)
    num = np.linalg.norm(gpu_vals - oracle_vals)
    den = np.linalg.norm(oracle_vals)
    rr = num / den if den > 0 else num
    _record(what, gpu_vals.size, max_rel=rr)
    assert rr <= PARAM_REL_RMS, f"{what}: rel-rms {rr:.3e}"
    return rr


def summary_lines():
    """One line per check label: elements, largest ulp distance, elements
    that passed only through the floor, largest relative error."""
    out = [f"{'check':58s} {'elements':>12s} {'max_ulp':>7s} {'floored':>8s} {'max_rel':>10s}"]
    for k in sorted(STATS):
        s = STATS[k]
        out.append(f"{k:58s} {s['n']:12d} {s['max_ulp']:7d} {s['floored']:8d} "
                   f"{s['max_rel']:10.3e}")
    return out
