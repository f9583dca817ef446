"""Parity bars between the HIP path and the binary64 oracle.

bf16 and fp16 outputs (same rule, each in its own format; for fp16 the
  ulp is 2^-11..2^-10 * |v| and the floor below still sits far above the
  float32 pipeline's error):
  the GPU value must be within 1 ulp of the correctly
  rounded oracle value (distance measured on the ordered integer image of the
  bit patterns, +0 == -0), or, for values produced by cancellation, within an
  absolute floor of 2^-16 times the row's scale.  The float32 pipeline's own
  error is a few float32 ulps of the scale of the terms that cancel (about
  2^-22 * scale); a bf16 ulp at |v| is 2^-8..2^-7 * |v|, so only outputs far
  below that scale can need the floor.  The row scale is the RMS of the
  oracle output, or for dx the larger of that and rstd * RMS(dy * gamma):
  dx = rstd * (g - c1 - x_hat * c2) is a difference of terms of size
  rstd * |g|, and for short rows it can cancel almost completely (H = 1
  RMSNorm: dx = rstd * g * eps / (x^2 + eps)).
fp32 outputs: |gpu - oracle| <= 1e-5 * max(|oracle|, row scale).
mean (fp32): |gpu - oracle| <= 1e-5 * max(|mean|, sqrt(var + eps)).
rstd (fp32): relative 1e-5.
dgamma/dbeta: relative RMS error ||gpu - oracle|| / ||oracle|| <= 5e-3.
h of the fused op: bit-exact to RNE(x + residual).
"""
import numpy as np

BF16_FLOOR = 2.0 ** -16
F32_REL = 1e-5
PARAM_REL_RMS = 5e-3


def ordered(bits_u16: np.ndarray) -> np.ndarray:
    """Map bfloat16 / binary16 bit patterns (sign-magnitude) to integers
    ordered like their values."""
    b = bits_u16.astype(np.int32)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def row_rms(v: np.ndarray) -> np.ndarray:
    v = np.atleast_2d(v)
    return np.sqrt(np.mean(v * v, axis=1, keepdims=True))


def _scale(oracle_vals, term_scale):
    s = row_rms(oracle_vals)
    if term_scale is not None:
        s = np.maximum(s, np.asarray(term_scale, dtype=np.float64).reshape(-1, 1))
    return s


def check_bf16(gpu_bits, oracle_vals, orc, what, term_scale=None, dtype="bf16"):
    """gpu_bits: uint16 [N, H] (bf16, or fp16 with dtype="f16");
    oracle_vals: float64 [N, H] (unrounded); term_scale: optional per-row
    scale of the terms that cancel."""
    gpu_bits = np.atleast_2d(gpu_bits)
    oracle_vals = np.atleast_2d(oracle_vals)
    want = orc.encode(oracle_vals, dtype)
    ulp = np.abs(ordered(gpu_bits) - ordered(want))
    gv = orc.decode(gpu_bits, dtype)
    floor = BF16_FLOOR * _scale(oracle_vals, term_scale)
    ok = (ulp <= 1) | (np.abs(gv - oracle_vals) <= floor)
    bad = np.argwhere(~ok)
    if bad.size:
        i, j = bad[0]
        raise AssertionError(
            f"{what}: {len(bad)} of {ok.size} elements off; first at "
            f"[{i},{j}] gpu={gv[i, j]!r} oracle={oracle_vals[i, j]!r} "
            f"ulp={ulp[i, j]}")
    return {"max_ulp": int(ulp.max()) if ulp.size else 0,
            "floored": int(np.sum((ulp > 1) & ok))}


def check_f32(gpu, oracle_vals, what, rel=F32_REL, term_scale=None):
    gpu = np.atleast_2d(np.asarray(gpu, dtype=np.float64))
    oracle_vals = np.atleast_2d(oracle_vals)
    scale = np.maximum(np.abs(oracle_vals), _scale(oracle_vals, term_scale))
    err = np.abs(gpu - oracle_vals)
    ok = err <= rel * scale
    bad = np.argwhere(~ok)
    if bad.size:
        i, j = bad[0]
        raise AssertionError(
            f"{what}: {len(bad)} of {ok.size} off; first at [{i},{j}] "
            f"gpu={gpu[i, j]!r} oracle={oracle_vals[i, j]!r}")
    return float(np.max(err / np.maximum(scale, 1e-300))) if err.size else 0.0


def check_out(gpu_host, oracle_vals, dtype, orc, what, term_scale=None):
    if dtype in ("bf16", "f16"):
        return check_bf16(gpu_host, oracle_vals, orc, what, term_scale, dtype)
    return check_f32(gpu_host, oracle_vals, what, term_scale=term_scale)


def dx_term_scale(dy, gamma, rstd):
    """Per-row scale of the terms dx is the difference of: rstd*RMS(dy*gamma)."""
    g = np.atleast_2d(dy) * np.asarray(gamma)[None, :]
    return np.asarray(rstd) * np.sqrt(np.mean(g * g, axis=1))


def check_mean(gpu, mean_o, var_o, eps, what):
    gpu = np.asarray(gpu, dtype=np.float64)
    scale = np.maximum(np.abs(mean_o), np.sqrt(var_o + eps))
    err = np.abs(gpu - mean_o)
    assert np.all(err <= F32_REL * scale), \
        f"{what}: max scaled err {np.max(err / scale):.3e}"


def check_rstd(gpu, rstd_o, what):
    gpu = np.asarray(gpu, dtype=np.float64)
    rel = np.abs(gpu - rstd_o) / np.abs(rstd_o)
    assert np.all(rel <= F32_REL), f"{what}: max rel err {rel.max():.3e}"


def check_param(gpu_vals, oracle_vals, what):
    gpu_vals = np.asarray(gpu_vals, dtype=np.float64)
    num = np.linalg.norm(gpu_vals - oracle_vals)
    den = np.linalg.norm(oracle_vals)
    rr = num / den if den > 0 else num
    assert rr <= PARAM_REL_RMS, f"{what}: rel-rms {rr:.3e}"
    return rr
