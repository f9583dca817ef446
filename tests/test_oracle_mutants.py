"""Mutation check for the oracle's pins: plant one plausible mistake at a time
in a copy of oracle.c (on the CPU), build it, and require that at least one
pin in tests/pins.py rejects it.  This shows that the pins constrain every
step of the oracle, not just that the oracle agrees with itself."""
import os
import subprocess

import pytest

import pins

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

# (name, exact snippet in oracle.c, replacement)
MUTANTS = [
    ("sample_variance", "*var = q / (double)H;",
     "*var = q / (double)(H > 1 ? H - 1 : 1);"),
    ("eps_outside_sqrt", "return 1.0 / sqrt(var + eps);",
     "return 1.0 / (sqrt(var) + eps);"),
    ("eps_counted_twice", "return 1.0 / sqrt(var + eps);",
     "return 1.0 / sqrt(var + 2.0 * eps);"),
    ("ln_no_mean_subtraction",
     "double xhat = (xr[j] - mu) * s;\n            yr[j]",
     "double xhat = xr[j] * s;\n            yr[j]"),
    ("ln_beta_dropped", "yr[j] = xhat * gamma[j] + (beta ? beta[j] : 0.0);",
     "yr[j] = xhat * gamma[j];"),
    ("rms_denominator", "return q / (double)H;", "return q / (double)(H + 1);"),
    ("fused_normalizes_x", "double s = rstd_of(row_mean_sq(hr, H), eps);",
     "double s = rstd_of(row_mean_sq(xr, H), eps);"),
    ("ln_bwd_drops_c1", "dxr[j] = s * (g - c1 - xhat * c2);",
     "dxr[j] = s * (g - xhat * c2);"),
    ("ln_bwd_c2_sign", "dxr[j] = s * (g - c1 - xhat * c2);",
     "dxr[j] = s * (g - c1 + xhat * c2);"),
    ("ln_bwd_c1_from_dy", "sg += g;", "sg += dyr[j];"),
    ("rms_bwd_c2_without_gamma",
     "sgx += dyr[j] * gamma[j] * (xr[j] * s);", "sgx += dyr[j] * (xr[j] * s);"),
    ("rms_bwd_missing_rstd", "dxr[j] = s * (g - xhat * c2);",
     "dxr[j] = (g - xhat * c2);"),
    ("dgamma_without_xhat", "g[j - j0] += dyr[j] * xhat;",
     "g[j - j0] += dyr[j];"),
    ("dgamma_uncentered", "double xhat = (xr[j] - mu) * rstd[r];",
     "double xhat = xr[j] * rstd[r];"),
    ("welford_m2_update", "q += d_old * (x[i] - m);", "q += d_old * d_old;"),
    ("merge_drops_delta_term",
     "*m2 = m2a + m2b + d * d * (na * nb / nn);", "*m2 = m2a + m2b;"),
    ("merge_wrong_weight", "*mean = ma + d * (nb / nn);",
     "*mean = ma + d * (na / nn);"),
    ("bf16_truncates", "double r = nearbyint(scaled);",
     "double r = trunc(scaled);"),
    ("bf16_ties_away", "double r = nearbyint(scaled);",
     "double r = round(scaled);"),
    ("bf16_no_subnormal_spacing", "if (k < -126) k = -126;", ";"),
    ("fused_bwd_drops_dh_in",
     "for (int64_t j = 0; j < H; ++j) dxr[j] += dh_in[r * lddh + j];", ";"),
    ("fused_bwd_dh_in_twice",
     "for (int64_t j = 0; j < H; ++j) dxr[j] += dh_in[r * lddh + j];",
     "for (int64_t j = 0; j < H; ++j) dxr[j] += 2.0 * dh_in[r * lddh + j];"),
    ("fused_bwd_c2_sign", "dxr[j] = s * (g - (hr[j] * s) * c2);",
     "dxr[j] = s * (g + (hr[j] * s) * c2);"),
    ("fused_bwd_c2_without_gamma",
     "sgx += dyr[j] * gamma[j] * (hr[j] * s);", "sgx += dyr[j] * (hr[j] * s);"),
    ("f16_truncates", "double r = nearbyint(ldexp(a, -q));",
     "double r = trunc(ldexp(a, -q));"),
    ("f16_no_subnormal_spacing", "if (k < -14) k = -14;", ";"),
    ("f16_no_overflow_to_inf", "if (rv > 65504.0)", "if (rv > 1e300)"),
    ("f16_decode_subnormal_scale", "v = ldexp((double)fr, -24);",
     "v = ldexp((double)fr, -25);"),
    ("f32_truncates", "out[i] = (float)in[i];",
     "{ out[i] = (float)in[i]; if (fabs((double)out[i]) > fabs(in[i])) "
     "out[i] = nextafterf(out[i], 0.0f); }"),
    ("f32_flushes_subnormals", "out[i] = (float)in[i];",
     "out[i] = fabs(in[i]) < 0x1p-126 ? 0.0f : (float)in[i];"),
]


def _build(tmp_path, name, old, new):
    from oracle.build import CFLAGS
    src = open(SRC).read()
    assert src.count(old) == 1, f"snippet for {name} not unique/present"
    mutated = src.replace(old, new)
    c = tmp_path / f"orc_{name}.c"
    so = tmp_path / f"liborc_{name}.so"
    c.write_text(mutated)
    subprocess.run(["gcc", *CFLAGS, str(c), "-o", str(so), "-lm"], check=True,
                   capture_output=True)
    return str(so)


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    import oracle
    orc = oracle.Oracle(_build(tmp_path, name, old, new))
    caught = []
    for check in pins.ALL_CHECKS:
        try:
            check(orc)
        except AssertionError:
            caught.append(check.__name__)
            break
    assert caught, f"no pin rejects mutant {name}"
