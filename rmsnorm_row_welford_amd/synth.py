"""Seeded synthetic inputs for the row-normalization workloads.

This module only draws numbers: it holds none of the normalization
arithmetic, and both the HIP path's tests and the CPU oracle read the bytes
it produces.

Recipe (per workload): numpy ``Generator(PCG64)`` streams, one child of
``SeedSequence(seed).spawn(6)`` per tensor, in the fixed order
[x, residual, dy, gamma, beta, dh] (child k depends only on seed and k, so a
tensor's values do not depend on which others a workload draws).  Each tensor is a binary64 standard-normal
draw z of its shape, mapped to ``mu + sigma * z`` (or the row-split mixture
for the cancellation workload), then rounded to the storage type: binary32
by numpy's round-to-nearest-even cast, bfloat16 and IEEE binary16 by torch's
CPU cast of that binary32 value (round-to-nearest-even).  bfloat16 and
binary16 arrays are carried as uint16 bit patterns, binary32 as float32.
gamma and beta take the workload's parameter type (``wdtype``, default: the
activation type).

Workloads (sizes and distributions as the normalization pages' benchmark
shapes and test lists describe them):

  ln_f32_64x1000       LayerNorm fwd+bwd, fp32, N=64, H=1000; x, dy ~ N(0,1),
                       gamma = 1 + N(0, 0.1), beta ~ N(0, 0.1), eps 1e-5
  fwd_bf16_8192x1024   LayerNorm and RMSNorm fwd, bf16, N=8192, H=1024;
                       rows [0, N/2) x ~ N(0,1), rows [N/2, N)
                       x = 50 + N(0, 0.01); gamma = 1 + N(0, 0.1); no beta;
                       eps 1e-5
  fused_bf16_32768x4096  fused add+RMSNorm fwd, bf16, (B=16, T=2048) -> N=32768,
                       H=4096; x, residual ~ N(0,1); gamma = 1 + N(0, 0.05);
                       eps 1e-6
  step_bf16_32768x1024  the benchmark step: x, residual, dy ~ N(0,1),
                       gamma = 1 + N(0, 0.1), beta ~ N(0, 0.1), eps 1e-5
  fused_bwd_bf16_32768x4096  fused add+RMSNorm fwd then bwd, bf16, the fused
                       forward's shape; x, residual, dy, dh ~ N(0,1) (dh: the
                       gradient reaching h through the residual stream);
                       gamma = 1 + N(0, 0.05); eps 1e-6
  mixed_bf16_f32w_32768x1024  LayerNorm/RMSNorm/fused fwd+bwd with bf16
                       activations and float32 gamma, beta, dgamma, dbeta;
                       distributions as step_bf16_32768x1024
  f16_32768x1024       the same in IEEE binary16 throughout
  rows_bf16_1048576x128  short rows (a normalization over a 128-wide head
                       dimension of 2^20 token-head rows): LayerNorm and
                       RMSNorm fwd+bwd, bf16, x, dy ~ N(0,1),
                       gamma = 1 + N(0, 0.1), beta ~ N(0, 0.1), eps 1e-5
  bwd_bf16_32768x1024, bwd_bf16_16384x2048  (tall-narrow)
  bwd_bf16_512x16384,  bwd_bf16_2048x16384  (wide)
                       LayerNorm and RMSNorm fwd+bwd, bf16; x, dy ~ N(0,1),
                       gamma = 1 + N(0, 0.1), beta ~ N(0, 0.1), eps 1e-5
"""
from dataclasses import dataclass
from typing import Dict, Optional, Tuple

import numpy as np

ORDER = ("x", "residual", "dy", "gamma", "beta", "dh")


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    N: int
    H: int
    dtype: str                 # activations: "bf16", "f16" or "f32"
    eps: float
    x: Tuple[float, float]     # (mu, sigma) of x
    gamma: Tuple[float, float]
    beta: Optional[Tuple[float, float]]
    residual: Optional[Tuple[float, float]] = None
    dy: Optional[Tuple[float, float]] = (0.0, 1.0)
    half_shifted: Optional[Tuple[float, float]] = None  # rows [N/2, N)
    dh: Optional[Tuple[float, float]] = None
    wdtype: Optional[str] = None   # gamma/beta storage; None = dtype


WORKLOADS: Dict[str, Workload] = {
    w.name: w for w in [
        Workload("ln_f32_64x1000", 1001, 64, 1000, "f32", 1e-5,
                 x=(0.0, 1.0), gamma=(1.0, 0.1), beta=(0.0, 0.1)),
        Workload("fwd_bf16_8192x1024", 1002, 8192, 1024, "bf16", 1e-5,
                 x=(0.0, 1.0), gamma=(1.0, 0.1), beta=None, dy=None,
                 half_shifted=(50.0, 0.01)),
        Workload("fused_bf16_32768x4096", 1003, 32768, 4096, "bf16", 1e-6,
                 x=(0.0, 1.0), gamma=(1.0, 0.05), beta=None,
                 residual=(0.0, 1.0), dy=None),
        Workload("fused_bwd_bf16_32768x4096", 1006, 32768, 4096, "bf16", 1e-6,
                 x=(0.0, 1.0), gamma=(1.0, 0.05), beta=None,
                 residual=(0.0, 1.0), dh=(0.0, 1.0)),
        Workload("bwd_bf16_32768x1024", 1004, 32768, 1024, "bf16", 1e-5,
                 x=(0.0, 1.0), gamma=(1.0, 0.1), beta=(0.0, 0.1)),
        # one full training-style pass at the headline shape: LN and RMS
        # forward, fused add+RMSNorm forward, LN and RMS backward
        Workload("step_bf16_32768x1024", 1004, 32768, 1024, "bf16", 1e-5,
                 x=(0.0, 1.0), gamma=(1.0, 0.1), beta=(0.0, 0.1),
                 residual=(0.0, 1.0)),
        Workload("mixed_bf16_f32w_32768x1024", 1007, 32768, 1024, "bf16", 1e-5,
                 x=(0.0, 1.0), gamma=(1.0, 0.1), beta=(0.0, 0.1),
                 residual=(0.0, 1.0), dh=(0.0, 1.0), wdtype="f32"),
        Workload("f16_32768x1024", 1008, 32768, 1024, "f16", 1e-5,
                 x=(0.0, 1.0), gamma=(1.0, 0.1), beta=(0.0, 0.1),
                 residual=(0.0, 1.0), dh=(0.0, 1.0)),
        Workload("rows_bf16_1048576x128", 1009, 1 << 20, 128, "bf16", 1e-5,
                 x=(0.0, 1.0), gamma=(1.0, 0.1), beta=(0.0, 0.1)),
        Workload("bwd_bf16_16384x2048", 1004, 16384, 2048, "bf16", 1e-5,
                 x=(0.0, 1.0), gamma=(1.0, 0.1), beta=(0.0, 0.1)),
        Workload("bwd_bf16_512x16384", 1005, 512, 16384, "bf16", 1e-5,
                 x=(0.0, 1.0), gamma=(1.0, 0.1), beta=(0.0, 0.1)),
        Workload("bwd_bf16_2048x16384", 1005, 2048, 16384, "bf16", 1e-5,
                 x=(0.0, 1.0), gamma=(1.0, 0.1), beta=(0.0, 0.1)),
        # the other shapes of the backward page's timing table (tall, square
        # and wide), bf16, both norms
        *[Workload(f"bwdtab_bf16_{n}x{h}", 1012 + i, n, h, "bf16", 1e-5,
                   x=(0.0, 1.0), gamma=(1.0, 0.1), beta=(0.0, 0.1))
          for i, (n, h) in enumerate([(8192, 1024), (16384, 1024), (2048, 4096),
                                      (4096, 4096), (8192, 4096), (1024, 8192)])],
        # rows past the register-resident plans: one that the LDS row cache
        # holds (x and dy of a 32768-element bf16 row: 128 KiB), one that no
        # cache holds (256 KiB rows, read twice)
        Workload("long_bf16_2048x32768", 1010, 2048, 32768, "bf16", 1e-5,
                 x=(0.0, 1.0), gamma=(1.0, 0.1), beta=(0.0, 0.1),
                 residual=(0.0, 1.0)),
        Workload("long_bf16_256x131072", 1011, 256, 131072, "bf16", 1e-5,
                 x=(0.0, 1.0), gamma=(1.0, 0.1), beta=(0.0, 0.1)),
    ]
}


def to_storage(a64: np.ndarray, dtype: str) -> np.ndarray:
    """Round a binary64 draw to the storage type (see module docstring)."""
    a32 = np.asarray(a64, dtype=np.float64).astype(np.float32)
    if dtype == "f32":
        return a32
    if dtype in ("bf16", "f16"):
        import torch
        tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
        t = torch.from_numpy(np.ascontiguousarray(a32)).to(tdt)
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    raise ValueError(f"unknown dtype {dtype!r}")


def _streams(seed: int):
    kids = np.random.SeedSequence(seed).spawn(len(ORDER))
    return {name: np.random.Generator(np.random.PCG64(k))
            for name, k in zip(ORDER, kids)}


def generate(w: Workload, N: Optional[int] = None, H: Optional[int] = None,
             seed: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Storage-typed arrays for workload ``w`` (optionally at another shape
    or seed, same distributions).  Keys present: x, gamma, and whichever of
    residual, dy, beta, dh the workload has."""
    N = w.N if N is None else N
    H = w.H if H is None else H
    rng = _streams(w.seed if seed is None else seed)
    out = {}
    z = rng["x"].standard_normal((N, H))
    xv = w.x[0] + w.x[1] * z
    if w.half_shifted is not None:
        lo = N // 2
        xv[lo:] = w.half_shifted[0] + w.half_shifted[1] * z[lo:]
    out["x"] = to_storage(xv, w.dtype)
    if w.residual is not None:
        mu, sd = w.residual
        out["residual"] = to_storage(
            mu + sd * rng["residual"].standard_normal((N, H)), w.dtype)
    if w.dy is not None:
        mu, sd = w.dy
        out["dy"] = to_storage(mu + sd * rng["dy"].standard_normal((N, H)),
                               w.dtype)
    wdt = w.wdtype or w.dtype
    mu, sd = w.gamma
    out["gamma"] = to_storage(mu + sd * rng["gamma"].standard_normal(H), wdt)
    if w.beta is not None:
        mu, sd = w.beta
        out["beta"] = to_storage(mu + sd * rng["beta"].standard_normal(H), wdt)
    if w.dh is not None:
        mu, sd = w.dh
        out["dh"] = to_storage(mu + sd * rng["dh"].standard_normal((N, H)),
                               w.dtype)
    return out


def device_normal(seed: int, shape, mu: float, sigma: float, dtype: str, device,
                  chunk_rows: int = 1 << 18):
    """A seeded draw made on the GPU, for tensors too large to draw on the
    host: ``mu + sigma * z`` with z from torch's generator for ``device``
    seeded with ``seed`` (binary32 standard normals, drawn in blocks of
    ``chunk_rows`` rows), rounded to the storage type by torch's cast
    (round-to-nearest-even).  Returns a torch tensor of that type on
    ``device``; the same seed and shape give the same bytes."""
    import torch
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[dtype]
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    out = torch.empty(shape, dtype=tdt, device=device)
    flat = out.view(-1, shape[-1]) if len(shape) > 1 else out.view(1, -1)
    for r0 in range(0, flat.shape[0], chunk_rows):
        r1 = min(r0 + chunk_rows, flat.shape[0])
        z = torch.randn((r1 - r0, flat.shape[1]), generator=gen, device=device,
                        dtype=torch.float32)
        flat[r0:r1] = (mu + sigma * z).to(tdt)
    return out


def custom(seed: int, N: int, H: int, dtype: str, x=(0.0, 1.0),
           gamma=(1.0, 0.1), beta=(0.0, 0.1), residual=(0.0, 1.0),
           dy=(0.0, 1.0), half_shifted=None, dh=(0.0, 1.0), wdtype=None
           ) -> Dict[str, np.ndarray]:
    """Arrays for an ad-hoc shape (edge cases, ragged tails)."""
    w = Workload("custom", seed, N, H, dtype, 1e-5, x=x, gamma=gamma,
                 beta=beta, residual=residual, dy=dy,
                 half_shifted=half_shifted, dh=dh, wdtype=wdtype)
    return generate(w)
