"""ln_bwd_noalloc (the LayerNorm backward whose partial rows live in the
library's static per-GPU array) against ln_bwd with a caller workspace,
through the C ABI: bit for bit the same dx, dgamma and dbeta, on two calls
in a row whose second input is smaller (the array keeps the first call's
contents), on the partial-row plans (tall and wide) and the column-sum
strategy (no partial rows).  The first call's result is also checked
against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import tolerance as tol
import rmsnorm_row_welford_amd as rn
from rmsnorm_row_welford_amd import synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _dev(a):
    return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(DEV)


def _case(seed, N, H):
    arr = synth.custom(seed, N, H, "bf16")
    x, dy, g = (_dev(arr[k]) for k in ("x", "dy", "gamma"))
    _, mean, rstd = rn.ln_fwd(x, g, None, 1e-5)
    return arr, x, dy, g, mean, rstd


def _both(x, dy, g, mean, rstd):
    N, H = x.shape
    bf = torch.bfloat16
    ws = torch.empty(max(1, rn.workspace_bytes(N, H, bf, True)), dtype=torch.uint8,
                     device=DEV)
    want = rn.ln_bwd(dy, x, g, mean, rstd, 1e-5, workspace=ws)
    # outputs preallocated and poisoned: the entry point must write them all
    dx = torch.full((N, H), 3.0, dtype=bf, device=DEV)
    dg = torch.full((H,), 3.0, dtype=bf, device=DEV)
    db = torch.full((H,), 3.0, dtype=bf, device=DEV)
    got = rn.ln_bwd_noalloc(dy, x, g, mean, rstd, 1e-5, dx=dx, dgamma=dg, dbeta=db)
    torch.cuda.synchronize()
    assert got[0].data_ptr() == dx.data_ptr()
    return want, got


# (first call, second smaller call): tall rows on the one-workgroup-per-CU
# plans (column-major partial rows), wide rows (row-major partial rows, the
# largest LayerNorm partial set: 256 x 16384 x 2 floats = the array's size),
# a short wide input that takes the column sums (no partial rows), rows
# past the register plans (column sums), and decode sizes (64 rows: partial
# rows of a few workgroups; one row: a single workgroup writes dgamma/dbeta
# itself).
CASES = [((32771, 1024), (4099, 1024)),
         ((4099, 16384), (1000, 2048)),
         ((2048, 16384), (300, 16384)),
         ((37, 32768), (5, 20480)),
         ((64, 4096), (1, 4096))]


@pytest.mark.parametrize("first,second", CASES)
def test_noalloc_matches_workspace_entry_point(orc, first, second):
    for k, (N, H) in enumerate((first, second)):
        print(f"ln_bwd_noalloc call {k + 1}: N={N} H={H}", flush=True)
        arr, x, dy, g, mean, rstd = _case(40 + k + H, N, H)
        want, got = _both(x, dy, g, mean, rstd)
        for w_, g_, name in zip(want, got, ("dx", "dgamma", "dbeta")):
            assert torch.equal(w_, g_), f"call {k + 1} ({N}x{H}): {name} differs"
        if k == 0:
            e = oracle.eps_at_boundary(1e-5)
            xd, dyd, gd = (orc.decode(arr[n], "bf16") for n in ("x", "dy", "gamma"))
            dx_o, dg_o, db_o, _, r_o = orc.ln_bwd(dyd, xd, gd, e)
            tol.check_out(got[0].cpu().view(torch.int16).numpy().view(np.uint16), dx_o,
                          "bf16", orc, "edge: no-alloc LN dx",
                          term_scale=tol.dx_term_scale(dyd, gd, r_o))
            for t, o, name in ((got[1], dg_o, "dgamma"), (got[2], db_o, "dbeta")):
                tol.check_param(orc.decode(t.cpu().view(torch.int16).numpy().view(np.uint16),
                                           "bf16"), o, f"edge: no-alloc LN {name}")


def test_noalloc_rejects_what_does_not_fit():
    """The array holds RN_NOALLOC_MAX_WORKSPACE_BYTES: every register-plan
    shape fits; a long-row shape whose LayerNorm partial rows need more
    (2048 x 32768: 256 partial rows of 32768 floats, twice) is refused with
    RN_EWORKSPACE, leaving the outputs untouched."""
    bf = torch.bfloat16
    cap = 32 << 20
    for H in (1024, 2048, 4096, 8192, 16384):
        assert rn.workspace_bytes(1 << 20, H, bf, True) <= cap
    N, H = 2048, 32768
    assert rn.workspace_bytes(N, H, bf, True) > cap
    x = torch.randn(N, H, device=DEV).to(bf)
    g = torch.ones(H, dtype=bf, device=DEV)
    _, mean, rstd = rn.ln_fwd(x, g, None, 1e-5)
    dx = torch.full((N, H), 3.0, dtype=bf, device=DEV)
    with pytest.raises(rn.RowNormError) as ei:
        rn.ln_bwd_noalloc(x, x, g, mean, rstd, 1e-5, dx=dx)
    assert ei.value.status == -4
    torch.cuda.synchronize()
    assert torch.all(dx == 3.0), "a refused call wrote its output"
