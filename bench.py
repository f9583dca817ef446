"""Benchmark: one step = the whole row-normalization hot path over one batch
at the headline shape (bf16, N=32768 rows, H=1024):

    LayerNorm fwd (y, mean, rstd)  ->  RMSNorm fwd (y, rstd)
    -> fused residual-add + RMSNorm fwd (y, h, rstd)
    -> LayerNorm bwd (dx, dgamma, dbeta)  ->  RMSNorm bwd (dx, dgamma)

Inputs are synthetic (rmsnorm_row_welford_amd.synth, workload
step_bf16_32768x1024) and resident in HBM before timing.

Cold data without cache sweeps: the step's tensors exist in M = 6 copies
("sets", about 3.4 GiB) and consecutive ops use consecutive sets, so every
launch reads data last touched about 1 GiB of traffic earlier, far beyond
the 256 MB Infinity Cache and 32 MB of L2.  The K timed steps run back to
back between two HIP events on the launch stream (ms_per_step = elapsed/K).
The per-op table times K launches of one op back to back over the rotating
sets, captured once in a HIP graph and replayed, each replay between two
events on the launch stream (median of 5): kernel time plus the gaps
between launches, without the per-call Python/ctypes overhead that would
otherwise exceed the kernel time of the small shapes; "us_eager" is the
same K launches issued one by one from Python.  --sweep adds the isolated
protocol (a 512 MiB read sweep before each op, events around the op alone),
which also pays each op's launch latency.

value = the step's algorithmic HBM bytes / ms_per_step.  Prints ONE JSON line
on stdout (diagnostics go to stderr).  One GPU only.

Outside the step, per_op also times (same protocol, same shape):
  fused_add_rms_bwd        the fused op's backward: dx from dy, the stored h,
                           the saved rstd and a residual-stream gradient dh_in
  fused_add_rms_fwd_inplace  the fused forward writing h over the residual
  unfused_add_rms          the unfused comparison: the library's add kernel
                           (h = x + r) then rms_fwd on h, 5 N H e bytes

shapes (not in the step): every op at the other workload shapes (16384x2048,
512x16384, 2048x16384 forward and backward; 8192x1024 forward without a
bias; the fused forward at 32768x4096), the other storage pairs at
32768x1024 (binary16 throughout; bf16 with float32 parameters: all six
ops) and short rows (1048576x128 forward and backward), each with enough
rotating copies that its data comes from HBM.  --shapes-only NAME[,NAME]
(or all) times just those and prints their table.  Each shape row also
carries the library copy's GB/s at that shape's own tensor size
(copy_same_size_GBps: launch and ramp weigh more on small tensors) and
each op's share of it (pct_copy_same_size).

decode (not in the step): the latency regime of a few rows (N = 1, 16, 64
at H = 4096, bf16, data in cache), every op, forward and backward: 50
back-to-back calls captured in one HIP graph and replayed, GPU time per call
(launch gaps included, host overhead excluded).
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_GBS = 8000.0          # MI355X HBM3E, published
WORKLOAD = "step_bf16_32768x1024"
FUSED_EPS = 1e-6
OPS = ("ln_fwd", "rms_fwd", "fused_add_rms_fwd", "ln_bwd", "rms_bwd")
EXTRA_OPS = ("fused_add_rms_bwd", "fused_add_rms_fwd_inplace", "unfused_add_rms")
# The other workload shapes of the normalization pages' test and benchmark
# lists, timed op by op outside the step (same cold protocol): tall-narrow
# and wide backward shapes (with the forwards at those shapes), the
# bias-free forward with half its rows constant, and the fused forward at
# (B=16, T=2048, H=4096).
# Beyond those: the other storage pairs at the headline shape (IEEE
# binary16 throughout; bf16 activations with float32 gamma/beta and their
# gradients) and short rows (2^20 rows of 128: a normalization over a head
# dimension), each for every op they have a workload for, and rows past the
# register-resident plans (32768 elements: cached in LDS between the two
# passes; 131072: read twice), and the other shapes of the backward page's
# timing table (8192x1024 ... 1024x8192).
NORM_OPS = ("ln_fwd", "rms_fwd", "ln_bwd", "rms_bwd")
ALL_OPS = NORM_OPS + ("fused_add_rms_fwd", "fused_add_rms_bwd")
SHAPES = (
    ("bwd_bf16_16384x2048", NORM_OPS),
    ("bwd_bf16_512x16384", NORM_OPS),
    ("bwd_bf16_2048x16384", NORM_OPS),
    ("fwd_bf16_8192x1024", ("ln_fwd", "rms_fwd")),
    ("fused_bf16_32768x4096", ("fused_add_rms_fwd",)),
    ("f16_32768x1024", ALL_OPS),
    ("mixed_bf16_f32w_32768x1024", ALL_OPS),
    ("rows_bf16_1048576x128", NORM_OPS),
    ("long_bf16_2048x32768", NORM_OPS + ("fused_add_rms_fwd",)),
    ("long_bf16_256x131072", NORM_OPS),
) + tuple((f"bwdtab_bf16_{n}x{h}", NORM_OPS)
          for n, h in ((8192, 1024), (16384, 1024), (2048, 4096), (4096, 4096), (8192, 4096),
                       (1024, 8192)))


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def alg_bytes(N, H, e, beta=True, ep=None):
    """Algorithmic HBM bytes of each op: every tensor read or written once.
    e: bytes per activation element; ep: per parameter element (gamma, beta
    and their gradients; default e); beta=False: LayerNorm without a bias."""
    ep = e if ep is None else ep
    return {
        "ln_fwd": 2 * N * H * e + (2 if beta else 1) * H * ep + 8 * N,  # x,y,gamma,beta,stats
        "rms_fwd": 2 * N * H * e + H * ep + 4 * N,             # x,y,gamma,rstd
        "fused_add_rms_fwd": 4 * N * H * e + H * ep + 4 * N,   # x,r,h,y,gamma,rstd
        "ln_bwd": 3 * N * H * e + 3 * H * ep + 8 * N,          # dy,x,dx,gamma,dg,db,stats
        "rms_bwd": 3 * N * H * e + 2 * H * ep + 4 * N,         # dy,x,dx,gamma,dg,rstd
        "fused_add_rms_bwd": 4 * N * H * e + 2 * H * ep + 4 * N,  # dy,h,dh_in,dx,gamma,dg,rstd
        "fused_add_rms_fwd_inplace": 4 * N * H * e + H * ep + 4 * N,
        # add: x, r read, h written; rms_fwd: h read, y written
        "unfused_add_rms": 5 * N * H * e + H * ep + 4 * N,
    }


_TORCH_DT = {"bf16": "bfloat16", "f16": "float16", "f32": "float32"}
_ESIZE = {"bf16": 2, "f16": 2, "f32": 4}


def counters_traffic(op, shape_tag):
    """HBM traffic per launch from the committed rocprofv3 counter summary,
    if it was taken on the current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", f"{op}_{shape_tag}.counters.json")
    if not os.path.exists(path):
        return None
    try:
        d = json.load(open(path))
    except Exception:
        return None
    from rmsnorm_row_welford_amd.profsum import kernel_source_digest
    if d.get("kernel_source_digest") != kernel_source_digest():
        return None
    return d.get("traffic_bytes_per_launch")


# what each op reads (inputs) and writes (outputs), by tensor key
_OP_INPUTS = {
    "ln_fwd": ("x",), "rms_fwd": ("x",), "fused_add_rms_fwd": ("x", "r"),
    "ln_bwd": ("x", "dy"), "rms_bwd": ("x", "dy"),
    "fused_add_rms_bwd": ("x", "r", "dy", "dh"),
    "fused_add_rms_fwd_inplace": ("x", "r_in"), "unfused_add_rms": ("x", "r"),
}
_OP_ROWS_OUT = {
    "ln_fwd": ("y",), "rms_fwd": ("y2",), "fused_add_rms_fwd": ("y3", "h"),
    "ln_bwd": ("dx",), "rms_bwd": ("dx2",), "fused_add_rms_bwd": ("dx3",),
    "fused_add_rms_fwd_inplace": ("y4",), "unfused_add_rms": ("y5", "h5"),
}
_OP_STATS_OUT = {
    "ln_fwd": ("mean", "rstd"), "rms_fwd": ("rstd2",), "fused_add_rms_fwd": ("rstd3",),
    "fused_add_rms_fwd_inplace": ("rstd4",), "unfused_add_rms": ("rstd5",),
}
# the forward whose saved statistics (and h) a backward op reads
_BWD_NEEDS_FWD = {"ln_bwd": "ln_fwd", "rms_bwd": "rms_fwd",
                  "fused_add_rms_bwd": "fused_add_rms_fwd"}


class Sets:
    """M copies of the tensors the given ops touch, on the GPU, and the ops
    bound to one copy each.  The forwards whose saved statistics a backward
    op reads run once per copy at set-up."""

    def __init__(self, rn, arr, eps, M, dev, ops, dtype="bf16", wdtype=None):
        import torch
        self.rn, self.eps, self.M = rn, eps, M
        bf = getattr(torch, _TORCH_DT[dtype])
        wt = getattr(torch, _TORCH_DT[wdtype or dtype])
        N, H = arr["x"].shape
        ops = list(ops)
        pre = [_BWD_NEEDS_FWD[o] for o in ops if o in _BWD_NEEDS_FWD]
        every = list(dict.fromkeys(pre + ops))

        def to_dev(a, t=bf):
            if a.dtype == np.uint16:      # 16-bit storage carried as bit patterns
                return torch.from_numpy(a.view(np.int16)).view(t).to(dev)
            return torch.from_numpy(a).to(dev)

        src = {"x": "x", "r": "residual", "r_in": "residual", "dy": "dy", "dh": "dy"}
        need_in = {k for o in every for k in _OP_INPUTS[o]}
        dev_src = {name: to_dev(arr[name]) for name in {src[k] for k in need_in}}
        base = {k: dev_src[src[k]] for k in need_in}
        self.g = to_dev(arr["gamma"], wt)
        self.b = to_dev(arr["beta"], wt) if "beta" in arr else None
        ws = {}
        if "ln_bwd" in ops:
            ws["ws_ln"] = rn.workspace_bytes(N, H, bf, True, wt)
        if "rms_bwd" in ops or "fused_add_rms_bwd" in ops:
            ws["ws_rms"] = rn.workspace_bytes(N, H, bf, False, wt)
        self.s = []
        for _ in range(M):
            t = {k: base[k].clone() for k in need_in}
            for o in every:
                for k in _OP_ROWS_OUT[o]:
                    t[k] = torch.empty((N, H), dtype=bf, device=dev)
                for k in _OP_STATS_OUT.get(o, ()):
                    t[k] = torch.empty(N, dtype=torch.float32, device=dev)
            for k in ("dg", "db", "dg2", "dg3"):
                t[k] = torch.empty(H, dtype=wt, device=dev)
            for k, nb in ws.items():
                t[k] = torch.empty(nb, dtype=torch.uint8, device=dev)
            self.s.append(t)
        del base, dev_src
        for i in range(M):       # saved statistics (and h) for the backward ops
            for o in dict.fromkeys(pre):
                self.run(o, i)

    def run(self, op, i):
        rn, t, g, b, eps = self.rn, self.s[i % self.M], self.g, self.b, self.eps
        if op == "ln_fwd":
            rn.ln_fwd(t["x"], g, b, eps, y=t["y"], mean=t["mean"], rstd=t["rstd"])
        elif op == "rms_fwd":
            rn.rms_fwd(t["x"], g, eps, y=t["y2"], rstd=t["rstd2"])
        elif op == "fused_add_rms_fwd":
            rn.fused_add_rms_fwd(t["x"], t["r"], g, FUSED_EPS, y=t["y3"], h=t["h"],
                                 rstd=t["rstd3"])
        elif op == "ln_bwd":
            rn.ln_bwd(t["dy"], t["x"], g, t["mean"], t["rstd"], eps, dx=t["dx"],
                      dgamma=t["dg"], dbeta=t["db"], workspace=t["ws_ln"])
        elif op == "rms_bwd":
            rn.rms_bwd(t["dy"], t["x"], g, t["rstd2"], eps, dx=t["dx2"],
                       dgamma=t["dg2"], workspace=t["ws_rms"])
        elif op == "fused_add_rms_bwd":
            rn.fused_add_rms_bwd(t["dy"], t["h"], g, t["rstd3"], FUSED_EPS,
                                 dh_in=t["dh"], dx=t["dx3"], dgamma=t["dg3"],
                                 workspace=t["ws_rms"])
        elif op == "fused_add_rms_fwd_inplace":
            rn.fused_add_rms_fwd(t["x"], t["r_in"], g, FUSED_EPS, y=t["y4"],
                                 h=t["r_in"], rstd=t["rstd4"])
        elif op == "unfused_add_rms":
            rn.add(t["x"], t["r"], out=t["h5"])
            rn.rms_fwd(t["h5"], g, FUSED_EPS, y=t["y5"], rstd=t["rstd5"])
        else:
            raise ValueError(op)


def time_steps(sets, ops, K, W):
    """ms per step: K steps back to back, consecutive ops on consecutive sets."""
    import torch
    stream = torch.cuda.current_stream()
    n = len(ops)
    for s in range(W):
        for j, op in enumerate(ops):
            sets.run(op, s * n + j)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for s in range(K):
        for j, op in enumerate(ops):
            sets.run(op, (W + s) * n + j)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return e0.elapsed_time(e1) / K, wall * 1e3 / K


def time_op(sets, op, K, reps=3):
    """us per launch of one op: K launches back to back over rotating sets,
    median over `reps` timed groups."""
    import torch
    stream = torch.cuda.current_stream()
    for i in range(sets.M):
        sets.run(op, i)
    out = []
    for r in range(reps):
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(K):
            sets.run(op, i)
        e1.record(stream)
        torch.cuda.synchronize()
        out.append(e0.elapsed_time(e1) * 1e3 / K)
    return float(np.median(out)), out


def time_op_graph(sets, op, K, reps=5):
    """us per launch of one op with the host out of the loop: K launches
    over the rotating sets captured once in a HIP graph; each of `reps`
    replays is timed between two events on the launch stream (kernels and
    the gaps between them, no per-call host overhead); the median."""
    import torch
    for i in range(sets.M):
        sets.run(op, i)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(K):
            sets.run(op, i)
    graph.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    out = []
    for _ in range(reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        graph.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        out.append(e0.elapsed_time(e1) * 1e3 / K)
    del graph
    return float(np.median(out))


def time_op_swept(sets, op, K, sweep):
    """Isolated protocol: read sweep of 512 MiB, then events around one op."""
    import torch
    stream = torch.cuda.current_stream()
    ms = []
    for i in range(K + 2):
        sweep.sum()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        sets.run(op, i)
        e1.record(stream)
        if i >= 2:
            ms.append((e0, e1))
    torch.cuda.synchronize()
    return float(np.median([a.elapsed_time(b) for a, b in ms])) * 1e3


def time_shapes(rn, dev, names=None, cold_bytes=1 << 30, K=24, only_ops=None):
    """Per-op times at the other workload shapes: for each, enough rotating
    copies that consecutive launches touch data last used about `cold_bytes`
    of traffic earlier (so it comes from HBM), K launches back to back.
    names: workloads to time (any synth workload; default: the SHAPES
    table); only_ops: restrict each workload to these ops (used to profile
    one op of one shape per kernel trace)."""
    import torch
    from rmsnorm_row_welford_amd import synth
    out = {}
    table = dict(SHAPES)
    todo = SHAPES if names is None else [(n, table.get(n, NORM_OPS)) for n in names]
    for name, ops in todo:
        if only_ops is not None:
            allowed = table.get(name, ALL_OPS)
            ops = tuple(o for o in only_ops if o in allowed)
            if not ops:
                continue
        w = synth.WORKLOADS[name]
        arr = synth.generate(w)
        N, H = w.N, w.H
        nb = alg_bytes(N, H, _ESIZE[w.dtype], beta="beta" in arr,
                       ep=_ESIZE[w.wdtype or w.dtype])
        per_launch = min(nb[o] for o in ops)
        M = int(min(32, max(3, -(-cold_bytes // per_launch) + 1)))
        sets = Sets(rn, arr, w.eps, M, dev, ops, w.dtype, w.wdtype)
        row = {"N": N, "H": H, "dtype": w.dtype, "param_dtype": w.wdtype or w.dtype,
               "sets": M}
        for k in ops:
            us = time_op_graph(sets, k, max(K, 2 * M))
            us_eager, _ = time_op(sets, k, max(K, 2 * M))
            gbs = nb[k] / (us * 1e-6) / 1e9
            row[k] = {"us": round(us, 3), "us_eager": round(us_eager, 3),
                      "alg_bytes": nb[k], "GBps": round(gbs, 1),
                      "pct_peak": round(100 * gbs / PEAK_GBS, 2)}
            log(f"{name:24s} {k:18s} {us:8.2f} us  {gbs:7.0f} GB/s  "
                f"{100 * gbs / PEAK_GBS:5.1f}% of peak")
        out[name] = row
        del sets, arr
        torch.cuda.empty_cache()
    return out


def bwd_plan(rn, N, H, dtype, wdtype, op, cus):
    """The backward's dgamma/dbeta reduction at (N, H) as the library sizes
    it: the partial rows its workspace holds (P_eff; 0 when none are needed:
    the column sums of the rows, or one workgroup writing dgamma/dbeta
    itself) and P_eff per CU (k)."""
    import torch
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}
    p = rn.bwd_partial_rows(N, H, tdt[dtype], op == "ln_bwd",
                            param_dtype=tdt[wdtype or dtype])
    return {"partial_rows": p, "per_cu": round(p / cus, 3),
            "reduction": "partial rows + kernel 2" if p else
                         "column sums or one workgroup (no partial rows)"}


def annotate(rn, dev, table, N, H, dtype, wdtype, copy_gbs):
    """Adds to each op's entry its share of the copy ceiling measured in
    the same run and, for the backward ops, the reduction's plan."""
    import torch
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    for k, v in table.items():
        if not isinstance(v, dict) or "GBps" not in v:
            continue
        v["pct_copy_ceiling"] = round(100 * v["GBps"] / copy_gbs, 1)
        if k in ("ln_bwd", "rms_bwd", "fused_add_rms_bwd"):
            v.update(bwd_plan(rn, N, H, dtype, wdtype, k, cus))


def decode_latency(rn, dev, H=4096, Ns=(1, 16, 64), K=50, reps=5):
    """us per call of every op at decode-size N, from graph replays (data in
    cache, so this is the launch-bound regime: kernels plus the gaps between
    them)."""
    import torch
    bf = torch.bfloat16
    out = {}
    for N in Ns:
        x = torch.randn(N, H, device=dev).to(bf)
        r = torch.randn(N, H, device=dev).to(bf)
        dy = torch.randn(N, H, device=dev).to(bf)
        g = (1 + 0.1 * torch.randn(H, device=dev)).to(bf)
        y, h, dx = torch.empty_like(x), torch.empty_like(x), torch.empty_like(x)
        rstd = torch.empty(N, dtype=torch.float32, device=dev)
        mean = torch.empty(N, dtype=torch.float32, device=dev)
        dg, db = torch.empty_like(g), torch.empty_like(g)
        rn.ln_fwd(x, g, None, 1e-6, y=y, mean=mean, rstd=rstd)
        ws = torch.empty(max(1, rn.workspace_bytes(N, H, bf, True),
                             rn.workspace_bytes(N, H, bf, False)),
                         dtype=torch.uint8, device=dev)
        ops = {
            "rms_fwd": lambda: rn.rms_fwd(x, g, 1e-6, y=y, rstd=rstd),
            "ln_fwd": lambda: rn.ln_fwd(x, g, None, 1e-6, y=y, rstd=rstd,
                                        save_stats=False),
            "fused_add_rms_fwd": lambda: rn.fused_add_rms_fwd(x, r, g, 1e-6, y=y,
                                                              h=h, rstd=rstd),
            "ln_bwd": lambda: rn.ln_bwd(dy, x, g, mean, rstd, 1e-6, dx=dx, dgamma=dg,
                                        dbeta=db, workspace=ws),
            "rms_bwd": lambda: rn.rms_bwd(dy, x, g, rstd, 1e-6, dx=dx, dgamma=dg,
                                          workspace=ws),
            "fused_add_rms_bwd": lambda: rn.fused_add_rms_bwd(
                dy, h, g, rstd, 1e-6, dh_in=r, dx=dx, dgamma=dg, workspace=ws),
        }
        for name, f in ops.items():
            f()
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                for _ in range(K):
                    f()
            graph.replay()
            torch.cuda.synchronize()
            stream = torch.cuda.current_stream()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                graph.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            out[f"{name}:{N}x{H}"] = round(e0.elapsed_time(e1) * 1e3 / (reps * K), 3)
            del graph
    return out


def stream_ceilings(rn, dev, nbytes=64 << 20, cold_bytes=1 << 30, K=24, reps=5,
                    kinds=("copy", "add")):
    """Plain streams measured like the ops: K launches over rotating buffers
    of `nbytes` (the step's tensor size) captured in a HIP graph, each replay
    timed between events on the launch stream, the median of `reps`.
    copy: one read and one write stream (the library's 16-byte copy); add:
    two reads and one write (the library's add over bf16 elements).  GB/s
    over the bytes read and written."""
    import torch
    M = int(max(3, -(-cold_bytes // (2 * nbytes)) + 1))
    bufs = [torch.ones(nbytes, dtype=torch.uint8, device=dev) for _ in range(3 * M)]
    bf = [b.view(torch.bfloat16) for b in bufs]

    def run(kind, i):
        j = 3 * (i % M)
        if kind == "copy":
            rn.copy(bufs[j], bufs[j + 1])
        else:
            rn.add(bf[j], bf[j + 1], out=bf[j + 2])

    out = {}
    stream = torch.cuda.current_stream()
    for kind, moved in (("copy", 2 * nbytes), ("add", 3 * nbytes)):
        if kind not in kinds:
            continue
        for i in range(M):
            run(kind, i)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(K):
                run(kind, i)
        graph.replay()
        torch.cuda.synchronize()
        us = []
        for _ in range(reps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            graph.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            us.append(e0.elapsed_time(e1) * 1e3 / K)
        del graph
        t = float(np.median(us))
        out[kind] = {"us": round(t, 3), "bytes": moved,
                     "GBps": round(moved / (t * 1e-6) / 1e9, 1)}
    del bufs, bf
    return out


def same_size_ceilings(rn, dev, shapes):
    """For each shape row: the library copy's GB/s at that shape's own
    tensor size (one read and one write stream of N*H*e bytes, same cold
    protocol), and each op's share of it.  Small tensors pay the launch and
    the ramp of the memory system on fewer bytes: this is what a plain
    one-pass stream of that size reaches, context rather than a bound (a
    persistent kernel can do better there)."""
    cache = {}
    for name, row in (shapes or {}).items():
        nb = row["N"] * row["H"] * _ESIZE[row["dtype"]]
        if nb not in cache:
            cache[nb] = stream_ceilings(rn, dev, nbytes=nb, kinds=("copy",))["copy"]["GBps"]
            log(f"copy at {nb >> 20} MiB per tensor: {cache[nb]:.0f} GB/s")
        row["copy_same_size_GBps"] = cache[nb]
        for v in row.values():
            if isinstance(v, dict) and "GBps" in v:
                v["pct_copy_same_size"] = round(100 * v["GBps"] / cache[nb], 1)


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo) and logical CPU count."""
    name = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                name = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return name, os.cpu_count()


def cpu_baseline(arr, eps, budget_s=12.0, budget_1t_s=8.0):
    """The oracle as it stands, on the host cores, on a bounded row sample of
    the same workload; GB/s over the sample's algorithmic bytes.  Timed with
    the oracle's default OpenMP thread count, then with one thread."""
    import oracle
    orc = oracle.default()
    N, H = arr["x"].shape
    e = oracle.eps_at_boundary(eps)
    ef = oracle.eps_at_boundary(FUSED_EPS)

    def one_pass(n):
        t0 = time.perf_counter()
        x = orc.decode(arr["x"][:n], "bf16")
        r = orc.decode(arr["residual"][:n], "bf16")
        dy = orc.decode(arr["dy"][:n], "bf16")
        g = orc.decode(arr["gamma"], "bf16")
        b = orc.decode(arr["beta"], "bf16")
        y, m, s = orc.ln_fwd(x, g, b, e)
        orc.encode(y, "bf16")
        y, s = orc.rms_fwd(x, g, e)
        orc.encode(y, "bf16")
        y, h, s = orc.fused_add_rms_fwd(x, r, g, ef)
        orc.encode(y, "bf16")
        orc.encode(h, "bf16")
        dx, dg, db, _, _ = orc.ln_bwd(dy, x, g, e)
        orc.encode(dx, "bf16")
        orc.encode(dg, "bf16")
        orc.encode(db, "bf16")
        dx, dg, _ = orc.rms_bwd(dy, x, g, e)
        orc.encode(dx, "bf16")
        orc.encode(dg, "bf16")
        return time.perf_counter() - t0

    def measure(budget):
        probe_rows = min(N, 256)
        per_row = one_pass(probe_rows) / probe_rows
        rows = int(min(N, max(probe_rows, budget / 3.0 / max(per_row, 1e-9))))
        t = float(np.median([one_pass(rows) for _ in range(3)]))
        return rows, t, sum(alg_bytes(rows, H, 2).values()) / t / 1e9

    threads = orc.num_threads()
    rows, t, gbs = measure(budget_s)
    orc.set_threads(1)
    rows1, t1, gbs1 = measure(budget_1t_s)
    orc.set_threads(threads)
    model, ncpu = cpu_model()
    return {
        "value": gbs,
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{rows} of {N} rows x H={H}: the full five-op step (bf16 "
                  f"decode/encode included), median of 3 passes, "
                  f"{t * 1e3:.1f} ms per pass on {threads} OpenMP threads",
        "one_thread": {"value": gbs1, "unit": "GB/s", "cores": 1,
                       "sample": f"{rows1} rows, median of 3 passes, "
                                 f"{t1 * 1e3:.1f} ms per pass"},
        "cpu_model": model,
        "logical_cpus": ncpu,
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--sets", type=int, default=6)
    ap.add_argument("--sweep", action="store_true",
                    help="also time each op isolated after a cache sweep")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", default=None, help="comma list of step ops")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the ops timed outside the step")
    ap.add_argument("--no-decode", action="store_true",
                    help="skip the decode-size latency table")
    ap.add_argument("--no-shapes", action="store_true",
                    help="skip the per-op table at the other workload shapes")
    ap.add_argument("--shapes-only", default=None,
                    help="comma list of shape workloads (or 'all'): time only "
                         "those, print their table as the JSON line, no step")
    ap.add_argument("--ops", default=None,
                    help="with --shapes-only: comma list of the ops to time")
    ap.add_argument("--decode-only", action="store_true",
                    help="time only the decode-size table and print it")
    ap.add_argument("--same-size-copy", action="store_true",
                    help="with --shapes-only: also time the copy at each "
                         "shape's tensor size (on by default in the full run)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="with --shapes-only: also run one 64 MiB rn_copy (the "
                         "known-size kernel that calibrates byte counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the row-normalization path has no "
              "multi-GPU part; run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import rmsnorm_row_welford_amd as rn
    from rmsnorm_row_welford_amd import synth

    if not os.path.exists(rn.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.decode_only:
        print(json.dumps({"decode_us_per_call": decode_latency(rn, dev)}), flush=True)
        return
    if args.shapes_only:
        names = None if args.shapes_only == "all" else args.shapes_only.split(",")
        only = None if not args.ops else args.ops.split(",")
        if args.calib_copy:
            a = torch.ones(64 << 20, dtype=torch.uint8, device=dev)
            b = torch.empty_like(a)
            rn.copy(a, b)
            torch.cuda.synchronize()
            del a, b
        shapes = time_shapes(rn, dev, names, only_ops=only)
        if args.same_size_copy:
            same_size_ceilings(rn, dev, shapes)
        print(json.dumps({"shapes": shapes}), flush=True)
        return
    w = synth.WORKLOADS[WORKLOAD]
    N, H = w.N, w.H
    t0 = time.time()
    arr = synth.generate(w)
    log(f"inputs generated in {time.time() - t0:.1f}s")
    ops = list(OPS) if not args.only else args.only.split(",")
    extras = [] if (args.no_extras or args.only) else list(EXTRA_OPS)
    sets = Sets(rn, arr, w.eps, args.sets, dev, ops + extras)
    nbytes = alg_bytes(N, H, 2)

    step_ms, wall_ms = time_steps(sets, ops, args.steps, args.warmup)
    step_bytes = sum(nbytes[k] for k in ops)
    value = step_bytes / (step_ms * 1e-3) / 1e9
    log(f"step: {step_ms * 1e3:.1f} us, {value:.0f} GB/s "
        f"({100 * value / PEAK_GBS:.1f}% of peak)")

    per_op = {}
    K = max(12, 2 * args.sets)
    for k in ops + extras:
        us = time_op_graph(sets, k, K)
        us_eager, _ = time_op(sets, k, K)
        gbs = nbytes[k] / (us * 1e-6) / 1e9
        per_op[k] = {"us": round(us, 3), "us_eager": round(us_eager, 3),
                     "alg_bytes": nbytes[k], "GBps": round(gbs, 1),
                     "pct_peak": round(100 * gbs / PEAK_GBS, 2)}
        if k in extras:
            per_op[k]["in_step"] = False
        log(f"{k:18s} {us:8.2f} us  {gbs:7.0f} GB/s  {100 * gbs / PEAK_GBS:5.1f}% of peak")
    if "unfused_add_rms" in per_op and "fused_add_rms_fwd" in per_op:
        sp = per_op["unfused_add_rms"]["us"] / per_op["fused_add_rms_fwd"]["us"]
        per_op["unfused_add_rms"]["fused_speedup"] = round(sp, 3)
        log(f"fused add+RMSNorm vs unfused (add, then rms_fwd): {sp:.2f}x")
    if args.sweep:
        sweep = torch.ones(128 << 20, dtype=torch.float32, device=dev)  # 512 MiB
        for k in ops:
            us = time_op_swept(sets, k, 10, sweep)
            per_op[k]["us_isolated_swept"] = round(us, 3)
            log(f"{k:18s} isolated after sweep: {us:8.2f} us")
        del sweep

    del sets
    torch.cuda.empty_cache()
    decode = None
    if not (args.no_decode or args.only):
        decode = decode_latency(rn, dev)
        for k, v in decode.items():
            log(f"decode {k:28s} {v:7.2f} us per call (graph replay)")
    shapes = None
    if not (args.no_shapes or args.only):
        shapes = time_shapes(rn, dev)
    ceil = stream_ceilings(rn, dev)
    copy_gbs = ceil["copy"]["GBps"]
    annotate(rn, dev, per_op, N, H, w.dtype, w.wdtype, copy_gbs)
    for name, row in (shapes or {}).items():
        annotate(rn, dev, row, row["N"], row["H"], row["dtype"], row["param_dtype"],
                 copy_gbs)
    same_size_ceilings(rn, dev, shapes)
    for k, v in ceil.items():
        log(f"{k} stream ceiling {v['GBps']:.0f} GB/s ({100 * v['GBps'] / PEAK_GBS:.1f}% of peak)")

    dom = max(ops, key=lambda k: per_op[k]["us"])
    achieved = nbytes[dom] / (per_op[dom]["us"] * 1e-6) / 1e9
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_GBS,
            "unit": "GB/s", "frac": round(achieved / PEAK_GBS, 4),
            "traffic": counters_traffic(dom, f"{N}x{H}"),
            "kernel": dom, "alg_bytes_per_launch": nbytes[dom],
            "us_per_launch": per_op[dom]["us"]}

    out = {
        "metric": "achieved HBM GB/s (% of peak) and us, LN/RMSNorm fwd+bwd bf16 32768x1024",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": WORKLOAD, "N": N, "H": H, "ops": ops,
                   "cache": f"cold: {args.sets} rotating tensor sets",
                   "parallelism": "single GPU"},
        "pct_peak": round(100.0 * value / PEAK_GBS, 2),
        "per_op": per_op,
        "copy_ceiling_GBps": round(copy_gbs, 1),
        "stream_ceilings": ceil,
        "decode_us_per_call": decode,
        "shapes": shapes,
        "wall_ms_per_step": round(wall_ms, 5),
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle baseline ...")
        out["cpu_baseline"] = cpu_baseline(arr, w.eps)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
