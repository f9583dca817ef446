"""Summaries of rocprofv3 output for profiles/.

  python -m rmsnorm_row_welford_amd.profsum trace <results.db> [title...]
      per-kernel call count and average/min/max duration (us) from a
      --kernel-trace database.
  python -m rmsnorm_row_welford_amd.profsum op <results.db> <op> [title...]
      one op of one shape (a trace of `bench.py --shapes-only W --ops OP`):
      each kernel's role (forward; backward kernel 1; backward kernel 2 or
      column sums; set-up: the forward that saves the backward's statistics,
      host copies), calls and median/average/min/max duration, and the
      op's device time per call: the sum of its kernels' medians.
  python -m rmsnorm_row_welford_amd.profsum pmc <results.db> [title...]
      per-kernel average counter value per dispatch from a --pmc database.
  python -m rmsnorm_row_welford_amd.profsum traffic <fetch.db> <write.db>
         <kernel-substring>[|<kernel-substring>...] <out.json> [calib-substring calib-bytes]
      HBM bytes per launch of each listed kernel (and their sum: the op's
      traffic per call; a pattern '=label' matches one kernel label exactly)
      from a FETCH_SIZE run and a
      WRITE_SIZE run (both KiB per dispatch), each scaled by what the same
      counter reads for the streaming copy kernel of known size
      (rn::copy16_kernel moving `calib-bytes` each way, 64 MiB by default:
      the size bench.py's stream ceilings and --calib-copy copy); written as JSON with
      a digest of the kernel sources it was measured on.
"""
import glob
import hashlib
import json
import os
import sqlite3
import sys

HERE = os.path.dirname(os.path.abspath(__file__))


def kernel_source_digest() -> str:
    """Digest of the HIP sources (csrc/*): counter figures are only valid
    for the kernels they were taken on."""
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(HERE, "csrc", "*"))):
        if os.path.isfile(p) and p.endswith((".h", ".hip")):
            h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def kernel_table(db: str):
    """Per kernel and launch shape (one template serves several row shapes,
    told apart by their grid): calls, average/min/max duration, share."""
    c = sqlite3.connect(db)
    rows = list(c.execute(
        "select name, grid_x / workgroup_x, grid_y, workgroup_x, count(*), "
        "avg(duration), min(duration), max(duration), sum(duration) from kernels "
        "group by name, grid_x, grid_y, workgroup_x order by sum(duration) desc"))
    tot = sum(r[8] for r in rows) or 1
    out = [f"{'kernel':90s} {'grid':>11s} {'wg':>5s} {'calls':>6s} {'avg_us':>9s} "
           f"{'min_us':>9s} {'max_us':>9s} {'pct':>6s}"]
    for name, gx, gy, wx, n, avg, mn, mx, s in rows:
        short = name if len(name) <= 90 else name[:87] + "..."
        grid = f"{gx}x{gy}"
        out.append(f"{short:90s} {grid:>11s} {wx:5d} {n:6d} {avg / 1e3:9.3f} "
                   f"{mn / 1e3:9.3f} {mx / 1e3:9.3f} {100 * s / tot:6.2f}")
    return out


def _role(name: str, op: str) -> str:
    """What a kernel is to `op` in a one-op trace."""
    bwd = op.endswith("_bwd")
    if any(k in name for k in ("bwd1_kernel", "bwd1_seg_kernel", "bwd_onchip_kernel",
                               "bwd_long_acc_kernel")):
        return "kernel 1" if bwd else "other"
    if "bwd2_" in name:
        return "kernel 2" if bwd else "other"
    if "bwd_colsum_kernel" in name:
        return "kernel 2 (column sums)" if bwd else "other"
    if any(k in name for k in ("fwd_kernel", "fwd_seg_kernel", "fwd_onchip_kernel",
                               "fwd_long_kernel")):
        return "set-up forward" if bwd else "forward"
    return "other"


def op_table(db: str, op: str):
    """Per kernel of a one-op trace: role, grid, calls, median/avg/min/max;
    then the op's device time per call (sum of the medians of its kernels)."""
    c = sqlite3.connect(db)
    rows = {}
    for name, gx, gy, wx, d in c.execute(
            "select name, grid_x / workgroup_x, grid_y, workgroup_x, duration from kernels"):
        rows.setdefault((name, gx, gy, wx), []).append(d / 1e3)
    out = [f"{'role':24s} {'kernel':80s} {'grid':>9s} {'wg':>5s} {'calls':>6s} "
           f"{'median':>8s} {'avg':>8s} {'min':>8s} {'max':>8s}"]
    total = 0.0
    for (name, gx, gy, wx), ds in sorted(rows.items(), key=lambda kv: -sum(kv[1])):
        role = _role(name, op)
        ds.sort()
        med = ds[len(ds) // 2] if len(ds) % 2 else 0.5 * (ds[len(ds) // 2 - 1] + ds[len(ds) // 2])
        if role in ("forward", "kernel 1", "kernel 2", "kernel 2 (column sums)"):
            total += med
        short = name if len(name) <= 80 else name[:77] + "..."
        out.append(f"{role:24s} {short:80s} {f'{gx}x{gy}':>9s} {wx:5d} {len(ds):6d} "
                   f"{med:8.3f} {sum(ds) / len(ds):8.3f} {ds[0]:8.3f} {ds[-1]:8.3f}")
    out.append(f"{op}: device time per call (sum of its kernels' medians) {total:.3f} us")
    return out, total


def _pmc_rows(db: str):
    """(kernel label, counter, dispatches, average per dispatch); a kernel
    launched with a 2-D grid (kernel 2 of LayerNorm: dgamma and dbeta) is
    labelled with its grid's y extent."""
    c = sqlite3.connect(db)
    cols = [r[1] for r in c.execute("pragma table_info(counters_collection)")]
    name_col = "kernel_name" if "kernel_name" in cols else "name"
    gy = "grid_size_y" if "grid_size_y" in cols else "1"
    q = (f"select {name_col}, {gy}, counter_name, count(distinct dispatch_id), "
         f"sum(value) / count(distinct dispatch_id) from counters_collection "
         f"group by {name_col}, {gy}, counter_name")
    out = []
    for name, y, cn, nd, v in c.execute(q):
        label = name if (y in (None, 1, "1")) else f"{name} [grid.y {y}]"
        out.append((label, cn, nd, v))
    return out


def pmc_table(db: str):
    out = [f"{'kernel':90s} {'counter':>14s} {'dispatches':>10s} {'avg_per_dispatch':>18s}"]
    for name, cn, nd, v in sorted(_pmc_rows(db)):
        short = name if len(name) <= 90 else name[:87] + "..."
        out.append(f"{short:90s} {cn:>14s} {nd:10d} {v:18.1f}")
    return out


def _counter(db, counter, substr):
    """Average per dispatch over the kernels whose label contains `substr`,
    or, for a pattern starting with '=', whose label is exactly the rest
    (LayerNorm's and RMSNorm's kernel 2 share a name and differ only by the
    grid suffix of the label)."""
    if substr.startswith("="):
        vals = [(n, nd, v) for n, cn, nd, v in _pmc_rows(db)
                if cn == counter and n == substr[1:]]
    else:
        vals = [(n, nd, v) for n, cn, nd, v in _pmc_rows(db)
                if cn == counter and substr in n]
    if not vals:
        raise SystemExit(f"no {counter} rows for kernels matching {substr!r} in {db}")
    tot_d = sum(nd for _, nd, _ in vals)
    return sum(nd * v for _, nd, v in vals) / tot_d, tot_d


def traffic(fetch_db, write_db, substr, out_json, calib="copy16_kernel",
            calib_bytes=64 << 20):
    """Bytes per launch of the kernels matching each of the substrings in
    `substr` (one string, or a list for an op made of several kernels, one
    launch each per call), their sum as the op's traffic per call."""
    subs = [substr] if isinstance(substr, str) else list(substr)
    f_c, _ = _counter(fetch_db, "FETCH_SIZE", calib)
    w_c, _ = _counter(write_db, "WRITE_SIZE", calib)
    f_scale = calib_bytes / f_c        # bytes per counter unit
    w_scale = calib_bytes / w_c
    kernels = []
    for sub in subs:
        f_k, nf = _counter(fetch_db, "FETCH_SIZE", sub)
        w_k, nw = _counter(write_db, "WRITE_SIZE", sub)
        kernels.append({"kernel_substring": sub,
                        "dispatches": {"fetch": nf, "write": nw},
                        "FETCH_SIZE_per_dispatch": f_k,
                        "WRITE_SIZE_per_dispatch": w_k,
                        "fetch_bytes_per_launch": f_k * f_scale,
                        "write_bytes_per_launch": w_k * w_scale})
    d = {
        "kernels": kernels,
        "calibration": {"kernel": calib, "bytes_each_way": calib_bytes,
                        "FETCH_SIZE": f_c, "WRITE_SIZE": w_c,
                        "fetch_bytes_per_unit": f_scale,
                        "write_bytes_per_unit": w_scale},
        "fetch_bytes_per_launch": sum(k["fetch_bytes_per_launch"] for k in kernels),
        "write_bytes_per_launch": sum(k["write_bytes_per_launch"] for k in kernels),
        "kernel_source_digest": kernel_source_digest(),
    }
    d["traffic_bytes_per_launch"] = d["fetch_bytes_per_launch"] + d["write_bytes_per_launch"]
    if len(kernels) == 1:      # the single-kernel form bench.py's roofline reads
        d["kernel_substring"] = subs[0]
    with open(out_json, "w") as fh:
        json.dump(d, fh, indent=1)
    return d


def main(argv):
    mode = argv[1]
    if mode == "traffic":
        # traffic <fetch.db> <write.db> <kernel-substring>[|substring...] <out.json>
        #         [calib-substring calib-bytes]
        extra = argv[6:]
        d = traffic(argv[2], argv[3], argv[4].split("|"), argv[5],
                    *(extra[:1]), *([int(extra[1])] if len(extra) > 1 else []))
        print(json.dumps(d, indent=1))
        return
    db = argv[2]
    if mode == "op":
        title = " ".join(argv[4:])
        lines = [f"# {title}"] if title else []
        lines += op_table(db, argv[3])[0]
        print("\n".join(lines))
        return
    title = " ".join(argv[3:])
    lines = [f"# {title}"] if title else []
    lines += kernel_table(db) if mode == "trace" else pmc_table(db)
    print("\n".join(lines))


if __name__ == "__main__":
    main(sys.argv)
