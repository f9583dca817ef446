"""Summarize rocprofv3 output (a rocpd SQLite database from --kernel-trace,
or one from a --pmc counter run) into the short text tables kept under
profiles/.

  python -m rmsnorm_row_welford_amd.profsum trace <run_results.db> [title...]
  python -m rmsnorm_row_welford_amd.profsum pmc <run_results.db> [title...]
"""
import sqlite3
import sys


def kernel_table(db: str):
    c = sqlite3.connect(db)
    rows = list(c.execute(
        "select name, count(*), avg(duration), min(duration), max(duration), "
        "sum(duration) from kernels group by name order by sum(duration) desc"))
    tot = sum(r[5] for r in rows) or 1
    out = [f"{'kernel':90s} {'calls':>6s} {'avg_us':>9s} {'min_us':>9s} "
           f"{'max_us':>9s} {'pct':>6s}"]
    for name, n, avg, mn, mx, s in rows:
        short = name if len(name) <= 90 else name[:87] + "..."
        out.append(f"{short:90s} {n:6d} {avg / 1e3:9.3f} {mn / 1e3:9.3f} "
                   f"{mx / 1e3:9.3f} {100 * s / tot:6.2f}")
    return out


def pmc_table(db: str):
    """Per kernel name: counter -> average value per dispatch."""
    c = sqlite3.connect(db)
    cols = [r[1] for r in c.execute("pragma table_info(counters_collection)")]
    name_col = "kernel_name" if "kernel_name" in cols else "name"
    q = (f"select {name_col}, counter_name, count(distinct dispatch_id), "
         f"sum(value) / count(distinct dispatch_id) from counters_collection "
         f"group by {name_col}, counter_name order by {name_col}, counter_name")
    out = [f"{'kernel':90s} {'counter':>14s} {'dispatches':>10s} {'avg_per_dispatch':>18s}"]
    for name, cn, nd, v in c.execute(q):
        short = name if len(name) <= 90 else name[:87] + "..."
        out.append(f"{short:90s} {cn:>14s} {nd:10d} {v:18.1f}")
    return out


def main(argv):
    mode, db = argv[1], argv[2]
    title = " ".join(argv[3:])
    lines = [f"# {title}"] if title else []
    lines += kernel_table(db) if mode == "trace" else pmc_table(db)
    print("\n".join(lines))


if __name__ == "__main__":
    main(sys.argv)
