"""Summaries of rocprofv3 output databases (kernel trace, PMC counters) as short text.

    python -m rejection_sampling_verify_specdec_amd.profsum trace DB [--cmd "..."]
    python -m rejection_sampling_verify_specdec_amd.profsum sequence DB --match k_cycle_ --count 9
    python -m rejection_sampling_verify_specdec_amd.profsum traffic FETCH_DB WRITE_DB \
        --kernel k_cycle_stats --calib-kernel copyBuffer --calib-bytes N --alg-bytes A \
        [--json profiles/KERNEL_WORKLOAD_traffic.json --workload c2 --cmd "..."]

``trace`` prints count / average / min / max duration per kernel; ``sequence`` the last
dispatches matching a name, in launch order, with durations and gaps; ``counters`` the
average per dispatch of every counter of a --pmc run for the named kernels. ``traffic`` turns the
FETCH_SIZE and WRITE_SIZE counters (KiB per dispatch) of a kernel into HBM bytes per
launch, scaled by what the same counters read for a plain copy kernel of known size (the
largest dispatch of the calibration kernel: the copy of N bytes), and optionally writes
the JSON summary that bench.py reads, stamped with the hash of the kernel sources.
"""

import argparse
import hashlib
import json
import os
import sqlite3
import sys

CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")


def source_hash() -> str:
    """Hash of every kernel source file: counters taken on other sources do not apply."""
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        h.update(f.encode())
        h.update(open(os.path.join(CSRC, f), "rb").read())
    return h.hexdigest()[:16]


def _kernels(db):
    con = sqlite3.connect(db)
    return con.execute("select name, count(*), avg(end-start), min(end-start), max(end-start) "
                       "from kernels group by name order by sum(end-start) desc").fetchall()


def trace(db, cmd=None, top=12):
    out = []
    if cmd:
        out.append(f"command: {cmd}")
    out.append(f"{'kernel':64s} {'calls':>6s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s}")
    for name, n, avg, mn, mx in _kernels(db)[:top]:
        out.append(f"{name[:64]:64s} {n:6d} {avg / 1e3:9.2f} {mn / 1e3:9.2f} {mx / 1e3:9.2f}")
    return "\n".join(out)


def sequence(db, match, count, cmd=None):
    """The last `count` dispatches whose kernel name contains `match`, in launch order, with
    each one's duration and the idle gap before it (one cycle's launches, say)."""
    con = sqlite3.connect(db)
    rows = [r for r in con.execute("select name, start, end from kernels order by start")
            if match in r[0]][-count:]
    out = [f"command: {cmd}"] if cmd else []
    out.append(f"{'kernel':48s} {'dur_us':>9s} {'gap_us':>9s}")
    prev = None
    for name, s, e in rows:
        gap = (s - prev) / 1e3 if prev is not None else 0.0
        out.append(f"{name.split('(')[0][:48]:48s} {(e - s) / 1e3:9.2f} {gap:9.2f}")
        prev = e
    if rows:
        out.append(f"{'span':48s} {(rows[-1][2] - rows[0][1]) / 1e3:9.2f}")
    return "\n".join(out)


def _pmc(db, counter):
    """Per-dispatch counter values: list of (kernel name, value)."""
    con = sqlite3.connect(db)
    views = {r[0] for r in con.execute("select name from sqlite_master")}
    if "counters_collection" in views:
        cols = [c[1] for c in con.execute("pragma table_info(counters_collection)")]
        name_col = "kernel_name" if "kernel_name" in cols else "name"
        val_col = "value" if "value" in cols else "counter_value"
        cnt_col = "counter_name" if "counter_name" in cols else "counter"
        rows = con.execute(f"select {name_col}, dispatch_id, sum({val_col}) from counters_collection "
                           f"where {cnt_col} = ? group by dispatch_id", (counter,)).fetchall()
        return [(r[0], r[2]) for r in rows]
    raise RuntimeError("no counters_collection view in " + db)


def counters(db, kernels, cmd=None):
    """Average per dispatch of every counter in a --pmc database, for each kernel whose
    name contains one of `kernels`."""
    con = sqlite3.connect(db)
    cols = [c[1] for c in con.execute("pragma table_info(counters_collection)")]
    name_col = "kernel_name" if "kernel_name" in cols else "name"
    val_col = "value" if "value" in cols else "counter_value"
    cnt_col = "counter_name" if "counter_name" in cols else "counter"
    rows = con.execute(f"select {name_col}, dispatch_id, {cnt_col}, sum({val_col}) from "
                       f"counters_collection group by dispatch_id, {cnt_col}").fetchall()
    out = [f"command: {cmd}"] if cmd else []
    for key in kernels:
        per = {}
        for name, disp, cnt, val in rows:
            if key in name:
                per.setdefault(cnt, {})[disp] = val
        if not per:
            continue
        n = max(len(v) for v in per.values())
        out.append(f"{key}: {n} dispatches, average per dispatch")
        for cnt in sorted(per):
            v = per[cnt]
            out.append(f"  {cnt:24s} {sum(v.values()) / len(v):16.1f}")
    return "\n".join(out)


def traffic(fetch_db, write_db, kernel, calib_kernel, calib_bytes, alg_bytes=None):
    f = _pmc(fetch_db, "FETCH_SIZE")
    w = _pmc(write_db, "WRITE_SIZE")
    sel = lambda rows, key: [v for n, v in rows if key in n]
    cf, cw = sel(f, calib_kernel), sel(w, calib_kernel)
    kf, kw = sel(f, kernel), sel(w, kernel)
    if not (cf and cw and kf and kw):
        raise RuntimeError("kernel or calibration copy not found in the counter databases")
    # the copy reads and writes calib_bytes: KiB reported -> bytes scale factors
    sf = calib_bytes / (max(cf) * 1024.0)
    sw = calib_bytes / (max(cw) * 1024.0)
    fetch = sum(kf) / len(kf) * 1024.0 * sf
    write = sum(kw) / len(kw) * 1024.0 * sw
    lines = [f"kernel {kernel}: {len(kf)} dispatches",
             f"calibration copy {calib_kernel}: {calib_bytes} bytes read and written; "
             f"FETCH_SIZE scale {sf:.4f}, WRITE_SIZE scale {sw:.4f}",
             f"FETCH bytes/launch {fetch:.4e}", f"WRITE bytes/launch {write:.4e}",
             f"total HBM bytes/launch {fetch + write:.4e}"]
    if alg_bytes:
        lines.append(f"algorithmic bytes/launch {alg_bytes:.4e}  ratio {(fetch + write) / alg_bytes:.4f}")
    info = {"kernel": kernel, "dispatches": len(kf), "fetch_scale": sf, "write_scale": sw,
            "fetch_bytes_per_launch": fetch, "write_bytes_per_launch": write,
            "bytes_per_launch": fetch + write, "algorithmic_bytes_per_launch": alg_bytes}
    return "\n".join(lines), info


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    t = sub.add_parser("trace")
    t.add_argument("db")
    t.add_argument("--cmd")
    q = sub.add_parser("sequence")
    q.add_argument("db")
    q.add_argument("--match", default="sd::")
    q.add_argument("--count", type=int, default=20)
    q.add_argument("--cmd")
    c = sub.add_parser("counters")
    c.add_argument("db")
    c.add_argument("--kernel", action="append", required=True)
    c.add_argument("--cmd")
    p = sub.add_parser("traffic")
    p.add_argument("fetch_db")
    p.add_argument("write_db")
    p.add_argument("--kernel", required=True)
    p.add_argument("--calib-kernel", required=True)
    p.add_argument("--calib-bytes", type=float, required=True)
    p.add_argument("--alg-bytes", type=float)
    p.add_argument("--json", help="write the summary bench.py reads")
    p.add_argument("--workload")
    p.add_argument("--cmd", help="the profiling command, recorded in the JSON")
    a = ap.parse_args(argv)
    if a.what == "trace":
        print(trace(a.db, a.cmd))
    elif a.what == "sequence":
        print(sequence(a.db, a.match, a.count, a.cmd))
    elif a.what == "counters":
        print(counters(a.db, a.kernel, a.cmd))
    else:
        text, info = traffic(a.fetch_db, a.write_db, a.kernel, a.calib_kernel, a.calib_bytes,
                             a.alg_bytes)
        print(text)
        if a.json:
            info.update(workload=a.workload, command=a.cmd, source_sha256_16=source_hash())
            with open(a.json, "w") as f:
                json.dump(info, f, indent=1)
                f.write("\n")


if __name__ == "__main__":
    sys.exit(main())
