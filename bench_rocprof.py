"""rocprofv3 helpers for bench.py: the copy-calibration workload and the summaries
kept under profiles/.

  python bench_rocprof.py copy [--mib 1024] [--reps 5]
      Runs a plain streaming kernel of known size on cuda:0: y = -x over float32
      tensors of --mib MiB (one read and one write of every byte, the traffic of
      a copy). Profiled with --pmc FETCH_SIZE / WRITE_SIZE it calibrates what
      those counters read per byte moved.

  python bench_rocprof.py kernels <rocprof_out_dir> --cmd "<command>" [--out FILE]
      Per-kernel duration table (calls, average, min, max, total) from a
      --kernel-trace run.

  python bench_rocprof.py traffic --fetch DIR --write DIR --copy-fetch DIR
      --copy-write DIR --kernel NAME --workload NAME --cmd "<cmds>" [--last N] [--out FILE]
      HBM bytes per launch of kernel NAME from two --pmc runs (FETCH_SIZE, then
      WRITE_SIZE), each scaled by the factor that the same counter shows for the
      copy workload (bytes moved / counter bytes). Writes JSON with the kernel
      source hash that bench.py checks before it reports the figure.

  python bench_rocprof.py counters <rocprof_out_dir> --cmd "<command>" [--last N] [--out FILE]
      Per-kernel averages of every counter of a --pmc run (all dispatches, and the
      last N of each kernel), with two derived figures: MFMA busy fraction (MFMA
      busy cycles over 1024 SIMDs x duration x the 2.4 GHz peak clock) and wait
      fraction (SQ_WAIT_ANY over SQ_WAVE_CYCLES).

The rocprofv3 output is its SQLite database (rocpd); only its `kernels` view
and `counters_collection` table are read.
"""
import argparse
import glob
import json
import os
import sqlite3
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))


def _dbs(d):
    out = sorted(glob.glob(os.path.join(d, "**", "*.db"), recursive=True))
    if not out:
        raise SystemExit(f"no rocprofv3 database under {d}")
    return out


def kernel_rows(d):
    """{kernel name: [durations in ns]} from a --kernel-trace run."""
    rows = {}
    for db in _dbs(d):
        con = sqlite3.connect(db)
        for name, dur in con.execute("select name, duration from kernels"):
            rows.setdefault(name, []).append(int(dur))
        con.close()
    return rows


def counter_rows(d, counter):
    """{kernel name: [value per dispatch, in dispatch order]} for one counter of a
    --pmc run."""
    rows = {}
    for db in _dbs(d):
        con = sqlite3.connect(db)
        q = ("select dispatch_id, kernel_name, sum(value) from counters_collection "
             "where counter_name = ? group by dispatch_id, kernel_name order by dispatch_id")
        for _, name, val in con.execute(q, (counter,)):
            rows.setdefault(name, []).append(float(val))
        con.close()
    return rows


def short(name, n=90):
    return name if len(name) <= n else name[:n - 3] + "..."


def cmd_copy(args):
    import torch

    n = args.mib * (1 << 20) // 4
    x = torch.randn(n, device="cuda:0")
    y = torch.empty_like(x)
    for _ in range(args.reps):
        torch.neg(x, out=y)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4,
                      "reps": args.reps}), flush=True)


def cmd_kernels(args):
    rows = kernel_rows(args.dir)
    lines = [f"# rocprofv3 kernel trace summary", f"command: {args.cmd}", "",
             f"{'kernel':90s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s} "
             f"{'total_ms':>10s}"]
    for name, d in sorted(rows.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"{short(name):90s} {len(d):6d} {sum(d) / len(d) / 1e3:10.1f} "
                     f"{min(d) / 1e3:10.1f} {max(d) / 1e3:10.1f} {sum(d) / 1e6:10.3f}")
    text = "\n".join(lines) + "\n"
    if args.out:
        with open(args.out, "w") as f:
            f.write(text)
    sys.stdout.write(text)


def _pick(rows, needle):
    hits = {k: v for k, v in rows.items() if needle in k}
    if len(hits) != 1:
        raise SystemExit(f"kernel {needle!r} matches {len(hits)} kernels: {list(hits)[:5]}")
    (name, vals), = hits.items()
    return name, vals


def cmd_traffic(args):
    sys.path.insert(0, ROOT)
    import bench

    kib = 1024.0
    _, cf = _pick(counter_rows(args.copy_fetch, "FETCH_SIZE"), args.copy_kernel)
    _, cw = _pick(counter_rows(args.copy_write, "WRITE_SIZE"), args.copy_kernel)
    copy_bytes = args.copy_mib * (1 << 20)
    f_factor = copy_bytes / (sum(cf) / len(cf) * kib)
    w_factor = copy_bytes / (sum(cw) / len(cw) * kib)
    name, kf = _pick(counter_rows(args.fetch, "FETCH_SIZE"), args.kernel)
    _, kw = _pick(counter_rows(args.write, "WRITE_SIZE"), args.kernel)
    if args.last:  # only the last dispatches (e.g. the calls bench.py times last)
        kf, kw = kf[-args.last:], kw[-args.last:]
    fetch = sum(kf) / len(kf) * kib * f_factor
    write = sum(kw) / len(kw) * kib * w_factor
    per_kernel = {}
    allw = counter_rows(args.write, "WRITE_SIZE")
    for kname, vals in counter_rows(args.fetch, "FETCH_SIZE").items():
        if "mk::" in kname and kname in allw:
            wv = allw[kname]
            per_kernel[short(kname, 70)] = {
                "fetch_bytes": round(sum(vals) / len(vals) * kib * f_factor),
                "write_bytes": round(sum(wv) / len(wv) * kib * w_factor)}
    out = {"kernel": name, "workload": args.workload, "kernel_sha": bench.kernel_sha(),
           "fetch_bytes_per_launch": round(fetch), "write_bytes_per_launch": round(write),
           "traffic_bytes_per_launch": round(fetch + write),
           "fetch_factor": round(f_factor, 4), "write_factor": round(w_factor, 4),
           "dispatches": {"fetch": len(kf), "write": len(kw)},
           "all_library_kernels": per_kernel,
           "copy_calibration": {"bytes_each_way": copy_bytes, "fetch_kib": sum(cf) / len(cf),
                                "write_kib": sum(cw) / len(cw)},
           "commands": args.cmd}
    text = json.dumps(out, indent=1) + "\n"
    if args.out:
        with open(args.out, "w") as f:
            f.write(text)
    sys.stdout.write(text)


def cmd_counters(args):
    per = {}  # kernel -> [(dispatch, {counter: value}, duration ns)]
    for db in _dbs(args.dir):
        con = sqlite3.connect(db)
        durs = dict(con.execute("select dispatch_id, duration from kernels"))
        vals = {}
        q = ("select dispatch_id, kernel_name, counter_name, sum(value) from counters_collection "
             "group by dispatch_id, kernel_name, counter_name order by dispatch_id")
        for did, name, cname, v in con.execute(q):
            vals.setdefault((did, name), {})[cname] = float(v)
        for (did, name), cs in sorted(vals.items()):
            per.setdefault(name, []).append((did, cs, durs.get(did, 0)))
        con.close()

    def summary(rows):
        n = len(rows)
        dur = sum(r[2] for r in rows) / n
        cs = {}
        for _, c, _ in rows:
            for k, v in c.items():
                cs[k] = cs.get(k, 0.0) + v / n
        out = {"dispatches": n, "avg_us": round(dur / 1e3, 1)}
        out.update({k: round(v) for k, v in sorted(cs.items())})
        if "SQ_VALU_MFMA_BUSY_CYCLES" in cs and dur > 0:
            out["mfma_busy_frac_at_2.4GHz"] = round(
                cs["SQ_VALU_MFMA_BUSY_CYCLES"] / (1024 * dur * 1e-9 * 2.4e9), 3)
        if cs.get("SQ_WAVE_CYCLES"):
            out["wait_frac"] = round(cs.get("SQ_WAIT_ANY", 0.0) / cs["SQ_WAVE_CYCLES"], 3)
        return out

    lines = ["# rocprofv3 counter summary", f"command: {args.cmd}", ""]
    for name, rows in sorted(per.items(), key=lambda kv: -sum(r[2] for r in kv[1])):
        if "mk::" not in name:
            continue
        lines.append(short(name, 100))
        lines.append(f"  all dispatches: {json.dumps(summary(rows))}")
        if args.last and len(rows) > args.last:
            lines.append(f"  last {args.last}: {json.dumps(summary(rows[-args.last:]))}")
    text = "\n".join(lines) + "\n"
    if args.out:
        with open(args.out, "w") as f:
            f.write(text)
    sys.stdout.write(text)


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    c = sub.add_parser("copy")
    c.add_argument("--mib", type=int, default=1024)
    c.add_argument("--reps", type=int, default=5)
    k = sub.add_parser("kernels")
    k.add_argument("dir")
    k.add_argument("--cmd", required=True)
    k.add_argument("--out")
    cn = sub.add_parser("counters")
    cn.add_argument("dir")
    cn.add_argument("--cmd", required=True)
    cn.add_argument("--last", type=int, default=4)
    cn.add_argument("--out")
    t = sub.add_parser("traffic")
    for a in ("--fetch", "--write", "--copy-fetch", "--copy-write", "--kernel", "--workload",
              "--cmd"):
        t.add_argument(a, required=True)
    t.add_argument("--copy-kernel", default="neg")
    t.add_argument("--copy-mib", type=int, default=1024)
    t.add_argument("--last", type=int, default=0,
                   help="use only the last N dispatches of the kernel")
    t.add_argument("--out")
    args = ap.parse_args()
    {"copy": cmd_copy, "kernels": cmd_kernels, "traffic": cmd_traffic,
     "counters": cmd_counters}[args.what](args)


if __name__ == "__main__":
    main()
